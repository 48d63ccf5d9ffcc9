"""The CPU code under AddressSanitizer and UndefinedBehaviorSanitizer: the
oracle (oracle/oracle.c) and the seeded generator (synth/synth.c) are built
with -fsanitize=address,undefined, and the oracle's pins and the generator's
tests run against those builds in a child process with the sanitizer
runtimes preloaded. Any out-of-bounds access, use after free or undefined
behaviour stops the child with an error. The plain-C consumer of the C ABI
(tests/c_abi/c_abi_check.c) is built the same way against them (it needs a
GPU to run)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=undefined"]


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                          check=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    d = tmp_path_factory.mktemp("san")
    libs = {}
    for name, src, extra in (("oracle", "oracle/oracle.c", ["-lm"]),
                             ("synth", "synth/synth.c", ["-lm", "-lpthread"])):
        out = str(d / f"lib{name}_san.so")
        subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC"] + SAN +
                       ["-o", out, os.path.join(ROOT, src)] + extra, check=True)
        libs[name] = out
    # reports go to files: pytest captures the child's stderr, and a process
    # that the sanitizer stops never prints what pytest captured
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS=f"detect_leaks=0:exitcode=86:log_path={d}/asan",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:exitcode=87:log_path={d}/ubsan",
               LSEC_ORACLE_LIB=libs["oracle"], LSEC_SYNTH_LIB=libs["synth"])
    return d, libs, env


def _reports(d):
    out = ""
    for n in sorted(os.listdir(d)):
        if n.startswith(("asan", "ubsan")):
            with open(os.path.join(d, n)) as f:
                out += f"--- {n}\n" + f.read()[:6000]
    return out


def _run_pins(env, *select):
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                           "-m", "not gpu"] + list(select), cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=900)


def test_sanitized_builds_are_the_ones_loaded(sanitized):
    _, libs, env = sanitized
    code = ("import oracle, synth; oracle._load(); synth._load(); "
            "print(open('/proc/self/maps').read())")
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-3000:]
    assert libs["oracle"] in res.stdout and libs["synth"] in res.stdout
    assert "libasan" in res.stdout


def test_oracle_pins_and_generator_under_sanitizers(sanitized):
    d, _, env = sanitized
    res = _run_pins(env, "tests/test_oracle.py", "tests/test_synth.py")
    tail = (res.stdout + res.stderr)[-3000:]
    assert res.returncode == 0, tail + _reports(d)
    assert " passed" in res.stdout and not _reports(d), tail + _reports(d)


def test_sanitizers_catch_a_planted_overflow(sanitized, tmp_path):
    """The harness has teeth: an oracle whose unpack writes each LSE one slot
    late (past the end of the array on the last row) stops the child with
    AddressSanitizer's exit status and report."""
    d, libs, env = sanitized
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    old = "memcpy(&lses[n * R + r], src + D * E, 4);"
    assert old in src
    bad = tmp_path / "oracle_bad.c"
    bad.write_text(src.replace(old, "memcpy(&lses[n * R + r + 1], src + D * E, 4);"))
    lib = str(tmp_path / "liboracle_bad.so")
    subprocess.run(["gcc", "-std=c11", "-shared", "-fPIC"] + SAN + ["-o", lib, str(bad), "-lm"],
                   check=True)
    logs = tmp_path / "logs"
    logs.mkdir()
    env = dict(env, LSEC_ORACLE_LIB=lib,
               ASAN_OPTIONS=f"detect_leaks=0:exitcode=86:log_path={logs}/asan")
    res = _run_pins(env, "tests/test_oracle.py", "-k", "pack_layout_and_round_trip")
    assert res.returncode == 86, res.stdout[-2000:]
    report = _reports(logs)
    assert "heap-buffer-overflow" in report and "oracle_unpack" in report, report


def test_c_consumer_builds_with_sanitizers(sanitized):
    d, libs, _ = sanitized
    lsec = os.path.join(ROOT, "lse_weighted_merge_combine_amd", "liblsec.so")
    if not os.path.exists(lsec):
        pytest.skip("liblsec.so is not built")
    out = str(d / "c_abi_check_san")
    res = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror"] + SAN +
                         ["-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                          "-I", "/opt/rocm/include",
                          "-o", out, os.path.join(ROOT, "tests", "c_abi", "c_abi_check.c"),
                          lsec, libs["oracle"], libs["synth"], "-L/opt/rocm/lib", "-lamdhip64",
                          "-lm", "-Wl,-rpath," + os.path.dirname(lsec)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    assert os.path.exists(out)
