"""Build step for liblsec.so (hipcc, gfx950) -- run from ``__graft_entry__.build()``."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblsec.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


# Translation units: the main one (row / element / corrected-partial / pack /
# unpack kernels, the host code and the C ABI), the measurement aids of
# lsec_floor.h, and the tiled combine once per element type (it holds most of
# the kernel instantiations). They compile in
# parallel and link into one shared library.
UNITS = [("lsec", os.path.join(PKG, "csrc", "lsec.hip"), []),
         ("lsec_floor", os.path.join(PKG, "csrc", "lsec_floor.hip"), [])] + [
    (f"lsec_tiled_{name}", os.path.join(PKG, "csrc", "lsec_tiled.hip"), [f"-DLSEC_TILED_DT={dt}"])
    for name, dt in (("bf16", 0), ("fp16", 1), ("fp32", 2))
]
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         "-I", INCLUDE, "-I", os.path.join(PKG, "csrc"),
         # packed fp32 VALU ops stay off (see the note at the top of lsec.hip)
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def build(verbose: bool = False) -> str:
    """Compile the csrc/ units into liblsec.so for gfx950 (always recompiles)."""
    import tempfile
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="lsec_build_") as tmp:
        procs = []
        objs = []
        for name, src, extra in UNITS:
            obj = os.path.join(tmp, name + ".o")
            objs.append(obj)
            procs.append((name, subprocess.Popen([cc] + FLAGS + extra + ["-c", "-o", obj, src],
                                                 stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                                 text=True)))
        errors = []
        for name, p in procs:
            out, err = p.communicate()
            if p.returncode != 0:
                errors.append(f"{name}: hipcc failed ({p.returncode}):\n{err}")
            elif verbose and err:
                print(err)
        if errors:
            raise RuntimeError("\n".join(errors))
        res = subprocess.run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", LIB + ".tmp"]
                             + objs, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed ({res.returncode}):\n{res.stderr}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
