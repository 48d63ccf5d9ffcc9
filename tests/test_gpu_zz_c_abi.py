"""liblsec.so driven from plain C (tests/c_abi/c_abi_check.c): hipMalloc'd
buffers, the seeded generator and the CPU oracle linked as C libraries, no
Python or PyTorch in the process. __graft_entry__.build() compiles it."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c_abi", "c_abi_check")


@pytest.mark.gpu
def test_c_consumer_of_the_c_abi():
    assert os.path.exists(BIN), "tests/c_abi/c_abi_check is missing: run __graft_entry__.build()"
    print("[case] c_abi_check", flush=True)
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(res.stdout)
    print(res.stderr)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "c_abi_check: ok" in res.stdout
