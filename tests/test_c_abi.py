"""The library used from plain C (tests/c_abi/fa_c_check.c, built by
__graft_entry__.build() with gcc against include/fa.h): argument errors on
the CPU, and fa_fwd on bf16 and fp32 shapes against the oracle on the GPU.
The program runs as a child process with its own time limit."""
import os
import subprocess

import pytest

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "fa_c_check")


def _run(*args, timeout):
    if not os.path.exists(BIN):
        pytest.fail("tests/c_abi/fa_c_check is not built: run __graft_entry__.build()")
    res = subprocess.run([BIN, *args], capture_output=True, text=True, timeout=timeout)
    print(res.stdout, res.stderr, flush=True)
    return res


def test_c_argument_errors():
    res = _run("args", timeout=60)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "null pointers -> -1" in res.stdout and "d = 96 -> -2" in res.stdout


@pytest.mark.gpu
def test_c_forward_parity():
    print("[c-abi] fa_c_check: bf16 (1,2,300,128) causal, bf16 (2,3,129,64), fp32 (1,1,77,64)", flush=True)
    res = _run(timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "all cases passed" in res.stdout
