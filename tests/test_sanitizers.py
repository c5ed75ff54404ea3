"""The C parts of the test infrastructure -- the fp64 oracle (oracle/fa_oracle.c)
and the input generator (fa_inputs/fa_gen.c) -- built with gcc's
AddressSanitizer and UndefinedBehaviorSanitizer (host code only) and run
under the CPU pin tests of both.  Any out-of-bounds access, use after free
or undefined behaviour (signed overflow, bad shift, misaligned access...)
aborts the run and fails this test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_TESTS = ["tests/test_oracle_pins.py", "tests/test_oracle_splitkv.py", "tests/test_oracle_bwd.py",
             "tests/test_oracle_fp8.py", "tests/test_inputs.py"]

PLUGIN = '''
import os
import fa_inputs
import oracle
# route both packages to the sanitized builds before their first call
oracle._LIB_PATH = os.environ["FA_SAN_ORACLE"]
fa_inputs.LIB_PATH = os.environ["FA_SAN_GEN"]
assert oracle._lib is None and fa_inputs._lib is None
'''


def _gcc_lib(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.mark.skipif(_gcc_lib("libasan.so") is None, reason="gcc's AddressSanitizer runtime is not installed")
def test_oracle_and_generator_under_asan_ubsan(tmp_path):
    flags = ["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
             "-I" + os.path.join(ROOT, "include")]
    libs = {}
    for key, src in (("FA_SAN_ORACLE", "oracle/fa_oracle.c"), ("FA_SAN_GEN", "fa_inputs/fa_gen.c")):
        out = str(tmp_path / (os.path.basename(src)[:-2] + "_san.so"))
        subprocess.run(flags + ["-o", out, os.path.join(ROOT, src), "-lm"], check=True)
        libs[key] = out
    (tmp_path / "fa_san_plugin.py").write_text(PLUGIN)
    env = dict(os.environ, **libs)
    env["LD_PRELOAD"] = _gcc_lib("libasan.so")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["PYTHONPATH"] = os.pathsep.join([str(tmp_path), ROOT, env.get("PYTHONPATH", "")])
    env["OMP_NUM_THREADS"] = "4"
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "fa_san_plugin",
                          "-p", "no:cacheprovider", *PIN_TESTS], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=900)
    report = (res.stdout + res.stderr)[-4000:]
    assert "AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, report
    assert res.returncode == 0, report
    assert " passed" in res.stdout, report
