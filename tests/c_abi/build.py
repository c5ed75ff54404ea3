"""Compile fa_c_check (plain C, gcc) against include/fa.h, the built library,
the C input generator and the C oracle; the binary sits next to this file."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BIN = os.path.join(HERE, "fa_c_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    lib_dir = os.path.join(ROOT, "io_aware_tiled_02_amd")
    oracle_dir = os.path.join(ROOT, "oracle")
    gen_dir = os.path.join(ROOT, "fa_inputs")
    tmp = BIN + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROOT, "include"), "-I" + oracle_dir, "-I" + os.path.join(ROCM, "include"),
           os.path.join(HERE, "fa_c_check.c"), "-o", tmp,
           "-L" + lib_dir, "-l:libfa_fwd.so", "-L" + oracle_dir, "-l:liboracle.so",
           "-L" + gen_dir, "-l:libfa_gen.so",
           "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           # the libraries are found next to the binary's tree wherever it is copied
           "-Wl,-rpath,$ORIGIN/../../io_aware_tiled_02_amd:$ORIGIN/../../oracle:$ORIGIN/../../fa_inputs:"
           + os.path.join(ROCM, "lib")]
    subprocess.run(cmd, check=True)
    os.replace(tmp, BIN)
    return BIN


if __name__ == "__main__":
    print(build())
