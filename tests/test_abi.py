"""The C-ABI library: it loads, exports what include/*.h declares, and rejects
bad arguments on the host before anything is enqueued (no GPU needed: every
call here returns before the first HIP call)."""
import glob
import os
import re

import pytest

import io_aware_tiled_02_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b(fa_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_function():
    lib = fa.load()
    names = _declared_functions()
    assert {"fa_fwd", "fa_strerror", "fa_last_hip_error", "fa_fwd_tiling"} <= names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"


def test_strerror_total():
    for code in (0, -1, -2, -3, -4, 7):
        assert isinstance(fa.fa_strerror(code), str) and fa.fa_strerror(code)


A = 1 << 20   # a fake 16-byte-aligned address: never dereferenced, the call fails first


@pytest.mark.parametrize("args,want", [
    ((0, A, A, A, A, 1, 1, 64, 64, 0.125, 0, 2), fa.FA_ERR_INVALID_ARG),   # null q
    ((A, A, A, A, 0, 1, 1, 64, 64, 0.125, 0, 2), fa.FA_ERR_INVALID_ARG),   # null lse
    ((A, A, A, A, A, 0, 1, 64, 64, 0.125, 0, 2), fa.FA_ERR_INVALID_ARG),   # B = 0
    ((A, A, A, A, A, 1, -1, 64, 64, 0.125, 0, 2), fa.FA_ERR_INVALID_ARG),  # H < 0
    ((A, A, A, A, A, 1, 1, 0, 64, 0.125, 0, 2), fa.FA_ERR_INVALID_ARG),    # L = 0
    ((A, A, A, A, A, 1, 1, 64, 64, 0.0, 0, 2), fa.FA_ERR_INVALID_ARG),     # scale 0
    ((A, A, A, A, A, 1, 1, 64, 64, -1.0, 0, 2), fa.FA_ERR_INVALID_ARG),    # scale < 0
    ((A, A, A, A, A, 1, 1, 64, 64, float("nan"), 0, 2), fa.FA_ERR_INVALID_ARG),
    ((A, A, A, A, A, 1, 1, 64, 64, float("inf"), 0, 2), fa.FA_ERR_INVALID_ARG),
    ((A, A, A, A, A, 1, 1, 64, 64, 0.125, 2, 2), fa.FA_ERR_INVALID_ARG),   # causal 2
    ((A, A, A, A, A, 1, 1, 64, 96, 0.125, 0, 2), fa.FA_ERR_UNSUPPORTED),   # d = 96
    ((A, A, A, A, A, 1, 1, 64, 256, 0.125, 0, 2), fa.FA_ERR_UNSUPPORTED),  # d = 256
    ((A, A, A, A, A, 1, 1, 64, 64, 0.125, 0, 3), fa.FA_ERR_UNSUPPORTED),   # dtype 3
    ((A, A, A, A, A, 1, 1, 64, 64, 0.125, 0, -1), fa.FA_ERR_UNSUPPORTED),
    ((A + 8, A, A, A, A, 1, 1, 64, 64, 0.125, 0, 2), fa.FA_ERR_ALIGN),     # q misaligned
    ((A, A, A, A + 2, A, 1, 1, 64, 64, 0.125, 0, 2), fa.FA_ERR_ALIGN),     # o misaligned
    ((A, A, A, A, A + 2, 1, 1, 64, 64, 0.125, 0, 2), fa.FA_ERR_ALIGN),     # lse misaligned
    ((A, A, A, A, A, 65536, 65536, 1 << 30, 128, 0.125, 0, 2), fa.FA_ERR_INVALID_ARG),  # overflow
])
def test_argument_errors(args, want):
    assert fa.fa_fwd(*args, 0) == want


def test_tiling_query():
    br, bc, wg = fa.fa_fwd_tiling(1, 32, 8192, 128, 0, fa.FA_BF16)
    assert br > 0 and bc > 0 and br % 32 == 0 and bc % 32 == 0
    assert wg == 32 * ((8192 + br - 1) // br)
    with pytest.raises(fa.FAError):
        fa.fa_fwd_tiling(1, 1, 64, 80, 0, fa.FA_BF16)
