"""GPU parity at the size limits of each entry point.

* grid limits: the forward and backward passes put (B*H, row block) on one
  grid dimension and take B*H beyond 65535; split-K/V and the FP8 quantiser
  put B*H on the second grid dimension, whose limit (65535) they accept
  exactly;
* a long sequence: L = 65536 in one head, non-causal and causal, checked on
  sampled rows (the first, the last and rows across the range).
Every case names itself before it touches the GPU.
"""
import numpy as np
import pytest

import fa_inputs as gen
import oracle
from parity_util import compare, run_gpu, say
from test_bwd_gpu import compare_grads, run_bwd
from test_fp8_gpu import _gpu_fwd_fp8, _gpu_quantize, compare_fp8, lse_tolerance
from test_splitkv_gpu import _run_splitkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import io_aware_tiled_02_amd as fa
    fa.load()


def _qkv(shape, seed, dtype=gen.BF16):
    return tuple(gen.fill(dtype, shape, seed, s) for s in range(3))


@pytest.mark.parametrize("causal", [0, 1])
def test_forward_beyond_65535_heads(causal):
    shape = (3, 21846, 3, 64)                     # B*H = 65538
    say(f"[limits] fa_fwd B*H=65538 L=3 d=64 causal={causal}")
    q, k, v = _qkv(shape, 61)
    o, lse = run_gpu(q, k, v, gen.BF16, 0.125, causal)
    o_ref, lse_ref = oracle.fwd(q, k, v, gen.BF16, 0.125, causal)
    compare(o, lse, o_ref, lse_ref, gen.BF16, "B*H=65538")


@pytest.mark.parametrize("dtype,d,causal", [(gen.BF16, 64, 0), (gen.BF16, 64, 1), (gen.F16, 128, 1)])
def test_forward_long_sequence(dtype, d, causal):
    L = 65536
    say(f"[limits] fa_fwd L={L} d={d} dtype={gen.DTYPE_NAMES[dtype]} causal={causal}")
    q, k, v = _qkv((1, 1, L, d), 62 + d, dtype)
    o, lse = run_gpu(q, k, v, dtype, d ** -0.5, causal)
    rows = np.unique(np.concatenate([[0, 1, L // 2, L - 1], gen.sample_rows(L, 12, 62)])).astype(np.int32)
    o_ref, lse_ref = oracle.fwd(q, k, v, dtype, d ** -0.5, causal, rows)
    compare(o[:, :, rows], lse[:, :, rows], o_ref, lse_ref, dtype, f"L={L}")


@pytest.mark.parametrize("causal", [0, 1])
def test_backward_beyond_65535_heads(causal):
    shape = (3, 21846, 3, 64)                     # B*H = 65538
    say(f"[limits] fa_bwd B*H=65538 L=3 d=64 causal={causal}")
    q, k, v = _qkv(shape, 63)
    g = gen.fill(gen.BF16, shape, 63, 3)
    got = run_bwd(q, k, v, g, gen.BF16, 0.125, causal)
    ref = oracle.bwd(q, k, v, g, gen.BF16, 0.125, causal)
    compare_grads(got, ref, "B*H=65538")


def test_splitkv_65535_heads():
    say("[limits] fa_fwd_splitkv B*H=65535 Lq=1 Lk=5 d=64")
    q = gen.fill(gen.BF16, (5, 13107, 1, 64), 64, 0)
    k = gen.fill(gen.BF16, (5, 13107, 5, 64), 64, 1)
    v = gen.fill(gen.BF16, (5, 13107, 5, 64), 64, 2)
    o, lse = _run_splitkv(q, k, v, gen.BF16, 0.125, 2)
    o_ref, lse_ref = oracle.attn_range(q, k, v, gen.BF16, 0.125, 0, 5)
    compare(o, lse, o_ref, lse_ref, gen.BF16, "splitkv B*H=65535")


def test_fp8_65535_heads():
    shape = (5, 13107, 2, 64)
    say("[limits] fa_quantize_fp8 + fa_fwd_fp8 B*H=65535 L=2 d=64")
    q, k, v = _qkv(shape, 65)
    g8, gs = _gpu_quantize(q, gen.BF16, 1)
    r8, rs = oracle.quantize_fp8(q, gen.BF16, 1)
    assert np.array_equal(g8, r8) and np.array_equal(gs.view(np.uint32), rs.view(np.uint32))
    k8, sk = oracle.quantize_fp8(k, gen.BF16, 32)
    o, lse = _gpu_fwd_fp8(r8, k8, rs, sk, v, gen.BF16, 0.125, 1, 1, 32)
    o_ref, lse_ref = oracle.fwd_fp8(r8, k8, rs, sk, v, gen.BF16, 0.125, 1, 1, 32)
    compare_fp8(o, lse, o_ref, lse_ref, lse_tolerance(64, 0.125, rs, sk), "fp8 B*H=65535")
