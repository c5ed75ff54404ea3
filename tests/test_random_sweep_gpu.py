"""Seeded random sweeps of every entry point against the oracle: forward
(all three types, random scale), split-K/V (automatic and given chunk
counts), backward and the FP8 path (random block sizes), each case a random
draw of type, head size, mask, batch, heads, length and input spread within
the range where its bar holds (fp32 at scores of moderate size; FP8 with
Q, K spreads up to 3).  Every case names itself before it touches the GPU."""
import math
import random

import numpy as np
import pytest

import fa_inputs as gen
import oracle
from parity_util import compare, run_gpu, say
from test_bwd_gpu import compare_grads, run_bwd
from test_fp8_gpu import _gpu_fwd_fp8, _gpu_quantize, compare_fp8, lse_tolerance
from test_splitkv_gpu import _inputs, _run_splitkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import io_aware_tiled_02_amd as fa
    fa.load()


def _cases(kind, n, seed):
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        d = rng.choice([64, 128])
        causal = rng.choice([0, 1])
        s = rng.randint(0, 10 ** 6)
        if kind == "fwd":
            dtype = rng.choice([gen.BF16, gen.F16, gen.F32])
            L = rng.choice([rng.randint(1, 300), rng.randint(300, 2000)])
            B, H = rng.randint(1, 2), rng.randint(1, 6)
            sigma = rng.choice([0.5, 1.0, 2.0]) if dtype == gen.F32 else rng.choice([0.5, 1.0, 2.0, 3.0])
            scale = rng.choice([1.0 / math.sqrt(d), rng.uniform(0.02, 0.3)])
            out.append((dtype, d, causal, B, H, L, sigma, round(scale, 5), s))
        elif kind == "splitkv":
            dtype = rng.choice([gen.BF16, gen.F16, gen.F32])
            B, H, Lq = rng.randint(1, 3), rng.randint(1, 12), rng.randint(1, 8)
            Lk = rng.choice([rng.randint(1, 300), rng.randint(300, 30000)])
            nsplit = rng.choice([0, 0, rng.randint(1, 48)])
            sigma = rng.choice([1.0, 3.0])
            scale = rng.choice([1.0 / math.sqrt(d), rng.uniform(0.02, 0.3)])
            out.append((dtype, d, B, H, Lq, Lk, nsplit, sigma, round(scale, 5), s))
        elif kind == "bwd":
            dtype = rng.choice([gen.BF16, gen.F16])
            L = rng.choice([rng.randint(1, 200), rng.randint(200, 900)])
            B, H = rng.randint(1, 2), rng.randint(1, 4)
            sigma = rng.choice([1.0, 2.0])
            out.append((dtype, d, causal, B, H, L, sigma, s))
        else:
            dtype = rng.choice([gen.BF16, gen.F16])
            L = rng.choice([rng.randint(1, 200), rng.randint(200, 1500)])
            B, H = rng.randint(1, 2), rng.randint(1, 6)
            bq = rng.choice([1, 128, rng.randint(1, 400)])
            bk = 32 * rng.randint(1, 10)
            sigma = rng.choice([0.5, 1.0, 3.0])
            scale = rng.choice([1.0 / math.sqrt(d), rng.uniform(0.02, 0.3)])
            out.append((dtype, d, causal, B, H, L, bq, bk, sigma, round(scale, 5), s))
    return out


@pytest.mark.parametrize("case", _cases("fwd", 24, 71))
def test_random_forward(case):
    dtype, d, causal, B, H, L, sigma, scale, s = case
    say(f"[sweep-fwd] {case}")
    shape = (B, H, L, d)
    q, k, v = gen.fill(dtype, shape, s, 0, sigma), gen.fill(dtype, shape, s, 1, sigma), gen.fill(dtype, shape, s, 2)
    o, lse = run_gpu(q, k, v, dtype, scale, causal)
    o_ref, lse_ref = oracle.fwd(q, k, v, dtype, scale, causal)
    compare(o, lse, o_ref, lse_ref, dtype, f"sweep-fwd {case}")


@pytest.mark.parametrize("case", _cases("splitkv", 24, 72))
def test_random_splitkv(case):
    dtype, d, B, H, Lq, Lk, nsplit, sigma, scale, s = case
    say(f"[sweep-splitkv] {case}")
    q, k, v = _inputs(B, H, Lq, Lk, d, dtype, s, sigma)
    o, lse = _run_splitkv(q, k, v, dtype, scale, nsplit)
    o_ref, lse_ref = oracle.attn_range(q, k, v, dtype, scale, 0, Lk)
    compare(o, lse, o_ref, lse_ref, dtype, f"sweep-splitkv {case}")


@pytest.mark.parametrize("case", _cases("bwd", 16, 73))
def test_random_backward(case):
    dtype, d, causal, B, H, L, sigma, s = case
    say(f"[sweep-bwd] {case}")
    shape = (B, H, L, d)
    q, k = gen.fill(dtype, shape, s, 0, sigma), gen.fill(dtype, shape, s, 1, sigma)
    v, g = gen.fill(dtype, shape, s, 2), gen.fill(dtype, shape, s, 3)
    scale = 1.0 / math.sqrt(d)
    got = run_bwd(q, k, v, g, dtype, scale, causal)
    ref = oracle.bwd(q, k, v, g, dtype, scale, causal)
    compare_grads(got, ref, f"sweep-bwd {case}")


@pytest.mark.parametrize("case", _cases("fp8", 20, 74))
def test_random_fp8(case):
    dtype, d, causal, B, H, L, bq, bk, sigma, scale, s = case
    say(f"[sweep-fp8] {case}")
    shape = (B, H, L, d)
    q, k, v = gen.fill(dtype, shape, s, 0, sigma), gen.fill(dtype, shape, s, 1, sigma), gen.fill(dtype, shape, s, 2)
    g8, gs = _gpu_quantize(q, dtype, bq)
    q8, sq = oracle.quantize_fp8(q, dtype, bq)
    assert np.array_equal(gs.view(np.uint32), sq.view(np.uint32)), "scales differ"
    assert np.count_nonzero(g8 != q8) == 0, "codes differ"
    k8, sk = oracle.quantize_fp8(k, dtype, bk)
    o, lse = _gpu_fwd_fp8(q8, k8, sq, sk, v, dtype, scale, causal, bq, bk)
    o_ref, lse_ref = oracle.fwd_fp8(q8, k8, sq, sk, v, dtype, scale, causal, bq, bk)
    compare_fp8(o, lse, o_ref, lse_ref, lse_tolerance(d, scale, sq, sk), f"sweep-fp8 {case}")
