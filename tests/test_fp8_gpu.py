"""GPU parity of the FP8 path through the C ABI against the oracle.

* fa_quantize_fp8: codes and scales bit-exact against oracle.quantize_fp8
  (the E4M3 decision is taken in float32 on both sides).
* fa_fwd_fp8: on quantised inputs that the oracle produced (codes and scales
  from oracle.quantize_fp8, never from the GPU), O and lse against
  oracle.fwd_fp8.
* both FP8 shapes at full size in the launch the bench times (GPU quantiser,
  then the FP8 forward): codes bit-exact on every element, O and lse on
  every row of every head.

Tolerances.  O: max-abs 2e-2, mean-abs 2e-3, as for the 16-bit forward.
lse: 1e-3 plus the score error of the FP8 matrix core.  gfx950's
32x32x64 E4M3 MFMA does not add its 64 products exactly: measured, its error
stays below 2^-11 of the largest product term, so a score (d/64 such
instructions) can be off by up to (d/64) 2^-11 scale max|q| max|k|, and lse
by as much.
"""
import math

import numpy as np
import pytest

import fa_inputs as gen
import oracle
from parity_util import TOL_LSE_16, TOL_MAX_ABS, TOL_MEAN_ABS, say, to_device, to_host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import io_aware_tiled_02_amd as fa
    fa.load()


def _dev_u8(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _gpu_quantize(x, dtype, block):
    import torch
    import io_aware_tiled_02_amd as fa
    B, H, L, d = x.shape
    xd = to_device(x, dtype)
    x8 = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
    sc = torch.empty((B * H, (L + block - 1) // block), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    rc = fa.fa_quantize_fp8(xd.data_ptr(), dtype, B, H, L, d, block, x8.data_ptr(), sc.data_ptr(), s.cuda_stream)
    assert rc == 0, f"fa_quantize_fp8 returned {rc}"
    s.synchronize()
    return x8.cpu().numpy(), sc.cpu().numpy()


def _gpu_fwd_fp8(q8, k8, sq, sk, v, dtype, scale, causal, bq, bk):
    import torch
    import io_aware_tiled_02_amd as fa
    B, H, L, d = q8.shape
    q8d, k8d = _dev_u8(q8), _dev_u8(k8)
    sqd, skd = (torch.from_numpy(np.ascontiguousarray(a)).to("cuda") for a in (sq, sk))
    vd = to_device(v, dtype)
    o = torch.empty_like(vd)
    lse = torch.empty((B, H, L), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    rc = fa.fa_fwd_fp8(q8d.data_ptr(), k8d.data_ptr(), sqd.data_ptr(), skd.data_ptr(), vd.data_ptr(), o.data_ptr(),
                       lse.data_ptr(), B, H, L, d, float(scale), int(causal), dtype, bq, bk, s.cuda_stream)
    assert rc == 0, f"fa_fwd_fp8 returned {rc}"
    s.synchronize()
    return to_host64(o, dtype), lse.cpu().numpy().astype(np.float64)


def lse_tolerance(d, scale, sq, sk):
    """1e-3 plus the FP8 MFMA bound (d/64) 2^-11 scale max|q| max|k|, with
    max|q| <= 448 max s_q (likewise k)."""
    return TOL_LSE_16 + (d / 64) * 2.0 ** -11 * scale * (448.0 * float(np.max(sq))) * (448.0 * float(np.max(sk)))


def compare_fp8(o, lse, o_ref, lse_ref, tol_lse, label):
    err = np.abs(o - o_ref)
    lerr = np.abs(lse - lse_ref)
    stats = dict(max_abs=float(err.max()), mean_abs=float(err.mean()), lse_max_abs=float(lerr.max()),
                 lse_tol=tol_lse)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), f"{label}: non-finite output"
    assert stats["max_abs"] <= TOL_MAX_ABS, f"{label}: O max abs err {stats['max_abs']:.3e}"
    assert stats["mean_abs"] <= TOL_MEAN_ABS, f"{label}: O mean abs err {stats['mean_abs']:.3e}"
    assert stats["lse_max_abs"] <= tol_lse, f"{label}: lse max abs err {stats['lse_max_abs']:.3e} > {tol_lse:.3e}"
    return stats


# ---- quantiser: bit-exact -------------------------------------------------------

@pytest.mark.parametrize("dtype", [gen.BF16, gen.F16])
@pytest.mark.parametrize("d", [64, 128])
def test_quantize_bit_exact(dtype, d):
    for (L, block, sigma) in [(1, 1, 1.0), (37, 16, 2.0), (128, 128, 1.0), (300, 64, 30.0), (300, 1000, 0.01),
                              (129, 7, 1.0), (520, 128, 3.0), (2150, 300, 1.0)]:
        say(f"[quant] dtype={gen.DTYPE_NAMES[dtype]} d={d} L={L} block={block} sigma={sigma}")
        x = gen.fill(dtype, (2, 3, L, d), 500 + L, 0, sigma)
        if L >= 2 * block:
            x[0, 1, block:2 * block] = 0                  # an all-zero block: scale 1, codes 0
        g8, gs = _gpu_quantize(x, dtype, block)
        r8, rs = oracle.quantize_fp8(x, dtype, block)
        assert np.array_equal(gs.view(np.uint32), rs.view(np.uint32)), "scales differ"
        bad = np.count_nonzero(g8 != r8)
        assert bad == 0, f"{bad} codes differ"


# ---- FP8 forward on the oracle's quantised inputs ---------------------------------

EDGE_L = [1, 17, 64, 65, 127, 128, 129, 255, 256, 257, 300, 600]


@pytest.mark.parametrize("dtype", [gen.BF16, gen.F16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [0, 1])
def test_fwd_fp8_edge_shapes(dtype, d, causal):
    scale = 1.0 / math.sqrt(d)
    for L in EDGE_L:
        say(f"[fp8] dtype={gen.DTYPE_NAMES[dtype]} d={d} causal={causal} L={L} blocks=128/128")
        shape = (1, 3, L, d)
        q = gen.fill(dtype, shape, 700 + L, 0, 1.5)
        k = gen.fill(dtype, shape, 700 + L, 1, 1.5)
        v = gen.fill(dtype, shape, 700 + L, 2)
        q8, sq = oracle.quantize_fp8(q, dtype, 128)
        k8, sk = oracle.quantize_fp8(k, dtype, 128)
        o, lse = _gpu_fwd_fp8(q8, k8, sq, sk, v, dtype, scale, causal, 128, 128)
        o_ref, lse_ref = oracle.fwd_fp8(q8, k8, sq, sk, v, dtype, scale, causal, 128, 128)
        compare_fp8(o, lse, o_ref, lse_ref, lse_tolerance(d, scale, sq, sk), f"L={L}")


@pytest.mark.parametrize("bq,bk", [(1, 32), (64, 64), (100, 96), (300, 256), (37, 160)])
@pytest.mark.parametrize("causal", [0, 1])
def test_fwd_fp8_block_sizes(bq, bk, causal):
    """Scale blocks that do not match the tiles: every query row and every
    32-key sub-tile reads its own block's scale."""
    B, H, L, d, dtype = 2, 2, 333, 128, gen.BF16
    scale = 1.0 / math.sqrt(d)
    say(f"[fp8-blocks] bq={bq} bk={bk} causal={causal} L={L}")
    q = gen.fill(dtype, (B, H, L, d), 800 + bq, 0, 2.0)
    k = gen.fill(dtype, (B, H, L, d), 800 + bq, 1, 2.0)
    v = gen.fill(dtype, (B, H, L, d), 800 + bq, 2)
    # spread the block scales: row r of Q and K times 2^(r mod 5 - 2)
    for r in range(L):
        f = 2.0 ** (r % 5 - 2)
        q[:, :, r] = gen.from_float64(gen.to_float64(q[:, :, r], dtype) * f, dtype)
        k[:, :, r] = gen.from_float64(gen.to_float64(k[:, :, r], dtype) * f, dtype)
    q8, sq = oracle.quantize_fp8(q, dtype, bq)
    k8, sk = oracle.quantize_fp8(k, dtype, bk)
    o, lse = _gpu_fwd_fp8(q8, k8, sq, sk, v, dtype, scale, causal, bq, bk)
    o_ref, lse_ref = oracle.fwd_fp8(q8, k8, sq, sk, v, dtype, scale, causal, bq, bk)
    compare_fp8(o, lse, o_ref, lse_ref, lse_tolerance(d, scale, sq, sk), f"bq={bq} bk={bk}")


def test_fwd_fp8_many_heads_remap():
    """B*H a multiple of 8 (heads grouped per XCD), ragged last tile, causal."""
    B, H, L, d, dtype = 2, 8, 700, 64, gen.F16
    say(f"[fp8-remap] B={B} H={H} L={L}")
    q = gen.fill(dtype, (B, H, L, d), 91, 0)
    k = gen.fill(dtype, (B, H, L, d), 91, 1)
    v = gen.fill(dtype, (B, H, L, d), 91, 2)
    q8, sq = oracle.quantize_fp8(q, dtype, 64)
    k8, sk = oracle.quantize_fp8(k, dtype, 64)
    o, lse = _gpu_fwd_fp8(q8, k8, sq, sk, v, dtype, 0.125, 1, 64, 64)
    o_ref, lse_ref = oracle.fwd_fp8(q8, k8, sq, sk, v, dtype, 0.125, 1, 64, 64)
    compare_fp8(o, lse, o_ref, lse_ref, lse_tolerance(d, 0.125, sq, sk), "remap")


# ---- the full FP8 shapes, in the bench's launch -----------------------------------

def _head(a, b, h):
    return np.ascontiguousarray(a[b:b + 1, h:h + 1])


@pytest.mark.parametrize("ci", range(len(gen.FP8)))
def test_fp8_workload(ci):
    import torch
    import io_aware_tiled_02_amd as fa
    cfg = gen.FP8[ci]
    say(f"[fp8-full] {cfg.name}")
    q, k, v = gen.make_fp8_inputs(cfg)
    qd, kd, vd = (to_device(x, cfg.dtype) for x in (q, k, v))
    q8d, sqd = fa.quantize_fp8(qd, cfg.block_q)
    k8d, skd = fa.quantize_fp8(kd, cfg.block_k)
    o, lse = fa.forward_fp8(q8d, k8d, sqd, skd, vd, cfg.scale, cfg.causal, cfg.block_q, cfg.block_k)
    torch.cuda.synchronize()
    q8, sq = oracle.quantize_fp8(q, cfg.dtype, cfg.block_q)
    k8, sk = oracle.quantize_fp8(k, cfg.dtype, cfg.block_k)
    assert np.array_equal(q8d.cpu().numpy(), q8) and np.array_equal(k8d.cpu().numpy(), k8), "codes differ"
    assert np.array_equal(sqd.cpu().numpy().view(np.uint32), sq.view(np.uint32))
    assert np.array_equal(skd.cpu().numpy().view(np.uint32), sk.view(np.uint32))
    o = to_host64(o, cfg.dtype)
    lse = lse.cpu().numpy().astype(np.float64)
    # every row of every head, against the oracle on the oracle's own codes
    o_ref, lse_ref = oracle.fwd_fp8(q8, k8, sq, sk, v, cfg.dtype, cfg.scale, cfg.causal, cfg.block_q, cfg.block_k)
    for b in range(cfg.B):
        for h in range(cfg.H):
            bh = b * cfg.H + h
            stats = compare_fp8(o[b, h], lse[b, h], o_ref[b, h], lse_ref[b, h],
                                lse_tolerance(cfg.d, cfg.scale, sq[bh], sk[bh]), f"{cfg.name} b={b} h={h}")
            if h in (0, cfg.H - 1):
                say(f"[fp8-full] b={b} h={h}: {stats}")
