"""GPU parity of the split-K/V (Flash-Decoding) path through the C ABI:
fa_fwd_splitkv against the oracle's attention over all keys, and fa_combine
against the oracle's merge.  Every case names itself before it touches the GPU.
"""
import math

import numpy as np
import pytest

import fa_inputs as gen
import oracle
from parity_util import compare, say, to_device, to_host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import io_aware_tiled_02_amd as fa
    fa.load()


def _run_splitkv(q, k, v, dtype, scale, nsplit):
    import torch
    import io_aware_tiled_02_amd as fa
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    qd, kd, vd = (to_device(x, dtype) for x in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device="cuda")
    need = fa.fa_splitkv_workspace_bytes(B, H, Lq, Lk, d, nsplit)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    rc = fa.fa_fwd_splitkv(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           B, H, Lq, Lk, d, float(scale), dtype, int(nsplit), ws.data_ptr(), need,
                           stream.cuda_stream)
    assert rc == 0, f"fa_fwd_splitkv returned {rc}: {fa.fa_strerror(rc)}"
    stream.synchronize()
    return to_host64(o, dtype), lse.cpu().numpy().astype(np.float64)


def _inputs(B, H, Lq, Lk, d, dtype, seed, sigma=1.0):
    q = gen.fill(dtype, (B, H, Lq, d), seed, 0, sigma)
    k = gen.fill(dtype, (B, H, Lk, d), seed, 1, sigma)
    v = gen.fill(dtype, (B, H, Lk, d), seed, 2)
    return q, k, v


@pytest.mark.parametrize("dtype", [gen.BF16, gen.F16, gen.F32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Lq", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("Lk,nsplit", [(1, 1), (5, 3), (63, 1), (64, 2), (65, 7), (1000, 0), (1000, 13),
                                       (4099, 5), (300, 40)])
def test_splitkv_small_shapes(dtype, d, Lq, Lk, nsplit):
    """Ragged chunk ends, chunks past the end (nsplit > keys / chunk), one
    key, every query-row count up to 8."""
    B, H = 2, 3
    label = f"splitkv {gen.DTYPE_NAMES[dtype]} d={d} Lq={Lq} Lk={Lk} nsplit={nsplit}"
    say(f"[splitkv] {label}")
    q, k, v = _inputs(B, H, Lq, Lk, d, dtype, seed=100 + Lq + Lk)
    scale = 1.0 / math.sqrt(d)
    o, lse = _run_splitkv(q, k, v, dtype, scale, nsplit)
    o_ref, lse_ref = oracle.attn_range(q, k, v, dtype, scale, 0, Lk)
    compare(o, lse, o_ref, lse_ref, dtype, label)


@pytest.mark.parametrize("sigma", [1.0, 3.0])
def test_splitkv_peaked_and_long(sigma):
    """Long K/V, several chunks, peaked scores (sigma 3 on Q and K)."""
    dtype, d = gen.BF16, 128
    q, k, v = _inputs(1, 4, 2, 20000, d, dtype, seed=77, sigma=sigma)
    say(f"[splitkv] peaked sigma={sigma} Lk=20000")
    o, lse = _run_splitkv(q, k, v, dtype, 1.0 / math.sqrt(d), 0)
    o_ref, lse_ref = oracle.attn_range(q, k, v, dtype, 1.0 / math.sqrt(d), 0, 20000)
    compare(o, lse, o_ref, lse_ref, dtype, f"peaked sigma={sigma}")


def test_splitkv_decode_workload():
    """The decoding workload at full size (B8 H32 Lq1 Lk16384 d128 bf16), the
    launch the bench times (automatic nsplit), checked on every head."""
    cfg = gen.DECODE
    say(f"[splitkv] workload {cfg.name}")
    q, k, v = gen.make_decode_qkv(cfg)
    o, lse = _run_splitkv(q, k, v, cfg.dtype, cfg.scale, 0)
    o_ref, lse_ref = oracle.attn_range(q, k, v, cfg.dtype, cfg.scale, 0, cfg.Lk)
    stats = compare(o, lse, o_ref, lse_ref, cfg.dtype, cfg.name)
    say(f"[splitkv] all {cfg.B * cfg.H} heads: {stats}")


@pytest.mark.parametrize("dtype", [gen.BF16, gen.F16, gen.F32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("nsplit", [1, 2, 7, 100])
def test_combine_against_oracle_merge(dtype, d, nsplit):
    """fa_combine on given partials (some empty, spread lse) vs oracle.merge."""
    import torch
    import io_aware_tiled_02_amd as fa
    B, H, Lq = 2, 3, 5
    rows = B * H * Lq
    say(f"[combine] {gen.DTYPE_NAMES[dtype]} d={d} nsplit={nsplit}")
    o_part = gen.normal(200 + nsplit, 0, nsplit * rows * d).reshape(nsplit, B, H, Lq, d).astype(np.float32)
    lse_part = (4.0 * gen.normal(200 + nsplit, 1, nsplit * rows)).reshape(nsplit, B, H, Lq).astype(np.float32)
    if nsplit > 1:
        lse_part[1, 0] = -np.inf                   # an empty part for every row of batch 0
    lse_part[:, 1, 2, 3] = -np.inf                 # one row with no keys at all
    o_ref, lse_ref = oracle.merge(o_part.astype(np.float64), lse_part.astype(np.float64))
    op = torch.from_numpy(o_part).cuda()
    lp = torch.from_numpy(lse_part).cuda()
    o = torch.empty((B, H, Lq, d), dtype={gen.F32: torch.float32, gen.F16: torch.float16,
                                          gen.BF16: torch.bfloat16}[dtype], device="cuda")
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    rc = fa.fa_combine(op.data_ptr(), lp.data_ptr(), nsplit, B, H, Lq, d, o.data_ptr(), lse.data_ptr(), dtype,
                       stream.cuda_stream)
    assert rc == 0, fa.fa_strerror(rc)
    stream.synchronize()
    o_h = to_host64(o, dtype)
    l_h = lse.cpu().numpy().astype(np.float64)
    # the all-empty row: o = 0, lse = -inf on both sides
    assert np.all(o_h[1, 2, 3] == 0.0) and l_h[1, 2, 3] == -np.inf and lse_ref[1, 2, 3] == -np.inf
    o_h[1, 2, 3] = o_ref[1, 2, 3] = 0.0
    l_h[1, 2, 3] = lse_ref[1, 2, 3] = 0.0
    # inputs are fp32 partials: the fp32 bar for fp32 output, the 16-bit bar
    # (output rounding) otherwise
    compare(o_h, l_h, o_ref, lse_ref, dtype, "combine")
