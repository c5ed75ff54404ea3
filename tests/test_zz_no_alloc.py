"""fa_fwd_splitkv_noalloc (the entry point that allocates nothing: its partial
results live in the library's own per-GPU array) through the C ABI, against
fa_fwd_splitkv (caller workspace) on the same inputs: two calls in a row, the
second smaller than the first, each bit-identical to the workspace entry
point and within the parity bar of the oracle.  Every case names itself
before it touches the GPU.
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


def _both(q, k, v, dtype, scale, nsplit, stream):
    """(noalloc o, lse), (workspace o, lse) as torch tensors, both on `stream`."""
    import torch
    import io_aware_tiled_02_amd as fa
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    qd, kd, vd = (to_device(x, dtype) for x in (q, k, v))
    torch.cuda.synchronize()
    o_n, o_w = torch.full_like(qd, float("nan")), torch.full_like(qd, float("nan"))
    l_n = torch.full((B, H, Lq), float("nan"), dtype=torch.float32, device="cuda")
    l_w = torch.full_like(l_n, float("nan"))
    need = fa.fa_splitkv_workspace_bytes(B, H, Lq, Lk, d, nsplit)
    assert 0 < need <= fa.FA_NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    rc = fa.fa_fwd_splitkv_noalloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o_n.data_ptr(), l_n.data_ptr(),
                                   B, H, Lq, Lk, d, float(scale), dtype, int(nsplit), stream.cuda_stream)
    assert rc == 0, f"fa_fwd_splitkv_noalloc returned {rc}: {fa.fa_strerror(rc)}"
    rc = fa.fa_fwd_splitkv(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o_w.data_ptr(), l_w.data_ptr(),
                           B, H, Lq, Lk, d, float(scale), dtype, int(nsplit), ws.data_ptr(), need,
                           stream.cuda_stream)
    assert rc == 0, f"fa_fwd_splitkv returned {rc}: {fa.fa_strerror(rc)}"
    stream.synchronize()
    return (o_n, l_n), (o_w, l_w)


def _check(q, k, v, dtype, scale, nsplit, stream, label):
    import torch
    (o_n, l_n), (o_w, l_w) = _both(q, k, v, dtype, scale, nsplit, stream)
    same_o = torch.equal(o_n.view(torch.int16), o_w.view(torch.int16)) if dtype != gen.F32 else \
        torch.equal(o_n.view(torch.int32), o_w.view(torch.int32))
    assert same_o, f"{label}: O differs from fa_fwd_splitkv"
    assert torch.equal(l_n.view(torch.int32), l_w.view(torch.int32)), f"{label}: lse differs from fa_fwd_splitkv"
    o_ref, lse_ref = oracle.attn_range(q, k, v, dtype, scale, 0, k.shape[2])
    stats = compare(to_host64(o_n, dtype), l_n.cpu().numpy().astype(np.float64), o_ref, lse_ref, dtype, label)
    say(f"[noalloc] {label}: bitwise equal to fa_fwd_splitkv; {stats}")


def test_noalloc_two_calls_second_smaller():
    import torch
    d, dtype = 128, gen.BF16
    # first call: the decoding shape (8 x 32 heads, one query row, 16K keys)
    cfg = gen.DECODE
    say(f"[noalloc] call 1: {cfg.name}, automatic nsplit")
    q, k, v = gen.make_decode_qkv(cfg)
    _check(q, k, v, cfg.dtype, cfg.scale, 0, torch.cuda.current_stream(), "call 1 (decode shape)")
    # second call: fewer heads, more query rows, fewer keys, on a side stream
    B, H, Lq, Lk, nsplit = 2, 3, 5, 3001, 7
    say(f"[noalloc] call 2: B={B} H={H} Lq={Lq} Lk={Lk} nsplit={nsplit} d={d} bf16, side stream")
    q = gen.fill(dtype, (B, H, Lq, d), 321, 0, 2.0)
    k = gen.fill(dtype, (B, H, Lk, d), 321, 1, 2.0)
    v = gen.fill(dtype, (B, H, Lk, d), 321, 2)
    side = torch.cuda.Stream()
    _check(q, k, v, dtype, 1.0 / math.sqrt(d), nsplit, side, "call 2 (smaller, side stream)")


def test_noalloc_other_types_and_ragged_chunks():
    import torch
    for dtype, d, Lq, Lk, nsplit in [(gen.F16, 64, 8, 999, 5), (gen.F32, 128, 1, 65, 7), (gen.F32, 64, 3, 1, 1)]:
        label = f"{gen.DTYPE_NAMES[dtype]} d={d} Lq={Lq} Lk={Lk} nsplit={nsplit}"
        say(f"[noalloc] {label}")
        q = gen.fill(dtype, (1, 4, Lq, d), 400 + Lk, 0)
        k = gen.fill(dtype, (1, 4, Lk, d), 400 + Lk, 1)
        v = gen.fill(dtype, (1, 4, Lk, d), 400 + Lk, 2)
        _check(q, k, v, dtype, 1.0 / math.sqrt(d), nsplit, torch.cuda.current_stream(), label)
