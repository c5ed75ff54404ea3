"""Launch behaviour of the backward, split-K/V and FP8 entry points on the GPU:
repeat launches are bitwise identical (no atomics, no order-dependent
reductions), outputs are fully overwritten whatever they held (NaN-filled
beforehand), and the work runs on the stream it is given (a side stream,
checked against the oracle).  Every case names itself before it touches the GPU.
"""
import numpy as np
import pytest

import fa_inputs as gen
import oracle
from parity_util import compare, say, to_device, to_host64
from test_bwd_gpu import compare_grads
from test_fp8_gpu import compare_fp8, lse_tolerance

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import io_aware_tiled_02_amd as fa
    fa.load()


def _bwd_call(fa, t, outs, ws, causal, stream):
    q, k, v, o, lse, g = t
    B, H, L, d = q.shape
    rc = fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), g.data_ptr(),
                   outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(), B, H, L, d, 0.125, causal,
                   gen.BF16, ws.data_ptr(), ws.numel(), stream.cuda_stream)
    assert rc == 0, fa.fa_strerror(rc)


@pytest.mark.parametrize("causal", [0, 1])
def test_backward_repeat_overwrite_side_stream(causal):
    import torch
    import io_aware_tiled_02_amd as fa
    B, H, L, d = 1, 3, 333, 64
    say(f"[behaviour] fa_bwd twice on a side stream, NaN-filled outputs, causal={causal}")
    qn, kn, vn, gn = (gen.fill(gen.BF16, (B, H, L, d), 71, s) for s in range(4))
    q, k, v, g = (to_device(x, gen.BF16) for x in (qn, kn, vn, gn))
    o, lse = fa.forward(q, k, v, 0.125, bool(causal))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, L), dtype=torch.uint8, device="cuda")
    runs = []
    for _ in range(2):
        outs = [torch.full_like(q, float("nan")) for _ in range(3)]
        torch.cuda.synchronize()
        _bwd_call(fa, (q, k, v, o, lse, g), outs, ws, causal, s)
        s.synchronize()
        runs.append(outs)
    for a, b in zip(*runs):
        assert torch.isfinite(a.float()).all() and torch.equal(a, b)
    got = [to_host64(x, gen.BF16) for x in runs[0]]
    ref = oracle.bwd(qn, kn, vn, gn, gen.BF16, 0.125, causal)
    compare_grads(got, ref, f"side stream causal={causal}")


def test_splitkv_repeat_overwrite_side_stream():
    import torch
    import io_aware_tiled_02_amd as fa
    B, H, Lq, Lk, d = 2, 4, 3, 3000, 128
    say("[behaviour] fa_fwd_splitkv twice on a side stream, NaN-filled outputs")
    qn = gen.fill(gen.BF16, (B, H, Lq, d), 72, 0)
    kn = gen.fill(gen.BF16, (B, H, Lk, d), 72, 1)
    vn = gen.fill(gen.BF16, (B, H, Lk, d), 72, 2)
    q, k, v = (to_device(x, gen.BF16) for x in (qn, kn, vn))
    s = torch.cuda.Stream()
    runs = []
    for _ in range(2):
        out = torch.full_like(q, float("nan"))
        lse = torch.full((B, H, Lq), float("nan"), device="cuda")
        ws = torch.full((fa.fa_splitkv_workspace_bytes(B, H, Lq, Lk, d, 0),), 255, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            fa.forward_splitkv(q, k, v, 0.09, out=out, lse=lse, workspace=ws, stream=s)
        s.synchronize()
        runs.append((out, lse))
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])
    o_ref, lse_ref = oracle.attn_range(qn, kn, vn, gen.BF16, 0.09, 0, Lk)
    compare(to_host64(runs[0][0], gen.BF16), runs[0][1].cpu().numpy().astype(np.float64), o_ref, lse_ref,
            gen.BF16, "splitkv side stream")


@pytest.mark.parametrize("causal", [0, 1])
def test_fp8_repeat_overwrite_side_stream(causal):
    import torch
    import io_aware_tiled_02_amd as fa
    B, H, L, d = 1, 3, 300, 128
    say(f"[behaviour] fa_quantize_fp8 + fa_fwd_fp8 twice on a side stream, NaN-filled outputs, causal={causal}")
    qn, kn, vn = (gen.fill(gen.BF16, (B, H, L, d), 73, s) for s in range(3))
    q, k, v = (to_device(x, gen.BF16) for x in (qn, kn, vn))
    s = torch.cuda.Stream()
    runs = []
    for _ in range(2):
        q8 = torch.full(q.shape, 0xFF, dtype=torch.uint8, device="cuda")     # E4M3 NaN codes
        k8 = torch.full(q.shape, 0xFF, dtype=torch.uint8, device="cuda")
        sq = torch.full((B * H, 3), float("nan"), device="cuda")
        sk = torch.full((B * H, 5), float("nan"), device="cuda")
        out = torch.full_like(v, float("nan"))
        lse = torch.full((B, H, L), float("nan"), device="cuda")
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            fa.quantize_fp8(q, 128, x8=q8, scales=sq, stream=s)
            fa.quantize_fp8(k, 64, x8=k8, scales=sk, stream=s)
            fa.forward_fp8(q8, k8, sq, sk, v, 0.1, bool(causal), 128, 64, out=out, lse=lse, stream=s)
        s.synchronize()
        runs.append((q8, k8, sq, sk, out, lse))
    for a, b in zip(*runs):
        assert torch.equal(a, b)
    r8q, rsq = oracle.quantize_fp8(qn, gen.BF16, 128)
    r8k, rsk = oracle.quantize_fp8(kn, gen.BF16, 64)
    q8, k8, sq, sk, out, lse = runs[0]
    assert np.array_equal(q8.cpu().numpy(), r8q) and np.array_equal(k8.cpu().numpy(), r8k)
    assert np.array_equal(sq.cpu().numpy().view(np.uint32), rsq.view(np.uint32))
    assert np.array_equal(sk.cpu().numpy().view(np.uint32), rsk.view(np.uint32))
    o_ref, lse_ref = oracle.fwd_fp8(r8q, r8k, rsq, rsk, vn, gen.BF16, 0.1, causal, 128, 64)
    compare_fp8(to_host64(out, gen.BF16), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref,
                lse_tolerance(d, 0.1, rsq, rsk), f"fp8 side stream causal={causal}")


def test_pending_error_of_another_call_is_not_reported():
    """A HIP error left pending on the thread by an unrelated call (here
    hipErrorNotReady from hipStreamQuery on a busy stream, when this HIP
    records it) is not reported by the library's launches: fa_fwd and fa_bwd
    return FA_OK and write correct results."""
    import ctypes
    import torch
    import io_aware_tiled_02_amd as fa
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipStreamQuery.argtypes = [ctypes.c_void_p]
    hip.hipStreamQuery.restype = ctypes.c_int
    hip.hipPeekAtLastError.restype = ctypes.c_int
    hip.hipGetLastError.restype = ctypes.c_int
    B, H, L, d = 1, 2, 300, 128
    say("[behaviour] fa_fwd / fa_bwd after a pending hipErrorNotReady")
    qn, kn, vn, gn = (gen.fill(gen.BF16, (B, H, L, d), 74, s) for s in range(4))
    q, k, v, g = (to_device(x, gen.BF16) for x in (qn, kn, vn, gn))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, L), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, L), dtype=torch.uint8, device="cuda")
    outs = [torch.full_like(q, float("nan")) for _ in range(3)]
    # a busy stream: a long forward pass, queried at once
    big = [torch.zeros((1, 32, 8192, 128), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    big_o = torch.empty_like(big[0])
    big_l = torch.empty((1, 32, 8192), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    torch.cuda.synchronize()
    hip.hipGetLastError()
    rc = fa.fa_fwd(big[0].data_ptr(), big[1].data_ptr(), big[2].data_ptr(), big_o.data_ptr(), big_l.data_ptr(),
                   1, 32, 8192, 128, 0.1, 0, gen.BF16, s.cuda_stream)
    assert rc == 0
    q_rc = hip.hipStreamQuery(ctypes.c_void_p(s.cuda_stream))
    pending = hip.hipPeekAtLastError()
    rc_f = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, L, d, 0.125, 0,
                     gen.BF16, s.cuda_stream)
    rc_b = fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), g.data_ptr(),
                     outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(), B, H, L, d, 0.125, 0, gen.BF16,
                     ws.data_ptr(), ws.numel(), s.cuda_stream)
    after = hip.hipPeekAtLastError()
    torch.cuda.synchronize()
    hip.hipGetLastError()
    say(f"[behaviour] hipStreamQuery -> {q_rc}, pending before {pending}, after {after}; fa_fwd {rc_f}, fa_bwd {rc_b}")
    assert rc_f == 0 and rc_b == 0, f"fa_fwd {rc_f}, fa_bwd {rc_b} with a pending error {pending}"
    o_ref, lse_ref = oracle.fwd(qn, kn, vn, gen.BF16, 0.125, 0)
    compare(to_host64(o, gen.BF16), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, gen.BF16, "pending error")
    ref = oracle.bwd(qn, kn, vn, gn, gen.BF16, 0.125, 0)
    compare_grads([to_host64(x, gen.BF16) for x in outs], ref, "pending error")
