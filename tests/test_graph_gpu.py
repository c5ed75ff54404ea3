"""Every entry point under HIP graph capture (torch.cuda.CUDAGraph).

The library allocates nothing and never synchronises, so a caller can record
its launches in a graph and replay them.  Each case captures the calls on
preallocated buffers, then replays the graph three times: on the captured
inputs, on new inputs copied into the same buffers, and on the first inputs
again after unrelated eager work and a device synchronisation.  Every replay
must equal, bit for bit, the same call made eagerly on the same inputs (the
kernels are deterministic).  Every case names itself before it touches the GPU.
"""
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


def _replays(inputs_a, inputs_b, static_in, outs, call):
    """Capture call() (which reads static_in, writes outs) and check three
    replays against eager calls on the same inputs."""
    import torch

    def load(vals):
        for dst, src in zip(static_in, vals):
            dst.copy_(src)

    def eager(vals):
        load(vals)
        call()
        torch.cuda.synchronize()
        return [o.clone() for o in outs]

    ref_b = eager(inputs_b)
    ref_a = eager(inputs_a)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                 # warm-up on a side stream, as torch asks before capture
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for o in outs:
        o.fill_(float("nan")) if o.is_floating_point() else o.fill_(0xAB)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    for o, r in zip(outs, ref_a):
        assert torch.equal(o, r), "replay 1 differs from the eager call"
    load(inputs_b)
    g.replay()
    torch.cuda.synchronize()
    for o, r in zip(outs, ref_b):
        assert torch.equal(o, r), "replay 2 (new inputs) differs from the eager call"
    junk = torch.arange(1 << 20, device="cuda", dtype=torch.float32)
    junk.mul_(1.5).add_(2.0)
    torch.cuda.synchronize()
    load(inputs_a)
    g.replay()
    torch.cuda.synchronize()
    for o, r in zip(outs, ref_a):
        assert torch.equal(o, r), "replay 3 differs from the eager call"
    return ref_a


@pytest.mark.parametrize("dtype,d,causal", [(gen.BF16, 128, 0), (gen.BF16, 128, 1), (gen.F16, 64, 1), (gen.F32, 64, 0)])
def test_forward_graph(dtype, d, causal):
    import torch
    import io_aware_tiled_02_amd as fa
    B, H, L = 2, 3, 333
    say(f"[graph] fa_fwd B={B} H={H} L={L} d={d} dtype={gen.DTYPE_NAMES[dtype]} causal={causal}")
    a = [gen.fill(dtype, (B, H, L, d), 81, s) for s in range(3)]
    b = [gen.fill(dtype, (B, H, L, d), 82, s) for s in range(3)]
    ta, tb = [to_device(x, dtype) for x in a], [to_device(x, dtype) for x in b]
    q, k, v = (torch.empty_like(x) for x in ta)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, L), dtype=torch.float32, device="cuda")
    ref = _replays(ta, tb, [q, k, v], [o, lse], lambda: fa.forward(q, k, v, 0.1, bool(causal), out=o, lse=lse))
    o_ref, lse_ref = oracle.fwd(a[0], a[1], a[2], dtype, 0.1, causal)
    compare(to_host64(ref[0], dtype), ref[1].cpu().numpy().astype(np.float64), o_ref, lse_ref, dtype,
            "graph forward")


def test_splitkv_graph():
    import torch
    import io_aware_tiled_02_amd as fa
    B, H, Lq, Lk, d = 2, 4, 3, 3000, 128
    say(f"[graph] fa_fwd_splitkv + fa_combine B={B} H={H} Lq={Lq} Lk={Lk} d={d}")
    shapes = [(B, H, Lq, d), (B, H, Lk, d), (B, H, Lk, d)]
    a = [gen.fill(gen.BF16, sh, 83, s) for s, sh in enumerate(shapes)]
    b = [gen.fill(gen.BF16, sh, 84, s) for s, sh in enumerate(shapes)]
    ta, tb = [to_device(x, gen.BF16) for x in a], [to_device(x, gen.BF16) for x in b]
    q, k, v = (torch.empty_like(x) for x in ta)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.fa_splitkv_workspace_bytes(B, H, Lq, Lk, d, 0), dtype=torch.uint8, device="cuda")
    ref = _replays(ta, tb, [q, k, v], [o, lse],
                   lambda: fa.forward_splitkv(q, k, v, 0.09, out=o, lse=lse, workspace=ws))
    o_ref, lse_ref = oracle.attn_range(a[0], a[1], a[2], gen.BF16, 0.09, 0, Lk)
    compare(to_host64(ref[0], gen.BF16), ref[1].cpu().numpy().astype(np.float64), o_ref, lse_ref, gen.BF16,
            "graph splitkv")


@pytest.mark.parametrize("causal", [0, 1])
def test_backward_graph(causal):
    import torch
    import io_aware_tiled_02_amd as fa
    B, H, L, d = 1, 3, 300, 128
    say(f"[graph] fa_fwd + fa_bwd B={B} H={H} L={L} d={d} causal={causal}")
    a = [gen.fill(gen.BF16, (B, H, L, d), 85, s) for s in range(4)]
    b = [gen.fill(gen.BF16, (B, H, L, d), 86, s) for s in range(4)]
    ta, tb = [to_device(x, gen.BF16) for x in a], [to_device(x, gen.BF16) for x in b]
    q, k, v, g = (torch.empty_like(x) for x in ta)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, L), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, L), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream

    def call():
        fa.forward(q, k, v, 0.125, bool(causal), out=o, lse=lse)
        rc = fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), g.data_ptr(),
                       dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, L, d, 0.125, causal, gen.BF16,
                       ws.data_ptr(), ws.numel(), stream().cuda_stream)
        assert rc == 0, fa.fa_strerror(rc)

    _replays(ta, tb, [q, k, v, g], [o, lse, dq, dk, dv], call)


def test_fp8_graph():
    import torch
    import io_aware_tiled_02_amd as fa
    B, H, L, d = 1, 3, 300, 128
    say(f"[graph] fa_quantize_fp8 + fa_fwd_fp8 B={B} H={H} L={L} d={d}")
    a = [gen.fill(gen.BF16, (B, H, L, d), 87, s) for s in range(3)]
    b = [gen.fill(gen.BF16, (B, H, L, d), 88, s) for s in range(3)]
    ta, tb = [to_device(x, gen.BF16) for x in a], [to_device(x, gen.BF16) for x in b]
    q, k, v = (torch.empty_like(x) for x in ta)
    q8 = torch.empty(q.shape, dtype=torch.uint8, device="cuda")
    k8 = torch.empty(q.shape, dtype=torch.uint8, device="cuda")
    sq = torch.empty((B * H, 3), dtype=torch.float32, device="cuda")
    sk = torch.empty((B * H, 5), dtype=torch.float32, device="cuda")
    o = torch.empty_like(v)
    lse = torch.empty((B, H, L), dtype=torch.float32, device="cuda")

    def call():
        fa.quantize_fp8(q, 128, x8=q8, scales=sq)
        fa.quantize_fp8(k, 64, x8=k8, scales=sk)
        fa.forward_fp8(q8, k8, sq, sk, v, 0.1, True, 128, 64, out=o, lse=lse)

    _replays(ta, tb, [q, k, v], [q8, k8, sq, sk, o, lse], call)
