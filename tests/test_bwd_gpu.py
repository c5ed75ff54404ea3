"""GPU parity of the backward pass (fa_bwd through the C ABI) against the
oracle's gradients.  The GPU backward takes o and lse from the GPU forward
pass (as a caller would); the oracle computes dQ, dK, dV from q, k, v and dO
alone.  Every case names itself before it touches the GPU.
"""
import math

import numpy as np
import pytest

import fa_inputs as gen
import oracle
from parity_util import say, to_device, to_host64

pytestmark = pytest.mark.gpu

# Gradient tolerance (16-bit storage, fp32 accumulation): relative to the
# largest reference magnitude of each gradient, max-abs <= 2e-2 and mean-abs
# <= 2e-3 -- the forward pass's bar, applied to gradients normalised by their
# scale (which changes with L).  The normalisation is floored at 0.1 x the
# largest magnitude of the three gradients, since a gradient can be exactly
# zero (one key: dQ = dK = 0) while rounding leaves ~1e-7 on the GPU.
TOL_MAX = 2e-2
TOL_MEAN = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import io_aware_tiled_02_amd as fa
    fa.load()


def run_bwd(q, k, v, g, dtype, scale, causal):
    import torch
    import io_aware_tiled_02_amd as fa
    B, H, L, d = q.shape
    qd, kd, vd, gd = (to_device(x, dtype) for x in (q, k, v, g))
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, L), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    rc = fa.fa_fwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, L, d,
                   float(scale), int(causal), dtype, s.cuda_stream)
    assert rc == 0, fa.fa_strerror(rc)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    need = fa.fa_bwd_workspace_bytes(B, H, L)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    rc = fa.fa_bwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(), gd.data_ptr(),
                   dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, L, d, float(scale), int(causal), dtype,
                   ws.data_ptr(), need, s.cuda_stream)
    assert rc == 0, fa.fa_strerror(rc)
    s.synchronize()
    return tuple(to_host64(x, dtype) for x in (dq, dk, dv))


def compare_grads(got, ref, label):
    stats = {}
    floor = 0.1 * max(float(np.abs(r).max()) for r in ref)
    for name, x, r in zip(("dq", "dk", "dv"), got, ref):
        assert np.all(np.isfinite(x)), f"{label}: non-finite {name}"
        scale = max(float(np.abs(r).max()), floor, 1e-30)
        err = np.abs(x - r)
        stats[name] = (float(err.max() / scale), float(err.mean() / scale))
    say(f"[bwd] {label}: " + " ".join(f"{n} max {a:.2e} mean {b:.2e}" for n, (a, b) in stats.items()))
    for n, (a, b) in stats.items():
        assert a <= TOL_MAX, f"{label}: {n} max-abs/scale {a:.3e}"
        assert b <= TOL_MEAN, f"{label}: {n} mean-abs/scale {b:.3e}"
    return stats


@pytest.mark.parametrize("dtype", [gen.BF16, gen.F16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("L", [1, 17, 64, 65, 127, 128, 129, 200, 300])
def test_bwd_small_shapes(L, causal, d, dtype):
    B, H = 2, 2
    label = f"{gen.DTYPE_NAMES[dtype]} d={d} L={L} causal={causal}"
    say(f"[bwd] {label}")
    shape = (B, H, L, d)
    q, k, v, g = (gen.fill(dtype, shape, 40 + L, s) for s in range(4))
    scale = 1.0 / math.sqrt(d)
    got = run_bwd(q, k, v, g, dtype, scale, causal)
    ref = oracle.bwd(q, k, v, g, dtype, scale, causal)
    compare_grads(got, ref, label)


def test_bwd_peaked():
    """Q, K ~ 3 N(0,1): peaked softmax rows."""
    dtype, d, L = gen.BF16, 128, 333
    shape = (1, 2, L, d)
    q, k = (gen.fill(dtype, shape, 50, s, 3.0) for s in range(2))
    v, g = (gen.fill(dtype, shape, 50, s) for s in range(2, 4))
    say("[bwd] peaked L=333")
    got = run_bwd(q, k, v, g, dtype, 1.0 / math.sqrt(d), 0)
    ref = oracle.bwd(q, k, v, g, dtype, 1.0 / math.sqrt(d), 0)
    compare_grads(got, ref, "peaked")


@pytest.mark.parametrize("idx", [0, 1])
def test_bwd_workload_all_heads(idx):
    """The backward shapes at full size, in the launch the bench times,
    checked on every head (every row of each), head by head."""
    cfg = gen.BWD[idx]
    say(f"[bwd] workload {cfg.name}")
    q, k, v, g = gen.make_bwd_inputs(cfg)
    got = run_bwd(q, k, v, g, cfg.dtype, cfg.scale, cfg.causal)
    ref = oracle.bwd(q, k, v, g, cfg.dtype, cfg.scale, cfg.causal)
    for b in range(cfg.B):
        for h in range(cfg.H):
            sl = lambda a: a[b:b + 1, h:h + 1]
            compare_grads(tuple(sl(x) for x in got), tuple(sl(x) for x in ref), f"{cfg.name} b={b} h={h}")
