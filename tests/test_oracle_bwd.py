"""Pins of the oracle's attention gradients (``oracle.bwd``).

Facts from outside the function: central finite differences of the pinned
forward oracle, a library routine (torch autograd through the CPU
scaled-dot-product attention in float64), and closed forms (one key, identical
keys, zero upstream gradient, linearity, the causal last key).
"""
import math

import numpy as np
import pytest
import torch

import fa_inputs as gen
import oracle

F64 = 3


def _inputs(B, H, L, d, seed, sigma=1.0):
    return tuple(gen.normal(seed, s, B * H * L * d, sigma if s < 2 else 1.0).reshape(B, H, L, d)
                 for s in range(4))


@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("L,d,scale", [(1, 3, 0.5), (4, 2, 1.3), (6, 5, 0.45)])
def test_gradients_match_finite_differences(L, d, scale, causal):
    """d/dx of sum(O (.) dO), by central differences of the forward oracle."""
    q, k, v, g = _inputs(1, 2, L, d, seed=31 + L)
    dq, dk, dv = oracle.bwd(q, k, v, g, F64, scale, causal)

    def loss(qq, kk, vv):
        o, _ = oracle.fwd(qq, kk, vv, F64, scale, causal)
        return float((o * g).sum())

    h = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy()
            xm = x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = loss(args["q"], args["k"], args["v"])
            args[name] = xm
            fm = loss(args["q"], args["k"], args["v"])
            num[idx] = (fp - fm) / (2 * h)
        assert np.max(np.abs(num - grad)) <= 1e-7, name


@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("sigma", [1.0, 3.0])
def test_gradients_match_torch_autograd(causal, sigma):
    """torch.nn.functional.scaled_dot_product_attention in float64 on the CPU,
    differentiated by autograd."""
    B, H, L, d = 2, 3, 37, 16
    q, k, v, g = _inputs(B, H, L, d, seed=5, sigma=sigma)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = oracle.bwd(q, k, v, g, F64, scale, causal)
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=bool(causal), scale=scale)
    out.backward(torch.tensor(g, dtype=torch.float64))
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.max(np.abs(mine - ref.numpy())) <= 1e-12 * max(1.0, float(ref.abs().max()))


@pytest.mark.parametrize("dtype", [gen.F32, gen.F16, gen.BF16])
def test_storage_types_widen_exactly(dtype):
    """16-bit and fp32 storage give the same gradients as their exact float64 widening."""
    shape = (1, 2, 19, 8)
    q, k, v, g = (gen.fill(dtype, shape, 9, s) for s in range(4))
    a = oracle.bwd(q, k, v, g, dtype, 0.35, 1)
    b = oracle.bwd(*(gen.to_float64(x, dtype) for x in (q, k, v, g)), F64, 0.35, 1)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_single_key_closed_form():
    """L = 1: P = 1, so dS = 0: dQ = dK = 0 and dV = dO."""
    q, k, v, g = _inputs(2, 2, 1, 8, seed=3)
    dq, dk, dv = oracle.bwd(q, k, v, g, F64, 0.9, 0)
    assert np.all(dq == 0.0) and np.all(dk == 0.0)
    assert np.allclose(dv, g, rtol=0, atol=1e-15)


def test_identical_keys_give_zero_dq():
    """Rows of dS sum to zero (sum_j P_ij (dP_ij - sum_k dP_ik P_ik) = 0), so
    with every key equal, dQ_i = scale * (sum_j dS_ij) k = 0."""
    q, k, v, g = _inputs(1, 2, 9, 8, seed=4)
    k[:] = k[:, :, :1]
    dq, dk, dv = oracle.bwd(q, k, v, g, F64, 0.6, 0)
    assert np.max(np.abs(dq)) <= 1e-13


def test_zero_and_scaled_upstream_gradient():
    """Gradients are linear in dO: zero for dO = 0, doubled for 2 dO."""
    q, k, v, g = _inputs(1, 2, 11, 4, seed=6)
    z = oracle.bwd(q, k, v, np.zeros_like(g), F64, 0.5, 1)
    assert all(np.all(x == 0.0) for x in z)
    a = oracle.bwd(q, k, v, g, F64, 0.5, 1)
    b = oracle.bwd(q, k, v, 2.0 * g, F64, 0.5, 1)
    for x, y in zip(a, b):
        assert np.allclose(2.0 * x, y, rtol=0, atol=1e-13)


def test_causal_last_key_sees_only_last_query():
    """Under the causal mask only the last query attends to the last key:
    dV_{L-1} = P_{L-1,L-1} dO_{L-1}."""
    q, k, v, g = _inputs(1, 1, 7, 4, seed=8)
    scale = 0.8
    _, _, dv = oracle.bwd(q, k, v, g, F64, scale, 1)
    s = scale * (k[0, 0] @ q[0, 0, -1])
    p_last = math.exp(s[-1] - s.max()) / np.exp(s - s.max()).sum()
    assert np.allclose(dv[0, 0, -1], p_last * g[0, 0, -1], rtol=0, atol=1e-14)
