"""Pins of the oracle's Flash-Decoding pieces: one K/V block's attention for a
few query rows (``oracle.attn_range``) and the merge of per-block results
(``oracle.merge``).

The facts checked come from outside those two functions: a pure-Python
evaluation of the attention definition, the already pinned full-attention
oracle, closed forms (one key, identical keys, equal partial results), and
the identities the merge must satisfy (a partition of the keys merges back to
attention over all of them; empty blocks are neutral; the order of the parts
does not matter).
"""
import math

import numpy as np
import pytest

import fa_inputs as gen
import oracle

F64 = 3


def _inputs(B, H, Lq, Lk, d, seed, sigma=1.0):
    q = gen.normal(seed, 0, B * H * Lq * d, sigma).reshape(B, H, Lq, d)
    k = gen.normal(seed, 1, B * H * Lk * d, sigma).reshape(B, H, Lk, d)
    v = gen.normal(seed, 2, B * H * Lk * d, 1.0).reshape(B, H, Lk, d)
    return q, k, v


def _python_attention(q, k, v, scale, a, b):
    """The definition, term by term, in Python floats: one query row q (d,)
    against keys a..b-1 of k, v (Lk, d)."""
    scores = []
    for j in range(a, b):
        scores.append(scale * sum(float(q[c]) * float(k[j, c]) for c in range(len(q))))
    m = max(scores)
    w = [math.exp(s - m) for s in scores]
    total = sum(w)
    out = [sum(w[t] * float(v[a + t, c]) for t in range(len(w))) / total for c in range(v.shape[1])]
    return out, m + math.log(total)


# ---- the block attention itself ---------------------------------------------

@pytest.mark.parametrize("rng_", [(0, 5), (2, 3), (1, 7), (0, 1)])
def test_range_matches_python_definition(rng_):
    """attn_range == the attention definition evaluated with Python floats."""
    a, b = rng_
    q, k, v = _inputs(1, 2, 3, 7, 4, seed=21)
    scale = 0.7
    o, lse = oracle.attn_range(q, k, v, F64, scale, a, b)
    for h in range(2):
        for i in range(3):
            ref_o, ref_l = _python_attention(q[0, h, i], k[0, h], v[0, h], scale, a, b)
            assert np.allclose(o[0, h, i], ref_o, rtol=0, atol=1e-13)
            assert abs(lse[0, h, i] - ref_l) <= 1e-13


@pytest.mark.parametrize("dtype", [gen.F32, gen.F16, gen.BF16, F64])
def test_range_over_all_keys_equals_full_attention(dtype):
    """With every key in the block and Lq = Lk, the block attention is the
    (separately pinned) full non-causal attention."""
    L, d = 29, 16
    shape = (2, 2, L, d)
    if dtype == F64:
        q, k, v = _inputs(2, 2, L, L, d, seed=3)
    else:
        q = gen.fill(dtype, shape, 3, 0)
        k = gen.fill(dtype, shape, 3, 1)
        v = gen.fill(dtype, shape, 3, 2)
    scale = 1.0 / math.sqrt(d)
    o1, l1 = oracle.attn_range(q, k, v, dtype, scale, 0, L)
    o2, l2 = oracle.fwd(q, k, v, dtype, scale, 0)
    assert np.max(np.abs(o1 - o2)) <= 1e-13
    assert np.max(np.abs(l1 - l2)) <= 1e-13


def test_range_single_key_closed_form():
    """One key: the output is that key's value row, lse its score."""
    q, k, v = _inputs(1, 3, 4, 9, 8, seed=5)
    scale = 0.4
    for j in (0, 4, 8):
        o, lse = oracle.attn_range(q, k, v, F64, scale, j, j + 1)
        for h in range(3):
            assert np.allclose(o[0, h], np.broadcast_to(v[0, h, j], (4, 8)), rtol=0, atol=1e-15)
            assert np.allclose(lse[0, h], scale * (q[0, h] @ k[0, h, j]), rtol=0, atol=1e-13)


def test_range_identical_keys_closed_form():
    """n identical keys: equal weights, so O is the mean of the block's value
    rows and lse = s + ln n."""
    q, k, v = _inputs(1, 1, 2, 12, 8, seed=8)
    k[:] = k[0, 0, 5]
    a, b = 3, 10
    o, lse = oracle.attn_range(q, k, v, F64, 0.5, a, b)
    assert np.allclose(o[0, 0], np.broadcast_to(v[0, 0, a:b].mean(axis=0), (2, 8)), rtol=0, atol=1e-14)
    s = 0.5 * (q[0, 0] @ k[0, 0, 5])
    assert np.allclose(lse[0, 0], s + math.log(b - a), rtol=0, atol=1e-13)


def test_range_empty_block_convention():
    q, k, v = _inputs(1, 2, 3, 6, 4, seed=9)
    o, lse = oracle.attn_range(q, k, v, F64, 1.0, 4, 4)
    assert np.all(o == 0.0)
    assert np.all(lse == -np.inf)


@pytest.mark.parametrize("bad", [(-1, 3), (2, 1), (0, 7)])
def test_range_rejects_bad_ranges(bad):
    q, k, v = _inputs(1, 1, 2, 6, 4, seed=1)
    with pytest.raises(ValueError):
        oracle.attn_range(q, k, v, F64, 1.0, *bad)


# ---- merge -------------------------------------------------------------------

@pytest.mark.parametrize("cuts", [
    [0, 37],                       # one part
    [0, 10, 20, 37],               # equal-ish parts
    [0, 1, 2, 3, 37],              # single-key parts
    [0, 0, 15, 15, 37, 37],        # empty parts in between and at the ends
    [0, 36, 37],                   # a one-key tail
])
@pytest.mark.parametrize("sigma", [1.0, 4.0])
def test_partition_merges_back_to_full_attention(cuts, sigma):
    """Attention over a partition of the keys, merged, equals attention over
    all of them (the Flash-Decoding identity)."""
    B, H, Lq, Lk, d = 2, 3, 5, 37, 16
    q, k, v = _inputs(B, H, Lq, Lk, d, seed=17, sigma=sigma)
    scale = 1.0 / math.sqrt(d)
    o_full, l_full = oracle.attn_range(q, k, v, F64, scale, 0, Lk)
    parts = [oracle.attn_range(q, k, v, F64, scale, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
    o, lse = oracle.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    assert np.max(np.abs(o - o_full)) <= 1e-12
    assert np.max(np.abs(lse - l_full)) <= 1e-12


def test_merge_two_equal_parts_closed_form():
    """Two parts with the same lse weigh equally: O is their average and the
    lse grows by ln 2."""
    rng = np.random.default_rng(2)
    o_parts = rng.standard_normal((2, 6, 8))
    lse_parts = np.broadcast_to(rng.standard_normal(6), (2, 6)).copy()
    o, lse = oracle.merge(o_parts, lse_parts)
    assert np.allclose(o, o_parts.mean(axis=0), rtol=0, atol=1e-15)
    assert np.allclose(lse, lse_parts[0] + math.log(2.0), rtol=0, atol=1e-15)


def test_merge_weights_follow_exp_of_lse():
    """Parts whose lse differ by ln 3 weigh 3 : 1 (weights exp(lse_s))."""
    o_parts = np.stack([np.full((1, 4), 2.0), np.full((1, 4), -6.0)])
    lse_parts = np.array([[0.5 + math.log(3.0)], [0.5]])
    o, lse = oracle.merge(o_parts, lse_parts)
    assert np.allclose(o, (3 * 2.0 + 1 * -6.0) / 4.0, rtol=0, atol=1e-14)
    assert np.allclose(lse, 0.5 + math.log(4.0), rtol=0, atol=1e-14)


def test_merge_single_part_and_empty_parts_are_neutral():
    rng = np.random.default_rng(3)
    o1 = rng.standard_normal((1, 5, 8))
    l1 = rng.standard_normal((1, 5))
    o, lse = oracle.merge(o1, l1)
    assert np.array_equal(o, o1[0]) and np.array_equal(lse, l1[0])
    empty_o = np.zeros((2, 5, 8))
    empty_l = np.full((2, 5), -np.inf)
    o, lse = oracle.merge(np.concatenate([empty_o[:1], o1, empty_o[1:]]),
                          np.concatenate([empty_l[:1], l1, empty_l[1:]]))
    assert np.allclose(o, o1[0], rtol=0, atol=1e-15) and np.allclose(lse, l1[0], rtol=0, atol=1e-15)
    o, lse = oracle.merge(empty_o, empty_l)
    assert np.all(o == 0.0) and np.all(lse == -np.inf)


def test_merge_is_order_independent():
    rng = np.random.default_rng(4)
    o_parts = rng.standard_normal((5, 7, 16))
    lse_parts = 3.0 * rng.standard_normal((5, 7))
    o1, l1 = oracle.merge(o_parts, lse_parts)
    perm = [3, 0, 4, 1, 2]
    o2, l2 = oracle.merge(o_parts[perm], lse_parts[perm])
    assert np.allclose(o1, o2, rtol=0, atol=1e-13) and np.allclose(l1, l2, rtol=0, atol=1e-13)
