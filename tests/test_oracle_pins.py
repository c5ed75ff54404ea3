"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each test names the fact it checks and where that fact comes from: a value a
page prints, a closed form, an invariant of softmax attention, a library
routine on a special case, or the independent brute-force twin.  Chosen so a
dropped term, a wrong sign or index, a transposed operand, a missing scale or
a wrong mask direction in the oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import fa_inputs as gen
import oracle
from oracle import tiled

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F64 = 3


def _fwd64(Q, K, V, scale, causal, rows=None):
    """Oracle on float64 (L, d) single-head inputs."""
    o, lse = oracle.fwd(Q[None, None], K[None, None], V[None, None], F64, scale, causal, rows)
    return o[0, 0], lse[0, 0]


def _rng_inputs(L, d, seed, sigma=1.0):
    q = gen.normal(seed, 0, L * d, sigma).reshape(L, d)
    k = gen.normal(seed, 1, L * d, sigma).reshape(L, d)
    v = gen.normal(seed, 2, L * d, 1.0).reshape(L, d)
    return q, k, v


# ---- P1: oracle == independent brute force on tiny shapes -------------------

@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("L", [1, 2, 3, 5, 16, 33, 64])
@pytest.mark.parametrize("d", [1, 4, 8, 64])
def test_p1_oracle_matches_brute_force(L, d, causal):
    B, H = 2, 2
    shape = (B, H, L, d)
    q = gen.fill(gen.F32, shape, 11, 0)
    k = gen.fill(gen.F32, shape, 11, 1)
    v = gen.fill(gen.F32, shape, 11, 2)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.fwd(q, k, v, gen.F32, scale, causal)
    ob, lb = oracle.brute(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), scale, causal)
    assert np.max(np.abs(o - ob)) <= 1e-13 * max(1.0, np.max(np.abs(ob)))
    assert np.max(np.abs(lse - lb)) <= 1e-13 * max(1.0, np.max(np.abs(lb)))


@pytest.mark.parametrize("dtype", [gen.F16, gen.BF16])
def test_p1_oracle_widening_of_16bit_storage(dtype):
    """The oracle's own bf16/fp16 decoding equals numpy's exact widening."""
    shape = (1, 3, 37, 16)
    q = gen.fill(dtype, shape, 5, 0, 2.0)
    k = gen.fill(dtype, shape, 5, 1, 2.0)
    v = gen.fill(dtype, shape, 5, 2)
    o, lse = oracle.fwd(q, k, v, dtype, 0.25, 1)
    ob, lb = oracle.brute(gen.to_float64(q, dtype), gen.to_float64(k, dtype), gen.to_float64(v, dtype), 0.25, 1)
    assert np.max(np.abs(o - ob)) <= 1e-13
    assert np.max(np.abs(lse - lb)) <= 1e-13


def test_p1_fp16_special_values_decode():
    """Subnormal, largest finite and signed values of binary16 decode exactly."""
    vals = np.array([0.0, -0.0, 6.0e-8, 6.1e-5, 65504.0, -2.5, 1.0 / 3.0], dtype=np.float16)
    L, d = vals.size, 1
    # one query with q = 0 makes softmax uniform: O = mean of V exactly (in fp64)
    q = np.zeros((1, 1, L, d), np.float16)
    k = np.zeros((1, 1, L, d), np.float16)
    v = vals.reshape(1, 1, L, d)
    o, _ = oracle.fwd(q, k, v, gen.F16, 1.0, 0)
    assert o[0, 0, 0, 0] == pytest.approx(float(np.mean(vals.astype(np.float64))), rel=1e-15)


# ---- P2: the NumPy toy whose difference a page prints -----------------------

def test_p2_numpy_toy_printed_difference():
    fx = json.load(open(os.path.join(GOLDEN, "p3_numpy_toy.json")))
    N, D, BLK = fx["N"], fx["D"], fx["BLOCK"]
    rs = np.random.RandomState(fx["seed"])  # legacy generator, as the page seeds it
    Q = rs.randn(N, D)
    K = rs.randn(N, D)
    V = rs.randn(N, D)
    scale = 1.0 / math.sqrt(D)
    o, _ = _fwd64(Q, K, V, scale, 0)
    O_t, _, _ = tiled.fa2_forward(Q, K, V, scale, Br=N, Bc=BLK)
    diff = float(np.max(np.abs(o - O_t)))
    assert diff <= fx["page_assert_atol"]
    # the page prints machine-zero agreement; ours must be of the same order
    assert diff <= 8 * fx["printed_max_abs_diff"]


# ---- P3: the 16-score / 4-blocks-of-4 walk-through -----------------------------

def test_p3_walkthrough_sixteen_scores():
    """Running (m, l) after four blocks equal the two-pass (max, sum exp); once
    the maximum stops changing the correction factor is exactly 1.0; and the
    normalised result equals the one-pass softmax of all 16 scores."""
    x = np.array([0.3, -1.2, 0.8, 0.1,
                  2.9, 0.5, 3.4, -0.7,     # the maximum (3.4) arrives in block 2
                  1.1, -2.0, 0.0, 2.2,
                  -0.4, 1.7, 3.3, 0.9])
    m, l, corr = tiled.online_softmax_stats(x, 4)
    assert corr[0] == 0.0
    assert corr[1] < 1.0
    assert corr[2] == 1.0 and corr[3] == 1.0
    assert m == x.max()
    assert l == pytest.approx(np.exp(x - x.max()).sum(), rel=1e-15)
    # the oracle on one query row whose scores are x: d = 16, q = e0,
    # k_j = x_j e0, v_j = e_j, scale 1, so O row 0 is the softmax row itself
    L = d = 16
    Q = np.zeros((L, d)); Q[:, 0] = 1.0
    K = np.zeros((L, d)); K[:, 0] = x
    V = np.eye(L)
    o, lse = _fwd64(Q, K, V, 1.0, 0)
    np.testing.assert_allclose(o[0], scipy.special.softmax(x), rtol=1e-14, atol=0)
    np.testing.assert_allclose(o[0], np.exp(x - m) / l, rtol=1e-14, atol=0)
    assert lse[0] == pytest.approx(scipy.special.logsumexp(x), rel=1e-15)


# ---- P4: softmax rows sum to one; equality with library softmax/logsumexp ----

@pytest.mark.parametrize("causal", [0, 1])
def test_p4_rows_are_softmax(causal):
    """With V = I (L <= d) the output row is the probability row itself."""
    L, d = 48, 64
    Q, K, _ = _rng_inputs(L, d, 21, sigma=1.5)
    V = np.zeros((L, d)); V[:, :L] = np.eye(L)
    scale = 0.3
    o, lse = _fwd64(Q, K, V, scale, causal)
    P = o[:, :L]
    assert np.all(np.abs(P.sum(axis=1) - 1.0) <= 1e-15 * L)
    S = scale * (Q @ K.T)
    if causal:
        S = np.where(np.triu(np.ones((L, L), bool), k=1), -np.inf, S)
    np.testing.assert_allclose(P, scipy.special.softmax(S, axis=1), rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(S, axis=1), rtol=1e-13)
    assert np.all(o[:, L:] == 0.0)


# ---- P5: constant K gives the mean of V -------------------------------------

@pytest.mark.parametrize("causal", [0, 1])
def test_p5_constant_keys(causal):
    L, d = 50, 8
    Q, _, V = _rng_inputs(L, d, 31)
    kvec = gen.normal(31, 9, d)
    K = np.tile(kvec, (L, 1))
    scale = 0.7
    o, lse = _fwd64(Q, K, V, scale, causal)
    for i in range(L):
        n = i + 1 if causal else L
        np.testing.assert_allclose(o[i], V[:n].mean(axis=0), rtol=1e-12, atol=1e-14)
        assert lse[i] == pytest.approx(scale * float(Q[i] @ kvec) + math.log(n), rel=1e-13, abs=1e-13)


# ---- P6: one dominant score selects its value row ----------------------------

def test_p6_dominant_score():
    L, d = 64, 16
    Q, K, V = _rng_inputs(L, d, 41, sigma=0.1)
    i, jstar = 10, 37
    K[jstar] = Q[i] * (200.0 / float(Q[i] @ Q[i]))   # s_{i,j*} = 200 * scale
    scale = 1.0
    o, lse = _fwd64(Q, K, V, scale, 0)
    s = scale * (Q[i] @ K.T)
    gap = s[jstar] - np.max(np.delete(s, jstar))
    assert gap >= 60.0
    np.testing.assert_allclose(o[i], V[jstar], rtol=0, atol=L * math.exp(-60.0) * 10 + 1e-14)
    assert lse[i] == pytest.approx(s[jstar], rel=1e-15)


# ---- P7: causal row 0 and L = 1 ----------------------------------------------

def test_p7_causal_first_row_and_single_key():
    L, d = 33, 8
    Q, K, V = _rng_inputs(L, d, 51)
    o, lse = _fwd64(Q, K, V, 0.4, 1)
    np.testing.assert_array_equal(o[0], V[0])
    assert lse[0] == pytest.approx(0.4 * float(Q[0] @ K[0]), rel=1e-15)
    o1, lse1 = _fwd64(Q[:1], K[:1], V[:1], 0.4, 0)
    np.testing.assert_array_equal(o1[0], V[0])


# ---- P8: V = ones gives ones; linearity in V ---------------------------------

@pytest.mark.parametrize("causal", [0, 1])
def test_p8_ones_and_linearity_in_v(causal):
    L, d = 40, 8
    Q, K, V1 = _rng_inputs(L, d, 61)
    V2 = gen.normal(61, 5, L * d).reshape(L, d)
    o_ones, _ = _fwd64(Q, K, np.ones((L, d)), 0.5, causal)
    np.testing.assert_allclose(o_ones, 1.0, rtol=0, atol=1e-15 * L)
    a, b = 1.75, -0.5
    o1, _ = _fwd64(Q, K, V1, 0.5, causal)
    o2, _ = _fwd64(Q, K, V2, 0.5, causal)
    o12, _ = _fwd64(Q, K, a * V1 + b * V2, 0.5, causal)
    np.testing.assert_allclose(o12, a * o1 + b * o2, rtol=0, atol=1e-13)


# ---- P9: shift invariance of softmax; permutation invariance over keys ------

@pytest.mark.parametrize("causal", [0, 1])
def test_p9_key_shift(causal):
    L, d = 40, 8
    Q, K, V = _rng_inputs(L, d, 71)
    u = gen.normal(71, 6, d)
    scale = 0.6
    o, lse = _fwd64(Q, K, V, scale, causal)
    o_s, lse_s = _fwd64(Q, K + u, V, scale, causal)
    np.testing.assert_allclose(o_s, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse_s, lse + scale * (Q @ u), rtol=0, atol=1e-12)


def test_p9_key_permutation():
    L, d = 40, 8
    Q, K, V = _rng_inputs(L, d, 81)
    perm = np.argsort(gen.uniform01(81, 3, 0, L))
    o, lse = _fwd64(Q, K, V, 0.6, 0)
    o_p, lse_p = _fwd64(Q, K[perm], V[perm], 0.6, 0)
    np.testing.assert_allclose(o_p, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse_p, lse, rtol=0, atol=1e-13)


def test_causal_mask_direction():
    """Changing a key after query i leaves row i unchanged; changing one before it does not."""
    L, d = 20, 8
    Q, K, V = _rng_inputs(L, d, 91)
    i = 9
    o, _ = _fwd64(Q, K, V, 0.5, 1)
    K2, V2 = K.copy(), V.copy()
    K2[i + 1:] += 3.0
    V2[i + 1:] -= 2.0
    o2, _ = _fwd64(Q, K2, V2, 0.5, 1)
    np.testing.assert_array_equal(o2[: i + 1], o[: i + 1])
    V3 = V.copy(); V3[i] += 1.0
    o3, _ = _fwd64(Q, K, V3, 0.5, 1)
    assert np.all(np.abs(o3[i] - o[i]) > 0)


def test_rows_subset_matches_full():
    L, d = 70, 16
    Q, K, V = _rng_inputs(L, d, 93)
    rows = gen.sample_rows(L, 12, 4)
    o, lse = _fwd64(Q, K, V, 0.25, 1)
    o_r, lse_r = _fwd64(Q, K, V, 0.25, 1, rows)
    np.testing.assert_array_equal(o_r, o[rows])
    np.testing.assert_array_equal(lse_r, lse[rows])


# ---- P10: the tiled algorithm (both orders) reaches the plain result ---------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Br,Bc", [(1, 1), (4, 4), (16, 8), (8, 16), (7, 5), (64, 64), (128, 32)])
def test_p10_tiled_models_are_exact(Br, Bc, causal):
    L, d = 100, 16
    Q, K, V = _rng_inputs(L, d, 101, sigma=2.0)
    scale = 1.0 / 4.0
    o, lse = _fwd64(Q, K, V, scale, int(causal))
    O2, lse2, _ = tiled.fa2_forward(Q, K, V, scale, Br, Bc, causal)
    O1, lse1 = tiled.fa1_forward(Q, K, V, scale, Br, Bc, causal)
    np.testing.assert_allclose(O2, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-13)
    np.testing.assert_allclose(O1, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse1, lse, rtol=0, atol=1e-13)


def test_p10_equivalence_shape_of_the_teaching_check():
    """The teaching check's shape (B=2, H=4, L=128, d=64, blocks 32x32) in fp64."""
    fx = json.load(open(os.path.join(GOLDEN, "p1_equivalence.json")))
    B, H, L, d, blk = fx["B"], fx["H"], fx["L"], fx["d"], fx["block"]
    shape = (B, H, L, d)
    q = gen.fill(gen.F32, shape, 42, 0)
    k = gen.fill(gen.F32, shape, 42, 1)
    v = gen.fill(gen.F32, shape, 42, 2)
    scale = 1.0 / math.sqrt(d)
    for causal in (0, 1):
        o, lse = oracle.fwd(q, k, v, gen.F32, scale, causal)
        for b in range(B):
            for h in range(H):
                Qh, Kh, Vh = (x[b, h].astype(np.float64) for x in (q, k, v))
                O1, _ = tiled.fa1_forward(Qh, Kh, Vh, scale, blk, blk, bool(causal))
                assert np.max(np.abs(O1 - o[b, h])) < fx["max_abs_tol"] * 1e-6


def test_oracle_rejects_bad_arguments():
    q = np.zeros((1, 1, 4, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.fwd(q, q, q, gen.F32, 1.0, 2)
    with pytest.raises(ValueError):
        oracle.fwd(q, q, q, gen.F32, 1.0, 0, rows=[4])
    with pytest.raises(TypeError):
        oracle.fwd(q, q, q, gen.BF16, 1.0, 0)
