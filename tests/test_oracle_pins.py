"""Pins of the float64 oracle against facts the pages and the mathematics fix.

Each test names the passage it follows.  They check the oracle against
something other than itself: closed forms, the glossary's worked example
(tests/golden/toy_linear_attention.json), brute force on tiny inputs and
invariances, chosen so that a dropped term, a wrong sign or index, a wrong
scale or a transposed factor in the oracle fails at least one of them.

[OAL] = "Not All Dimensions Are Equal: Outlier-Aware Attention Linearization
with Grouped Quadratic Kernels" (arXiv 2610.13674).
[GLOSSARY] = "Linear attention" (SelfMadeQuant glossary).
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import oal_oracle as O


def _rand_L(rng, G, diag="pos"):
    n = G + 1
    L = np.tril(rng.normal(0, 0.6, size=(n, n)))
    if diag == "pos":
        L[np.diag_indices(n)] = np.abs(np.diag(L)) + 0.3
    elif diag == "zero":
        L[np.diag_indices(n)] = 0.0
    elif diag == "neg":
        L[np.diag_indices(n)] = -np.abs(np.diag(L)) - 0.1
    # junk above the diagonal must be ignored ([OAL] §4.3: L is lower triangular)
    L = L + np.triu(rng.normal(0, 5.0, size=(n, n)), 1)
    return L


def _rand_groups(rng, d, G):
    """Random map of d dims onto groups 1..G with every group non-empty."""
    g = np.concatenate([np.arange(1, G + 1), rng.integers(1, G + 1, size=d - G)])
    return rng.permutation(g)


# --- P1: positivity, [OAL] §4.3 (kappa >= eps > 0 since L L^T is PSD) -------

@pytest.mark.parametrize("G", [1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("diag", ["pos", "zero", "neg"])
def test_p1_kappa_positive(G, diag):
    rng = np.random.default_rng(100 + G)
    d = 16
    L = _rand_L(rng, G, diag)
    g = _rand_groups(rng, d, G)
    eps = 1e-3
    q = rng.normal(size=(400, d)) * rng.uniform(0.1, 10, size=(1, d))
    k = rng.normal(size=(400, d)) * rng.uniform(0.1, 10, size=(1, d))
    kap = O.kappa_grouped(q, k, L, g, G, eps)
    assert np.all(kap >= eps)
    # sharper: ||L^T s_bar||^2 >= sigma_min(L)^2 ||s_bar||^2 >= sigma_min(L)^2
    smin = np.linalg.svd(np.tril(L), compute_uv=False).min()
    assert np.all(kap >= eps + smin ** 2 * (1 - 1e-12))


def test_p1_zero_L_gives_eps():
    rng = np.random.default_rng(1)
    q, k = rng.normal(size=(10, 8)), rng.normal(size=(10, 8))
    g = _rand_groups(rng, 8, 3)
    kap = O.kappa_grouped(q, k, np.zeros((4, 4)), g, 3, 0.25)
    assert np.array_equal(kap, np.full(10, 0.25))


# --- P2: constant values give that constant (weights are a convex combination)

def test_p2_constant_values():
    rng = np.random.default_rng(2)
    N, d, G = 97, 64, 4
    q = rng.normal(size=(N, d)) * 3
    k = rng.normal(size=(N, d)) * 3
    v = np.full((N, 64), -1.75)
    L = _rand_L(rng, G)
    y = O.causal_attention(q, k, v, L, _rand_groups(rng, d, G), G, 1e-6, row_block=32)
    np.testing.assert_allclose(y, -1.75, rtol=1e-14, atol=0)


# --- P3: L = e0 e0^T gives kappa = 1 + eps, so y_i is the causal prefix mean -

def test_p3_prefix_mean():
    rng = np.random.default_rng(3)
    N, d, G = 130, 64, 5
    q, k, v = rng.normal(size=(N, d)), rng.normal(size=(N, d)), rng.normal(size=(N, 64))
    L = np.zeros((G + 1, G + 1))
    L[0, 0] = 1.0
    y = O.causal_attention(q, k, v, L, _rand_groups(rng, d, G), G, 0.3, row_block=50)
    expect = np.cumsum(v, axis=0) / np.arange(1, N + 1)[:, None]
    np.testing.assert_allclose(y, expect, rtol=1e-13, atol=1e-14)


# --- P4: the first output is the first value ([OAL] Eq. 5 sums j <= i) -------

def test_p4_first_row():
    rng = np.random.default_rng(4)
    q, k, v = rng.normal(size=(5, 64)), rng.normal(size=(5, 64)), rng.normal(size=(5, 64))
    y = O.causal_attention(q, k, v, _rand_L(rng, 3), _rand_groups(rng, 64, 3), 3, 1e-6)
    np.testing.assert_allclose(y[0], v[0], rtol=1e-15, atol=0)


# --- P5: the glossary's toy example ([GLOSSARY] "An equality within one kernel")

def _toy(golden_dir):
    with open(os.path.join(golden_dir, "toy_linear_attention.json")) as f:
        return json.load(f)


def test_p5_toy_kappa_dim_and_state(golden_dir):
    t = _toy(golden_dir)
    q = np.array(t["q"])
    K = np.array(t["keys"])
    v = np.array(t["values"])[:, None]
    d = 2
    # identity feature map == kappa_dim with a = 0, b_r = sqrt(d_h), C = 0:
    # sum_r b_r x_r = sum_r q_r k_r
    a, b, C = 0.0, np.full(d, math.sqrt(d)), np.zeros((d, d))
    sims = O.kappa_dim(q[None, :], K, a, b, C)
    np.testing.assert_allclose(sims, t["similarities"], rtol=1e-15)
    np.testing.assert_allclose(sims / sims.sum(), t["weights"], rtol=1e-15)
    # aggregate-then-read: H1 columns are S (value channel) and z (ones channel)
    state = O.canonical_state(K, v)
    H1 = state[1:1 + d]
    np.testing.assert_allclose(H1[:, 0], t["S"], rtol=0, atol=0)
    np.testing.assert_allclose(H1[:, 1], t["z"], rtol=0, atol=0)
    # the recurrence's last-row readout gives numerator 8, denominator 3, y = 8/3
    Q = np.stack([q, q])
    y, ut = O.recurrence(Q, K, v, a, b, C, return_parts=True)
    np.testing.assert_allclose(ut[-1], [t["numerator"], t["denominator"]], rtol=1e-15)
    np.testing.assert_allclose(y[-1, 0], t["y"], rtol=1e-15)
    assert abs(y[-1, 0] - t["y_printed"]) < 5e-5
    # direct causal sum at the last position gives the same value
    yd = O.causal_attention_rows(q[None, :], [1], K, v,
                                 np.diag([0.0, 1.0, math.sqrt(2.0)]),
                                 np.array([1, 2]), 2, 0.0)
    np.testing.assert_allclose(yd[0, 0], t["y"], rtol=1e-15)


@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.5, 3.0])
def test_p5_toy_oal_native(golden_dir, eps):
    """g = (1, 2), L = diag(0, 1, sqrt 2): kappa = eps + s_1^2 + 2 s_2^2 with
    s_r = q_r k_r / sqrt 2, i.e. (2 + eps, 1 + eps), so y = (8 + 6 eps)/(3 + 2 eps)."""
    t = _toy(golden_dir)
    q = np.array(t["q"])
    K = np.array(t["keys"])
    v = np.array(t["values"])[:, None]
    L = np.diag([0.0, 1.0, math.sqrt(2.0)])
    g = np.array([1, 2])
    kap = O.kappa_grouped(q[None, :], K, L, g, 2, eps)
    np.testing.assert_allclose(kap, [2 + eps, 1 + eps], rtol=1e-15)
    y = O.causal_attention(np.stack([q, q]), K, v, L, g, 2, eps)
    np.testing.assert_allclose(y[1, 0], (8 + 6 * eps) / (3 + 2 * eps), rtol=1e-15)
    # causal form: the first position sees only the first key and value
    assert y[0, 0] == pytest.approx(t["values"][0], rel=1e-15)
    # the expanded coefficients reproduce the same weights
    a, b, C = O.expand_coeffs(L, g, 2, eps)
    np.testing.assert_allclose(O.kappa_dim(q[None, :], K, a, b, C), [2 + eps, 1 + eps],
                               rtol=1e-15)


# --- P6: direct sum == Algorithm 1 recurrence ([OAL] App. D Eq. 25) ----------

@pytest.mark.parametrize("d,N,G", [(4, 24, 2), (8, 20, 4), (8, 9, 1), (64, 5, 6)])
@pytest.mark.parametrize("packed", [False, True])
def test_p6_direct_equals_recurrence(d, N, G, packed):
    rng = np.random.default_rng(600 + d + N + G)
    q = rng.normal(size=(N, d)) * rng.uniform(0.5, 4, size=(1, d))
    k = rng.normal(size=(N, d)) * rng.uniform(0.5, 4, size=(1, d))
    v = rng.normal(size=(N, 3))
    L = _rand_L(rng, G)
    g = _rand_groups(rng, d, G)
    eps = 0.01
    y_direct = O.causal_attention(q, k, v, L, g, G, eps)
    a, b, C = O.expand_coeffs(L, g, G, eps)
    y_rec = O.recurrence(q, k, v, a, b, C, packed=packed)
    np.testing.assert_allclose(y_rec, y_direct, rtol=1e-11, atol=1e-12)


# --- P7: the Hadamard-diagonal identity ([OAL] Eq. 4, proof in App. D) ------

def test_p7_hd_identity_on_recurrence_numerator():
    rng = np.random.default_rng(7)
    N, d, dv = 6, 4, 3
    Q, K, V = rng.normal(size=(N, d)), rng.normal(size=(N, d)), rng.normal(size=(N, dv))
    lhs = ((Q @ K.T) * (Q @ K.T)) @ V                       # [(QK^T).(QK^T)] V
    rhs = np.stack([np.diag(Q @ K.T @ np.diag(V[:, l]) @ K @ Q.T) for l in range(dv)], 1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12)
    # kappa_dim with a = 0, b = 0, C_rt = d_h is (q.k)^2, so the recurrence's
    # numerator after all N tokens must equal row i of the left side
    a, b, C = 0.0, np.zeros(d), np.full((d, d), float(d))
    for i in range(N):
        Qi = np.vstack([Q[:N - 1], Q[i]])    # query i read at the last position
        for packed in (False, True):
            _, ut = O.recurrence(Qi, K, V, a, b, C, packed=packed, return_parts=True)
            np.testing.assert_allclose(ut[-1, :dv], lhs[i], rtol=1e-12)
            np.testing.assert_allclose(ut[-1, dv], np.sum((K @ Q[i]) ** 2), rtol=1e-12)


# --- P8: the learned global kernel embeds into OAL for any partition ---------
#         ([OAL] App. D Eq. 23; Taylor 1 + s + s^2/2, [OAL] §2)

@pytest.mark.parametrize("G", [1, 2, 4, 6])
def test_p8_global_embedding(G):
    rng = np.random.default_rng(800 + G)
    d = 32
    Lg = np.tril(rng.normal(size=(2, 2)))
    Mg = Lg @ Lg.T
    # grouped factor [E^T Lg | 0] with E = [[1, 0..0], [0, 1..1]]: lower triangular
    L = np.zeros((G + 1, G + 1))
    L[0, :2] = Lg[0]
    L[1:, :2] = Lg[1]
    g = _rand_groups(rng, d, G)
    q, k = rng.normal(size=(300, d)) * 2, rng.normal(size=(300, d)) * 2
    s = np.sum(q * k, axis=1) / math.sqrt(d)
    eps = 0.02
    expect = eps + Mg[0, 0] + 2 * Mg[0, 1] * s + Mg[1, 1] * s ** 2
    np.testing.assert_allclose(O.kappa_grouped(q, k, L, g, G, eps), expect, rtol=1e-12)
    # Taylor: M_global = [[1, 1/2], [1/2, 1/2]] gives eps + 1 + s + s^2 / 2
    Lt = np.linalg.cholesky(np.array([[1.0, 0.5], [0.5, 0.5]]))
    L2 = np.zeros((G + 1, G + 1))
    L2[0, :2] = Lt[0]
    L2[1:, :2] = Lt[1]
    np.testing.assert_allclose(O.kappa_grouped(q, k, L2, g, G, eps),
                               eps + 1 + s + s ** 2 / 2, rtol=1e-12)


# --- P9: invariance under a joint relabelling of dimensions and groups ------

def test_p9_permutation_invariance():
    rng = np.random.default_rng(9)
    N, d, G = 40, 64, 5
    q = rng.normal(size=(N, d)) * rng.uniform(0.5, 6, size=(1, d))
    k = rng.normal(size=(N, d)) * rng.uniform(0.5, 6, size=(1, d))
    v = rng.normal(size=(N, 8))
    L = _rand_L(rng, G)
    g = _rand_groups(rng, d, G)
    eps = 1e-4
    y = O.causal_attention(q, k, v, L, g, G, eps)
    pi = rng.permutation(d)                       # dimension permutation
    sigma = np.concatenate([[0], 1 + rng.permutation(G)])   # new label of old group
    P = np.zeros((G + 1, G + 1))
    P[sigma, np.arange(G + 1)] = 1.0
    Lf = np.tril(L)
    M2 = P @ (Lf @ Lf.T) @ P.T
    L2 = np.linalg.cholesky(M2)
    g2 = sigma[g][pi]
    y2 = O.causal_attention(q[:, pi], k[:, pi], v, L2, g2, G, eps)
    np.testing.assert_allclose(y2, y, rtol=1e-11, atol=1e-12)


# --- P10: state and parameter counts ([OAL] App. D) -------------------------

def test_p10_counts():
    assert O.state_size(64, 64) == 139425
    assert O.state_size(64, 64) * 4 == 557700
    assert O.ordered_state_size(64, 64) == 270465
    assert O.lower_factor_params(4) == 15
    assert O.lower_factor_params(5) == 21
    assert len(O.packed_pairs(64)) == 2080
    rng = np.random.default_rng(10)
    st = O.canonical_state(rng.normal(size=(3, 64)), rng.normal(size=(3, 64)))
    assert st.shape == (2145, 65) and st.size == 139425


# --- P11: grouped-query sharing ([OAL] App. D: GQA shares KV states) --------

def test_p11_gqa_mapping():
    rng = np.random.default_rng(11)
    B, Hq, Hkv, N, d = 2, 6, 2, 17, 64
    q = rng.normal(size=(B, Hq, N, d))
    k = rng.normal(size=(B, Hkv, N, d))
    v = rng.normal(size=(B, Hkv, N, 8))
    L = np.stack([_rand_L(rng, 3) for _ in range(Hq)])
    g = np.stack([_rand_groups(rng, d, 3) for _ in range(Hq)])
    G = np.full(Hq, 3)
    y = O.causal_attention_gqa(q, k, v, L, g, G, 1e-6)
    rep = Hq // Hkv
    y_rep = O.causal_attention_gqa(q, np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1),
                                   L, g, G, 1e-6)
    np.testing.assert_array_equal(y, y_rep)
    # and the mapping is contiguous: head 2 reads KV head 0, head 3 reads KV head 1
    y3 = O.causal_attention(q[1, 3], k[1, 1], v[1, 1], L[3], g[3], 3, 1e-6)
    np.testing.assert_array_equal(y[1, 3], y3)


# --- P12: coefficient expansion == the grouped kernel ([OAL] App. D Eq. 24) --

@pytest.mark.parametrize("G", [1, 2, 3, 4, 5, 6])
def test_p12_expand_matches_grouped_kernel(G):
    rng = np.random.default_rng(1200 + G)
    d = 64
    L = _rand_L(rng, G, diag="neg" if G % 2 else "pos")
    g = _rand_groups(rng, d, G)
    eps = 0.125
    q = rng.normal(size=(500, d)) * rng.uniform(0.2, 12, size=(1, d))
    k = rng.normal(size=(500, d)) * rng.uniform(0.2, 12, size=(1, d))
    a, b, C = O.expand_coeffs(L, g, G, eps)
    assert np.allclose(C, C.T)
    np.testing.assert_allclose(O.kappa_dim(q, k, a, b, C),
                               O.kappa_grouped(q, k, L, g, G, eps), rtol=1e-12)


# --- P13: the matrix-product row evaluator == the pairwise definition -------

def test_p13_rows_match_pairwise_definition():
    rng = np.random.default_rng(13)
    N, d, G = 23, 64, 4
    q = rng.normal(size=(N, d)) * 3
    k = rng.normal(size=(N, d)) * 3
    v = rng.normal(size=(N, 5))
    L = _rand_L(rng, G)
    g = _rand_groups(rng, d, G)
    eps = 1e-3
    y = O.causal_attention(q, k, v, L, g, G, eps, row_block=7)
    for i in range(N):
        w = np.array([O.kappa_grouped(q[i], k[j], L, g, G, eps) for j in range(i + 1)])
        np.testing.assert_allclose(y[i], (w @ v[: i + 1]) / w.sum(), rtol=1e-12)


# --- P14: the canonical state read out with the packed multiplicities equals
#          the direct numerator/denominator ([OAL] Eq. 6 and App. D) ---------

def test_p14_canonical_state_readout():
    rng = np.random.default_rng(14)
    N, d, G = 9, 64, 3
    q = rng.normal(size=(d,)) * 2
    k = rng.normal(size=(N, d)) * 2
    v = rng.normal(size=(N, 64))
    L = _rand_L(rng, G)
    g = _rand_groups(rng, d, G)
    eps = 1e-5
    st = O.canonical_state(k, v)
    a, b, C = O.expand_coeffs(L, g, G, eps)
    ut = a * st[0] + sum(b[r] * q[r] / math.sqrt(d) * st[1 + r] for r in range(d))
    for p, (r, t) in enumerate(O.packed_pairs(d)):
        m = 1.0 if r == t else 2.0
        ut = ut + m * C[r, t] * q[r] * q[t] / d * st[1 + d + p]
    _, num, den = O.causal_attention_rows(q[None], [N - 1], k, v, L, g, G, eps,
                                          return_parts=True)
    np.testing.assert_allclose(ut[:64], num[0], rtol=1e-11, atol=1e-9)
    np.testing.assert_allclose(ut[64], den[0], rtol=1e-12)


# --- P15: the dimension-specific kernel ([OAL] §4.1, Eq. 3) with arbitrary a, b,
#          C: direct sum == Algorithm 1 recurrence; the grouped kernel is the
#          special case of [OAL] §4.3; closed forms -----------------------------

def _rand_dim(rng, d, skew=1.0):
    """a, b, C with [[a, b^T/2], [b/2, sym(C)]] positive definite (so kappa_dim > 0)
    and no group structure, plus an antisymmetric part of C, which Eq. 3 ignores."""
    R = rng.normal(size=(d + 1, d + 1)) * rng.uniform(0.2, 1.5, size=(d + 1, 1))
    Mp = R @ R.T / (d + 1) + 0.05 * np.eye(d + 1)
    A = rng.normal(size=(d, d))
    return float(Mp[0, 0]), 2.0 * Mp[0, 1:], Mp[1:, 1:] + skew * (A - A.T)


@pytest.mark.parametrize("d,N", [(4, 15), (8, 12), (64, 5)])
def test_p15_dim_direct_equals_recurrence(d, N):
    rng = np.random.default_rng(1500 + d + N)
    q = rng.normal(size=(N, d)) * rng.uniform(0.5, 3, size=(1, d))
    k = rng.normal(size=(N, d)) * rng.uniform(0.5, 3, size=(1, d))
    v = rng.normal(size=(N, 5))
    a, b, C = _rand_dim(rng, d)
    y_direct = O.causal_attention_dim(q, k, v, a, b, C)
    y_rec = O.recurrence(q, k, v, a, b, C, packed=False)   # full C, unsymmetrised
    np.testing.assert_allclose(y_direct, y_rec, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("G", [1, 3, 6])
def test_p15_dim_reduces_to_grouped(G):
    rng = np.random.default_rng(1510 + G)
    N, d = 40, 64
    q = rng.normal(size=(N, d)) * 2
    k = rng.normal(size=(N, d)) * 2
    v = rng.normal(size=(N, 64))
    L = _rand_L(rng, G)
    g = _rand_groups(rng, d, G)
    a, b, C = O.expand_coeffs(L, g, G, 1e-3)
    np.testing.assert_allclose(O.causal_attention_dim(q, k, v, a, b, C),
                               O.causal_attention(q, k, v, L, g, G, 1e-3), rtol=1e-10, atol=1e-12)


def test_p15_dim_closed_forms():
    rng = np.random.default_rng(1520)
    N, d = 30, 64
    q = rng.normal(size=(N, d))
    k = rng.normal(size=(N, d))
    v = rng.normal(size=(N, 64))
    # b = 0, C = 0: equal weights, the causal prefix mean
    y = O.causal_attention_dim(q, k, v, 0.7, np.zeros(d), np.zeros((d, d)))
    np.testing.assert_allclose(y, np.cumsum(v, axis=0) / np.arange(1, N + 1)[:, None], rtol=1e-12)
    # a = 0, b = 0, C = d I: kappa = sum_r (q_r k_r)^2, written out for one row
    y = O.causal_attention_dim(q, k, v, 0.0, np.zeros(d), d * np.eye(d))
    w = ((q[17][None, :] * k[:18]) ** 2).sum(axis=1)
    np.testing.assert_allclose(y[17], w @ v[:18] / w.sum(), rtol=1e-12)
    # the antisymmetric part of C leaves every output unchanged
    a, b, C = _rand_dim(rng, d, skew=0.0)
    A = rng.normal(size=(d, d)) * 3
    np.testing.assert_allclose(O.causal_attention_dim(q, k, v, a, b, C + A - A.T),
                               O.causal_attention_dim(q, k, v, a, b, C), rtol=1e-11, atol=1e-13)


# --- P16: the backward oracle against central finite differences of the
#          (pinned) forward oracles: every gradient, both parameterisations ------

def _fd(f, x, h=1e-6):
    """Central differences of the scalar function f at every entry of x."""
    x = np.array(x, dtype=np.float64)
    out = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        xp = x.copy(); xp[idx] += h
        xm = x.copy(); xm[idx] -= h
        out[idx] = (f(xp) - f(xm)) / (2 * h)
    return out


def test_p16_dim_grad_matches_finite_differences():
    rng = np.random.default_rng(1600)
    N, d, dv = 9, 4, 3
    q = rng.normal(size=(N, d)) * 1.5
    k = rng.normal(size=(N, d)) * 1.5
    v = rng.normal(size=(N, dv))
    dy = rng.normal(size=(N, dv))
    a, b, C = _rand_dim(rng, d, skew=0.7)
    dq, dk, dvv, da, db, dC = O.causal_attention_dim_grad(q, k, v, a, b, C, dy)
    loss = lambda q_, k_, v_, a_, b_, C_: float(np.sum(dy * O.causal_attention_dim(q_, k_, v_, a_, b_, C_)))
    np.testing.assert_allclose(dq, _fd(lambda x: loss(x, k, v, a, b, C), q), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dk, _fd(lambda x: loss(q, x, v, a, b, C), k), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dvv, _fd(lambda x: loss(q, k, x, a, b, C), v), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(da, _fd(lambda x: loss(q, k, v, float(x), b, C), np.array(a)), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(db, _fd(lambda x: loss(q, k, v, a, x, C), b), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dC, _fd(lambda x: loss(q, k, v, a, b, x), C), rtol=1e-6, atol=1e-8)
    assert np.allclose(dC, dC.T)


@pytest.mark.parametrize("G", [1, 3])
def test_p16_grouped_L_grad_matches_finite_differences(G):
    rng = np.random.default_rng(1610 + G)
    N, d = 8, 8
    q = rng.normal(size=(N, d)) * 1.5
    k = rng.normal(size=(N, d)) * 1.5
    v = rng.normal(size=(N, 5))
    dy = rng.normal(size=(N, 5))
    L = _rand_L(rng, G)
    g = _rand_groups(rng, d, G)
    eps = 1e-3
    a, b, C = O.expand_coeffs(L, g, G, eps)
    _, _, _, da, db, dC = O.causal_attention_dim_grad(q, k, v, a, b, C, dy)
    dL = O.grouped_coeff_grad(L, g, G, da, db, dC)
    fd = _fd(lambda x: float(np.sum(dy * O.causal_attention(q, k, v, x, g, G, eps))), L)
    fd = np.tril(fd)          # entries above the diagonal do not enter (the oracle ignores them)
    np.testing.assert_allclose(dL, fd, rtol=1e-6, atol=1e-8)


def test_p16_row_restriction_equals_zeroed_dy():
    rng = np.random.default_rng(1620)
    N, d = 12, 8
    q, k, v = rng.normal(size=(N, d)), rng.normal(size=(N, d)), rng.normal(size=(N, 4))
    dy = rng.normal(size=(N, 4))
    a, b, C = _rand_dim(rng, d)
    rows = [3, 7, 8, 11]
    dz = np.zeros_like(dy)
    dz[rows] = dy[rows]
    full = O.causal_attention_dim_grad(q, k, v, a, b, C, dz)
    part = O.causal_attention_dim_grad(q, k, v, a, b, C, dy, rows=rows)
    for x, y in zip(full, part):
        np.testing.assert_allclose(np.asarray(y), np.asarray(x), rtol=1e-12, atol=1e-14)
