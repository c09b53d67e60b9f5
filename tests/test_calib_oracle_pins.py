"""Pins of the calibration oracle ([OAL] App. B Eq. 20, App. D Eq. 23; Adam,
Kingma and Ba 2015, Algorithm 1) against finite differences, closed forms and
a convex test problem.  CPU only."""

import math

import numpy as np
import pytest

from oracle import calib_oracle as K
from oracle import oal_oracle as O


def _case(seed, N=10, d=8, G=2):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(N, d)) * 1.5
    k = rng.normal(size=(N, d)) * 1.5
    v = rng.normal(size=(N, 5))
    g = np.concatenate([np.arange(1, G + 1), rng.integers(1, G + 1, size=d - G)])
    g = rng.permutation(g)
    L = np.tril(rng.normal(0, 0.6, size=(G + 1, G + 1)))
    L[np.diag_indices(G + 1)] = np.abs(np.diag(L)) + 0.3
    y_ref = rng.normal(size=(N, 5)) * 0.5
    return q, k, v, g, L, y_ref


def test_loss_grad_matches_finite_differences():
    q, k, v, g, L, y_ref = _case(1)
    G, eps = 2, 1e-3
    pos = [0, 3, 4, 9]
    loss, dL = K.output_match_loss_grad(q, k, v, y_ref, pos, L, g, G, eps)

    def f(Lx):
        y = O.causal_attention_rows(q[pos], pos, k, v, Lx, g, G, eps)
        return float(np.sum((y - y_ref[pos]) ** 2) / (2 * len(pos)))

    assert math.isclose(loss, f(L), rel_tol=1e-12)
    fd = np.zeros_like(L)
    h = 1e-6
    for i in range(L.shape[0]):
        for j in range(i + 1):
            Lp = L.copy(); Lp[i, j] += h
            Lm = L.copy(); Lm[i, j] -= h
            fd[i, j] = (f(Lp) - f(Lm)) / (2 * h)
    np.testing.assert_allclose(dL, fd, rtol=1e-6, atol=1e-9)


def test_loss_zero_at_own_output():
    q, k, v, g, L, _ = _case(2)
    y_self = O.causal_attention(q, k, v, L, g, 2, 1e-3)
    loss, dL = K.output_match_loss_grad(q, k, v, y_self, [1, 5, 7], L, g, 2, 1e-3)
    assert loss < 1e-28
    assert np.abs(dL).max() < 1e-13


def test_adam_first_step_closed_form():
    # m_hat = g and v_hat = g^2 after one step: the update is lr g / (|g| + eps)
    rng = np.random.default_rng(3)
    L = rng.normal(size=(3, 3))
    g = rng.normal(size=(3, 3))
    mask = K.param_mask((3, 3), 2)
    L1, m, v = K.adam_step(L, g, np.zeros((3, 3)), np.zeros((3, 3)), 1, mask, lr=0.02, clip=1e9)
    expect = np.where(mask, L - 0.02 * g / (np.abs(g) + 1e-8), L)
    np.testing.assert_allclose(L1, expect, rtol=1e-12, atol=1e-15)
    assert np.all(L1[~mask] == L[~mask])


def test_adam_clips_to_norm():
    g = np.zeros((3, 3)); g[1, 0] = 12.0; g[2, 2] = 16.0          # norm 20
    mask = K.param_mask((3, 3), 2)
    _, m, v = K.adam_step(np.zeros((3, 3)), g, np.zeros((3, 3)), np.zeros((3, 3)), 1, mask, clip=10.0)
    np.testing.assert_allclose(m[1, 0], 0.1 * 6.0)
    np.testing.assert_allclose(m[2, 2], 0.1 * 8.0)
    np.testing.assert_allclose(v[2, 2], 0.001 * 64.0)


def test_adam_minimises_a_quadratic():
    target = np.array([[0.7, 0.0], [-1.3, 2.1]])
    mask = K.param_mask((2, 2), 1)
    x = np.zeros((2, 2)); m = np.zeros((2, 2)); v = np.zeros((2, 2))
    for t in range(1, 2001):
        x, m, v = K.adam_step(x, x - target, m, v, t, mask, lr=0.02)
    np.testing.assert_allclose(x[mask], target[mask], atol=1e-3)


def test_taylor_start_is_the_second_order_polynomial():
    rng = np.random.default_rng(4)
    d, G = 16, 3
    g = rng.permutation(np.concatenate([np.arange(1, G + 1), rng.integers(1, G + 1, size=d - G)]))
    L = K.taylor_L(G, g_max=5)
    q, k = rng.normal(size=d), rng.normal(size=d)
    s = q @ k / math.sqrt(d)
    kap = O.kappa_grouped(q, k, L, g, G, 0.0)
    assert math.isclose(kap, 1 + s + s * s / 2, rel_tol=1e-12)
    assert np.all(L[G + 1:] == 0) and np.all(L[:, 2:] == 0)


def test_global_embedding_reproduces_eq23():
    rng = np.random.default_rng(5)
    d, G, eps = 16, 4, 1e-3
    g = rng.permutation(np.concatenate([np.arange(1, G + 1), rng.integers(1, G + 1, size=d - G)]))
    F = rng.normal(size=(2, 2))
    Mg = F @ F.T + 0.1 * np.eye(2)
    L = K.global_embedding_L(Mg, G)
    for _ in range(5):
        q, k = rng.normal(size=d), rng.normal(size=d)
        s = q @ k / math.sqrt(d)
        expect = eps + Mg[0, 0] + 2 * Mg[0, 1] * s + Mg[1, 1] * s * s
        assert math.isclose(O.kappa_grouped(q, k, L, g, G, eps), expect, rel_tol=1e-12)


def test_calibration_loop_lowers_the_loss():
    # fit L to the outputs of a different L of the same groups: the loss falls
    q, k, v, g, L, _ = _case(6, N=24)
    L_true = L.copy(); L_true[2, 1] += 0.8; L_true[1, 0] -= 0.5
    y_ref = O.causal_attention(q, k, v, L_true, g, 2, 1e-3)
    rng = np.random.default_rng(7)
    sched = [(0, rng.choice(24, size=8, replace=False)) for _ in range(150)]
    Ls, losses = K.calibrate([(q, k, v, y_ref)], L, g, 2, 1e-3, sched, lr=0.02)
    assert np.mean(losses[-10:]) < 0.2 * np.mean(losses[:10])
