"""Pins of the softmax oracle and the fidelity metrics against closed forms
([OAL] §3 exact attention; App. C, Eqs. 21-22).  CPU only."""

import math

import numpy as np

from oracle import softmax_oracle as S


def _rand(seed, n, d):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n, d)), rng.standard_normal((n, d)), rng.standard_normal((n, d))


def test_constant_values_pass_through():
    # a convex combination of equal vectors is that vector
    q, k, _ = _rand(1, 37, 64)
    c = np.linspace(-2.0, 3.0, 64)
    v = np.tile(c, (37, 1))
    np.testing.assert_allclose(S.softmax_attention(q, k, v), v, rtol=0, atol=1e-12)


def test_zero_queries_give_prefix_means():
    # all scores 0: uniform weights over j <= i
    _, k, v = _rand(2, 50, 64)
    q = np.zeros((50, 64))
    y = S.softmax_attention(q, k, v)
    expect = np.cumsum(v, axis=0) / np.arange(1, 51)[:, None]
    np.testing.assert_allclose(y, expect, rtol=1e-12, atol=1e-12)


def test_one_dominant_key():
    # q_i . k_3 / 8 exceeds every other score by 60: y_i = v_3 for i >= 3, while
    # the rows before 3 never see key 3
    rng = np.random.default_rng(3)
    n, d = 12, 64
    k = rng.standard_normal((n, d)) * 0.01
    u = np.zeros(d)
    u[5] = 1.0
    k[3] = 60.0 * math.sqrt(d) * u
    q = np.tile(u, (n, 1))
    v = rng.standard_normal((n, d))
    y = S.softmax_attention(q, k, v)
    np.testing.assert_allclose(y[3:], np.tile(v[3], (n - 3, 1)), rtol=0, atol=1e-20 + 1e-24)
    assert np.abs(y[:3] - v[3]).max() > 0.1


def test_two_tokens_written_out():
    q, k, v = _rand(4, 2, 64)
    y = S.softmax_attention(q, k, v)
    s0 = q[1] @ k[0] / 8.0
    s1 = q[1] @ k[1] / 8.0
    w1 = 1.0 / (1.0 + math.exp(s0 - s1))                 # logistic form of two weights
    np.testing.assert_allclose(y[0], v[0], rtol=1e-14)
    np.testing.assert_allclose(y[1], w1 * v[1] + (1.0 - w1) * v[0], rtol=1e-12)


def test_row_blocks_do_not_change_the_result():
    q, k, v = _rand(5, 300, 64)
    np.testing.assert_allclose(S.softmax_attention(q, k, v, row_block=7),
                               S.softmax_attention(q, k, v, row_block=512), rtol=1e-12, atol=1e-14)


def test_gqa_head_mapping():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((2, 6, 20, 64))
    k = rng.standard_normal((2, 2, 20, 64))
    v = rng.standard_normal((2, 2, 20, 64))
    y = S.softmax_attention_gqa(q, k, v)
    np.testing.assert_allclose(y[1, 4], S.softmax_attention(q[1, 4], k[1, 1], v[1, 1]), rtol=1e-14)
    np.testing.assert_allclose(y[0, 2], S.softmax_attention(q[0, 2], k[0, 0], v[0, 0]), rtol=1e-14)


def test_fidelity_metrics():
    rng = np.random.default_rng(7)
    a = rng.standard_normal((3, 10, 4))
    b = rng.standard_normal((5, 2))
    assert S.fidelity([a, b], [a, b]) == (0.0, 0.0)
    # doubling every output: RelMSE 1 for every sequence, MSE = mean square of Y
    mse, rel = S.fidelity([2 * a, 2 * b], [a, b])
    assert math.isclose(rel, 1.0, rel_tol=1e-14)
    assert math.isclose(mse, (np.mean(a ** 2) + np.mean(b ** 2)) / 2, rel_tol=1e-14)
    # a constant shift c: MSE c^2; RelMSE c^2 n_b / ||Y_b||^2 averaged over sequences
    mse, rel = S.fidelity([a + 0.5, b + 0.5], [a, b])
    assert math.isclose(mse, 0.25, rel_tol=1e-14)
    assert math.isclose(rel, (0.25 * a.size / np.sum(a ** 2) + 0.25 * b.size / np.sum(b ** 2)) / 2,
                        rel_tol=1e-14)
