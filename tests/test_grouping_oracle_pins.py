"""Pins of the grouping oracle ([OAL] Eq. 2 and App. B, Eq. 16-19) against
closed forms, profiles with known cuts, hand-counted bootstrap support and the
G_min fallback rules.  CPU only."""

import math

import numpy as np

from oracle import grouping_oracle as GR


def test_contribution_closed_forms():
    rng = np.random.default_rng(1)
    n, d = 9, 16
    a = rng.uniform(0.5, 3.0, size=d)
    b = rng.uniform(0.5, 3.0, size=d)
    q = a * rng.choice([-1.0, 1.0], size=(n, d))          # |q_ir| = a_r at every position
    k = b * rng.choice([-1.0, 1.0], size=(n, d))
    np.testing.assert_allclose(GR.contribution_prompt(q, k), a * b / math.sqrt(d), rtol=1e-12)
    # one token: the single pair (0, 0)
    np.testing.assert_allclose(GR.contribution_prompt(q[:1] * 2, k[:1]),
                               np.abs(2 * q[0] * k[0]) / 4.0, rtol=1e-12)
    # equal weights per prompt, not per pair: a 1-token and a 9-token prompt
    chi = GR.contribution([(q[:1], k[:1]), (q, k)])
    np.testing.assert_allclose(chi, 0.5 * (GR.contribution_prompt(q[:1], k[:1]) +
                                           GR.contribution_prompt(q, k)), rtol=1e-12)


def test_sort_order_and_candidates():
    assert GR.sort_order([3.0, 1.0, 3.0, 1.0, 2.0]) == [1, 3, 4, 0, 2]
    assert GR.candidate_cuts(64, 0.25) == list(range(48, 64))
    assert GR.candidate_cuts(64, 0.5) == list(range(32, 64))
    assert GR.candidate_cuts(64, 0.001) == [63]
    assert GR.candidate_cuts(64, 1.0) == list(range(1, 64))


def _perm_profile(seed, levels):
    rng = np.random.default_rng(seed)
    perm = rng.permutation(len(levels))
    chi = np.empty(len(levels))
    chi[perm] = levels                 # dim perm[t] holds the t-th smallest level
    return chi, perm


def test_staircase_gives_its_natural_cuts():
    levels = np.array([1.0] * 58 + [4.0, 4.0, 16.0, 16.0, 64.0, 64.0])
    chi, perm = _perm_profile(2, levels)
    prompts = np.tile(chi, (5, 1))                       # identical prompts: support 1
    boot = np.random.default_rng(3).integers(0, 5, size=(50, 5))
    labels, G, cuts, rho, sup = GR.group_head(prompts, boot, 0.25, 1.5, 0.9, 2)
    assert cuts == [58, 60, 62] and G == 4
    assert rho[58] == 4.0 and rho[59] == 1.0 and sup[58] == 1.0
    want = np.empty(64, dtype=int)
    want[perm] = [1] * 58 + [2, 2, 3, 3, 4, 4]
    assert list(want) == labels


def test_bootstrap_support_counted_by_hand():
    # two prompts whose outlier dims differ: dim 5 large in prompt 0, dim 9 in 1
    base = np.ones(16)
    p0, p1 = base.copy(), base.copy()
    p0[5], p0[9] = 10.0, 3.0
    p1[5], p1[9] = 3.0, 10.0
    chi_p = np.stack([p0, p1])
    chi = chi_p.mean(axis=0)                             # dims 5 and 9 tie at 6.5
    pi = GR.sort_order(chi)
    assert pi[-2:] == [5, 9]
    boot = [(0, 0), (0, 1), (1, 0), (1, 1)]              # every replicate of P = 2 once
    sup = GR.bootstrap_support(chi_p, pi, [14, 15], boot, 1.5, 1e-12)
    # k = 14 (bulk | {5, 9}): min(upper) / max(lower) = 3, 6.5, 6.5, 3 -> all >= 1.5
    # k = 15 ({.., 5} | {9}): chi9 / max(chi5, 1) = 0.3, 1, 1, 3.33 -> only (1, 1) passes
    assert sup[14] == 1.0 and sup[15] == 0.25


def test_fallback_reaches_g_min_by_support_then_gap():
    levels = np.array([1.0] * 60 + [1.2, 1.3, 1.3 * 1.2, 1.3 * 1.2 * 1.1])
    chi, perm = _perm_profile(4, levels)
    prompts = np.tile(chi, (3, 1))
    boot = [(0, 1, 2)] * 10
    labels, G, cuts, rho, sup = GR.group_head(prompts, boot, 0.25, 1.5, 0.9, 2)
    # no natural cut (every gap < 1.5), every support 0: the largest gap wins
    assert all(s == 0.0 for s in sup.values())
    assert G == 2 and cuts == [max(rho, key=lambda k: (rho[k], -k))]
    assert cuts == [60]                                  # 1.2 / 1.0 is the largest gap


def test_fallback_ties_keep_candidate_order():
    cuts = [10, 11, 12, 13]
    rho = {10: 1.2, 11: 1.4, 12: 1.4, 13: 1.1}
    sup = {10: 0.5, 11: 0.2, 12: 0.2, 13: 0.5}
    # support first: 10 and 13 tie at 0.5, rho breaks it (1.2 > 1.1); then 11 before 12
    assert GR.select_cuts(cuts, rho, sup, 1.5, 0.9, 2) == [10]
    assert GR.select_cuts(cuts, rho, sup, 1.5, 0.9, 3) == [10, 13]
    assert GR.select_cuts(cuts, rho, sup, 1.5, 0.9, 4) == [10, 11, 13]
    rho2 = {10: 1.2, 11: 1.2, 12: 1.2, 13: 1.2}
    sup2 = {10: 0.3, 11: 0.3, 12: 0.3, 13: 0.3}
    assert GR.select_cuts(cuts, rho2, sup2, 1.5, 0.9, 3) == [10, 11]
