"""Float64 / plain-Python CPU oracle for the dimension grouping of [OAL]: the
contribution scores of Eq. 2 and the bootstrap tail-cut grouping of App. B
(Eq. 16-19).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check in
``__graft_entry__`` and ``bench.py``'s ``cpu_baseline`` leg may import this
module.  It shares no code with the HIP path and imports nothing from it.

Sources: [OAL] "Not All Dimensions Are Equal: Outlier-Aware Attention
Linearization with Grouped Quadratic Kernels", §3.1 (Eq. 2, the contribution of
dimension r on input p over its causal pair set, averaged with equal weight over
the P calibration inputs) and App. B "Dimension grouping" (sorting, the tail of
candidate cuts, Eq. 16 gap, Eq. 17 bootstrap separation, Eq. 18 support, natural
cuts, the G_min fallback, Eq. 19 groups).

Readings: Eq. 2 takes |q_{p,i,r} k_{p,j,r}| (the absolute
value that the HTML rendering and the second record show; the first PDF record
lost it); positions and dimensions are 0-based here, the cut k of the pages
(1-based, separating pi_1..pi_k from pi_{k+1}..pi_d) is the same integer k; the
fallback ranks unused candidates by (S_k, rho_k) descending and keeps the
candidate order (ascending k) on exact ties.

Pins: ``tests/test_grouping_oracle_pins.py``.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = ["contribution_prompt", "contribution", "sort_order", "candidate_cuts", "gaps",
           "bootstrap_support", "select_cuts", "groups_from_cuts", "group_head"]


def contribution_prompt(q, k):
    """chi_{p,r} of Eq. 2 for one prompt and one head: the mean over the causal
    pairs (i, j), j <= i, of |q_ir k_jr| / sqrt(d_h), pair by pair."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    n, d = q.shape
    acc = np.zeros(d)
    count = 0
    for i in range(n):
        for j in range(i + 1):
            acc += np.abs(q[i] * k[j])
            count += 1
    return acc / (count * math.sqrt(d))


def contribution(prompts):
    """chi_r of Eq. 2: equal-weight mean of chi_{p,r} over the prompts [(q, k), ...]."""
    return np.mean([contribution_prompt(q, k) for q, k in prompts], axis=0)


def sort_order(chi):
    """pi: dimensions by increasing chi, stable (ties keep the dimension order)."""
    return sorted(range(len(chi)), key=lambda r: (chi[r], r))


def candidate_cuts(d, alpha):
    """k in {max(1, d - m), .., d - 1}, m = ceil(alpha d)."""
    m = math.ceil(alpha * d)
    return list(range(max(1, d - m), d))


def gaps(chi, pi, cuts, eps):
    """Eq. 16: rho_k = chi_{pi_{k+1}} / max(chi_{pi_k}, eps), 1-based pi."""
    return {k: chi[pi[k]] / max(chi[pi[k - 1]], eps) for k in cuts}


def bootstrap_support(chi_prompts, pi, cuts, boot_idx, tau, eps):
    """Eq. 17-18: for replicate b with prompt indices I_b (with repetition),
    chi^(b) = mean over I_b of chi_{p,.}; R_k^(b) = min over U_k of chi^(b) /
    max(max over L_k of chi^(b), eps) with L_k = {pi_1..pi_k}, U_k the rest, the
    order pi of the full sample kept fixed; S_k = fraction of b with R_k >= tau."""
    chi_prompts = np.asarray(chi_prompts, dtype=np.float64)
    support = {k: 0 for k in cuts}
    for idx in boot_idx:
        chib = np.mean(chi_prompts[list(idx)], axis=0)
        for k in cuts:
            lower = [chib[pi[t]] for t in range(k)]
            upper = [chib[pi[t]] for t in range(k, len(pi))]
            if min(upper) / max(max(lower), eps) >= tau:
                support[k] += 1
    return {k: support[k] / len(boot_idx) for k in cuts}


def select_cuts(cuts, rho, support, tau, gamma, g_min):
    """Natural cuts (rho_k >= tau and S_k >= gamma); if they give fewer than
    g_min groups, add unused candidates by descending (S_k, rho_k), exact ties in
    candidate order, until g_min groups.  Returns the sorted cut list."""
    chosen = [k for k in cuts if rho[k] >= tau and support[k] >= gamma]
    if len(chosen) + 1 < g_min:
        rest = [k for k in cuts if k not in chosen]
        rest = sorted(rest, key=lambda k: (-support[k], -rho[k], cuts.index(k)))
        for k in rest:
            if len(chosen) + 1 >= g_min:
                break
            chosen.append(k)
    return sorted(chosen)


def groups_from_cuts(pi, cuts):
    """Eq. 19: with k_0 = 0 < k_1 < .. < k_{G-1} < k_G = d, group g holds
    pi_{k_{g-1}+1} .. pi_{k_g}; returns the label (1..G) of every dimension."""
    d = len(pi)
    bounds = [0] + list(cuts) + [d]
    label = [0] * d
    for g in range(1, len(bounds)):
        for t in range(bounds[g - 1], bounds[g]):
            label[pi[t]] = g
    return label


def group_head(chi_prompts, boot_idx, alpha, tau, gamma, g_min, eps=1e-12):
    """The whole grouping of one head from its per-prompt scores [P][d]:
    returns (labels, n_groups, cuts, rho, support)."""
    chi_prompts = np.asarray(chi_prompts, dtype=np.float64)
    chi = chi_prompts.mean(axis=0)
    d = chi.shape[0]
    pi = sort_order(chi)
    cuts = candidate_cuts(d, alpha)
    rho = gaps(chi, pi, cuts, eps)
    support = bootstrap_support(chi_prompts, pi, cuts, boot_idx, tau, eps)
    chosen = select_cuts(cuts, rho, support, tau, gamma, g_min)
    labels = groups_from_cuts(pi, chosen)
    return labels, len(chosen) + 1, chosen, rho, support
