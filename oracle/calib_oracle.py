"""Float64 CPU oracle for the coefficient calibration of [OAL] App. B (Eq. 20):
output matching of the causal OAL output to softmax attention, optimised with
Adam under gradient-norm clipping.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check in
``__graft_entry__`` and ``bench.py``'s ``cpu_baseline`` leg may import this
module.  It shares no code with the HIP path and imports nothing from it.

Sources:

* [OAL] "Not All Dimensions Are Equal: Outlier-Aware Attention Linearization
  with Grouped Quadratic Kernels": App. B "Coefficient calibration" (Eq. 20, the
  output-matching objective over causal query positions; Adam at learning rate
  0.02, 32 sampled query positions per update, gradient norm clipped at 10,
  validation every 100 updates, early stopping after 400 updates without
  improvement) and App. D (the learned global quadratic, Eq. 23, and its
  embedding into the grouped parameterisation; the second-order Taylor start).
* Adam: Kingma and Ba, "Adam: A Method for Stochastic Optimization" (ICLR 2015),
  Algorithm 1 (bias-corrected first and second moment estimates).

Readings: the per-update objective is Eq. 20 restricted to
the sampled positions S of one sequence, averaged over them:
loss = (1 / (2 |S|)) sum_{i in S} ||y^_i - y_i^softmax||^2; the clipping norm is
the Euclidean norm of one head's gradient over the entries of L that are
parameters (the lower triangle of the leading (G+1) block); Adam uses
beta1 = 0.9, beta2 = 0.999, eps = 1e-8 (the pages give only the learning rate).

Pins: ``tests/test_calib_oracle_pins.py``.
"""

from __future__ import annotations

import math

import numpy as np

from oracle import oal_oracle as O

__all__ = ["output_match_loss_grad", "param_mask", "adam_step", "taylor_L", "global_embedding_L",
           "calibrate"]


def output_match_loss_grad(q, k, v, y_ref, positions, L, group_map, n_groups, eps):
    """One head, one sequence: loss = (1/(2|S|)) sum_{i in S} ||y^_i - y_ref_i||^2
    ([OAL] Eq. 20 on the sampled positions S) and its gradient with respect to L,
    through the gradient oracle (dy_i = (y^_i - y_ref_i) / |S| on S, zero
    elsewhere) and the grouped map.  Returns (loss, dL)."""
    positions = np.asarray(sorted(set(int(p) for p in positions)), dtype=np.int64)
    n_s = len(positions)
    y = O.causal_attention_rows(np.asarray(q, dtype=np.float64)[positions], positions, k, v, L,
                                group_map, n_groups, eps)
    diff = y - np.asarray(y_ref, dtype=np.float64)[positions]
    loss = float(np.sum(diff ** 2) / (2.0 * n_s))
    dy = np.zeros((np.asarray(q).shape[0], np.asarray(v).shape[1]))
    dy[positions] = diff / n_s
    a, b, C = O.expand_coeffs(L, group_map, n_groups, eps)
    _, _, _, da, db, dC = O.causal_attention_dim_grad(q, k, v, a, b, C, dy, rows=positions)
    return loss, O.grouped_coeff_grad(L, group_map, n_groups, da, db, dC)


def param_mask(shape, n_groups):
    """The entries of L that are parameters: lower triangle of the leading
    (G+1) x (G+1) block ([OAL] §4.3: L is lower triangular)."""
    m = np.zeros(shape, dtype=bool)
    n = n_groups + 1
    m[:n, :n] = np.tril(np.ones((n, n), dtype=bool))
    return m


def adam_step(L, g, m, v, t, mask, lr=0.02, beta1=0.9, beta2=0.999, eps=1e-8, clip=10.0):
    """Clip g to Euclidean norm <= clip over the masked entries, then one Adam
    update (Kingma and Ba, Algorithm 1) of those entries; t is the 1-based step.
    Returns (L, m, v) as new arrays."""
    L = np.array(L, dtype=np.float64)
    g = np.where(mask, np.asarray(g, dtype=np.float64), 0.0)
    norm = math.sqrt(float(np.sum(g ** 2)))
    if norm > clip:
        g = g * (clip / norm)
    m = np.where(mask, beta1 * np.asarray(m, dtype=np.float64) + (1 - beta1) * g, 0.0)
    v = np.where(mask, beta2 * np.asarray(v, dtype=np.float64) + (1 - beta2) * g * g, 0.0)
    m_hat = m / (1 - beta1 ** t)
    v_hat = v / (1 - beta2 ** t)
    L = np.where(mask, L - lr * m_hat / (np.sqrt(v_hat) + eps), L)
    return L, m, v


def taylor_L(n_groups, g_max=None):
    """L of the second-order Taylor start exp(s) ~ 1 + s + s^2/2 with s = q.k/sqrt(d_h)
    in the grouped form ([OAL] App. D: the global polynomial a + b s + c s^2 with
    M_00 = a - eps ~ 1, M_{0g} = b/2 = 1/2, M_{gh} = c = 1/2 for all groups):
    rows g >= 1 of L are (1/2, 1/2, 0, ...), row 0 is (1, 0, ...)."""
    g_max = n_groups if g_max is None else g_max
    L = np.zeros((g_max + 1, g_max + 1))
    L[0, 0] = 1.0
    L[1:n_groups + 1, 0] = 0.5
    L[1:n_groups + 1, 1] = 0.5
    return L


def global_embedding_L(M_global, n_groups, g_max=None):
    """Embed a learned global quadratic M_global (2x2, PSD; [OAL] App. D Eq. 23)
    into the grouped parameterisation: M_00 = m00, M_{0g} = M_{g0} = m01,
    M_{gh} = m11 for all groups, factored as L with rows g >= 1 equal to
    (m01 / l00, l11, 0, ...) where l00 = sqrt(m00), l11 = sqrt(m11 - m01^2 / m00)."""
    g_max = n_groups if g_max is None else g_max
    M_global = np.asarray(M_global, dtype=np.float64)
    l00 = math.sqrt(M_global[0, 0])
    l10 = M_global[0, 1] / l00
    l11 = math.sqrt(max(M_global[1, 1] - l10 * l10, 0.0))
    L = np.zeros((g_max + 1, g_max + 1))
    L[0, 0] = l00
    L[1:n_groups + 1, 0] = l10
    L[1:n_groups + 1, 1] = l11
    return L


def calibrate(train, L0, group_map, n_groups, eps, schedule, lr=0.02, clip=10.0):
    """Adam on one head's L over a fixed schedule of updates; ``train`` is a list
    of (q, k, v, y_ref) and ``schedule`` a list of (sequence index, positions).
    Returns the list of L after each update and the list of losses."""
    L = np.array(L0, dtype=np.float64)
    mask = param_mask(L.shape, n_groups)
    m = np.zeros_like(L)
    v = np.zeros_like(L)
    Ls, losses = [], []
    for t, (si, pos) in enumerate(schedule, start=1):
        q, k, vv, y_ref = train[si]
        loss, g = output_match_loss_grad(q, k, vv, y_ref, pos, L, group_map, n_groups, eps)
        L, m, v = adam_step(L, g, m, v, t, mask, lr=lr, clip=clip)
        Ls.append(L.copy())
        losses.append(loss)
    return Ls, losses
