"""Float64 CPU oracle for the exact softmax attention that OAL approximates, and
for the fidelity metrics the pages report against it.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check in
``__graft_entry__`` and ``bench.py`` may import this module.  It shares no code
with the HIP path and imports nothing from it.

Sources (cited by title and section/equation):

* [OAL] "Not All Dimensions Are Equal: Outlier-Aware Attention Linearization
  with Grouped Quadratic Kernels": the exact (softmax) attention of §3 with
  scores q_i . k_j / sqrt(d_h) over the causal prefix j <= i, and the
  frozen-attention error metrics of App. C, Eqs. 21-22.

Every function is pinned in ``tests/test_softmax_oracle_pins.py`` against closed
forms (constant values, zero queries, one dominant key, two tokens written out,
metrics of scaled and shifted outputs).
"""

from __future__ import annotations

import math

import numpy as np

__all__ = ["softmax_attention", "softmax_attention_gqa", "fidelity"]


def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, d_h: int | None = None,
                      row_block: int = 512) -> np.ndarray:
    """Causal softmax attention of one head ([OAL] §3): for every i,
    y_i = sum_{j <= i} exp(s_ij) v_j / sum_{j <= i} exp(s_ij), s_ij = q_i . k_j / sqrt(d_h).
    q [N, d_h], k [N, d_h], v [N, d_v]; float64.  Each row subtracts its largest
    score before the exponential (the ratio is unchanged)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    d_h = q.shape[1] if d_h is None else d_h
    y = np.empty((n, v.shape[1]), dtype=np.float64)
    for i0 in range(0, n, row_block):
        i1 = min(n, i0 + row_block)
        s = q[i0:i1] @ k[:i1].T / math.sqrt(d_h)             # [rows, keys]
        rows = np.arange(i0, i1)[:, None]
        s = np.where(np.arange(i1)[None, :] <= rows, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        y[i0:i1] = (p @ v[:i1]) / p.sum(axis=1, keepdims=True)
    return y


def softmax_attention_gqa(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Grouped-query layout: q [B, Hq, N, d], k/v [B, Hkv, N, d]; query head h
    reads KV head h // (Hq / Hkv)."""
    B, Hq = q.shape[:2]
    Hkv = k.shape[1]
    rep = Hq // Hkv
    out = np.empty(q.shape[:3] + (v.shape[-1],), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            out[b, h] = softmax_attention(q[b, h], k[b, h // rep], v[b, h // rep])
    return out


def fidelity(approx, exact) -> tuple[float, float]:
    """[OAL] App. C: over sequences b = 1..B (the outputs of all heads of one
    sequence in one array each), MSE = mean_b ||Y^_b - Y_b||_F^2 / n_b (n_b the
    number of output elements of sequence b, Eq. 21) and
    RelMSE = mean_b ||Y^_b - Y_b||_F^2 / ||Y_b||_F^2 (Eq. 22)."""
    mse, rel = [], []
    for a, e in zip(approx, exact):
        a = np.asarray(a, dtype=np.float64)
        e = np.asarray(e, dtype=np.float64)
        err = float(np.sum((a - e) ** 2))
        mse.append(err / e.size)
        rel.append(err / float(np.sum(e ** 2)))
    return float(np.mean(mse)), float(np.mean(rel))
