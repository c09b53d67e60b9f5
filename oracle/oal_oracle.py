"""Float64 CPU oracle for OAL causal attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import this
module.  It shares no code with the HIP path and imports nothing from it: every
function here is a plain, slow restatement of the method's definitions in
float64 numpy.

Sources (cited by title and section/equation throughout):

* [OAL] "Not All Dimensions Are Equal: Outlier-Aware Attention Linearization
  with Grouped Quadratic Kernels" (Sun, Wu, Wang, Hu; arXiv 2610.13674).
* [GLOSSARY] "Linear attention" (SelfMadeQuant glossary), sections "Aggregate
  first, query second", "An equality within one kernel" and "A running state
  must respect the forecast clock".

Notation follows [OAL]: queries/keys are d_h-vectors, values d_v-vectors, the
per-dimension contribution is x_r = q_r k_r / sqrt(d_h) ([OAL] §4.1), groups are
labelled 1..G by a map g(r) ([OAL] §4.2) and s_bar = [1, s_1, .., s_G] with
s_g = sum_{r in group g} x_r ([OAL] §4.3).

Readings of the pages that this module fixes:

* causal sums include the current position j = i ([OAL] Eq. 5 sums over j <= i;
  Algorithm 1 adds token i to the states before its readout; [GLOSSARY] running
  state "including the current position");
* the 1/sqrt(d_h) scale uses the full head dimension for every group;
* only the lower triangle of L is used (entries above the diagonal are ignored);
* eps enters once per (i, j) weight through a = eps + M_00.

Every function has a pin in ``tests/test_oracle_pins.py`` that checks it against
something other than itself (closed forms, the glossary's worked example, brute
force on tiny inputs); none is "parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "lower_factor",
    "group_sums",
    "kappa_grouped",
    "expand_coeffs",
    "kappa_dim",
    "causal_attention",
    "causal_attention_rows",
    "causal_attention_gqa",
    "causal_attention_dim_rows",
    "causal_attention_dim",
    "causal_attention_dim_grad",
    "grouped_coeff_grad",
    "recurrence",
    "canonical_state",
    "packed_pairs",
    "state_size",
    "ordered_state_size",
    "lower_factor_params",
]


# ---------------------------------------------------------------------------
# Kernel definitions
# ---------------------------------------------------------------------------

def lower_factor(L: np.ndarray) -> np.ndarray:
    """The lower-triangular factor L of [OAL] §4.3 ("a learnable lower-triangular
    matrix L of size (G+1)x(G+1)"); entries above the diagonal are ignored."""
    return np.tril(np.asarray(L, dtype=np.float64))


def group_sums(x: np.ndarray, group_map: np.ndarray, n_groups: int) -> np.ndarray:
    """s_bar = [1, s_1, .., s_G] with s_g = sum of x_r over the dimensions r of
    group g ([OAL] §4.2 and the definition of s_bar under Eq. 7).

    ``x`` has the d_h contributions on its last axis; the result has G+1 entries
    on its first axis."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(group_map)
    out = np.empty((n_groups + 1,) + x.shape[:-1], dtype=np.float64)
    out[0] = 1.0
    for grp in range(1, n_groups + 1):
        out[grp] = x[..., g == grp].sum(axis=-1)
    return out


def kappa_grouped(q, k, L, group_map, n_groups, eps, d_h=None) -> np.ndarray:
    """kappa_OAL(q, k) = eps + s_bar^T L L^T s_bar  ([OAL] §4.3, Eq. 7).

    q and k broadcast against each other over leading axes; the last axis is
    the head dimension."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    d_h = q.shape[-1] if d_h is None else d_h
    x = q * k / math.sqrt(d_h)                      # [OAL] §4.1
    s_bar = group_sums(x, group_map, n_groups)      # [G+1, ...]
    Lf = lower_factor(L)[: n_groups + 1, : n_groups + 1]
    M = Lf @ Lf.T
    quad = np.einsum("uv,u...,v...->...", M, s_bar, s_bar)
    return eps + quad


def expand_coeffs(L, group_map, n_groups, eps):
    """Coefficient map of the positive group-aware kernel ([OAL] §4.3, the line
    after "set M = L L^T"): a = eps + M_00, b_r = 2 M_{0,g(r)},
    C_rt = M_{g(r),g(t)}.  Returns (a, b[d_h], C[d_h, d_h]) in the
    dimension-wise form of [OAL] Eq. 3."""
    Lf = lower_factor(L)[: n_groups + 1, : n_groups + 1]
    M = Lf @ Lf.T
    g = np.asarray(group_map, dtype=np.int64)
    a = float(eps + M[0, 0])
    b = 2.0 * M[0, g]
    C = M[np.ix_(g, g)]
    return a, b, C


def kappa_dim(q, k, a, b, C, d_h=None) -> np.ndarray:
    """kappa_dim(q, k) = a + sum_r b_r x_r + sum_{r,t} C_rt x_r x_t with
    x_r = q_r k_r / sqrt(d_h)  ([OAL] §4.1, Eq. 3)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    d_h = q.shape[-1] if d_h is None else d_h
    x = q * k / math.sqrt(d_h)
    lin = x @ np.asarray(b, dtype=np.float64)
    quad = np.einsum("...r,rt,...t->...", x, np.asarray(C, dtype=np.float64), x)
    return a + lin + quad


# ---------------------------------------------------------------------------
# Causal attention: the direct O(N^2) sum (the oracle proper)
# ---------------------------------------------------------------------------

def causal_attention_rows(q_rows, positions, k, v, L, group_map, n_groups, eps,
                          return_parts=False):
    """Causal OAL attention for selected query rows, evaluated directly.

    For query row q_i at 0-based position p_i the output is
    y_i = sum_{j <= p_i} kappa(q_i, k_j) v_j / sum_{j <= p_i} kappa(q_i, k_j)
    ([OAL] §2 linear-attention normalisation with the causal prefix of Eq. 5,
    the kernel of Eq. 7; [OAL] App. D Eq. 25 shows the linear-time readout of
    Eq. 6 equals exactly this sum).  Each row is independent, so the rows are
    simply evaluated side by side; no sum is reordered.

    q_rows: [R, d_h]; positions: [R] ints; k: [N, d_h]; v: [N, d_v].
    Returns y [R, d_v] (and, with return_parts, the numerator [R, d_v] and the
    denominator [R])."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    positions = np.asarray(positions, dtype=np.int64)
    R, d_h = q_rows.shape
    if R == 0:
        z = np.zeros((0, v.shape[1]))
        return (z, z, np.zeros(0)) if return_parts else z
    n_keys = int(positions.max()) + 1
    kk = k[:n_keys]
    g = np.asarray(group_map)
    # s_bar for every (row, key) pair: s_g[i, j] = sum_{r in group g} q_ir k_jr
    # / sqrt(d_h), i.e. a matrix product restricted to the group's columns.
    s_bar = np.empty((n_groups + 1, R, n_keys), dtype=np.float64)
    s_bar[0] = 1.0
    for grp in range(1, n_groups + 1):
        cols = g == grp
        s_bar[grp] = (q_rows[:, cols] @ kk[:, cols].T) / math.sqrt(d_h)
    Lf = lower_factor(L)[: n_groups + 1, : n_groups + 1]
    M = Lf @ Lf.T
    # kappa = eps + s_bar^T M s_bar  ([OAL] Eq. 7), for every (row, key) pair
    kap = np.full((R, n_keys), float(eps))
    for u_ in range(n_groups + 1):
        for v_ in range(n_groups + 1):
            if M[u_, v_] != 0.0:
                kap += M[u_, v_] * s_bar[u_] * s_bar[v_]
    del s_bar
    mask = np.arange(n_keys)[None, :] <= positions[:, None]   # j <= i
    kap = np.where(mask, kap, 0.0)
    num = kap @ v[:n_keys]
    den = kap.sum(axis=1)
    y = num / den[:, None]
    if return_parts:
        return y, num, den
    return y


def causal_attention(q, k, v, L, group_map, n_groups, eps, row_block=256):
    """Causal OAL attention of one head over a whole sequence, direct sum.

    q: [N, d_h]; k: [N, d_h]; v: [N, d_v]; returns y [N, d_v].  Rows are
    processed ``row_block`` at a time only to bound memory; each row is the
    definition in :func:`causal_attention_rows`."""
    q = np.asarray(q, dtype=np.float64)
    N = q.shape[0]
    y = np.empty((N, np.asarray(v).shape[1]), dtype=np.float64)
    for i0 in range(0, N, row_block):
        i1 = min(N, i0 + row_block)
        y[i0:i1] = causal_attention_rows(q[i0:i1], np.arange(i0, i1), k, v, L,
                                         group_map, n_groups, eps)
    return y


def causal_attention_dim_rows(q_rows, positions, k, v, a, b, C, return_parts=False):
    """Causal attention with the dimension-specific kernel of [OAL] §4.1 (Eq. 3),
    arbitrary a, b_r, C_rt: for query row q_i at 0-based position p_i,
    y_i = sum_{j <= p_i} kappa_dim(q_i, k_j) v_j / sum_{j <= p_i} kappa_dim(q_i, k_j)
    (the normalisation of [OAL] §2 over the causal prefix of Eq. 5).  One row at a
    time, each through :func:`kappa_dim`; C need not be symmetric.

    q_rows: [R, d_h]; positions: [R]; k: [N, d_h]; v: [N, d_v].  Returns y [R, d_v]
    (and, with return_parts, the numerator [R, d_v] and denominator [R])."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    positions = np.asarray(positions, dtype=np.int64)
    R = q_rows.shape[0]
    num = np.zeros((R, v.shape[1]))
    den = np.zeros(R)
    for i in range(R):
        n_keys = int(positions[i]) + 1
        kap = kappa_dim(q_rows[i][None, :], k[:n_keys], a, b, C)      # [n_keys]
        num[i] = kap @ v[:n_keys]
        den[i] = kap.sum()
    y = num / den[:, None] if R else np.zeros((0, v.shape[1]))
    if return_parts:
        return y, num, den
    return y


def causal_attention_dim(q, k, v, a, b, C):
    """:func:`causal_attention_dim_rows` for every row of one head's sequence."""
    q = np.asarray(q, dtype=np.float64)
    return causal_attention_dim_rows(q, np.arange(q.shape[0]), k, v, a, b, C)


def causal_attention_dim_grad(q, k, v, a, b, C, dy, rows=None):
    """Gradients of the causal attention of :func:`causal_attention_dim` (the
    dimension-specific kernel of [OAL] Eq. 3) for the loss sum_i dy_i . y_i, by
    differentiating the direct sum term by term (the chain rule written out).

    Per row i, with den_i = sum_{j<=i} kappa_ij and u_j = [v_j; 1]:
    g_i = [dy_i / den_i ; -(dy_i . y_i) / den_i] is the gradient with respect to
    the unnormalised [numerator; denominator] of row i, and alpha_ij = g_i . u_j
    the gradient with respect to kappa_ij.  With x_ij = q_i o k_j / sqrt(d_h) and
    w_ij = b + 2 sym(C) x_ij (the gradient of kappa_ij with respect to x_ij):
      dv_j = sum_{i>=j} kappa_ij g_i[:d_v]
      dq_i = sum_{j<=i} alpha_ij k_j o w_ij / sqrt(d_h)
      dk_j = sum_{i>=j} alpha_ij q_i o w_ij / sqrt(d_h)
      da = sum alpha_ij,  db = sum alpha_ij x_ij,  dC = sum alpha_ij x_ij x_ij^T.
    Returns (dq, dk, dv, da, db, dC); dC is symmetric (only sym(C) enters kappa).

    ``rows`` restricts the loss to those query rows (dy of the other rows taken
    as zero): then dq is exact on those rows, and dk_j, dv_j are exact for every
    key j whose rows i >= j are all included."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    N, d_h = q.shape
    d_v = v.shape[1]
    sq = math.sqrt(d_h)
    Cs = 0.5 * (C + C.T)
    u = np.concatenate([v, np.ones((N, 1))], axis=1)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    da = 0.0
    db = np.zeros(d_h)
    dC = np.zeros((d_h, d_h))
    for i in (range(N) if rows is None else sorted(set(int(r) for r in rows))):
        x = q[i][None, :] * k[: i + 1] / sq                       # [i+1, d_h]
        kap = a + x @ b + ((x @ C) * x).sum(axis=1)              # x_j^T C x_j per key
        ut = kap @ u[: i + 1]
        den = ut[d_v]
        y = ut[:d_v] / den
        g = np.append(dy[i] / den, -(dy[i] @ y) / den)
        alpha = u[: i + 1] @ g                                     # [i+1]
        w = b[None, :] + 2.0 * x @ Cs                              # [i+1, d_h]
        dq[i] = (alpha[:, None] * k[: i + 1] * w).sum(axis=0) / sq
        dk[: i + 1] += alpha[:, None] * q[i][None, :] * w / sq
        dv[: i + 1] += kap[:, None] * g[None, :d_v]
        da += alpha.sum()
        db += alpha @ x
        dC += (alpha[:, None] * x).T @ x
    return dq, dk, dv, da, db, dC


def grouped_coeff_grad(L, group_map, n_groups, da, db, dC):
    """Gradient with respect to L of a loss whose gradient with respect to the
    dimension-wise coefficients (a, b, C) of [OAL] Eq. 3 is (da, db, dC), through
    the grouped map of [OAL] §4.3 (a = eps + M_00, b_r = 2 M_{0,g(r)},
    C_rt = M_{g(r),g(t)}, M = L L^T).  In the group sums s_bar the kernel is
    eps + sum_uv M_uv s_bar_u s_bar_v, so the gradient with respect to the entry
    M_uv is sum alpha s_bar_u s_bar_v: dM_00 = da, dM_{0,gam} = dM_{gam,0} =
    sum_{r in gam} db_r, dM_{gam,del} = sum_{r in gam, t in del} dC_rt; then
    dL = (dM + dM^T) L, of which the lower triangle is returned (the entries of L
    above its diagonal are not parameters).  Shape as L."""
    L = np.asarray(L, dtype=np.float64)
    n = n_groups + 1
    g = np.asarray(group_map, dtype=np.int64)
    dM = np.zeros((n, n))
    dM[0, 0] = da
    for gam in range(1, n):
        cols = g == gam
        dM[0, gam] = dM[gam, 0] = np.sum(np.asarray(db)[cols])
        for dlt in range(1, n):
            dM[gam, dlt] = np.sum(np.asarray(dC)[np.ix_(cols, g == dlt)])
    Lf = lower_factor(L)[:n, :n]
    out = np.zeros_like(L)
    out[:n, :n] = np.tril((dM + dM.T) @ Lf)
    return out


def causal_attention_gqa(q, k, v, L, group_map, n_groups, eps, heads=None):
    """Grouped-query causal OAL attention.

    q: [B, Hq, N, d_h]; k, v: [B, Hkv, N, d]; L: [Hq, >=G+1, >=G+1];
    group_map: [Hq, d_h]; n_groups: [Hq].  Query head h reads KV head
    floor(h / (Hq / Hkv)) (contiguous grouped-query mapping; [OAL] App. D notes
    KV states can be shared across the query heads of a group).
    ``heads`` optionally restricts the evaluation to a list of (b, h) pairs;
    the other outputs are left as NaN."""
    q = np.asarray(q)
    B, Hq, N, _ = q.shape
    Hkv = np.asarray(k).shape[1]
    assert Hq % Hkv == 0
    rep = Hq // Hkv
    y = np.full((B, Hq, N, np.asarray(v).shape[-1]), np.nan)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in pairs:
        kv = h // rep
        y[b, h] = causal_attention(q[b, h], k[b, kv], v[b, kv], L[h],
                                   group_map[h], int(n_groups[h]), eps)
    return y


# ---------------------------------------------------------------------------
# Algorithm 1: the Hadamard-diagonal recurrence (used by the pins)
# ---------------------------------------------------------------------------

def packed_pairs(d_h: int):
    """The (r, t) pairs with r <= t in row-major order: the rows of the
    packed-symmetric H2 ([OAL] App. D, "Exact state and parameter counts")."""
    return [(r, t) for r in range(d_h) for t in range(r, d_h)]


def recurrence(q, k, v, a, b, C, packed=False, return_parts=False):
    """[OAL] Algorithm 1, causal evaluation, one token at a time.

    Token i is appended as u_i = [v_i; 1]; H0 += u_i, H1_r += k_{i,r} u_i,
    H2_rt += k_{i,r} k_{i,t} u_i ([OAL] Eq. 5); then
    u~_i = a H0 + (1/sqrt d_h) sum_r b_r q_{i,r} H1_r
           + (1/d_h) sum_{r,t} C_rt q_{i,r} q_{i,t} H2_rt        ([OAL] Eq. 6)
    and y_i = u~_{i,1:d_v} / u~_{i,d_v+1}.

    With ``packed`` the H2 state keeps only r <= t and the readout weights a
    diagonal pair once and an off-diagonal pair twice ([OAL] App. D).  Both
    forms must agree with :func:`causal_attention`."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    N, d_h = q.shape
    d_v = v.shape[1]
    W = d_v + 1
    H0 = np.zeros(W)
    H1 = np.zeros((d_h, W))
    pairs = packed_pairs(d_h)
    H2 = np.zeros((len(pairs), W)) if packed else np.zeros((d_h, d_h, W))
    y = np.empty((N, d_v))
    ut_all = np.empty((N, W))
    sq = math.sqrt(d_h)
    for i in range(N):
        u = np.append(v[i], 1.0)
        H0 += u
        for r in range(d_h):
            H1[r] += k[i, r] * u
        if packed:
            for p, (r, t) in enumerate(pairs):
                H2[p] += k[i, r] * k[i, t] * u
        else:
            for r in range(d_h):
                for t in range(d_h):
                    H2[r, t] += k[i, r] * k[i, t] * u
        ut = a * H0
        for r in range(d_h):
            ut = ut + (b[r] * q[i, r] / sq) * H1[r]
        if packed:
            for p, (r, t) in enumerate(pairs):
                mult = 1.0 if r == t else 2.0
                ut = ut + (mult * C[r, t] * q[i, r] * q[i, t] / d_h) * H2[p]
        else:
            for r in range(d_h):
                for t in range(d_h):
                    ut = ut + (C[r, t] * q[i, r] * q[i, t] / d_h) * H2[r, t]
        ut_all[i] = ut
        y[i] = ut[:d_v] / ut[d_v]
    if return_parts:
        return y, ut_all
    return y


def canonical_state(k, v):
    """The prefix state after all tokens of k, v, in the packed canonical row
    order used by the library's state export: row 0 is H0, rows 1..d_h are
    H1_r, then one row per pair r <= t of H2 in row-major pair order; each row
    has d_v + 1 columns (value channels, then the all-ones channel).  Built
    token by token from [OAL] Eq. 5 with u_j = [v_j; 1]."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, d_h = k.shape
    W = v.shape[1] + 1
    pairs = packed_pairs(d_h)
    rows = np.zeros((1 + d_h + len(pairs), W))
    for j in range(N):
        u = np.append(v[j], 1.0)
        rows[0] += u
        rows[1:1 + d_h] += k[j][:, None] * u[None, :]
        for p, (r, t) in enumerate(pairs):
            rows[1 + d_h + p] += k[j, r] * k[j, t] * u
    return rows


# ---------------------------------------------------------------------------
# Counts ([OAL] App. D, "Exact state and parameter counts")
# ---------------------------------------------------------------------------

def state_size(d_h: int, d_v: int) -> int:
    """Entries of one packed-symmetric state: (1 + d_h + d_h(d_h+1)/2)(d_v+1)."""
    return (1 + d_h + d_h * (d_h + 1) // 2) * (d_v + 1)


def ordered_state_size(d_h: int, d_v: int) -> int:
    """Entries of one ordered-pair state: (1 + d_h + d_h^2)(d_v+1)."""
    return (1 + d_h + d_h * d_h) * (d_v + 1)


def lower_factor_params(n_groups: int) -> int:
    """Learned parameters of L per head: (G+1)(G+2)/2."""
    return (n_groups + 1) * (n_groups + 2) // 2
