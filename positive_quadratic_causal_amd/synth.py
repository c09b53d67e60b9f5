"""Seeded synthetic inputs for the OAL workloads.

This module only draws random numbers: it holds none of the method's
arithmetic, so both the HIP path's tests/bench and the float64 oracle can take
their inputs from it.  Every tensor is a pure function of (workload id, stream
kind, batch index, head index), so any single head can be regenerated on its
own (which is what the sampled parity checks of the large workloads rely on).

The shapes follow the head configurations of the OAL paper's runtime
benchmark (App. E: Qwen2.5-0.5B, 14 query / 2 KV heads, d_h = d_v = 64) and a
Llama-3.2-1B-shaped layer (32 query / 8 KV heads).  The value distributions
imitate the query-key outlier structure of the paper's §3 / Fig. 1-2 (a few
dimensions carrying most of the dot product): q, k ~ N(0, 1) with a handful of
per-head outlier dimensions scaled by 8-20 (x12 in the tiny case), v ~ N(0, 1).
They stand in for the real Qwen/Llama attention states and WikiText prompts of
the paper, which are not available here.

Recipe:

* streams: ``numpy.random.default_rng(SeedSequence([20261202, wid, kind, b, h]))``
  with kind 0 = structure (shared by the whole workload), 1 = q, 2 = k, 3 = v;
* q/k/v are standard normal float32, multiplied per dimension by the head's
  outlier scales (U[8, 20] unless a workload sets another range; U[2.5, 4.5]
  gives the outlier dims about 43 % of sum_r |q_r k_r|, near the 46-49 % of
  [OAL] Table 4, and a score spread of about 3), then rounded to bfloat16
  (round to nearest even) for the bf16 workloads;
* L per query head: (G+1)x(G+1) lower triangular, N(0, 0.3^2) entries, diagonal
  replaced by |.| + 0.5, zero above the diagonal; eps = 1e-6;
* groups are labelled 1..G, group 1 being the bulk of non-outlier dimensions;
* dimension-specific coefficients (stream kind 4, one per query head): with
  F ~ N(0, 1)^{65x65} and P = F F^T / 65 + 0.05 I, a = P_00, b_r = 2 P_0r and
  C = P_{1:,1:} + 0.3 (A - A^T), A ~ N(0, 1)^{64x64}: a positive definite form in
  [1, x] plus an antisymmetric part, all float32.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED = 20261202
D_H = 64
D_V = 64
G_MAX = 6

KIND_STRUCT, KIND_Q, KIND_K, KIND_V, KIND_DIM = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    seq_len: int            # prefill tokens
    dtype: str              # "f32" or "bf16"
    decode_steps: int = 0   # single-token steps after the prefill
    eps: float = 1e-6
    grouping: str = "qwen"  # "tiny", "qwen" (G = 4) or "llama" (G in 2..6)
    outlier_scale: tuple = (8.0, 20.0)   # U[lo, hi] factor of the outlier dims of q and k
    d_h: int = D_H
    d_v: int = D_V
    chunks: tuple = (128,)

    @property
    def total_len(self) -> int:
        return self.seq_len + self.decode_steps


WORKLOADS = {
    0: Workload(0, "tiny single head fp32, N=256", 1, 1, 1, 256, "f32",
                grouping="tiny"),
    1: Workload(1, "Qwen2.5-0.5B-shaped layer 14/2, N=2048", 1, 14, 2, 2048,
                "bf16", grouping="qwen"),
    2: Workload(2, "Llama-3.2-1B-shaped layer 32/8, B=4, N=4096", 4, 32, 8,
                4096, "bf16", grouping="llama"),
    3: Workload(3, "Qwen2.5-0.5B-shaped long-context prefill 14/2, N=32768", 1,
                14, 2, 32768, "bf16", grouping="qwen", chunks=(64, 128, 256)),
    4: Workload(4, "Llama-3.2-1B-shaped batched decode 32/8, B=64, 8192+256", 64,
                32, 8, 8192, "bf16", decode_steps=256, grouping="llama"),
}


def _rng(wid: int, kind: int, b: int = 0, h: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([SEED, wid, kind, b, h]))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32)


@dataclass
class Structure:
    """Per-workload structure: outlier dims/scales, group maps and L factors."""
    q_scale: np.ndarray      # [Hq, d_h] float32 multipliers
    k_scale: np.ndarray      # [Hkv, d_h]
    n_groups: np.ndarray     # [Hq] int32, G_h
    group_map: np.ndarray    # [Hq, d_h] int32, values 1..G_h
    L: np.ndarray            # [Hq, G_MAX+1, G_MAX+1] float32, lower triangular
    eps: float
    outliers: list = field(default_factory=list)   # per KV head: outlier dims


def random_L(rng: np.random.Generator, n_groups: int) -> np.ndarray:
    """Lower-triangular (G+1)x(G+1): N(0, 0.3^2) entries, diagonal |.| + 0.5,
    embedded in a (G_MAX+1)^2 zero matrix."""
    n = n_groups + 1
    Lh = rng.normal(0.0, 0.3, size=(n, n))
    Lh = np.tril(Lh)
    Lh[np.diag_indices(n)] = np.abs(np.diag(Lh)) + 0.5
    out = np.zeros((G_MAX + 1, G_MAX + 1), dtype=np.float32)
    out[:n, :n] = Lh
    return out


def dim_coefficients(w: Workload):
    """(a [Hq], b [Hq, 64], C [Hq, 64, 64]) float32 for the dimension-specific kernel:
    the form [[a, b^T / 2], [b / 2, sym(C)]] is positive definite, so the kernel is
    positive for every q, k, and C carries an antisymmetric part as well."""
    d = w.d_h
    a = np.empty(w.n_q_heads, dtype=np.float32)
    b = np.empty((w.n_q_heads, d), dtype=np.float32)
    C = np.empty((w.n_q_heads, d, d), dtype=np.float32)
    for h in range(w.n_q_heads):
        rng = _rng(w.wid, KIND_DIM, 0, h)
        F = rng.standard_normal((d + 1, d + 1))
        P = F @ F.T / (d + 1) + 0.05 * np.eye(d + 1)
        A = rng.standard_normal((d, d))
        a[h] = P[0, 0]
        b[h] = 2.0 * P[0, 1:]
        C[h] = P[1:, 1:] + 0.3 * (A - A.T)
    return a, b, C


def structure(w: Workload) -> Structure:
    rng = _rng(w.wid, KIND_STRUCT)
    Hq, Hkv, d = w.n_q_heads, w.n_kv_heads, w.d_h
    rep = Hq // Hkv
    q_scale = np.ones((Hq, d), dtype=np.float32)
    k_scale = np.ones((Hkv, d), dtype=np.float32)
    n_groups = np.zeros(Hq, dtype=np.int32)
    group_map = np.ones((Hq, d), dtype=np.int32)
    L = np.zeros((Hq, G_MAX + 1, G_MAX + 1), dtype=np.float32)
    outliers = []
    if w.grouping == "tiny":
        dims = [3, 17, 40, 61]
        q_scale[:, dims] = 12.0
        k_scale[:, dims] = 12.0
        n_groups[:] = 4
        group_map[:, [3, 17]] = 2
        group_map[:, 40] = 3
        group_map[:, 61] = 4
        for h in range(Hq):
            L[h] = random_L(rng, 4)
        outliers = [dims] * Hkv
    else:
        for kv in range(Hkv):
            heads = range(kv * rep, (kv + 1) * rep)
            if w.grouping == "qwen":
                n_out = int(rng.integers(3, 7))          # 3..6 outlier dims
                sizes = {}
                for h in heads:
                    cuts = np.sort(rng.choice(np.arange(1, n_out), size=2,
                                              replace=False))
                    sizes[h] = np.diff(np.concatenate([[0], cuts, [n_out]]))
            else:  # llama: G_h in 2..6, outlier group sizes 1..3
                sizes = {}
                for h in heads:
                    G = int(rng.integers(2, 7))
                    sizes[h] = rng.integers(1, 4, size=G - 1)
                n_out = int(max(int(np.sum(s)) for s in sizes.values()))
            O = rng.choice(d, size=n_out, replace=False)
            outliers.append(sorted(int(x) for x in O))
            k_scale[kv, O] = rng.uniform(*w.outlier_scale, size=n_out)
            for h in heads:
                q_scale[h, O] = rng.uniform(*w.outlier_scale, size=n_out)
                s = sizes[h]
                G = len(s) + 1
                n_groups[h] = G
                members = rng.permutation(O)[: int(np.sum(s))]
                start = 0
                for gi, sz in enumerate(s):
                    group_map[h, members[start:start + sz]] = gi + 2
                    start += sz
                L[h] = random_L(rng, G)
    return Structure(q_scale, k_scale, n_groups, group_map, L, w.eps, outliers)


def _stream(w: Workload, kind: int, b: int, h: int, n_tokens: int) -> np.ndarray:
    x = _rng(w.wid, kind, b, h).standard_normal((n_tokens, w.d_h), dtype=np.float32)
    return x


def head_tensor(w: Workload, st: Structure, kind: int, b: int, h: int,
                n_tokens: int | None = None) -> np.ndarray:
    """Tokens 0..n_tokens-1 of one (batch, head) stream: q (kind 1, query head
    h), k (kind 2, KV head h) or v (kind 3, KV head h).  float32, already
    rounded to bfloat16 for bf16 workloads."""
    n = w.total_len if n_tokens is None else n_tokens
    x = _stream(w, kind, b, h, n)
    if kind == KIND_Q:
        x = x * st.q_scale[h][None, :]
    elif kind == KIND_K:
        x = x * st.k_scale[h][None, :]
    if w.dtype == "bf16":
        x = round_bf16(x)
    return np.ascontiguousarray(x, dtype=np.float32)


def full_tensor(w: Workload, st: Structure, kind: int, t0: int = 0,
                t1: int | None = None) -> np.ndarray:
    """[B, H, t1-t0, d] for q (H = Hq) or k/v (H = Hkv), tokens t0..t1-1."""
    t1 = w.total_len if t1 is None else t1
    H = w.n_q_heads if kind == KIND_Q else w.n_kv_heads
    out = np.empty((w.batch, H, t1 - t0, w.d_h), dtype=np.float32)
    for b in range(w.batch):
        for h in range(H):
            out[b, h] = head_tensor(w, st, kind, b, h, t1)[t0:t1]
    return out


def small_workload(wid: int, name: str, batch: int, n_q_heads: int, n_kv_heads: int,
                   seq_len: int, dtype: str, grouping: str = "llama",
                   decode_steps: int = 0, eps: float = 1e-6,
                   outlier_scale: tuple = (8.0, 20.0)) -> Workload:
    """Ad-hoc workload (edge cases, ragged sizes) with its own seed id."""
    return Workload(wid, name, batch, n_q_heads, n_kv_heads, seq_len, dtype,
                    decode_steps=decode_steps, eps=eps, grouping=grouping,
                    outlier_scale=outlier_scale)
