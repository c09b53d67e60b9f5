"""Helpers shared by the GPU parity tests: build device inputs from the seeded
generator, run the library through its C ABI binding, and evaluate the float64
oracle on the same values."""

from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import oal_oracle as O
from positive_quadratic_causal_amd import synth

# Tolerances on rel-L2 = ||y_gpu - y_ref|| / ||y_ref|| (float64), fixed by the
# accuracy targets for the two input precisions.
TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def tol_for(w: synth.Workload) -> float:
    return TOL_F32 if w.dtype == "f32" else TOL_BF16


def torch_dtype(w: synth.Workload):
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


class Case:
    """Device tensors and coefficients of one workload (tokens [0, n_tokens))."""

    def __init__(self, w: synth.Workload, n_tokens: int | None = None, with_q: bool = True,
                 device: str = "cuda"):
        self.w = w
        self.st = synth.structure(w)
        self.n = w.total_len if n_tokens is None else n_tokens
        dt = torch_dtype(w)
        self.device = device
        if with_q:
            self.q = torch.from_numpy(synth.full_tensor(w, self.st, synth.KIND_Q, 0, self.n)).to(
                device=device, dtype=dt)
        else:
            self.q = None
        self.k = torch.from_numpy(synth.full_tensor(w, self.st, synth.KIND_K, 0, self.n)).to(
            device=device, dtype=dt)
        self.v = torch.from_numpy(synth.full_tensor(w, self.st, synth.KIND_V, 0, self.n)).to(
            device=device, dtype=dt)
        self.n_groups = torch.from_numpy(self.st.n_groups.astype(np.int32)).to(device)
        self.group_map = torch.from_numpy(self.st.group_map.astype(np.int32)).to(device)
        self.L = torch.from_numpy(self.st.L.astype(np.float32)).to(device)

    def coeffs(self):
        from positive_quadratic_causal_amd import oal
        return oal.oal_expand_coeffs(self.n_groups, self.group_map, self.L, self.w.eps)

    # ---- oracle side -------------------------------------------------------
    def head_qkv(self, b: int, h: int, n: int | None = None):
        """float64 q (query head h), k, v (its KV head) for batch b, regenerated
        from the seeded streams (identical values to what the GPU consumed)."""
        n = self.n if n is None else n
        rep = self.w.n_q_heads // self.w.n_kv_heads
        kv = h // rep
        q = synth.head_tensor(self.w, self.st, synth.KIND_Q, b, h, n).astype(np.float64)
        k = synth.head_tensor(self.w, self.st, synth.KIND_K, b, kv, n).astype(np.float64)
        v = synth.head_tensor(self.w, self.st, synth.KIND_V, b, kv, n).astype(np.float64)
        return q, k, v

    def oracle_head(self, b: int, h: int, n: int | None = None):
        q, k, v = self.head_qkv(b, h, n)
        return O.causal_attention(q, k, v, self.st.L[h].astype(np.float64), self.st.group_map[h],
                                  int(self.st.n_groups[h]), self.w.eps)

    def oracle_rows(self, b: int, h: int, positions):
        positions = np.asarray(positions)
        q, k, v = self.head_qkv(b, h, int(positions.max()) + 1)
        return O.causal_attention_rows(q[positions], positions, k, v,
                                       self.st.L[h].astype(np.float64), self.st.group_map[h],
                                       int(self.st.n_groups[h]), self.w.eps)
