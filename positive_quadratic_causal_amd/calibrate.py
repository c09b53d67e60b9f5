"""Calibration of L by output matching ([OAL] App. B, Eq. 20) on the GPU.

The host only schedules: it draws each update's sequence and causal query
positions from a seeded generator, runs validation every ``val_every`` updates,
keeps each head's best L and stops early.  Every arithmetic step runs in the
library's kernels: the sampled rows' loss and gradient (``oal_calib_grad``), the
clipped Adam step (``oal_adam_step``), the softmax targets
(``oal_softmax_attention``), the validation outputs and errors
(``oal_expand_coeffs``, ``oal_prefill``, ``oal_output_mse``) and the embedding of
the learned global kernel (``oal_embed_global``).

Protocol of the pages (App. B "Coefficient-calibration settings"): Adam at
learning rate 0.02 without a scheduler, up to 1000 updates per initialisation,
fp32 parameters, gradient norm clipped at 10, one training sequence and 32
causal query positions per update, validation every 100 updates, early stopping
after 400 updates without improvement, the lowest-validation-error checkpoint
kept per query head.  Starts (App. D): the second-order Taylor polynomial, the
learned global quadratic embedded in the grouped form, or a Gaussian
perturbation of either.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

from positive_quadratic_causal_amd import oal

__all__ = ["Sequence", "taylor_L", "perturbed", "softmax_targets", "validation_mse", "calibrate",
           "learned_global", "calibrate_protocol"]


@dataclass
class Sequence:
    """One sequence of a layer: q [1, Hq, N, 64], k, v [1, Hkv, N, 64] on the GPU."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    y_ref: torch.Tensor | None = None     # softmax output [1, Hq, N, 64] fp32


def taylor_L(n_groups: np.ndarray, g_max: int) -> np.ndarray:
    """Per head the L of exp(s) ~ 1 + s + s^2 / 2 in the grouped form ([OAL] App.
    D: M_00 = 1, M_0g = M_gh = 1/2): row 0 = (1, 0, ..), rows 1..G = (1/2, 1/2, 0, ..)."""
    Hq = len(n_groups)
    L = np.zeros((Hq, g_max + 1, g_max + 1), dtype=np.float32)
    for h, G in enumerate(n_groups):
        L[h, 0, 0] = 1.0
        L[h, 1:G + 1, 0] = 0.5
        L[h, 1:G + 1, 1] = 0.5
    return L


def perturbed(L: np.ndarray, n_groups: np.ndarray, sigma: float, seed: int) -> np.ndarray:
    """L plus N(0, sigma^2) on every parameter entry (lower triangle of the leading
    (G+1) block): a start that is not confined to the rank-2 family of the Taylor
    and learned-global starts (their zero columns receive no gradient)."""
    rng = np.random.default_rng(seed)
    out = np.array(L, dtype=np.float32, copy=True)
    for h, G in enumerate(n_groups):
        n = G + 1
        out[h, :n, :n] += np.tril(rng.normal(0.0, sigma, size=(n, n))).astype(np.float32)
    return out


def softmax_targets(seqs: list[Sequence]) -> None:
    for s in seqs:
        if s.y_ref is None:
            s.y_ref = torch.empty(s.q.shape, dtype=torch.float32, device=s.q.device)
            oal.oal_softmax_attention(s.q, s.k, s.v, s.y_ref)


def validation_mse(seqs: list[Sequence], n_groups: torch.Tensor, group_map: torch.Tensor,
                   L: torch.Tensor, eps: float, chunk: int = 128) -> torch.Tensor:
    """Per-head MSE of the OAL output against the softmax targets, averaged over
    the sequences (device tensor [Hq])."""
    coeffs = oal.oal_expand_coeffs(n_groups, group_map, L, eps)
    total = None
    for s in seqs:
        y = torch.empty(s.q.shape, dtype=torch.float32, device=s.q.device)
        oal.oal_prefill(s.q, s.k, s.v, coeffs, chunk=chunk, y=y)
        mse = oal.oal_output_mse(y, s.y_ref)
        total = mse if total is None else total + mse
    return total / len(seqs)


@dataclass
class CalibResult:
    L: torch.Tensor                      # best L per head [Hq, g+1, g+1]
    best_mse: np.ndarray                 # its validation MSE per head
    updates: int                         # updates run
    val_history: list = field(default_factory=list)    # (update, per-head MSE)
    loss_history: np.ndarray | None = None             # per update, per head


def calibrate(train: list[Sequence], val: list[Sequence], n_groups: torch.Tensor,
              group_map: torch.Tensor, L0: torch.Tensor, eps: float, *, lr: float = 0.02,
              max_updates: int = 1000, n_pos: int = 32, val_every: int = 100,
              patience: int = 400, clip: float = 10.0, seed: int = 0) -> CalibResult:
    softmax_targets(train)
    softmax_targets(val)
    dev = L0.device
    Hq = L0.shape[0]
    N = train[0].q.shape[2]
    rng = np.random.default_rng(seed)
    seq_idx = rng.integers(0, len(train), size=max_updates)
    pos = np.stack([np.sort(rng.choice(N, size=n_pos, replace=False)) for _ in range(max_updates)])
    pos_d = torch.from_numpy(pos.astype(np.int32)).to(dev)
    L = L0.clone()
    m = torch.zeros_like(L)
    v = torch.zeros_like(L)
    dL = torch.empty_like(L)
    losses = torch.empty((max_updates, Hq), dtype=torch.float32, device=dev)
    ws = oal.alloc_workspace(oal.oal_calib_workspace_bytes(Hq, n_pos), dev)
    best = validation_mse(val, n_groups, group_map, L, eps).cpu().numpy()
    best_L = L.clone()
    last_improve = np.zeros(Hq, dtype=np.int64)
    history = [(0, best.copy())]
    t = 0
    for t in range(1, max_updates + 1):
        s = train[int(seq_idx[t - 1])]
        oal.oal_calib_grad(s.q, s.k, s.v, s.y_ref, pos_d[t - 1], n_groups, group_map, L, eps,
                           dL=dL, loss=losses[t - 1], workspace=ws)
        oal.oal_adam_step(n_groups, L, dL, m, v, t, lr=lr, clip_norm=clip)
        if t % val_every == 0:
            mse = validation_mse(val, n_groups, group_map, L, eps).cpu().numpy()
            history.append((t, mse.copy()))
            better = mse < best
            best = np.where(better, mse, best)
            last_improve = np.where(better, t, last_improve)
            for h in np.nonzero(better)[0]:
                best_L[h] = L[h]
            if np.all(t - last_improve >= patience):
                break
    torch.cuda.synchronize()
    return CalibResult(best_L, best, t, history, losses[:t].cpu().numpy())


def learned_global(train: list[Sequence], val: list[Sequence], n_q_heads: int, eps: float,
                   **kw) -> CalibResult:
    """The learned global quadratic ([OAL] App. D): the same calibration with every
    dimension in one group (G = 1, L 2 x 2), from its Taylor start."""
    dev = train[0].q.device
    ng1 = torch.ones((n_q_heads,), dtype=torch.int32, device=dev)
    gm1 = torch.ones((n_q_heads, 64), dtype=torch.int32, device=dev)
    L1 = torch.from_numpy(taylor_L(np.ones(n_q_heads, dtype=np.int64), 1)).to(dev)
    return calibrate(train, val, ng1, gm1, L1, eps, **kw)


@dataclass
class ProtocolResult:
    L: torch.Tensor                      # per head the best of the starts
    best_mse: np.ndarray                 # its validation MSE
    chosen: list                         # per head the name of the winning start
    starts: dict                         # name -> CalibResult (and the start L)


def calibrate_protocol(train: list[Sequence], val: list[Sequence], n_groups: torch.Tensor,
                       group_map: torch.Tensor, eps: float, *, g_max: int = 6,
                       sigma: float = 0.05, seed: int = 0, **kw) -> ProtocolResult:
    """The three starts of [OAL] App. B: the learned global quadratic embedded into
    the grouped form (``oal_embed_global``), the second-order Taylor start, and a
    Gaussian perturbation of the embedded global start; each calibrated with
    ``calibrate`` and the best start kept per head by validation MSE."""
    Hq = n_groups.shape[0]
    dev = n_groups.device
    ng_host = n_groups.cpu().numpy()
    glob = learned_global(train, val, Hq, eps, seed=seed, **kw)
    emb = oal.oal_embed_global(n_groups, glob.L, g_max)
    starts = {"global_embedding": emb,
              "taylor": torch.from_numpy(taylor_L(ng_host, g_max)).to(dev),
              "global_perturbed": torch.from_numpy(perturbed(emb.cpu().numpy(), ng_host, sigma,
                                                             seed + 1)).to(dev)}
    results = {"learned_global_G1": glob}
    best_L, best, chosen = None, None, None
    for i, (name, L0) in enumerate(starts.items()):
        res = calibrate(train, val, n_groups, group_map, L0, eps, seed=seed + 10 + i, **kw)
        results[name] = res
        if best is None:
            best_L, best, chosen = res.L.clone(), res.best_mse.copy(), [name] * Hq
            continue
        for h in np.nonzero(res.best_mse < best)[0]:
            best_L[h] = res.L[h]
            best[h] = res.best_mse[h]
            chosen[h] = name
    return ProtocolResult(best_L, best, chosen, {"results": results, "starts": starts})
