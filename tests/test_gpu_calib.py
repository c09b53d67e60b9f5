"""GPU parity of the calibration kernels ([OAL] App. B, Eq. 20): the sampled-row
loss and dL (oal_calib_grad), the clipped Adam step (oal_adam_step), the output
MSE, and a short update schedule from the Taylor start, each against the float64
calibration oracle (pinned in tests/test_calib_oracle_pins.py)."""

import numpy as np
import pytest
import torch

from oracle import calib_oracle as K
from oracle import softmax_oracle as S
from positive_quadratic_causal_amd import synth

from gpu_util import Case, announce, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def oal():
    from positive_quadratic_causal_amd import oal as mod
    return mod


def _targets(case, b=0):
    """float64 softmax outputs of every head (the oracle), as fp32."""
    w = case.w
    return np.stack([S.softmax_attention(*case.head_qkv(b, h)) for h in range(w.n_q_heads)])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_calib_grad_matches_oracle(oal, dtype):
    w = synth.small_workload(900, "calib", 1, 6, 2, 300, dtype, grouping="llama", eps=1e-3)
    announce(f"calib grad 6/2 N=300 {dtype}, 16 positions")
    case = Case(w)
    y_ref = _targets(case).astype(np.float32)
    pos = np.sort(np.random.default_rng(901).choice(300, size=16, replace=False)).astype(np.int32)
    dL, loss = oal.oal_calib_grad(case.q, case.k, case.v, torch.from_numpy(y_ref).cuda(),
                                  torch.from_numpy(pos).cuda(), case.n_groups, case.group_map,
                                  case.L, w.eps)
    torch.cuda.synchronize()
    dL, loss = dL.cpu().numpy(), loss.cpu().numpy()
    for h in range(6):
        q, k, v = case.head_qkv(0, h)
        G = int(case.st.n_groups[h])
        lo, gr = K.output_match_loss_grad(q, k, v, y_ref[h].astype(np.float64), pos,
                                          case.st.L[h].astype(np.float64), case.st.group_map[h], G,
                                          w.eps)
        assert abs(loss[h] - lo) <= 1e-4 * lo, (h, loss[h], lo)
        assert rel_l2(dL[h], gr) <= 1e-4, h


def test_adam_step_matches_oracle(oal):
    announce("adam step, 5 steps, clipping active on the first")
    rng = np.random.default_rng(910)
    n_groups = np.array([2, 6, 4], dtype=np.int32)
    L = rng.normal(size=(3, 7, 7)).astype(np.float32)
    Ld, md, vd = (torch.from_numpy(x).cuda() for x in (L, np.zeros_like(L), np.zeros_like(L)))
    ng = torch.from_numpy(n_groups).cuda()
    Lr = [L[h].astype(np.float64) for h in range(3)]
    mr = [np.zeros((7, 7)) for _ in range(3)]
    vr = [np.zeros((7, 7)) for _ in range(3)]
    for t in range(1, 6):
        g = (rng.normal(size=(3, 7, 7)) * (8.0 if t == 1 else 0.3)).astype(np.float32)
        oal.oal_adam_step(ng, Ld, torch.from_numpy(g).cuda(), md, vd, t)
        for h in range(3):
            mask = K.param_mask((7, 7), int(n_groups[h]))
            Lr[h], mr[h], vr[h] = K.adam_step(Lr[h], g[h], mr[h], vr[h], t, mask)
    torch.cuda.synchronize()
    got = Ld.cpu().numpy()
    for h in range(3):
        np.testing.assert_allclose(got[h], Lr[h], rtol=1e-5, atol=1e-6)


def test_output_mse(oal):
    announce("output mse, B=2 5 heads N=77")
    rng = np.random.default_rng(920)
    y = rng.normal(size=(2, 5, 77, 64)).astype(np.float32)
    r = rng.normal(size=(2, 5, 77, 64)).astype(np.float32)
    got = oal.oal_output_mse(torch.from_numpy(y).cuda(), torch.from_numpy(r).cuda()).cpu().numpy()
    expect = ((y.astype(np.float64) - r) ** 2).mean(axis=(0, 2, 3))
    np.testing.assert_allclose(got, expect, rtol=1e-5)


def test_update_schedule_matches_oracle(oal):
    """Eight updates from the Taylor start on two sequences of one layer: L after
    the schedule against the oracle's loop on the same schedule."""
    w = synth.small_workload(930, "calib loop", 2, 2, 1, 120, "f32", grouping="llama", eps=1e-3)
    announce("calibration schedule, 2 heads N=120, 8 updates from the Taylor start")
    case = Case(w)
    from positive_quadratic_causal_amd.calibrate import taylor_L
    L0 = taylor_L(case.st.n_groups, 6)
    y_ref = [_targets(case, b).astype(np.float32) for b in range(2)]
    rng = np.random.default_rng(931)
    sched = [(int(rng.integers(2)), np.sort(rng.choice(120, size=12, replace=False))) for _ in range(8)]
    Ld = torch.from_numpy(L0).cuda()
    m = torch.zeros_like(Ld)
    v = torch.zeros_like(Ld)
    for t, (b, pos) in enumerate(sched, start=1):
        dL, _ = oal.oal_calib_grad(case.q[b], case.k[b], case.v[b], torch.from_numpy(y_ref[b]).cuda(),
                                   torch.from_numpy(pos.astype(np.int32)).cuda(), case.n_groups,
                                   case.group_map, Ld, w.eps)
        oal.oal_adam_step(case.n_groups, Ld, dL, m, v, t)
    torch.cuda.synchronize()
    got = Ld.cpu().numpy()
    for h in range(2):
        G = int(case.st.n_groups[h])
        train = [case.head_qkv(b, h) + (y_ref[b][h].astype(np.float64),) for b in range(2)]
        Ls, _ = K.calibrate(train, L0[h].astype(np.float64), case.st.group_map[h], G, w.eps, sched)
        assert rel_l2(got[h], Ls[-1]) <= 1e-4, h
        assert rel_l2(Ls[-1], L0[h]) > 1e-3       # the schedule really moved L


def test_embed_global_matches_oracle(oal):
    """oal_embed_global against the oracle's embedding of Eq. 23, and the embedded
    grouped kernel equal to the global one on a pair."""
    announce("learned-global embedding, 5 heads")
    rng = np.random.default_rng(940)
    n_groups = np.array([1, 2, 4, 6, 3], dtype=np.int32)
    Lg = np.zeros((5, 2, 2), dtype=np.float32)
    Lg[:, 0, 0] = rng.uniform(0.5, 1.5, size=5)
    Lg[:, 1, 0] = rng.normal(size=5)
    Lg[:, 1, 1] = rng.uniform(0.2, 1.0, size=5)
    L = oal.oal_embed_global(torch.from_numpy(n_groups).cuda(), torch.from_numpy(Lg).cuda(), 6)
    torch.cuda.synchronize()
    got = L.cpu().numpy()
    for h in range(5):
        Lg64 = Lg[h].astype(np.float64)
        ref = K.global_embedding_L(Lg64 @ Lg64.T, int(n_groups[h]), 6)
        np.testing.assert_allclose(got[h], ref, rtol=1e-6, atol=1e-7)
