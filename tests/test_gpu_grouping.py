"""GPU parity of the dimension grouping ([OAL] Eq. 2; App. B Eq. 16-19):
oal_contribution_scores against the pair-by-pair oracle, and
oal_bootstrap_grouping against the oracle's grouping fed the same per-prompt
scores and bootstrap indices: labels, group counts and supports identical
(integer decisions, taken in double precision on both sides)."""

import numpy as np
import pytest
import torch

from oracle import grouping_oracle as GR
from positive_quadratic_causal_amd import synth

from gpu_util import announce

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def oal():
    from positive_quadratic_causal_amd import oal as mod
    return mod


def _prompts(w, lengths):
    """Concatenate prompts b = 0.. of the workload (each its own token streams,
    same outlier structure) to q [Hq, T, 64], k [Hkv, T, 64] plus offsets."""
    st = synth.structure(w)
    qs = [[synth.head_tensor(w, st, synth.KIND_Q, b, h, n) for h in range(w.n_q_heads)]
          for b, n in enumerate(lengths)]
    ks = [[synth.head_tensor(w, st, synth.KIND_K, b, h, n) for h in range(w.n_kv_heads)]
          for b, n in enumerate(lengths)]
    q = np.concatenate([np.stack(x) for x in qs], axis=1)
    k = np.concatenate([np.stack(x) for x in ks], axis=1)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return st, q, k, off


def _dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_contribution_scores_match_oracle(oal, dtype):
    w = synth.small_workload(960, "contrib", 6, 6, 2, 1, dtype, grouping="llama",
                             outlier_scale=(2.5, 4.5))
    lengths = [1, 17, 64, 100, 0, 200]
    announce(f"contribution scores, 6 prompts (one empty), 6/2 heads, {dtype}")
    st, q, k, off = _prompts(w, lengths)
    chi_p, chi = oal.oal_contribution_scores(_dev(q, dtype), _dev(k, dtype), torch.from_numpy(off).cuda())
    torch.cuda.synchronize()
    chi_p, chi = chi_p.cpu().numpy(), chi.cpu().numpy()
    for p, n in enumerate(lengths):
        for h in range(6):
            if n == 0:
                assert np.all(chi_p[p, h] == 0.0)
                continue
            qq = q[h, off[p]:off[p + 1]].astype(np.float64)
            kk = k[h // 3, off[p]:off[p + 1]].astype(np.float64)
            ref = GR.contribution_prompt(qq, kk)
            np.testing.assert_allclose(chi_p[p, h], ref, rtol=2e-6, atol=1e-12)
    np.testing.assert_allclose(chi, chi_p.astype(np.float64).mean(axis=0), rtol=1e-6)


@pytest.mark.parametrize("alpha,gamma", [(0.25, 0.9), (0.5, 0.5)])
def test_grouping_matches_oracle(oal, alpha, gamma):
    w = synth.small_workload(970, "grouping", 40, 14, 2, 1, "bf16", grouping="qwen",
                             outlier_scale=(2.5, 4.5))
    lengths = list(np.random.default_rng(971).integers(32, 160, size=40))
    announce(f"bootstrap grouping, 40 prompts, 14 heads, B=1000, alpha={alpha} gamma={gamma}")
    st, q, k, off = _prompts(w, lengths)
    chi_p, _ = oal.oal_contribution_scores(_dev(q, "bf16"), _dev(k, "bf16"), torch.from_numpy(off).cuda())
    boot = np.random.default_rng(972).integers(0, 40, size=(1000, 40)).astype(np.int32)
    tau, g_min, eps = 1.5, 2, 1e-12
    gm, ng, sup, gap = oal.oal_bootstrap_grouping(chi_p, torch.from_numpy(boot).cuda(), alpha, tau,
                                                  gamma, g_min, eps)
    torch.cuda.synchronize()
    cp = chi_p.cpu().numpy().astype(np.float64)
    gm, ng, sup, gap = gm.cpu().numpy(), ng.cpu().numpy(), sup.cpu().numpy(), gap.cpu().numpy()
    gamma32 = float(np.float32(gamma))
    for h in range(14):
        labels, G, cuts, rho, support = GR.group_head(cp[:, h], boot, alpha, tau, gamma32, g_min, eps)
        assert list(gm[h]) == labels, h
        assert ng[h] == G, h
        for kk in cuts:
            assert sup[h, kk] == np.float32(support[kk])
        for kk, r in rho.items():
            assert abs(gap[h, kk] - r) <= 1e-6 * r
        # the dims outside the bulk group are exactly the head's synthetic outlier dims
        assert set(np.nonzero(gm[h] >= 2)[0]) == set(st.outliers[h // 7]), h


def test_grouping_staircase(oal):
    """The oracle pin's staircase profile through the kernel: cuts at 58, 60, 62."""
    announce("bootstrap grouping, staircase profile")
    levels = np.array([1.0] * 58 + [4.0, 4.0, 16.0, 16.0, 64.0, 64.0], dtype=np.float32)
    perm = np.random.default_rng(2).permutation(64)
    chi = np.empty(64, dtype=np.float32)
    chi[perm] = levels
    chi_p = np.tile(chi, (5, 3, 1))                      # 5 prompts, 3 heads
    boot = np.random.default_rng(3).integers(0, 5, size=(50, 5)).astype(np.int32)
    gm, ng, sup, _ = oal.oal_bootstrap_grouping(torch.from_numpy(chi_p).cuda(),
                                                torch.from_numpy(boot).cuda(), 0.25, 1.5, 0.9, 2)
    torch.cuda.synchronize()
    want = np.empty(64, dtype=np.int32)
    want[perm] = [1] * 58 + [2, 2, 3, 3, 4, 4]
    for h in range(3):
        assert np.array_equal(gm[h].cpu().numpy(), want)
    assert list(ng.cpu().numpy()) == [4, 4, 4]
