"""Full-size batched decode (Llama-shaped 32/8, batch 64, 8192 prefilled tokens,
256 single-token steps) checked on sampled outputs against the oracle's direct
sum over all keys up to each step."""

import numpy as np
import pytest
import torch

from positive_quadratic_causal_amd import synth

from gpu_util import Case, announce, rel_l2, tol_for

pytestmark = pytest.mark.gpu


def test_decode_batched_full_size_sampled():
    from positive_quadratic_causal_amd import oal
    w = synth.WORKLOADS[4]
    announce("decode B=64 32/8 after 8192 tokens, 256 steps, bf16 (sampled outputs)")
    case = Case(w, with_q=False)
    n0 = w.seq_len
    coeffs = case.coeffs()
    st = oal.oal_state_alloc(w.batch, w.n_kv_heads)
    oal.oal_prefill(None, case.k[:, :, :n0].contiguous(), case.v[:, :, :n0].contiguous(), coeffs,
                    chunk=128, state=st, want_output=False)
    q = torch.from_numpy(synth.full_tensor(w, case.st, synth.KIND_Q, n0, n0 + w.decode_steps)).to(
        device="cuda", dtype=torch.bfloat16)
    ys = torch.empty((w.batch, w.n_q_heads, w.decode_steps, 64), dtype=torch.bfloat16, device="cuda")
    for s in range(w.decode_steps):
        t = n0 + s
        ys[:, :, s] = oal.oal_decode_step(q[:, :, s].contiguous(), case.k[:, :, t].contiguous(),
                                          case.v[:, :, t].contiguous(), coeffs, st)
    torch.cuda.synchronize()
    y = ys.float().cpu().numpy()
    assert np.all(np.isfinite(y))
    rng = np.random.default_rng(4)
    steps = np.array([0, 1, 2, 63, 64, 100, 127, 128, 254, 255])
    # every query head once (so every KV head's state and every GQA slot), each with
    # a random sequence of the batch, plus the two corners
    pairs = [(0, 0), (63, 31)] + [(int(rng.integers(64)), h) for h in range(32)]
    for b, h in pairs:
        ref = case.oracle_rows(b, h, n0 + steps)
        err = rel_l2(y[b, h, steps], ref)
        rows = np.linalg.norm(y[b, h, steps] - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
        assert err <= tol_for(w) and rows.max() <= tol_for(w), (b, h, err, rows.max())
