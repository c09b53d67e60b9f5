"""GPU parity of the dimension-specific kernel path ([OAL] §4.1, Eq. 3: arbitrary
a, b_r, C_rt): oal_dim_coeffs + oal_prefill_dim + oal_decode_step against the
float64 oracle's direct sum with the same kernel.  Bars: rel-L2 1e-4 per head for
fp32 inputs and outputs; 2e-2 for bf16 (the oracle takes the same bf16 input
values, so the error is the fp32 arithmetic plus the output rounding)."""

import numpy as np
import pytest
import torch

from oracle import oal_oracle as O
from positive_quadratic_causal_amd import synth

from gpu_util import Case, announce, rel_l2, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def oal():
    from positive_quadratic_causal_amd import oal as mod
    return mod


def _dim(case):
    a, b, C = synth.dim_coefficients(case.w)
    dev = "cuda"
    return (a, b, C), (torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev),
                       torch.from_numpy(C).to(dev))


def _oracle_rows(case, coef, b, h, positions):
    a, bb, C = coef
    positions = np.asarray(positions)
    q, k, v = case.head_qkv(b, h, int(positions.max()) + 1)
    return O.causal_attention_dim_rows(q[positions], positions, k, v, float(a[h]),
                                       bb[h].astype(np.float64), C[h].astype(np.float64))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [64, 128, 256])
@pytest.mark.parametrize("n", [1, 100, 300])
def test_dim_prefill_parity(oal, dtype, chunk, n):
    w = synth.small_workload(700 + n, "dim", 2, 6, 2, n, dtype, grouping="llama")
    announce(f"prefill_dim B=2 6/2 N={n} {dtype} chunk={chunk}")
    case = Case(w)
    coef, (a, b, C) = _dim(case)
    coeffs = oal.oal_dim_coeffs(a, b, C)
    y = torch.empty(tuple(case.q.shape), dtype=torch.float32, device="cuda")
    oal.oal_prefill_dim(case.q, case.k, case.v, coeffs, chunk=chunk, y=y)
    torch.cuda.synchronize()
    yc = y.cpu().numpy()
    assert np.all(np.isfinite(yc))
    tol = tol_for(w)
    rows = np.arange(n) if n <= 100 else np.unique(np.r_[0:3, chunk - 1:chunk + 2, n - 40:n] % n)
    for bi, h in [(0, 0), (0, 4), (1, 2), (1, 5)]:
        ref = _oracle_rows(case, coef, bi, h, rows)
        err = rel_l2(yc[bi, h, rows], ref)
        assert err <= tol, (bi, h, err)


def test_dim_state_chaining_and_decode(oal):
    """Prefill in two calls (state carried), then three decode steps, all with the
    same dimension-specific record; each output row against the oracle's row at its
    absolute position."""
    w = synth.small_workload(720, "dim chain", 1, 7, 1, 333, "f32", decode_steps=3)
    announce("prefill_dim 7/1 N=200+133, then 3 decode steps, f32")
    case = Case(w)
    coef, (a, b, C) = _dim(case)
    coeffs = oal.oal_dim_coeffs(a, b, C)
    state = oal.oal_state_alloc(1, 1)
    n0, n1 = 200, 333
    ya = oal.oal_prefill_dim(case.q[:, :, :n0].contiguous(), case.k[:, :, :n0].contiguous(),
                             case.v[:, :, :n0].contiguous(), coeffs, chunk=128, state=state)
    yb = oal.oal_prefill_dim(case.q[:, :, n0:n1].contiguous(), case.k[:, :, n0:n1].contiguous(),
                             case.v[:, :, n0:n1].contiguous(), coeffs, chunk=64, state=state)
    yd = [oal.oal_decode_step(case.q[:, :, t].contiguous(), case.k[:, :, t].contiguous(),
                              case.v[:, :, t].contiguous(), coeffs, state) for t in range(n1, n1 + 3)]
    torch.cuda.synchronize()
    assert state.tokens == n1 + 3
    for h in (0, 3, 6):
        pos = np.r_[0, 150, 199, 200, 260, 332, 333, 334, 335]
        ref = _oracle_rows(case, coef, 0, h, pos)
        got = np.concatenate([ya[0, h, [0, 150, 199]].cpu().numpy(),
                              yb[0, h, [0, 60, 132]].cpu().numpy(),
                              np.stack([d[0, h].cpu().numpy() for d in yd])])
        err = rel_l2(got, ref)
        assert err <= 1e-4, (h, err)
    state.free()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_grouped_record_through_prefill_dim(oal, dtype):
    """The general path evaluates a grouped record (from oal_expand_coeffs) too: it
    matches the grouped oracle and oal_prefill."""
    w = synth.small_workload(730, "dim grouped", 1, 6, 2, 250, dtype, grouping="llama")
    announce(f"prefill_dim with a grouped record, 6/2 N=250 {dtype}")
    case = Case(w)
    coeffs = case.coeffs()
    y_dim = torch.empty(tuple(case.q.shape), dtype=torch.float32, device="cuda")
    y_grp = torch.empty_like(y_dim)
    oal.oal_prefill_dim(case.q, case.k, case.v, coeffs, chunk=128, y=y_dim)
    oal.oal_prefill(case.q, case.k, case.v, coeffs, chunk=128, y=y_grp)
    torch.cuda.synchronize()
    tol = tol_for(w)
    for h in range(6):
        ref = case.oracle_head(0, h)
        assert rel_l2(y_dim[0, h].cpu().numpy(), ref) <= tol
        assert rel_l2(y_grp[0, h].cpu().numpy(), ref) <= tol


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_grouped_prefill_poisons_a_dim_record(oal, dtype):
    """oal_prefill's readouts evaluate grouped records only: the binding refuses the
    buffer that oal_dim_coeffs filled, and the library itself (reached here through
    another tensor over the same memory) yields NaN outputs rather than a silently
    wrong value."""
    w = synth.small_workload(740, "dim misuse", 1, 2, 1, 150, dtype)
    announce(f"oal_prefill with a dimension-specific record, {dtype}")
    case = Case(w)
    _, (a, b, C) = _dim(case)
    coeffs = oal.oal_dim_coeffs(a, b, C)
    with pytest.raises(ValueError, match="dimension-specific"):
        oal.oal_prefill(case.q, case.k, case.v, coeffs, chunk=64)
    y = oal.oal_prefill(case.q, case.k, case.v, coeffs[:], chunk=64)
    torch.cuda.synchronize()
    assert torch.isnan(y.float()).all()


def test_dim_qwen_2048_sampled_rows(oal):
    w = synth.WORKLOADS[1]
    announce("prefill_dim Qwen-shaped 14/2 N=2048 bf16, sampled rows")
    case = Case(w)
    coef, (a, b, C) = _dim(case)
    coeffs = oal.oal_dim_coeffs(a, b, C)
    y = torch.empty(tuple(case.q.shape), dtype=torch.float32, device="cuda")
    oal.oal_prefill_dim(case.q, case.k, case.v, coeffs, chunk=128, y=y)
    torch.cuda.synchronize()
    rows = np.r_[0, 1, 127, 128, 1000, 1500, 2046, 2047]
    for h in (0, 7, 13):
        ref = _oracle_rows(case, coef, 0, h, rows)
        assert rel_l2(y[0, h, rows].cpu().numpy(), ref) <= 2e-2
