"""oal_prefill_fresh: a prefill of a sequence that starts empty, written into a
state whatever it held ([OAL] Algorithm 1 from step 5).  With bf16 inputs the
builder starts from zero without reading the state; the outputs, the state and
its token count must equal oal_state_reset followed by oal_prefill, bit for bit."""

import pytest
import torch

from positive_quadratic_causal_amd import synth

from gpu_util import Case, announce

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def oal():
    from positive_quadratic_causal_amd import oal as mod
    return mod


def _dirty(oal, case, n):
    st = oal.oal_state_alloc(case.w.batch, case.w.n_kv_heads)
    oal.oal_prefill(None, case.k[:, :, :n].contiguous(), case.v[:, :, :n].contiguous(), None,
                    chunk=128, state=st, want_output=False)
    return st


@pytest.mark.parametrize("dtype,chunk,n", [("bf16", 64, 700), ("bf16", 128, 1000),
                                           ("bf16", 256, 1300), ("f32", 128, 300)])
def test_fresh_prefill_equals_reset_then_prefill(oal, dtype, chunk, n):
    w = synth.small_workload(880 + chunk, "fresh prefill", 2, 4, 2, n, dtype)
    announce(f"oal_prefill_fresh vs reset + oal_prefill, 4/2 N={n} {dtype} chunk={chunk}")
    case = Case(w)
    coeffs = case.coeffs()
    a = _dirty(oal, case, 200)
    b = _dirty(oal, case, 300)
    y1 = oal.oal_prefill_fresh(case.q, case.k, case.v, coeffs, a, chunk=chunk)
    oal.oal_state_reset(b)
    y2 = oal.oal_prefill(case.q, case.k, case.v, coeffs, chunk=chunk, state=b)
    s1, s2 = oal.oal_state_export(a), oal.oal_state_export(b)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.equal(s1, s2)
    assert oal.oal_state_tokens(a) == n == oal.oal_state_tokens(b)
    # state only (no outputs; with fp32 inputs the state-only pass adds in another
    # order), and a continuation from the fresh state
    oal.oal_prefill_fresh(None, case.k, case.v, None, a, chunk=chunk, want_output=False)
    s3 = oal.oal_state_export(a)
    if dtype == "bf16":
        assert torch.equal(s3, s2)
    else:
        assert (s3 - s2).norm() <= 1e-6 * s2.norm()
    c = oal.oal_state_alloc(w.batch, w.n_kv_heads)
    oal.oal_prefill_fresh(None, case.k[:, :, :n // 2].contiguous(), case.v[:, :, :n // 2].contiguous(),
                          None, c, chunk=chunk, want_output=False)
    oal.oal_prefill(None, case.k[:, :, n // 2:].contiguous(), case.v[:, :, n // 2:].contiguous(),
                    None, chunk=chunk, state=c, want_output=False)
    full = oal.oal_state_export(c)
    torch.cuda.synchronize()
    tol = 1e-5 if dtype == "f32" else 4e-3
    assert (full - s2).norm() <= tol * s2.norm()


def test_fresh_prefill_of_no_tokens_clears(oal):
    w = synth.small_workload(890, "fresh empty", 1, 4, 2, 100, "bf16")
    announce("oal_prefill_fresh with seq_len 0 clears the state")
    case = Case(w)
    a = _dirty(oal, case, 100)
    empty = case.k[:, :, :0].contiguous()
    oal.oal_prefill_fresh(None, empty, case.v[:, :, :0].contiguous(), None, a, want_output=False)
    torch.cuda.synchronize()
    assert oal.oal_state_export(a).abs().max().item() == 0.0
    assert oal.oal_state_tokens(a) == 0
