"""oal_prefill_noalloc (the prefill entry point that allocates nothing: its
workspace is the library's static device array) against oal_prefill with a
caller-supplied workspace, through the C ABI: the same kernels on the same inputs,
so outputs and states must agree bit for bit.  Two calls in a row, the second
with a smaller input, so that the second runs on whatever the first left in the
shared array; bf16 (matrix-core path) and fp32 (vector path) inputs."""

import numpy as np
import pytest
import torch

from positive_quadratic_causal_amd import synth

from gpu_util import Case, announce, rel_l2, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def oal():
    from positive_quadratic_causal_amd import oal as mod
    return mod


def _pair(oal, case, chunk, with_state):
    """(y, exported state) from oal_prefill and from oal_prefill_noalloc."""
    out = []
    for fn in ("ws", "noalloc"):
        y = torch.empty(case.q.shape, dtype=case.q.dtype, device="cuda")
        st = oal.oal_state_alloc(case.w.batch, case.w.n_kv_heads) if with_state else None
        if st is not None:   # continue from a state holding the first 70 tokens
            oal.oal_prefill(None, case.k[:, :, :70].contiguous(), case.v[:, :, :70].contiguous(), None,
                            chunk=chunk, state=st, want_output=False)
        if fn == "ws":
            oal.oal_prefill(case.q, case.k, case.v, case.coeffs(), chunk=chunk, state=st, y=y)
        else:
            oal.oal_prefill_noalloc(case.q, case.k, case.v, case.coeffs(), chunk=chunk, state=st, y=y)
        torch.cuda.synchronize()
        out.append((y, oal.oal_state_export(st) if st is not None else None))
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_prefill_two_calls(oal, dtype):
    big = synth.small_workload(700, "noalloc big", 1, 14, 2, 4096, dtype, grouping="qwen")
    small = synth.small_workload(701, "noalloc small", 2, 4, 2, 300, dtype)
    for w, chunk, with_state in ((big, 128, False), (small, 64, True)):
        need = oal.oal_prefill_workspace_bytes(w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, chunk,
                                               oal.OAL_BF16 if dtype == "bf16" else oal.OAL_F32, True)
        announce(f"noalloc prefill B={w.batch} {w.n_q_heads}/{w.n_kv_heads} N={w.seq_len} chunk={chunk} "
                 f"{dtype} state={with_state} (workspace {need} of {oal.oal_prefill_noalloc_scratch_bytes()} B)")
        assert 0 < need <= oal.oal_prefill_noalloc_scratch_bytes()
        case = Case(w)
        (y_ws, s_ws), (y_na, s_na) = _pair(oal, case, chunk, with_state)
        assert torch.equal(y_na, y_ws)
        if with_state:
            assert torch.equal(s_na, s_ws)
        # and the outputs are right (two heads against the float64 oracle)
        if not with_state:
            yc = y_na.float().cpu().numpy()
            for h in (0, w.n_q_heads - 1):
                assert rel_l2(yc[0, h], case.oracle_head(0, h)) <= tol_for(w)


def test_noalloc_rejects_sizes_beyond_its_array(oal):
    """The Qwen-shaped N = 32768 prefill needs more workspace than the array holds:
    the call fails on the host with a clear error and launches nothing."""
    w = synth.WORKLOADS[3]
    need = oal.oal_prefill_workspace_bytes(1, 14, 2, w.seq_len, 128, oal.OAL_BF16, True)
    assert need > oal.oal_prefill_noalloc_scratch_bytes()
    q = torch.zeros((1, 14, w.seq_len, 64), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 2, w.seq_len, 64), dtype=torch.bfloat16, device="cuda")
    coeffs = torch.zeros((14, oal.COEF_WORDS), dtype=torch.float32, device="cuda")
    y = torch.full_like(q, 7.0)
    with pytest.raises(oal.OALError) as ei:
        oal.oal_prefill_noalloc(q, kv, kv, coeffs, chunk=128, y=y)
    assert ei.value.status == oal.OAL_ERR_UNSUPPORTED and "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
