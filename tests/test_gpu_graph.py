"""The prefill step (coefficient expansion, state reset, chunked prefill; no
memset, allocation or synchronisation inside) captured in a HIP graph: every
replay, with eager work and synchronisation between replays, reproduces the
eager outputs and final state bit for bit."""

import pytest
import torch

from positive_quadratic_causal_amd import synth

from gpu_util import Case, announce

pytestmark = pytest.mark.gpu


def test_prefill_step_graph_replays_match_eager():
    from positive_quadratic_causal_amd import oal
    w = synth.WORKLOADS[1]
    announce("HIP graph of the prefill step, Qwen-shaped 14/2 N=2048, 4 replays")
    case = Case(w)
    ng, gm, L = case.n_groups, case.group_map, case.L
    coeffs = oal.oal_expand_coeffs(ng, gm, L, w.eps)
    state = oal.oal_state_alloc(1, 2)
    y = torch.empty(tuple(case.q.shape), dtype=torch.bfloat16, device="cuda")
    ws = oal.alloc_workspace(oal.oal_prefill_workspace_bytes(1, 14, 2, w.seq_len, 128,
                                                             oal.OAL_BF16, True))

    def step():
        oal.oal_expand_coeffs(ng, gm, L, w.eps, coeffs)
        oal.oal_state_reset(state)
        oal.oal_prefill(case.q, case.k, case.v, coeffs, chunk=128, state=state, y=y, workspace=ws)

    step()
    torch.cuda.synchronize()
    y_ref = y.clone()
    st_ref = oal.oal_state_export(state)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        y.zero_()                      # eager work between replays
        oal.oal_state_reset(state)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), rep
        assert torch.equal(oal.oal_state_export(state), st_ref), rep
    state.free()
