"""GPU parity of the chunk-256 readout in each of its launch layouts.

The readout's items (unit x chunk, head group) run per XCD in rounds of two
workgroups per CU.  Items that fill at most half of one round run as half
workgroups (one 32-token tile per wave, two workgroups per item); other item
counts run whole workgroups.  On a 256-CU device (64 slots per XCD) the
Qwen-shaped 14/2 layer gives: N = 2048, 14 items per XCD, half workgroups;
N = 9216, 63 items per XCD, whole workgroups.  Every layout is checked against
the float64 oracle, and the two layouts against each other on shared tokens."""

import numpy as np
import pytest
import torch

from positive_quadratic_causal_amd import synth

from gpu_util import TOL_BF16, Case, announce, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def oal():
    from positive_quadratic_causal_amd import oal as mod
    return mod


def _rows_ok(y, ref, what):
    rows = np.linalg.norm(y - ref, axis=-1) / np.maximum(np.linalg.norm(ref, axis=-1), 1e-30)
    assert rel_l2(y, ref) <= TOL_BF16, (what, rel_l2(y, ref))
    assert rows.max() <= TOL_BF16, (what, int(np.argmax(rows)), float(rows.max()))


def _qwen(n):
    return synth.small_workload(330, f"Qwen-shaped 14/2 N={n}", 1, 14, 2, n, "bf16", grouping="qwen")


def test_half_workgroups_all_heads_2048(oal):
    """N = 2048: 14 items per XCD, all as half workgroups; every head, every row."""
    w = _qwen(2048)
    announce("readout layouts: Qwen-shaped 14/2 N=2048 chunk=256 (half workgroups), all heads")
    case = Case(w)
    y = oal.oal_prefill(case.q, case.k, case.v, case.coeffs(), chunk=256)
    torch.cuda.synchronize()
    yc = y.float().cpu().numpy()
    assert np.all(np.isfinite(yc))
    for h in range(14):
        _rows_ok(yc[0, h], case.oracle_head(0, h), h)


def test_whole_workgroups_9216_against_half_2048(oal):
    """N = 9216 (whole workgroups only) against the oracle on sampled rows of every
    head, and its first 2048 tokens against the half-workgroup run of those tokens
    alone (causal: the same outputs up to rounding)."""
    w = _qwen(9216)
    announce("readout layouts: Qwen-shaped 14/2 N=9216 chunk=256 (whole workgroups) vs N=2048 (half)")
    case = Case(w)
    y = oal.oal_prefill(case.q, case.k, case.v, case.coeffs(), chunk=256)
    n0 = 2048
    y0 = oal.oal_prefill(case.q[:, :, :n0].contiguous(), case.k[:, :, :n0].contiguous(),
                         case.v[:, :, :n0].contiguous(), case.coeffs(), chunk=256)
    torch.cuda.synchronize()
    yc = y.float().cpu().numpy()
    y0c = y0.float().cpu().numpy()
    assert np.all(np.isfinite(yc)) and np.all(np.isfinite(y0c))
    # the two launch layouts agree far inside the accuracy bar
    assert rel_l2(y0c, yc[:, :, :n0]) <= 2e-3, rel_l2(y0c, yc[:, :, :n0])
    rng = np.random.default_rng(5)
    edges = np.arange(256, 9216, 256)
    rows = np.unique(np.concatenate([rng.integers(0, 9216, 24), edges, edges - 1, [0, 9215]]))
    for h in range(14):
        _rows_ok(yc[0, h, rows], case.oracle_rows(0, h, rows), h)


@pytest.mark.parametrize("n", [1000, 4700])
def test_half_workgroups_ragged(oal, n):
    """Ragged lengths (a partial last chunk), fp32 outputs: B = 3, 6/2 heads gives
    9 items per XCD at N = 1000 (half workgroups) and 45 at N = 4700 (whole ones)."""
    w = synth.small_workload(331, f"ragged B=3 6/2 N={n}", 3, 6, 2, n, "bf16", grouping="qwen")
    announce(f"readout layouts: ragged B=3 6/2 N={n} chunk=256 fp32 out")
    case = Case(w)
    y = torch.empty((3, 6, n, 64), dtype=torch.float32, device="cuda")
    oal.oal_prefill(case.q, case.k, case.v, case.coeffs(), chunk=256, y=y)
    torch.cuda.synchronize()
    yc = y.cpu().numpy()
    assert np.all(np.isfinite(yc))
    for b, h in [(0, 0), (1, 2), (2, 3), (2, 5)]:
        _rows_ok(yc[b, h], case.oracle_head(b, h), (b, h))
