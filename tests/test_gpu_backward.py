"""GPU parity of the prefill backward (oal_prefill_backward, oal_coeffs_backward)
against the float64 gradient oracle, which is pinned against finite differences
of the forward oracles.  Loss sum_i dy_i . y_i with seeded dy; bars as for the
forward: rel-L2 1e-4 (fp32 inputs) and 2e-2 (bf16 inputs; the oracle takes the
same bf16 values, so the error is the fp32 arithmetic)."""

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


def _dy(seed, shape):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


def _grouped_abc(case, h):
    st = case.st
    return O.expand_coeffs(st.L[h].astype(np.float64), st.group_map[h], int(st.n_groups[h]),
                           case.w.eps)


def _oracle_grads(case, dy, coef_of_head, rows=None):
    """Per query head oracle gradients; dk, dv summed over the heads of each KV
    head, da, db, dC over the batch."""
    w = case.w
    rep = w.n_q_heads // w.n_kv_heads
    n = case.n
    dq = np.zeros((w.batch, w.n_q_heads, n, 64))
    dk = np.zeros((w.batch, w.n_kv_heads, n, 64))
    dv = np.zeros((w.batch, w.n_kv_heads, n, 64))
    da = np.zeros(w.n_q_heads)
    db = np.zeros((w.n_q_heads, 64))
    dC = np.zeros((w.n_q_heads, 64, 64))
    for b in range(w.batch):
        for h in range(w.n_q_heads):
            q, k, v = case.head_qkv(b, h)
            a, bb, C = coef_of_head(h)
            g = O.causal_attention_dim_grad(q, k, v, a, bb, C, dy[b, h], rows=rows)
            dq[b, h] = g[0]
            dk[b, h // rep] += g[1]
            dv[b, h // rep] += g[2]
            da[h] += g[3]
            db[h] += g[4]
            dC[h] += g[5]
    return dq, dk, dv, da, db, dC


def _run(oal, case, dy, coeffs, chunk):
    dyt = torch.from_numpy(dy).cuda()
    out = oal.oal_prefill_backward(case.q, case.k, case.v, coeffs, dyt, chunk=chunk)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [64, 128])
@pytest.mark.parametrize("n", [1, 70, 200])
def test_backward_grouped_small(oal, dtype, chunk, n):
    w = synth.small_workload(800 + n, "bwd", 2, 6, 2, n, dtype, grouping="llama")
    announce(f"backward B=2 6/2 N={n} {dtype} chunk={chunk}")
    case = Case(w)
    dy = _dy(801 + n, (2, 6, n, 64))
    got = _run(oal, case, dy, case.coeffs(), chunk)
    ref = _oracle_grads(case, dy, lambda h: _grouped_abc(case, h))
    tol = tol_for(w)
    names = ["dq", "dk", "dv", "da", "db", "dC"]
    for name, g_, r_ in zip(names, got, ref):
        assert np.all(np.isfinite(g_)), name
        if n == 1 and name != "dv":
            # one token: y_0 = v_0 whatever q and k are, so these gradients are 0
            # (alpha_00 = g_0 . u_0 = 0); only rounding remains
            assert np.abs(g_).max() <= 1e-4 * max(1.0, np.abs(ref[2]).max()), name
            continue
        err = rel_l2(g_, r_)
        assert err <= tol, (name, err)
    # dL through the grouped map, against the oracle's chain rule on the oracle's (da, db, dC)
    dL = oal.oal_coeffs_backward(case.n_groups, case.group_map, case.L,
                                 *[torch.from_numpy(np.asarray(x, dtype=np.float32)).cuda()
                                   for x in ref[3:]])
    torch.cuda.synchronize()
    dLr = np.stack([O.grouped_coeff_grad(case.st.L[h].astype(np.float64), case.st.group_map[h],
                                         int(case.st.n_groups[h]), ref[3][h], ref[4][h], ref[5][h])
                    for h in range(6)])
    if n > 1:
        assert rel_l2(dL.cpu().numpy(), dLr) <= 1e-5


@pytest.mark.parametrize("chunk", [64, 128])
def test_backward_single_group(oal, chunk):
    """G = 1 (one group holding every dim): the learned-global kernel through the
    backward, where the matrix-core pair kernel has one group-sum chain and two
    weighted terms (v = 0, 1)."""
    w = synth.small_workload(870, "bwd global", 1, 4, 2, 150, "f32")
    announce(f"backward G=1 4/2 N=150 f32 chunk={chunk}")
    case = Case(w)
    rng = np.random.default_rng(13)
    for h in range(4):
        case.st.n_groups[h] = 1
        case.st.group_map[h] = 1
        case.st.L[h] = synth.random_L(rng, 1)
    case.n_groups = torch.from_numpy(case.st.n_groups.astype(np.int32)).to("cuda")
    case.group_map = torch.from_numpy(case.st.group_map.astype(np.int32)).to("cuda")
    case.L = torch.from_numpy(case.st.L.astype(np.float32)).to("cuda")
    dy = _dy(871, (1, 4, 150, 64))
    got = _run(oal, case, dy, case.coeffs(), chunk)
    ref = _oracle_grads(case, dy, lambda h: _grouped_abc(case, h))
    for name, g_, r_ in zip(["dq", "dk", "dv", "da", "db", "dC"], got, ref):
        err = rel_l2(g_, r_)
        assert err <= 1e-4, (name, err)


def test_backward_dimension_specific_record(oal):
    w = synth.small_workload(830, "bwd dim", 1, 7, 1, 150, "f32")
    announce("backward with a dimension-specific record, 7/1 N=150 f32 chunk=64")
    case = Case(w)
    a, b, C = synth.dim_coefficients(w)
    coeffs = oal.oal_dim_coeffs(*(torch.from_numpy(x).cuda() for x in (a, b, C)))
    dy = _dy(831, (1, 7, 150, 64))
    got = _run(oal, case, dy, coeffs, 64)
    ref = _oracle_grads(case, dy, lambda h: (float(a[h]), b[h].astype(np.float64),
                                             C[h].astype(np.float64)))
    for name, g_, r_ in zip(["dq", "dk", "dv", "da", "db", "dC"], got, ref):
        err = rel_l2(g_, r_)
        assert err <= 1e-4, (name, err)


@pytest.mark.parametrize("chunk", [64, 128])
def test_backward_mixed_records(oal, chunk):
    """Grouped and dimension-specific records in the same GQA groups: at chunk 64
    the grouped heads take the matrix-core pair kernel and the others the vector
    kernels, and the key side adds one pair part for the former and four for the
    latter."""
    w = synth.small_workload(860, "bwd mixed", 1, 6, 2, 150, "f32", grouping="llama")
    announce(f"backward with mixed records, 6/2 N=150 f32 chunk={chunk}")
    case = Case(w)
    a, b, C = synth.dim_coefficients(w)
    grouped = case.coeffs()
    dim = oal.oal_dim_coeffs(*(torch.from_numpy(x).cuda() for x in (a, b, C)))
    is_dim = [h % 2 == 1 for h in range(6)]   # each KV group holds both kinds
    coeffs = torch.stack([dim[h] if is_dim[h] else grouped[h] for h in range(6)]).contiguous()
    dy = _dy(861, (1, 6, 150, 64))
    got = _run(oal, case, dy, coeffs, chunk)

    def coef(h):
        if is_dim[h]:
            return float(a[h]), b[h].astype(np.float64), C[h].astype(np.float64)
        return _grouped_abc(case, h)

    ref = _oracle_grads(case, dy, coef)
    for name, g_, r_ in zip(["dq", "dk", "dv", "da", "db", "dC"], got, ref):
        err = rel_l2(g_, r_)
        assert err <= 1e-4, (name, err)


def test_backward_without_coefficient_gradients(oal):
    w = synth.small_workload(840, "bwd nocoef", 1, 4, 2, 130, "bf16")
    announce("backward without coefficient gradients, 4/2 N=130 bf16")
    case = Case(w)
    dy = torch.from_numpy(_dy(841, (1, 4, 130, 64))).cuda()
    full = oal.oal_prefill_backward(case.q, case.k, case.v, case.coeffs(), dy, chunk=64)
    part = oal.oal_prefill_backward(case.q, case.k, case.v, case.coeffs(), dy, chunk=64,
                                    want_coeff_grad=False)
    torch.cuda.synchronize()
    for x, y in zip(full[:3], part[:3]):
        assert torch.equal(x, y)
    assert part[3] is None


def test_backward_qwen_2048_sampled(oal):
    """Full-size Qwen-shaped layer: dq on sampled rows and dk, dv on keys in the
    last two chunks (whose rows i >= j are all evaluated by the oracle), so both the
    prefix-state and the suffix-state paths are checked at this size."""
    w = synth.WORKLOADS[1]
    announce("backward Qwen-shaped 14/2 N=2048 bf16 chunk=64, sampled rows and keys")
    case = Case(w)
    n = w.seq_len
    dy = _dy(850, (1, 14, n, 64))
    got = _run(oal, case, dy, case.coeffs(), 64)
    rows_q = [0, 63, 64, 1000, 1937]
    tail0 = n - 100
    rows = sorted(set(rows_q) | set(range(tail0, n)))
    keys = list(range(tail0, n))
    rep = 7
    for h in (0, 9):
        q, k, v = case.head_qkv(0, h)
        a, bb, C = _grouped_abc(case, h)
        g = O.causal_attention_dim_grad(q, k, v, a, bb, C, dy[0, h], rows=rows)
        assert rel_l2(got[0][0, h, rows_q], g[0][rows_q]) <= 2e-2
    for kv in (0, 1):
        dk = np.zeros((n, 64))
        dv = np.zeros((n, 64))
        for h in range(kv * rep, kv * rep + rep):
            q, k, v = case.head_qkv(0, h)
            a, bb, C = _grouped_abc(case, h)
            g = O.causal_attention_dim_grad(q, k, v, a, bb, C, dy[0, h], rows=range(tail0, n))
            dk += g[1]
            dv += g[2]
        assert rel_l2(got[1][0, kv, keys], dk[keys]) <= 2e-2
        assert rel_l2(got[2][0, kv, keys], dv[keys]) <= 2e-2
