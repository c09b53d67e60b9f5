"""CPU checks of the Python binding's argument validation: a tensor of the wrong
shape, dtype or device, a short workspace or a state of the wrong size raises
ValueError before any device pointer reaches the library.  The tensors here are
CPU tensors passed off as GPU ones (the device test is patched), and every
computing entry point of the library is replaced by a recorder that fails the
test if it is ever reached."""

import os

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "positive_quadratic_causal_amd", "liboal.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="liboal.so not built")

COMPUTE = ("oal_expand_coeffs", "oal_dim_coeffs", "oal_prefill", "oal_prefill_fresh", "oal_prefill_dim",
           "oal_decode_step", "oal_prefill_backward", "oal_coeffs_backward",
           "oal_softmax_attention", "oal_state_export", "oal_calib_grad", "oal_adam_step",
           "oal_output_mse", "oal_embed_global", "oal_contribution_scores",
           "oal_bootstrap_grouping")


@pytest.fixture
def oal(monkeypatch):
    from positive_quadratic_causal_amd import oal as mod
    reached = []
    for name in COMPUTE:
        monkeypatch.setattr(mod._lib, name, lambda *a, _n=name: reached.append(_n) or 0)
    monkeypatch.setattr(mod, "_on_gpu", lambda t: True)
    monkeypatch.setattr(mod, "_stream", lambda t=None: None)
    mod._reached = reached
    yield mod
    del mod._reached


def fake_state(oal, b, h):
    """An OalState look-alike whose handle is never freed (nor dereferenced: every
    call that could take it is a recorder here)."""
    class Fake(oal.OalState):
        def __init__(self):
            self.handle, self.batch, self.n_kv_heads = 1, b, h

        def __del__(self):
            pass
    return Fake()


bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32


def qkv(B=1, Hq=4, Hkv=2, N=16, dt=bf):
    return (torch.zeros(B, Hq, N, 64, dtype=dt), torch.zeros(B, Hkv, N, 64, dtype=dt),
            torch.zeros(B, Hkv, N, 64, dtype=dt))


def coeffs(oal, Hq=4):
    return torch.zeros(Hq, oal.COEF_WORDS, dtype=f32)


def test_prefill_rejects_mismatches(oal):
    q, k, v = qkv()
    c = coeffs(oal)
    cases = [
        dict(q=q.float(), k=k, v=v, coeffs=c),                        # q dtype != k dtype
        dict(q=q, k=k, v=v.float(), coeffs=c),                        # v dtype
        dict(q=q[:, :, :8].contiguous(), k=k, v=v, coeffs=c),         # q length != N
        dict(q=q, k=k, v=v[:, :, :8].contiguous(), coeffs=c),         # v length
        dict(q=q, k=k, v=torch.zeros(1, 2, 16, 32, dtype=bf), coeffs=c),   # d_v
        dict(q=q, k=k, v=v, coeffs=coeffs(oal, 3)),                   # coeffs rows < Hq
        dict(q=q, k=k, v=v, coeffs=c.to(torch.float64)),              # coeffs dtype
        dict(q=q, k=k, v=v, coeffs=None),                             # coeffs missing
        dict(q=q, k=k, v=v, coeffs=c, y=torch.zeros(1, 4, 15, 64, dtype=bf)),    # y shape
        dict(q=q, k=k, v=v, coeffs=c, y=torch.zeros(1, 4, 16, 64, dtype=torch.float16)),
        dict(q=q, k=k, v=v, coeffs=c, workspace=torch.zeros(16, dtype=torch.uint8)),  # short
        dict(q=q.transpose(2, 3), k=k, v=v, coeffs=c),                # not contiguous
        dict(q=None, k=k, v=v, coeffs=c),                             # output wanted, no q
    ]
    for kw in cases:
        with pytest.raises(ValueError):
            oal.oal_prefill(**kw)
        with pytest.raises(ValueError):
            oal.oal_prefill_dim(**kw)
    assert not oal._reached
    # the well-formed call does reach the library (the checks are not vacuous)
    oal.oal_prefill(q, k, v, c, workspace=torch.zeros(1 << 26, dtype=torch.uint8))
    assert oal._reached == ["oal_prefill"]


def test_prefill_rejects_a_state_of_another_size(oal):
    q, k, v = qkv()

    with pytest.raises(ValueError):
        oal.oal_prefill(q, k, v, coeffs(oal), state=fake_state(oal, 2, 2))
    with pytest.raises(ValueError):
        oal.oal_prefill_fresh(q, k, v, coeffs(oal), fake_state(oal, 2, 2))
    with pytest.raises(ValueError):
        oal.oal_prefill_fresh(q, k, v, coeffs(oal), None)
    with pytest.raises(ValueError):
        oal.oal_decode_step(q[:, :, 0].contiguous(), k[:, :, 0].contiguous(), v[:, :, 0].contiguous(),
                            coeffs(oal), fake_state(oal, 1, 1))
    with pytest.raises(ValueError):
        oal.oal_state_export(fake_state(oal, 1, 2), out=torch.zeros(1, 2, 2145, 64, dtype=f32))
    assert not oal._reached


def test_decode_rejects_mismatches(oal):
    q, k, v = (t[:, :, 0].contiguous() for t in qkv())
    c = coeffs(oal)
    with pytest.raises(ValueError):
        oal.oal_decode_step(q, k, v, c, None)
    st = fake_state(oal, 1, 2)
    for args in [(q.float(), k, v, c), (q, k[:, :1].contiguous(), v, c), (q, k, v[:, :, :32].contiguous(), c),
                 (q, k, v, coeffs(oal, 2))]:
        with pytest.raises(ValueError):
            oal.oal_decode_step(*args, state=st)
    assert not oal._reached
    oal.oal_decode_step(q, k, v, c, st)
    assert oal._reached == ["oal_decode_step"]


def test_other_calls_reject_mismatches(oal):
    q, k, v = qkv()
    c = coeffs(oal)
    with pytest.raises(ValueError):      # dy shape
        oal.oal_prefill_backward(q, k, v, c, torch.zeros(1, 4, 15, 64, dtype=f32))
    with pytest.raises(ValueError):      # dy dtype
        oal.oal_prefill_backward(q, k, v, c, torch.zeros(1, 4, 16, 64, dtype=bf))
    with pytest.raises(ValueError):      # Hkv of v != k
        oal.oal_softmax_attention(q, k, torch.zeros(1, 1, 16, 64, dtype=bf))
    L = torch.zeros(4, 7, 7, dtype=f32)
    with pytest.raises(ValueError):      # group map width
        oal.oal_expand_coeffs(torch.ones(4, dtype=i32), torch.ones(4, 32, dtype=i32), L, 1e-6)
    with pytest.raises(ValueError):      # n_groups dtype
        oal.oal_expand_coeffs(torch.ones(4, dtype=torch.int64), torch.ones(4, 64, dtype=i32), L, 1e-6)
    with pytest.raises(ValueError):      # C shape
        oal.oal_dim_coeffs(torch.zeros(4, dtype=f32), torch.zeros(4, 64, dtype=f32),
                           torch.zeros(4, 64, 32, dtype=f32))
    with pytest.raises(ValueError):      # offsets dtype
        oal.oal_contribution_scores(q[0], k[0], torch.zeros(3, dtype=torch.int64))
    with pytest.raises(ValueError):      # bootstrap indices of another prompt count
        oal.oal_bootstrap_grouping(torch.zeros(5, 4, 64, dtype=f32), torch.zeros(10, 4, dtype=i32))
    with pytest.raises(ValueError):      # y_ref shape
        oal.oal_output_mse(torch.zeros(1, 4, 16, 64, dtype=f32), torch.zeros(1, 4, 8, 64, dtype=f32))
    assert not oal._reached


def test_grouped_prefill_refuses_a_dimension_specific_record(oal):
    """A buffer that oal_dim_coeffs filled last is refused by the grouped prefill
    calls on the host (the library could only make the outputs NaN); once
    oal_expand_coeffs refills it, it is accepted again."""
    q, k, v = qkv()
    c = coeffs(oal)
    a, b, C = torch.zeros(4, dtype=f32), torch.zeros(4, 64, dtype=f32), torch.zeros(4, 64, 64, dtype=f32)
    oal.oal_dim_coeffs(a, b, C, c)
    for call in (lambda: oal.oal_prefill(q, k, v, c),
                 lambda: oal.oal_prefill_fresh(q, k, v, c, fake_state(oal, 1, 2)),
                 lambda: oal.oal_prefill_noalloc(q, k, v, c, y=torch.zeros(1, 4, 16, 64, dtype=bf))):
        with pytest.raises(ValueError, match="dimension-specific"):
            call()
    assert "oal_prefill" not in oal._reached and "oal_prefill_fresh" not in oal._reached
    ng, gm, L = torch.ones(4, dtype=i32), torch.zeros(4, 64, dtype=i32), torch.zeros(4, 7, 7, dtype=f32)
    oal.oal_expand_coeffs(ng, gm, L, 1e-6, c)
    oal._refuse_dim_record(c)   # accepted again
