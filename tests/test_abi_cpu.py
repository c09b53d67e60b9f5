"""CPU checks of the C ABI: the library loads, exports every function that
include/oal.h declares, and rejects invalid arguments on the host before any
HIP call (no compute runs here: this host has no GPU)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "positive_quadratic_causal_amd", "liboal.so")
HEADER = os.path.join(ROOT, "include", "oal.h")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="liboal.so not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(oal_[a-z_]+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("oal_expand_coeffs", "oal_prefill", "oal_decode_step", "oal_state_alloc"):
        assert required in names


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(LIB)
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_names_match_the_abi():
    from positive_quadratic_causal_amd import oal
    for n in _declared_functions():
        assert hasattr(oal, n), n
        assert n in oal.EXPORTED


def _lib():
    from positive_quadratic_causal_amd import oal
    return oal._lib, oal


def test_sizes():
    lib, oal = _lib()
    assert lib.oal_coeffs_bytes(14, 64, 6) == 14 * oal.COEF_WORDS * 4
    assert lib.oal_coeffs_bytes(14, 32, 6) == 0
    assert lib.oal_coeffs_bytes(14, 64, 7) == 0
    assert lib.oal_prefill_workspace_bytes(1, 14, 2, 0, 64, 64, 128, oal.OAL_BF16, 1) == 0
    assert lib.oal_prefill_workspace_bytes(1, 14, 3, 100, 64, 64, 128, oal.OAL_BF16, 1) == 0
    assert lib.oal_prefill_workspace_bytes(1, 14, 2, 100, 64, 64, 100, oal.OAL_BF16, 1) == 0
    assert lib.oal_prefill_workspace_bytes(1, 14, 2, 100, 64, 64, 0, oal.OAL_BF16, 1) > 0
    assert lib.oal_prefill_workspace_bytes(1, 14, 2, 100, 64, 64, 0, oal.OAL_F32, 1) > 0
    assert lib.oal_prefill_workspace_bytes(1, 14, 2, 100, 64, 64, 0, oal.OAL_F32, 0) == 0
    # state only: scratch for the segment sums and the staged fp16 copy of k and v
    # (as large as the inputs), far less than the per-chunk tiles
    so = lib.oal_prefill_workspace_bytes(64, 32, 8, 8192, 64, 64, 128, oal.OAL_BF16, 0)
    wo = lib.oal_prefill_workspace_bytes(64, 32, 8, 8192, 64, 64, 128, oal.OAL_BF16, 1)
    kv_bytes = 2 * 64 * 8 * 8192 * 64 * 2
    assert kv_bytes <= so < kv_bytes + wo / 10 < wo / 5
    assert lib.oal_prefill_workspace_bytes(1, 14, 2, 32768, 64, 64, 128, oal.OAL_BF16, 0) > 0
    assert lib.oal_state_bytes(None) == 0
    assert lib.oal_state_tokens(None) == -1


P = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


@pytest.mark.parametrize("args,expect", [
    # batch, Hq, Hkv, N, d_h, d_v, in_dt, q, k, v, coeffs, chunk, state, y, out_dt, ws, wsb
    ((0, 14, 2, 16, 64, 64, 1, P, P, P, P, 0, None, P, 1, P, 1 << 30), 1),
    ((1, 14, 3, 16, 64, 64, 1, P, P, P, P, 0, None, P, 1, P, 1 << 30), 1),
    ((1, 14, 2, 16, 32, 64, 1, P, P, P, P, 0, None, P, 1, P, 1 << 30), 2),
    ((1, 14, 2, 16, 64, 64, 7, P, P, P, P, 0, None, P, 1, P, 1 << 30), 1),
    ((1, 14, 2, 16, 64, 64, 1, P, P, P, P, 100, None, P, 1, P, 1 << 30), 1),
    ((1, 14, 2, -1, 64, 64, 1, P, P, P, P, 0, None, P, 1, P, 1 << 30), 1),
    ((1, 14, 2, 16, 64, 64, 1, P, P, P, P, 0, None, None, 1, P, 1 << 30), 1),  # nothing to do
    ((1, 14, 2, 16, 64, 64, 1, None, P, P, P, 0, None, P, 1, P, 1 << 30), 1),  # q null
    ((1, 14, 2, 16, 64, 64, 1, P, P, P, P, 0, None, P, 1, P, 10), 1),          # ws too small
    ((1, 14, 2, 16, 64, 64, 1, P, P, P, P, 0, None, P, 1, None, 1 << 30), 1),  # ws null
    ((1, 14, 2, 16, 64, 64, 1, P, P, P, P, 0, None, P, 1, ctypes.c_void_p(0x1010), 1 << 30), 1),
])
@pytest.mark.parametrize("entry", ["oal_prefill", "oal_prefill_dim"])
def test_prefill_rejects_invalid_arguments(args, expect, entry):
    lib, oal = _lib()
    st = getattr(lib, entry)(*args, None)
    assert st == expect, lib.oal_last_error()
    assert lib.oal_last_error()


def test_prefill_fresh_needs_a_state():
    lib, oal = _lib()
    assert lib.oal_prefill_fresh(1, 14, 2, 16, 64, 64, 1, P, P, P, P, 0, None, P, 1, P, 1 << 30,
                                 None) == 1
    assert b"state" in lib.oal_last_error()


def test_prefill_empty_sequence_is_a_noop():
    lib, oal = _lib()
    assert lib.oal_prefill(1, 14, 2, 0, 64, 64, 1, P, P, P, P, 0, None, P, 1, None, 0, None) == 0
    assert lib.oal_prefill_dim(1, 14, 2, 0, 64, 64, 1, P, P, P, P, 0, None, P, 1, None, 0, None) == 0


def test_dim_entries_sizes_and_checks():
    lib, oal = _lib()
    # the general path's workspace: one prefix state per (unit, chunk), any input dtype
    per_state = 65 * 2176 * 4
    assert lib.oal_prefill_dim_workspace_bytes(1, 14, 2, 300, 64, 64, 128, 1) == 2 * 3 * per_state
    assert lib.oal_prefill_dim_workspace_bytes(1, 14, 2, 300, 64, 64, 0, 0) == 0
    assert lib.oal_prefill_dim_workspace_bytes(1, 14, 2, 300, 64, 64, 96, 1) == 0
    assert lib.oal_prefill_dim_workspace_bytes(1, 14, 3, 300, 64, 64, 128, 1) == 0
    assert lib.oal_dim_coeffs(0, 64, P, P, P, P, None) == 1
    assert lib.oal_dim_coeffs(2, 32, P, P, P, P, None) == 2
    assert lib.oal_dim_coeffs(2, 64, P, None, P, P, None) == 1
    assert lib.oal_dim_coeffs(2, 64, P, P, P, None, None) == 1


def test_decode_and_expand_reject_invalid_arguments():
    lib, oal = _lib()
    assert lib.oal_decode_step(1, 14, 2, 64, 64, 1, P, P, P, P, None, P, 1, None) == 1
    assert lib.oal_decode_step(1, 14, 4, 64, 64, 1, P, P, P, P, P, P, 1, None) == 1
    assert lib.oal_decode_step(1, 14, 2, 48, 64, 1, P, P, P, P, P, P, 1, None) == 2
    assert lib.oal_expand_coeffs(4, 64, 6, P, P, P, 0.0, P, None) == 1      # eps must be > 0
    assert lib.oal_expand_coeffs(4, 64, 7, P, P, P, 1e-6, P, None) == 2     # g_max <= 6
    assert lib.oal_expand_coeffs(4, 64, 6, None, P, P, 1e-6, P, None) == 1
    assert lib.oal_state_alloc(1, 2, 64, 64, None) == 1
    out = ctypes.c_void_p()
    assert lib.oal_state_alloc(0, 2, 64, 64, ctypes.byref(out)) == 1
    assert lib.oal_state_alloc(1, 2, 64, 32, ctypes.byref(out)) == 2
    assert lib.oal_state_free(None) == 0
    for s in range(5):
        assert lib.oal_status_string(s).startswith(b"OAL_")


def test_softmax_rejects_invalid_arguments():
    lib, oal = _lib()
    # batch, Hq, Hkv, N, d_h, d_v, in_dt, q, k, v, y, out_dt, stream
    assert lib.oal_softmax_attention(1, 14, 2, 16, 64, 64, 0, P, P, P, P, 1, None) == 2   # fp32 in
    assert lib.oal_softmax_attention(1, 14, 3, 16, 64, 64, 1, P, P, P, P, 1, None) == 1   # Hq % Hkv
    assert lib.oal_softmax_attention(1, 14, 2, 16, 32, 64, 1, P, P, P, P, 1, None) == 2   # d_h
    assert lib.oal_softmax_attention(1, 14, 2, 16, 64, 64, 1, None, P, P, P, 1, None) == 1
    assert lib.oal_softmax_attention(1, 14, 2, -1, 64, 64, 1, P, P, P, P, 1, None) == 1
    assert lib.oal_softmax_attention(1, 14, 2, 0, 64, 64, 1, P, P, P, P, 1, None) == 0     # no-op


def test_backward_entries_sizes_and_checks():
    lib, oal = _lib()
    assert lib.oal_prefill_backward_workspace_bytes(1, 14, 2, 300, 64, 64, 256) == 0
    assert lib.oal_prefill_backward_workspace_bytes(1, 14, 2, 0, 64, 64, 128) == 0
    ws = lib.oal_prefill_backward_workspace_bytes(1, 14, 2, 300, 64, 64, 128)
    assert ws >= 2 * 2 * 3 * 65 * 2176 * 4
    # batch, Hq, Hkv, N, d_h, d_v, in_dt, q, k, v, coeffs, dy, chunk, dq, dk, dv, da, db, dC, ws, wsb, stream
    ok = (1, 14, 2, 16, 64, 64, 1, P, P, P, P, P, 0, P, P, P, P, P, P, P, 1 << 40, None)
    def call(**kw):
        args = list(ok)
        for i, x in kw.items():
            args[int(i[1:])] = x
        return lib.oal_prefill_backward(*args)
    assert call(a12=256) == 1                    # chunk 256 not supported by the backward
    assert call(a2=3) == 1                       # Hq % Hkv
    assert call(a4=32) == 2                      # d_h
    assert call(a11=None) == 1                   # dy null
    assert call(a17=None) == 1                   # coefficient outputs: all or none
    assert call(a20=10) == 1                     # workspace too small
    assert call(a19=ctypes.c_void_p(0x1010)) == 1  # misaligned workspace
    assert lib.oal_coeffs_backward(2, 64, 7, P, P, P, P, P, P, P, None) == 2
    assert lib.oal_coeffs_backward(2, 64, 6, P, P, None, P, P, P, P, None) == 1


def test_calibration_entries_checks():
    lib, oal = _lib()
    assert lib.oal_calib_workspace_bytes(14, 32) >= 14 * 32 * 49 * 4
    assert lib.oal_calib_workspace_bytes(0, 32) == 0
    # Hq, Hkv, N, d_h, d_v, in_dt, q, k, v, y_ref, pos, n_pos, g_max, ng, gm, L, eps, dL, loss, ws, wsb, stream
    ok = [14, 2, 100, 64, 64, 1, P, P, P, P, P, 32, 6, P, P, P, 1e-6, P, P, P, 1 << 30, None]
    def call(**kw):
        args = list(ok)
        for i, x in kw.items():
            args[int(i[1:])] = x
        return lib.oal_calib_grad(*args)
    assert call(a1=3) == 1            # Hq % Hkv
    assert call(a11=0) == 1           # n_pos
    assert call(a12=7) == 2           # g_max
    assert call(a16=0.0) == 1         # eps
    assert call(a9=None) == 1         # y_ref
    assert call(a20=8) == 1           # workspace too small
    assert lib.oal_adam_step(2, 6, P, P, P, P, P, 0, 0.02, 0.9, 0.999, 1e-8, 10.0, None) == 1   # step 0
    assert lib.oal_adam_step(2, 6, P, P, P, P, P, 1, 0.02, 1.0, 0.999, 1e-8, 10.0, None) == 1   # beta1
    assert lib.oal_output_mse(1, 2, 0, 64, P, P, P, None) == 1


def test_grouping_entries_checks():
    lib, oal = _lib()
    # Hq, Hkv, P, T, d_h, in_dt, q, k, offsets, chi_p, chi, stream
    assert lib.oal_contribution_scores(6, 4, 3, 10, 64, 1, P, P, P, P, P, None) == 1   # Hq % Hkv
    assert lib.oal_contribution_scores(6, 2, 0, 10, 64, 1, P, P, P, P, P, None) == 1   # no prompts
    assert lib.oal_contribution_scores(6, 2, 3, 10, 32, 1, P, P, P, P, P, None) == 2   # d_h
    assert lib.oal_contribution_scores(6, 2, 3, 10, 64, 1, P, None, P, P, P, None) == 1
    # Hq, P, d_h, chi_p, B, boot, alpha, tau, gamma, g_min, eps, gm, ng, sup, gap, stream
    ok = [6, 40, 64, P, 1000, P, 0.25, 1.5, 0.9, 2, 1e-12, P, P, None, None, None]
    def call(**kw):
        args = list(ok)
        for i, x in kw.items():
            args[int(i[1:])] = x
        return lib.oal_bootstrap_grouping(*args)
    assert call(a1=257) == 2          # more prompts than the kernel stages
    assert call(a4=0) == 1            # no replicates
    assert call(a6=0.0) == 1          # alpha
    assert call(a8=1.5) == 1          # gamma
    assert call(a9=0) == 1            # g_min
    assert call(a12=None) == 1        # n_groups


def test_noalloc_prefill_rejects_oversized_calls_on_the_host():
    """oal_prefill_noalloc checks its scratch limit before any HIP call (so this
    runs without a GPU): a workspace beyond the static array is refused."""
    lib, oal = _lib()
    cap = lib.oal_prefill_noalloc_scratch_bytes()
    assert cap == 128 << 20
    need = lib.oal_prefill_workspace_bytes(1, 14, 2, 32768, 64, 64, 128, oal.OAL_BF16, 1)
    assert need > cap
    st = lib.oal_prefill_noalloc(1, 14, 2, 32768, 64, 64, oal.OAL_BF16, P, P, P, P, 128, None, P,
                                 oal.OAL_BF16, None)
    assert st == oal.OAL_ERR_UNSUPPORTED
    assert b"scratch" in lib.oal_last_error()
