"""ctypes binding of liboal.so (the C ABI declared in include/oal.h).

Argument marshalling only: every step of the computation runs in the library's
HIP kernels.  Tensors are torch CUDA (HIP) tensors, which supply device memory;
calls are enqueued on torch's current stream of the tensors' device.  Importing
this module raises if liboal.so has not been built; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
import weakref

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboal.so")

OAL_OK, OAL_ERR_INVALID_ARG, OAL_ERR_UNSUPPORTED, OAL_ERR_OUT_OF_MEMORY, OAL_ERR_HIP = range(5)
OAL_F32, OAL_BF16 = 0, 1

# coefficient record layout (words), mirrors include/oal.h
COEF_A, COEF_EPS, COEF_NG = 0, 1, 2
COEF_BP, COEF_GMAP, COEF_M, COEF_L = 16, 80, 144, 208
COEF_ELL, COEF_CM, COEF_CP, COEF_MG, COEF_GPACK = 272, 720, 4816, 6896, 7344
COEF_WORDS = 7424

D_H = 64
D_V = 64
D_CANON = 2145


class OALError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with positive_quadratic_causal_amd.build.build() "
            "(hipcc --offload-arch=gfx950); there is no non-HIP fallback")
    lib = ctypes.CDLL(LIB_PATH)
    c_int, c_size, c_void, c_float = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
    sigs = {
        "oal_coeffs_bytes": (c_size, [c_int, c_int, c_int]),
        "oal_expand_coeffs": (c_int, [c_int, c_int, c_int, c_void, c_void, c_void, c_float,
                                      c_void, c_void]),
        "oal_dim_coeffs": (c_int, [c_int, c_int, c_void, c_void, c_void, c_void, c_void]),
        "oal_state_alloc": (c_int, [c_int, c_int, c_int, c_int, ctypes.POINTER(c_void)]),
        "oal_state_reset": (c_int, [c_void, c_void]),
        "oal_state_free": (c_int, [c_void]),
        "oal_state_copy": (c_int, [c_void, c_void, c_void]),
        "oal_state_bytes": (c_size, [c_void]),
        "oal_state_tokens": (ctypes.c_int64, [c_void]),
        "oal_state_export": (c_int, [c_void, c_void, c_void]),
        "oal_prefill_workspace_bytes": (c_size, [c_int, c_int, c_int, c_int, c_int, c_int,
                                                 c_int, c_int, c_int]),
        "oal_prefill": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_void, c_void,
                                c_void, c_void, c_int, c_void, c_void, c_int, c_void, c_size,
                                c_void]),
        "oal_prefill_fresh": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_void,
                                      c_void, c_void, c_void, c_int, c_void, c_void, c_int, c_void,
                                      c_size, c_void]),
        "oal_prefill_noalloc_scratch_bytes": (c_size, []),
        "oal_prefill_noalloc": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_void,
                                        c_void, c_void, c_void, c_int, c_void, c_void, c_int,
                                        c_void]),
        "oal_prefill_dim_workspace_bytes": (c_size, [c_int, c_int, c_int, c_int, c_int, c_int,
                                                     c_int, c_int]),
        "oal_prefill_dim": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_void,
                                    c_void, c_void, c_void, c_int, c_void, c_void, c_int, c_void,
                                    c_size, c_void]),
        "oal_prefill_backward_workspace_bytes": (c_size, [c_int] * 7),
        "oal_prefill_backward": (c_int, [c_int] * 7 + [c_void] * 5 + [c_int] + [c_void] * 6
                                 + [c_void, c_size, c_void]),
        "oal_coeffs_backward": (c_int, [c_int, c_int, c_int] + [c_void] * 7 + [c_void]),
        "oal_contribution_scores": (c_int, [c_int] * 6 + [c_void] * 5 + [c_void]),
        "oal_bootstrap_grouping": (c_int, [c_int] * 3 + [c_void, c_int, c_void] + [c_float] * 3
                                   + [c_int, c_float] + [c_void] * 4 + [c_void]),
        "oal_calib_workspace_bytes": (c_size, [c_int, c_int]),
        "oal_calib_grad": (c_int, [c_int] * 6 + [c_void] * 5 + [c_int, c_int] + [c_void] * 3
                           + [c_float] + [c_void] * 3 + [c_size, c_void]),
        "oal_adam_step": (c_int, [c_int, c_int] + [c_void] * 5 + [c_int] + [c_float] * 5 + [c_void]),
        "oal_output_mse": (c_int, [c_int] * 4 + [c_void] * 3 + [c_void]),
        "oal_embed_global": (c_int, [c_int, c_int, c_void, c_int, c_void, c_void, c_void]),
        "oal_decode_step": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_void, c_void,
                                    c_void, c_void, c_void, c_void, c_int, c_void]),
        "oal_softmax_attention": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_void,
                                          c_void, c_void, c_void, c_int, c_void]),
        "oal_profile_enable": (c_int, [c_int]),
        "oal_profile_filter": (c_int, [ctypes.c_char_p]),
        "oal_profile_reset": (c_int, []),
        "oal_profile_query": (c_int, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                      ctypes.POINTER(ctypes.c_int64)]),
        "oal_status_string": (ctypes.c_char_p, [c_int]),
        "oal_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()

EXPORTED = ("oal_coeffs_bytes", "oal_expand_coeffs", "oal_dim_coeffs", "oal_state_alloc",
            "oal_state_reset", "oal_state_free", "oal_state_copy", "oal_state_bytes",
            "oal_state_tokens", "oal_state_export", "oal_prefill_workspace_bytes", "oal_prefill",
            "oal_prefill_fresh",
            "oal_prefill_noalloc_scratch_bytes", "oal_prefill_noalloc",
            "oal_prefill_dim_workspace_bytes", "oal_prefill_dim",
            "oal_prefill_backward_workspace_bytes", "oal_prefill_backward", "oal_coeffs_backward",
            "oal_calib_workspace_bytes", "oal_calib_grad", "oal_adam_step", "oal_output_mse",
            "oal_embed_global",
            "oal_contribution_scores", "oal_bootstrap_grouping",
            "oal_decode_step", "oal_softmax_attention", "oal_profile_enable", "oal_profile_reset",
            "oal_profile_query", "oal_profile_filter",
            "oal_status_string", "oal_last_error")


def _status_name(status: int) -> str:
    return _lib.oal_status_string(status).decode()


def _check(status: int) -> None:
    if status != OAL_OK:
        raise OALError(status, _lib.oal_last_error().decode())


def _stream(t: torch.Tensor | None = None):
    dev = t.device if t is not None and t.is_cuda else None
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not _on_gpu(t):
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return OAL_F32
    if t.dtype == torch.bfloat16:
        return OAL_BF16
    raise ValueError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _on_gpu(t: torch.Tensor) -> bool:
    return t.is_cuda


def _expect(t: torch.Tensor | None, name: str, shape: tuple | None = None, dtypes=None,
            device: torch.device | None = None, optional: bool = False) -> None:
    """Raises ValueError unless t is a contiguous GPU tensor of the given shape
    (None entries match any size), one of the given dtypes and on the given device.
    Every check runs before any device pointer is handed to the library, so a
    mismatched tensor never reaches a kernel."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if not _on_gpu(t):
        raise ValueError(f"{name} must be on the GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {tuple(dtypes)}")
    if shape is not None:
        if t.dim() != len(shape) or any(e is not None and int(d) != e for d, e in zip(t.shape, shape)):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected "
                             f"{tuple('*' if e is None else e for e in shape)}")


_IN_DTYPES = (torch.float32, torch.bfloat16)
_F32 = (torch.float32,)
_I32 = (torch.int32,)


def _expect_coeffs(coeffs: torch.Tensor | None, n_q_heads: int, device, optional: bool = False) -> None:
    _expect(coeffs, "coeffs", None, _F32, device, optional)
    if coeffs is not None and (coeffs.dim() != 2 or coeffs.shape[0] < n_q_heads
                               or coeffs.shape[1] != COEF_WORDS):
        raise ValueError(f"coeffs has shape {tuple(coeffs.shape)}, expected ({n_q_heads}, {COEF_WORDS})")


def _expect_state(state, batch: int, n_kv_heads: int) -> None:
    if state is None:
        return
    if not isinstance(state, OalState) or not state.handle:
        raise ValueError("state must be a live OalState")
    if state.batch != batch or state.n_kv_heads != n_kv_heads:
        raise ValueError(f"state holds ({state.batch}, {state.n_kv_heads}) units, "
                         f"expected ({batch}, {n_kv_heads})")


def _expect_workspace(ws: torch.Tensor | None, nbytes: int, device) -> None:
    if ws is None:
        return
    _expect(ws, "workspace", None, (torch.uint8,), device)
    if ws.numel() < nbytes:
        raise ValueError(f"workspace holds {ws.numel()} bytes, {nbytes} needed")


# ---------------------------------------------------------------------------


# Buffers that oal_dim_coeffs filled last (keyed by address, holding the tensor
# weakly): the grouped prefill calls refuse them on the host, since the library
# reads a record's kind only on the device (where it can only make the outputs NaN).
_DIM_RECORDS: dict = {}


def _mark_record(coeffs: torch.Tensor, dimension_specific: bool) -> None:
    if dimension_specific:
        _DIM_RECORDS[coeffs.data_ptr()] = weakref.ref(coeffs)
    else:
        _DIM_RECORDS.pop(coeffs.data_ptr(), None)


def _refuse_dim_record(coeffs: torch.Tensor | None) -> None:
    if coeffs is None:
        return
    ref = _DIM_RECORDS.get(coeffs.data_ptr())
    if ref is not None and ref() is coeffs:
        raise ValueError("coeffs holds a dimension-specific record (oal_dim_coeffs): "
                         "the grouped prefill cannot evaluate it; use oal_prefill_dim")


def oal_coeffs_bytes(n_q_heads: int, d_h: int = D_H, g_max: int = 6) -> int:
    return int(_lib.oal_coeffs_bytes(n_q_heads, d_h, g_max))


def oal_expand_coeffs(n_groups: torch.Tensor, group_map: torch.Tensor, L: torch.Tensor,
                      eps: float, coeffs: torch.Tensor | None = None) -> torch.Tensor:
    """n_groups int32 [Hq], group_map int32 [Hq, 64], L float32 [Hq, g+1, g+1].
    Returns (or fills) the coefficient buffer as a float32 tensor [Hq, COEF_WORDS]."""
    _expect(L, "L", (None, None, None), _F32)
    Hq, g_max = L.shape[0], L.shape[-1] - 1
    dev = L.device
    _expect(L, "L", (Hq, g_max + 1, g_max + 1))
    _expect(n_groups, "n_groups", (Hq,), _I32, dev)
    _expect(group_map, "group_map", (Hq, D_H), _I32, dev)
    if coeffs is None:
        coeffs = torch.empty((Hq, COEF_WORDS), dtype=torch.float32, device=dev)
    _expect_coeffs(coeffs, Hq, dev)
    _check(_lib.oal_expand_coeffs(Hq, group_map.shape[-1], g_max, _ptr(n_groups), _ptr(group_map),
                                  _ptr(L), float(eps), _ptr(coeffs), _stream(L)))
    _mark_record(coeffs, False)
    return coeffs


def oal_dim_coeffs(a: torch.Tensor, b: torch.Tensor, C: torch.Tensor,
                   coeffs: torch.Tensor | None = None) -> torch.Tensor:
    """Dimension-specific coefficients: a float32 [Hq], b float32 [Hq, 64],
    C float32 [Hq, 64, 64].  Returns (or fills) a coefficient buffer [Hq, COEF_WORDS]
    for oal_prefill_dim and oal_decode_step."""
    _expect(a, "a", (None,), _F32)
    Hq, dev = a.shape[0], a.device
    _expect(b, "b", (Hq, D_H), _F32, dev)
    _expect(C, "C", (Hq, D_H, D_H), _F32, dev)
    if coeffs is None:
        coeffs = torch.empty((Hq, COEF_WORDS), dtype=torch.float32, device=dev)
    _expect_coeffs(coeffs, Hq, dev)
    _check(_lib.oal_dim_coeffs(Hq, D_H, _ptr(a), _ptr(b), _ptr(C), _ptr(coeffs), _stream(a)))
    _mark_record(coeffs, True)
    return coeffs


class OalState:
    """Owns an oal_state* (library-owned device memory)."""

    def __init__(self, batch: int, n_kv_heads: int, d_h: int = D_H, d_v: int = D_V):
        h = ctypes.c_void_p()
        _check(_lib.oal_state_alloc(batch, n_kv_heads, d_h, d_v, ctypes.byref(h)))
        self.handle = h
        self.batch = batch
        self.n_kv_heads = n_kv_heads

    @property
    def nbytes(self) -> int:
        return int(_lib.oal_state_bytes(self.handle))

    @property
    def tokens(self) -> int:
        return int(_lib.oal_state_tokens(self.handle))

    def free(self) -> None:
        if self.handle:
            _check(_lib.oal_state_free(self.handle))
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            if self.handle:
                _lib.oal_state_free(self.handle)
        except Exception:
            pass


def oal_state_alloc(batch: int, n_kv_heads: int, d_h: int = D_H, d_v: int = D_V) -> OalState:
    return OalState(batch, n_kv_heads, d_h, d_v)


def oal_state_reset(state: OalState) -> None:
    _expect_state(state, getattr(state, "batch", -1), getattr(state, "n_kv_heads", -1))
    _check(_lib.oal_state_reset(state.handle, _stream()))


def oal_state_free(state: OalState) -> None:
    state.free()


def oal_state_copy(dst: OalState, src: OalState) -> None:
    _expect_state(src, getattr(src, "batch", -1), getattr(src, "n_kv_heads", -1))
    _expect_state(dst, src.batch, src.n_kv_heads)
    _check(_lib.oal_state_copy(dst.handle, src.handle, _stream()))


def oal_state_export(state: OalState, out: torch.Tensor | None = None,
                     device: str | torch.device = "cuda") -> torch.Tensor:
    """Canonical packed state, float32 [B, Hkv, 2145, 65]."""
    _expect_state(state, getattr(state, "batch", -1), getattr(state, "n_kv_heads", -1))
    if out is None:
        out = torch.empty((state.batch, state.n_kv_heads, D_CANON, D_V + 1), dtype=torch.float32,
                          device=device)
    _expect(out, "out", (state.batch, state.n_kv_heads, D_CANON, D_V + 1), _F32)
    _check(_lib.oal_state_export(state.handle, _ptr(out), _stream(out)))
    return out


def oal_prefill_workspace_bytes(batch: int, n_q_heads: int, n_kv_heads: int, seq_len: int,
                                chunk: int = 0, in_dtype: int = OAL_BF16,
                                with_output: bool = True) -> int:
    return int(_lib.oal_prefill_workspace_bytes(batch, n_q_heads, n_kv_heads, seq_len, D_H, D_V,
                                                chunk, in_dtype, 1 if with_output else 0))


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor | None:
    """A device buffer of at least nbytes (torch's allocator aligns to 512 B)."""
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _prefill_args(q, k, v, coeffs, state, y, want_output):
    """Shapes of a prefill call, checked: k, v [B, Hkv, N, 64] of one input dtype;
    q [B, Hq, N, 64] of that dtype and coeffs [Hq, COEF_WORDS] when outputs are
    wanted; y [B, Hq, N, 64] fp32 or bf16 (allocated in q's dtype if not given)."""
    _expect(k, "k", (None, None, None, D_H), _IN_DTYPES)
    B, Hkv, N, _ = k.shape
    dev = k.device
    _expect(v, "v", (B, Hkv, N, D_V), (k.dtype,), dev)
    if want_output or q is not None:
        _expect(q, "q", (B, None, N, D_H), (k.dtype,), dev)
        Hq = q.shape[1]
        _expect_coeffs(coeffs, Hq, dev, optional=not want_output)
    else:
        Hq = coeffs.shape[0] if coeffs is not None else Hkv
        _expect_coeffs(coeffs, Hq, dev, optional=True)
    _expect_state(state, B, Hkv)
    if want_output:
        if y is None:
            y = torch.empty((B, Hq, N, D_V), dtype=q.dtype, device=dev)
        _expect(y, "y", (B, Hq, N, D_V), _IN_DTYPES, dev)
    elif y is not None:
        raise ValueError("y given with want_output=False")
    return B, Hkv, N, Hq, y


def oal_prefill(q: torch.Tensor | None, k: torch.Tensor, v: torch.Tensor, coeffs: torch.Tensor | None,
                chunk: int = 0, state: OalState | None = None, y: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None, want_output: bool = True) -> torch.Tensor | None:
    """q [B, Hq, N, 64] (or None with want_output=False), k/v [B, Hkv, N, 64].
    Returns y [B, Hq, N, 64] in q's dtype unless y is given or want_output is False."""
    return _prefill_call(_lib.oal_prefill, q, k, v, coeffs, chunk, state, y, workspace, want_output)


def oal_prefill_fresh(q: torch.Tensor | None, k: torch.Tensor, v: torch.Tensor,
                      coeffs: torch.Tensor | None, state: OalState, chunk: int = 0,
                      y: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                      want_output: bool = True) -> torch.Tensor | None:
    """oal_prefill of a sequence that starts empty, written into state (its contents
    on entry are ignored and replaced)."""
    if state is None:
        raise ValueError("oal_prefill_fresh needs a state")
    return _prefill_call(_lib.oal_prefill_fresh, q, k, v, coeffs, chunk, state, y, workspace,
                         want_output)


def _prefill_call(fn, q, k, v, coeffs, chunk, state, y, workspace, want_output):
    _refuse_dim_record(coeffs)
    B, Hkv, N, Hq, y = _prefill_args(q, k, v, coeffs, state, y, want_output)
    dh, dv = D_H, D_V
    in_dt = _dtype_code(k)
    out_dt = _dtype_code(y) if y is not None else OAL_F32
    ws_bytes = oal_prefill_workspace_bytes(B, Hq, Hkv, N, chunk, in_dt, y is not None)
    if workspace is None:
        workspace = alloc_workspace(ws_bytes, k.device)
    _expect_workspace(workspace, ws_bytes, k.device)
    _check(fn(B, Hq, Hkv, N, dh, dv, in_dt, _ptr(q), _ptr(k), _ptr(v), _ptr(coeffs),
              chunk, state.handle if state is not None else None, _ptr(y), out_dt,
              _ptr(workspace) if workspace is not None else None,
              workspace.numel() if workspace is not None else 0, _stream(k)))
    return y


def oal_prefill_noalloc_scratch_bytes() -> int:
    return int(_lib.oal_prefill_noalloc_scratch_bytes())


def oal_prefill_noalloc(q: torch.Tensor | None, k: torch.Tensor, v: torch.Tensor,
                        coeffs: torch.Tensor | None, chunk: int = 0, state: OalState | None = None,
                        y: torch.Tensor | None = None, want_output: bool = True) -> torch.Tensor | None:
    """oal_prefill without a workspace argument: the library's static scratch array
    serves instead, and the call allocates nothing.  y must be given when outputs
    are wanted (the caller owns every buffer)."""
    if want_output and y is None:
        raise ValueError("oal_prefill_noalloc allocates nothing: pass y")
    _refuse_dim_record(coeffs)
    B, Hkv, N, Hq, y = _prefill_args(q, k, v, coeffs, state, y, want_output)
    out_dt = _dtype_code(y) if y is not None else OAL_F32
    _check(_lib.oal_prefill_noalloc(B, Hq, Hkv, N, D_H, D_V, _dtype_code(k), _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(coeffs), chunk, state.handle if state is not None else None,
                                    _ptr(y), out_dt, _stream(k)))
    return y


def oal_prefill_dim_workspace_bytes(batch: int, n_q_heads: int, n_kv_heads: int, seq_len: int,
                                    chunk: int = 0, with_output: bool = True) -> int:
    return int(_lib.oal_prefill_dim_workspace_bytes(batch, n_q_heads, n_kv_heads, seq_len, D_H,
                                                    D_V, chunk, 1 if with_output else 0))


def oal_prefill_dim(q: torch.Tensor | None, k: torch.Tensor, v: torch.Tensor,
                    coeffs: torch.Tensor | None, chunk: int = 0, state: OalState | None = None,
                    y: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                    want_output: bool = True) -> torch.Tensor | None:
    """Prefill for any coefficient record (dimension-specific ones included); same
    shapes and semantics as oal_prefill."""
    B, Hkv, N, Hq, y = _prefill_args(q, k, v, coeffs, state, y, want_output)
    dh, dv = D_H, D_V
    out_dt = _dtype_code(y) if y is not None else OAL_F32
    ws_bytes = oal_prefill_dim_workspace_bytes(B, Hq, Hkv, N, chunk, y is not None)
    if workspace is None:
        workspace = alloc_workspace(ws_bytes, k.device)
    _expect_workspace(workspace, ws_bytes, k.device)
    _check(_lib.oal_prefill_dim(B, Hq, Hkv, N, dh, dv, _dtype_code(k), _ptr(q), _ptr(k), _ptr(v),
                                _ptr(coeffs), chunk, state.handle if state is not None else None,
                                _ptr(y), out_dt, _ptr(workspace) if workspace is not None else None,
                                workspace.numel() if workspace is not None else 0, _stream(k)))
    return y


def oal_prefill_backward_workspace_bytes(batch: int, n_q_heads: int, n_kv_heads: int,
                                         seq_len: int, chunk: int = 0) -> int:
    return int(_lib.oal_prefill_backward_workspace_bytes(batch, n_q_heads, n_kv_heads, seq_len,
                                                         D_H, D_V, chunk))


def oal_prefill_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, coeffs: torch.Tensor,
                         dy: torch.Tensor, chunk: int = 0, want_coeff_grad: bool = True,
                         out: tuple | None = None, workspace: torch.Tensor | None = None):
    """Gradients of sum(dy * y) for y = the prefill of (q, k, v) from an empty state.
    q [B, Hq, N, 64], k/v [B, Hkv, N, 64] (fp32 or bf16), dy [B, Hq, N, 64] fp32.
    Returns (dq, dk, dv, da, db, dC), all fp32 (the last three None unless
    want_coeff_grad); out may supply the six output tensors."""
    _expect(q, "q", (None, None, None, D_H), _IN_DTYPES)
    B, Hq, N, dh = q.shape
    dev = q.device
    _expect(k, "k", (B, None, N, D_H), (q.dtype,), dev)
    Hkv = k.shape[1]
    dv_ = D_V
    _expect(v, "v", (B, Hkv, N, D_V), (q.dtype,), dev)
    _expect_coeffs(coeffs, Hq, dev)
    _expect(dy, "dy", (B, Hq, N, D_V), _F32, dev)
    if out is None:
        f32 = dict(dtype=torch.float32, device=dev)
        out = (torch.empty((B, Hq, N, dh), **f32), torch.empty((B, Hkv, N, dh), **f32),
               torch.empty((B, Hkv, N, dv_), **f32),
               torch.empty((Hq,), **f32) if want_coeff_grad else None,
               torch.empty((Hq, dh), **f32) if want_coeff_grad else None,
               torch.empty((Hq, dh, dh), **f32) if want_coeff_grad else None)
    dq, dk, dv, da, db, dC = out
    _expect(dq, "dq", (B, Hq, N, D_H), _F32, dev)
    _expect(dk, "dk", (B, Hkv, N, D_H), _F32, dev)
    _expect(dv, "dv", (B, Hkv, N, D_V), _F32, dev)
    _expect(da, "da", (Hq,), _F32, dev, optional=True)
    _expect(db, "db", (Hq, D_H), _F32, dev, optional=True)
    _expect(dC, "dC", (Hq, D_H, D_H), _F32, dev, optional=True)
    if not ((da is None) == (db is None) == (dC is None)):
        raise ValueError("da, db and dC are given together or not at all")
    ws_bytes = oal_prefill_backward_workspace_bytes(B, Hq, Hkv, N, chunk)
    if workspace is None:
        workspace = alloc_workspace(ws_bytes, dev)
    _expect_workspace(workspace, ws_bytes, dev)
    _check(_lib.oal_prefill_backward(B, Hq, Hkv, N, dh, dv_, _dtype_code(q), _ptr(q), _ptr(k),
                                     _ptr(v), _ptr(coeffs), _ptr(dy), chunk, _ptr(dq), _ptr(dk),
                                     _ptr(dv), _ptr(da), _ptr(db), _ptr(dC),
                                     _ptr(workspace) if workspace is not None else None,
                                     workspace.numel() if workspace is not None else 0, _stream(q)))
    return dq, dk, dv, da, db, dC


def oal_coeffs_backward(n_groups: torch.Tensor, group_map: torch.Tensor, L: torch.Tensor,
                        da: torch.Tensor, db: torch.Tensor, dC: torch.Tensor,
                        dL: torch.Tensor | None = None) -> torch.Tensor:
    """dL [Hq, g+1, g+1] from (da, db, dC) through the grouped map (L as for
    oal_expand_coeffs)."""
    _expect(L, "L", (None, None, None), _F32)
    Hq, g_max, dev = L.shape[0], L.shape[-1] - 1, L.device
    _expect(L, "L", (Hq, g_max + 1, g_max + 1))
    _expect(n_groups, "n_groups", (Hq,), _I32, dev)
    _expect(group_map, "group_map", (Hq, D_H), _I32, dev)
    _expect(da, "da", (Hq,), _F32, dev)
    _expect(db, "db", (Hq, D_H), _F32, dev)
    _expect(dC, "dC", (Hq, D_H, D_H), _F32, dev)
    if dL is None:
        dL = torch.empty_like(L)
    _expect(dL, "dL", tuple(L.shape), _F32, dev)
    _check(_lib.oal_coeffs_backward(Hq, D_H, g_max, _ptr(n_groups), _ptr(group_map), _ptr(L),
                                    _ptr(da), _ptr(db), _ptr(dC), _ptr(dL), _stream(L)))
    return dL


def oal_contribution_scores(q: torch.Tensor, k: torch.Tensor, offsets: torch.Tensor,
                            want_mean: bool = True):
    """q [Hq, T, 64], k [Hkv, T, 64] (prompts concatenated along T), offsets int32
    [P+1].  Returns (chi_prompt [P, Hq, 64], chi [Hq, 64] or None)."""
    _expect(q, "q", (None, None, D_H), _IN_DTYPES)
    Hq, T, dh = q.shape
    _expect(k, "k", (None, T, D_H), (q.dtype,), q.device)
    _expect(offsets, "offsets", (None,), _I32, q.device)
    P = offsets.numel() - 1
    chi_p = torch.empty((P, Hq, dh), dtype=torch.float32, device=q.device)
    chi = torch.empty((Hq, dh), dtype=torch.float32, device=q.device) if want_mean else None
    _check(_lib.oal_contribution_scores(Hq, k.shape[0], P, T, dh, _dtype_code(q), _ptr(q), _ptr(k),
                                        _ptr(offsets), _ptr(chi_p), _ptr(chi), _stream(q)))
    return chi_p, chi


def oal_bootstrap_grouping(chi_prompt: torch.Tensor, boot_idx: torch.Tensor, alpha: float = 0.25,
                           tau: float = 1.5, gamma: float = 0.9, g_min: int = 2,
                           eps: float = 1e-12, want_stats: bool = True):
    """chi_prompt [P, Hq, 64], boot_idx int32 [B, P].  Returns (group_map int32
    [Hq, 64], n_groups int32 [Hq], support [Hq, 64], gap [Hq, 64])."""
    _expect(chi_prompt, "chi_prompt", (None, None, D_H), _F32)
    P, Hq, dh = chi_prompt.shape
    dev = chi_prompt.device
    _expect(boot_idx, "boot_idx", (None, P), _I32, dev)
    gm = torch.empty((Hq, dh), dtype=torch.int32, device=dev)
    ng = torch.empty((Hq,), dtype=torch.int32, device=dev)
    sup = torch.empty((Hq, dh), dtype=torch.float32, device=dev) if want_stats else None
    gap = torch.empty((Hq, dh), dtype=torch.float32, device=dev) if want_stats else None
    _check(_lib.oal_bootstrap_grouping(Hq, P, dh, _ptr(chi_prompt), boot_idx.shape[0], _ptr(boot_idx),
                                       float(alpha), float(tau), float(gamma), int(g_min), float(eps),
                                       _ptr(gm), _ptr(ng), _ptr(sup), _ptr(gap), _stream(chi_prompt)))
    return gm, ng, sup, gap


def oal_calib_workspace_bytes(n_q_heads: int, n_pos: int) -> int:
    return int(_lib.oal_calib_workspace_bytes(n_q_heads, n_pos))


def oal_calib_grad(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, y_ref: torch.Tensor,
                   positions: torch.Tensor, n_groups: torch.Tensor, group_map: torch.Tensor,
                   L: torch.Tensor, eps: float, dL: torch.Tensor | None = None,
                   loss: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """One sequence: q [Hq, N, 64], k/v [Hkv, N, 64] (or with a leading batch of 1),
    y_ref [Hq, N, 64] fp32, positions int32 [n_pos].  Returns (dL, loss)."""
    if q.dim() == 4:
        q, k, v = q[0], k[0], v[0]
    if y_ref.dim() == 4:
        y_ref = y_ref[0]
    _expect(q, "q", (None, None, D_H), _IN_DTYPES)
    Hq, N, dh = q.shape
    dev = q.device
    _expect(k, "k", (None, N, D_H), (q.dtype,), dev)
    Hkv = k.shape[0]
    _expect(v, "v", (Hkv, N, D_V), (q.dtype,), dev)
    _expect(y_ref, "y_ref", (Hq, N, D_V), _F32, dev)
    _expect(positions, "positions", (None,), _I32, dev)
    n_pos = positions.numel()
    _expect(L, "L", (Hq, None, None), _F32, dev)
    g_max = L.shape[-1] - 1
    _expect(L, "L", (Hq, g_max + 1, g_max + 1))
    _expect(n_groups, "n_groups", (Hq,), _I32, dev)
    _expect(group_map, "group_map", (Hq, D_H), _I32, dev)
    if dL is None:
        dL = torch.empty_like(L)
    _expect(dL, "dL", tuple(L.shape), _F32, dev)
    if loss is None:
        loss = torch.empty((Hq,), dtype=torch.float32, device=L.device)
    _expect(loss, "loss", (Hq,), _F32, dev)
    ws_bytes = oal_calib_workspace_bytes(Hq, n_pos)
    if workspace is None:
        workspace = alloc_workspace(ws_bytes, L.device)
    _expect_workspace(workspace, ws_bytes, dev)
    _check(_lib.oal_calib_grad(Hq, Hkv, N, dh, v.shape[-1], _dtype_code(q), _ptr(q), _ptr(k), _ptr(v),
                               _ptr(y_ref), _ptr(positions), n_pos, g_max, _ptr(n_groups),
                               _ptr(group_map), _ptr(L), float(eps), _ptr(dL), _ptr(loss),
                               _ptr(workspace), workspace.numel(), _stream(L)))
    return dL, loss


def oal_adam_step(n_groups: torch.Tensor, L: torch.Tensor, dL: torch.Tensor, m: torch.Tensor,
                  v: torch.Tensor, step: int, lr: float = 0.02, beta1: float = 0.9,
                  beta2: float = 0.999, eps: float = 1e-8, clip_norm: float = 10.0) -> None:
    """In place on L, m, v (all [Hq, g+1, g+1] fp32)."""
    _expect(L, "L", (None, None, None), _F32)
    dev = L.device
    _expect(n_groups, "n_groups", (L.shape[0],), _I32, dev)
    for t, nm in ((dL, "dL"), (m, "m"), (v, "v")):
        _expect(t, nm, tuple(L.shape), _F32, dev)
    _check(_lib.oal_adam_step(n_groups.shape[0], L.shape[-1] - 1, _ptr(n_groups), _ptr(L), _ptr(dL),
                              _ptr(m), _ptr(v), int(step), float(lr), float(beta1), float(beta2),
                              float(eps), float(clip_norm), _stream(L)))


def oal_embed_global(n_groups: torch.Tensor, L_global: torch.Tensor, g_max: int = 6,
                     L: torch.Tensor | None = None) -> torch.Tensor:
    """L_global [Hq, g+1, g+1] (a G = 1 calibration's L); returns the grouped start
    L [Hq, g_max+1, g_max+1]."""
    _expect(n_groups, "n_groups", (None,), _I32)
    Hq = n_groups.shape[0]
    _expect(L_global, "L_global", (Hq, None, None), _F32, n_groups.device)
    if L is None:
        L = torch.empty((Hq, g_max + 1, g_max + 1), dtype=torch.float32, device=L_global.device)
    _expect(L, "L", (Hq, g_max + 1, g_max + 1), _F32, n_groups.device)
    _check(_lib.oal_embed_global(Hq, g_max, _ptr(n_groups), L_global.shape[-1], _ptr(L_global), _ptr(L),
                                 _stream(L)))
    return L


def oal_output_mse(y: torch.Tensor, y_ref: torch.Tensor, mse: torch.Tensor | None = None) -> torch.Tensor:
    """y, y_ref [B, Hq, N, d_v] fp32; returns the per-head MSE [Hq]."""
    _expect(y, "y", (None, None, None, D_V), _F32)
    B, Hq, N, dv = y.shape
    _expect(y_ref, "y_ref", tuple(y.shape), _F32, y.device)
    if mse is None:
        mse = torch.empty((Hq,), dtype=torch.float32, device=y.device)
    _expect(mse, "mse", (Hq,), _F32, y.device)
    _check(_lib.oal_output_mse(B, Hq, N, dv, _ptr(y), _ptr(y_ref), _ptr(mse), _stream(y)))
    return mse


def oal_decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, coeffs: torch.Tensor,
                    state: OalState, y: torch.Tensor | None = None) -> torch.Tensor:
    """q [B, Hq, 64], k/v [B, Hkv, 64]; returns y [B, Hq, 64]."""
    _expect(q, "q", (None, None, D_H), _IN_DTYPES)
    B, Hq, dh = q.shape
    dev = q.device
    _expect(k, "k", (B, None, D_H), (q.dtype,), dev)
    Hkv = k.shape[1]
    dv = D_V
    _expect(v, "v", (B, Hkv, D_V), (q.dtype,), dev)
    _expect_coeffs(coeffs, Hq, dev)
    if state is None:
        raise ValueError("state is required")
    _expect_state(state, B, Hkv)
    if y is None:
        y = torch.empty((B, Hq, dv), dtype=q.dtype, device=q.device)
    _expect(y, "y", (B, Hq, D_V), _IN_DTYPES, dev)
    _check(_lib.oal_decode_step(B, Hq, Hkv, dh, dv, _dtype_code(q), _ptr(q), _ptr(k), _ptr(v),
                                _ptr(coeffs), state.handle, _ptr(y), _dtype_code(y), _stream(q)))
    return y


def oal_softmax_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                          y: torch.Tensor | None = None) -> torch.Tensor:
    """Exact causal softmax attention (the reference OAL approximates): q [B, Hq, N, 64],
    k/v [B, Hkv, N, 64] in bf16; returns y [B, Hq, N, 64] in q's dtype unless y is given."""
    _expect(q, "q", (None, None, None, D_H), _IN_DTYPES)
    B, Hq, N, dh = q.shape
    dev = q.device
    _expect(k, "k", (B, None, N, D_H), (q.dtype,), dev)
    Hkv = k.shape[1]
    dv = D_V
    _expect(v, "v", (B, Hkv, N, D_V), (q.dtype,), dev)
    if y is None:
        y = torch.empty((B, Hq, N, dv), dtype=q.dtype, device=q.device)
    _expect(y, "y", (B, Hq, N, D_V), _IN_DTYPES, dev)
    _check(_lib.oal_softmax_attention(B, Hq, Hkv, N, dh, dv, _dtype_code(q), _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(y), _dtype_code(y), _stream(q)))
    return y


def oal_status_string(status: int) -> str:
    return _status_name(status)


def oal_last_error() -> str:
    return _lib.oal_last_error().decode()


def oal_state_bytes(state: OalState) -> int:
    return state.nbytes


def oal_state_tokens(state: OalState) -> int:
    return state.tokens


def oal_profile_enable(enable: bool = True) -> None:
    _check(_lib.oal_profile_enable(1 if enable else 0))


def oal_profile_filter(kernel: str | None = None) -> None:
    """Record profiling events around the named kernel only (None: every kernel)."""
    _check(_lib.oal_profile_filter(kernel.encode() if kernel else None))


def oal_profile_reset() -> None:
    _check(_lib.oal_profile_reset())


def oal_profile_query(kernel: str | None = None) -> tuple[float, int]:
    """(total milliseconds, launches) of the named kernel since the last reset."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(_lib.oal_profile_query(kernel.encode() if kernel else None, ctypes.byref(ms),
                                  ctypes.byref(n)))
    return ms.value, n.value
