"""Taylor-state attention on MI355X (gfx950): thin Python binding of libtaylor_attn.so.

The method is "A Taylor-Series Route to Linear-Time Transformers with a Fixed
Number of Recurrent States" (arXiv 2610.20637): causal attention whose
exponential kernel is replaced by its n-term Taylor polynomial, evaluated
through n symmetric tensor-power states (sections 3.1-3.5).

Every step of the computation runs in the library's HIP kernels; this module
only checks tensor arguments, passes raw device pointers and the current HIP
stream through the C ABI declared in ``include/taylor_attn.h``, and turns error
codes into exceptions.  PyTorch provides device memory and streams.  There is
no fallback: if the library is missing, importing this package fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "LIB_PATH", "TaylorError", "state_width", "state_numel", "new_state", "state_init",
    "state_views", "prefill_workspace_bytes", "prefill", "decode", "set_phase_events",
    "prefill_check", "set_wait_limit", "debug_fill_lds", "softmax_prefill", "softmax_decode",
    "softmax_decode_workspace_bytes",
    "prefill_noalloc", "state_bf16_bytes", "new_state_bf16", "state_to_bf16", "state_bf16_views",
    "decode_bf16state", "hybrid_fill_window", "hybrid_decode", "EXPORTED_SYMBOLS",
]

# TAYLOR_ATTN_LIB names another build of the same library to load instead (the
# CPU test that runs the ABI tests against an AddressSanitizer build of the
# host code uses it)
LIB_PATH = os.environ.get("TAYLOR_ATTN_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                              "libtaylor_attn.so")

TAYLOR_F32, TAYLOR_BF16 = 0, 1
_CODES = {0: "TAYLOR_OK", -1: "TAYLOR_EINVAL", -2: "TAYLOR_EUNSUPPORTED", -3: "TAYLOR_EHIP", -4: "TAYLOR_ETIMEOUT"}

EXPORTED_SYMBOLS = (
    "taylor_state_width", "taylor_state_numel", "taylor_state_init", "taylor_prefill_workspace_bytes",
    "taylor_attn_prefill", "taylor_attn_decode", "taylor_last_error", "taylor_set_phase_events",
    "taylor_prefill_check", "taylor_set_wait_limit", "taylor_softmax_prefill",
    "taylor_softmax_decode_workspace_bytes", "taylor_softmax_decode", "taylor_attn_prefill_noalloc",
    "taylor_state_bf16_bytes", "taylor_state_to_bf16", "taylor_attn_decode_bf16state",
    "taylor_hybrid_fill_window", "taylor_hybrid_decode", "taylor_debug_fill_lds",
)


class TaylorError(RuntimeError):
    """A call into libtaylor_attn.so returned an error code."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"{_CODES.get(code, code)}: {msg}")
        self.code = code


if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
        "(or python recurrent_state_phi_amd/build.py) first")

_lib = ctypes.CDLL(LIB_PATH)
_vp, _i, _f, _sz, _i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_int64
_lib.taylor_state_width.argtypes = [_i, _i]
_lib.taylor_state_width.restype = _i64
_lib.taylor_state_numel.argtypes = [_i, _i, _i]
_lib.taylor_state_numel.restype = _i64
_lib.taylor_state_init.argtypes = [_vp, _i, _i, _i, _i, _i, _vp]
_lib.taylor_state_init.restype = _i
_lib.taylor_prefill_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i, _i]
_lib.taylor_prefill_workspace_bytes.restype = _sz
_lib.taylor_attn_prefill.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _i, _i, _vp, _sz, _vp]
_lib.taylor_attn_prefill.restype = _i
_lib.taylor_attn_prefill_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _i, _i, _vp]
_lib.taylor_attn_prefill_noalloc.restype = _i
_lib.taylor_state_bf16_bytes.argtypes = [_i, _i, _i]
_lib.taylor_state_bf16_bytes.restype = _i64
_lib.taylor_state_to_bf16.argtypes = [_vp, _vp, _i, _i, _i, _i, _i, _vp]
_lib.taylor_state_to_bf16.restype = _i
_lib.taylor_attn_decode_bf16state.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i,
                                              _i, _vp]
_lib.taylor_attn_decode_bf16state.restype = _i
_lib.taylor_hybrid_fill_window.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp]
_lib.taylor_hybrid_fill_window.restype = _i
_lib.taylor_hybrid_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _i, _vp]
_lib.taylor_hybrid_decode.restype = _i
_lib.taylor_attn_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _vp]
_lib.taylor_attn_decode.restype = _i
_lib.taylor_last_error.argtypes = []
_lib.taylor_last_error.restype = ctypes.c_char_p
_lib.taylor_set_phase_events.argtypes = [_vp, _i]
_lib.taylor_set_phase_events.restype = _i
_lib.taylor_prefill_check.argtypes = [_vp, _sz, _vp]
_lib.taylor_prefill_check.restype = _i
_lib.taylor_set_wait_limit.argtypes = [_i]
_lib.taylor_set_wait_limit.restype = _i
_lib.taylor_debug_fill_lds.argtypes = [ctypes.c_uint, _vp]
_lib.taylor_debug_fill_lds.restype = _i
_lib.taylor_softmax_prefill.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _vp]
_lib.taylor_softmax_prefill.restype = _i
_lib.taylor_softmax_decode_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]
_lib.taylor_softmax_decode_workspace_bytes.restype = _sz
_lib.taylor_softmax_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _i, _vp, _sz,
                                       _vp]
_lib.taylor_softmax_decode.restype = _i


def raw_library() -> ctypes.CDLL:
    """The loaded ctypes handle (for tests that call the C ABI directly)."""
    return _lib


def _check(code: int):
    if code != 0:
        raise TaylorError(code, _lib.taylor_last_error().decode())


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return TAYLOR_F32
    if t == torch.bfloat16:
        return TAYLOR_BF16
    raise TypeError(f"unsupported dtype {t}; use torch.float32 or torch.bfloat16")


def _stream_ptr(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: torch.Tensor) -> int:
    return t.data_ptr()


def state_width(d: int, n: int) -> int:
    """D = sum_{m<n} C(d+m-1, m), rows of the stacked state."""
    return int(_lib.taylor_state_width(d, n))


def state_numel(d: int, d_v: int, n: int) -> int:
    """Floats per head: D * (d_v + 1)."""
    return int(_lib.taylor_state_numel(d, d_v, n))


def state_init(state: torch.Tensor, B: int, H: int, n: int, d: int = 16, d_v: int = 64):
    """Zero the state through the library (enqueued on the current stream)."""
    _check(_lib.taylor_state_init(_ptr(state), B, H, d, d_v, n, _stream_ptr(state.device)))


def new_state(B: int, H: int, n: int, d: int = 16, d_v: int = 64, device="cuda") -> torch.Tensor:
    """A zeroed float32 state buffer for B*H heads (flat; see :func:`state_views`)."""
    st = torch.empty(B * H * state_numel(d, d_v, n), dtype=torch.float32, device=device)
    state_init(st, B, H, n, d, d_v)
    return st


def state_views(state: torch.Tensor, B: int, H: int, n: int, d: int = 16, d_v: int = 64):
    """(S [B,H,D,d_v], T [B,H,D]) views of a flat state buffer."""
    D = state_width(d, n)
    S = state[: B * H * D * d_v].view(B, H, D, d_v)
    T = state[B * H * D * d_v: B * H * D * (d_v + 1)].view(B, H, D)
    return S, T


def prefill_workspace_bytes(B: int, H: int, N: int, n: int, chunk: int, d: int = 16, d_v: int = 64) -> int:
    r = int(_lib.taylor_prefill_workspace_bytes(B, H, N, d, d_v, n, chunk))
    if r == ctypes.c_size_t(-1).value:
        raise TaylorError(-1, "invalid arguments to taylor_prefill_workspace_bytes")
    return r


def _check_tensor(name, t, shape, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA/HIP tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, state: torch.Tensor, n: int, a: float,
            chunk: int = 64, out_dtype: torch.dtype | None = None, out: torch.Tensor | None = None,
            workspace: torch.Tensor | None = None, check: bool = False) -> torch.Tensor:
    """Chunked prefill; adds the tokens to ``state`` in place and returns o [B,H,N,d_v].

    Without ``workspace`` one is allocated for the call when the plan needs
    it.  ``check=True`` waits for the call and raises TaylorError
    (TAYLOR_ETIMEOUT) if a bounded wait between workgroups ran out, whichever
    workspace was used; otherwise a caller who wants that report passes its
    own workspace and calls :func:`prefill_check` on it later.
    """
    B, H, N, d = q.shape
    d_v = v.shape[-1]
    _check_tensor("q", q, (B, H, N, d))
    _check_tensor("k", k, (B, H, N, d), q.dtype)
    _check_tensor("v", v, (B, H, N, d_v), q.dtype)
    _check_tensor("state", state, (B * H * state_numel(d, d_v, n),), torch.float32)
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((B, H, N, d_v), dtype=out_dtype, device=q.device)
    _check_tensor("out", out, (B, H, N, d_v), out_dtype)
    need = prefill_workspace_bytes(B, H, N, n, chunk, d, d_v)
    if need and workspace is None:
        workspace = torch.empty(need // 4 + 4, dtype=torch.float32, device=q.device)
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.taylor_attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(state), B, H, N, d, d_v, n,
                                    float(a), chunk, _dtype_code(q.dtype), _dtype_code(out_dtype), ws_ptr,
                                    ws_bytes, _stream_ptr(q.device)))
    if check:
        prefill_check(workspace)
    return out


def prefill_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, state: torch.Tensor, n: int, a: float,
                    chunk: int = 64, out_dtype: torch.dtype | None = None,
                    out: torch.Tensor | None = None) -> torch.Tensor:
    """prefill() through taylor_attn_prefill_noalloc: the library's fixed per-device
    scratch instead of a workspace (pass ``out`` to allocate nothing here either)."""
    B, H, N, d = q.shape
    d_v = v.shape[-1]
    _check_tensor("q", q, (B, H, N, d))
    _check_tensor("k", k, (B, H, N, d), q.dtype)
    _check_tensor("v", v, (B, H, N, d_v), q.dtype)
    _check_tensor("state", state, (B * H * state_numel(d, d_v, n),), torch.float32)
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((B, H, N, d_v), dtype=out_dtype, device=q.device)
    _check_tensor("out", out, (B, H, N, d_v), out_dtype)
    _check(_lib.taylor_attn_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(state), B, H, N, d, d_v, n,
                                            float(a), chunk, _dtype_code(q.dtype), _dtype_code(out_dtype),
                                            _stream_ptr(q.device)))
    return out


def decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, state: torch.Tensor, n: int, a: float,
           out_dtype: torch.dtype | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """One decode step per head: q, k [B,H,d], v [B,H,d_v]; returns o [B,H,d_v]."""
    B, H, d = q.shape
    d_v = v.shape[-1]
    _check_tensor("q", q, (B, H, d))
    _check_tensor("k", k, (B, H, d), q.dtype)
    _check_tensor("v", v, (B, H, d_v), q.dtype)
    _check_tensor("state", state, (B * H * state_numel(d, d_v, n),), torch.float32)
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((B, H, d_v), dtype=out_dtype, device=q.device)
    _check_tensor("out", out, (B, H, d_v), out_dtype)
    _check(_lib.taylor_attn_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(state), B, H, d, d_v, n, float(a),
                                   _dtype_code(q.dtype), _dtype_code(out_dtype), _stream_ptr(q.device)))
    return out


def set_phase_events(events) -> None:
    """Record 4 HIP events around the prefill phases (see taylor_set_phase_events); None turns it off."""
    if events is None:
        _check(_lib.taylor_set_phase_events(None, 0))
        return
    arr = (ctypes.c_void_p * 4)(*[e.cuda_event for e in events])
    _check(_lib.taylor_set_phase_events(ctypes.cast(arr, ctypes.c_void_p), 4))


def prefill_check(workspace: torch.Tensor | None) -> None:
    """Wait for the current stream and raise TaylorError (TAYLOR_ETIMEOUT) if a wait
    between workgroups ran out in the last prefill that used ``workspace``."""
    if workspace is None:
        return
    _check(_lib.taylor_prefill_check(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream_ptr(workspace.device)))


def set_wait_limit(polls: int) -> int:
    """Test hook: polls before a wait between workgroups gives up; returns the previous value."""
    prev = _lib.taylor_set_wait_limit(int(polls))
    if prev < 0:
        raise TaylorError(-1, _lib.taylor_last_error().decode())
    return prev


def debug_fill_lds(pattern: int, device="cuda") -> None:
    """Test hook: fill every CU's LDS with a 32-bit pattern on the device's current
    stream, so that the next kernel there starts from it (see taylor_debug_fill_lds)."""
    _check(_lib.taylor_debug_fill_lds(int(pattern) & 0xFFFFFFFF, _stream_ptr(torch.device(device))))


# ---- exact causal softmax attention (the comparison method, Eq. (1)) ----------
def softmax_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, a: float,
                    out_dtype: torch.dtype | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """Causal softmax attention over q, k [B,H,N,d], v [B,H,N,d_v]; returns o [B,H,N,d_v]."""
    B, H, N, d = q.shape
    d_v = v.shape[-1]
    _check_tensor("q", q, (B, H, N, d))
    _check_tensor("k", k, (B, H, N, d), q.dtype)
    _check_tensor("v", v, (B, H, N, d_v), q.dtype)
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((B, H, N, d_v), dtype=out_dtype, device=q.device)
    _check_tensor("out", out, (B, H, N, d_v), out_dtype)
    _check(_lib.taylor_softmax_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, N, d, d_v, float(a),
                                       _dtype_code(q.dtype), _dtype_code(out_dtype), _stream_ptr(q.device)))
    return out


def softmax_decode_workspace_bytes(B: int, H: int, cap: int, d: int = 16, d_v: int = 64) -> int:
    r = int(_lib.taylor_softmax_decode_workspace_bytes(B, H, cap, d, d_v))
    if r == ctypes.c_size_t(-1).value:
        raise TaylorError(-1, "invalid arguments to taylor_softmax_decode_workspace_bytes")
    return r


def softmax_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   pos: int, a: float, workspace: torch.Tensor, out_dtype: torch.dtype | None = None,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    """One decode step against the cache: writes k, v [B,H,d / d_v] at ``pos`` of
    k_cache [B,H,cap,d] / v_cache [B,H,cap,d_v] and attends over 0..pos."""
    B, H, d = q.shape
    d_v = v.shape[-1]
    cap = k_cache.shape[2]
    _check_tensor("q", q, (B, H, d))
    _check_tensor("k", k, (B, H, d), q.dtype)
    _check_tensor("v", v, (B, H, d_v), q.dtype)
    _check_tensor("k_cache", k_cache, (B, H, cap, d), q.dtype)
    _check_tensor("v_cache", v_cache, (B, H, cap, d_v), q.dtype)
    _check_tensor("workspace", workspace, (workspace.numel(),), torch.float32)
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((B, H, d_v), dtype=out_dtype, device=q.device)
    _check_tensor("out", out, (B, H, d_v), out_dtype)
    _check(_lib.taylor_softmax_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(k_cache), _ptr(v_cache), B, H,
                                      int(pos), cap, d, d_v, float(a), _dtype_code(q.dtype), _dtype_code(out_dtype),
                                      _ptr(workspace), workspace.numel() * 4, _stream_ptr(q.device)))
    return out


# ---- bfloat16 state storage with an exact window of recent tokens ------------
def state_bf16_bytes(d: int, d_v: int, n: int) -> int:
    """Bytes per head of a bfloat16 state (bfloat16 S, float32 T)."""
    return int(_lib.taylor_state_bf16_bytes(d, d_v, n))


def new_state_bf16(B: int, H: int, n: int, d: int = 16, d_v: int = 64, device="cuda") -> torch.Tensor:
    """An uninitialised bfloat16-state buffer (uint8, see :func:`state_bf16_views`)."""
    return torch.empty(B * H * state_bf16_bytes(d, d_v, n), dtype=torch.uint8, device=device)


def state_to_bf16(state: torch.Tensor, state_bf16: torch.Tensor, B: int, H: int, n: int, d: int = 16,
                  d_v: int = 64) -> torch.Tensor:
    """Round a float32 state into a bfloat16-state buffer (enqueued on the current stream)."""
    _check_tensor("state", state, (B * H * state_numel(d, d_v, n),), torch.float32)
    _check_tensor("state_bf16", state_bf16, (B * H * state_bf16_bytes(d, d_v, n),), torch.uint8)
    _check(_lib.taylor_state_to_bf16(_ptr(state), _ptr(state_bf16), B, H, d, d_v, n, _stream_ptr(state.device)))
    return state_bf16


def state_bf16_views(state_bf16: torch.Tensor, B: int, H: int, n: int, d: int = 16, d_v: int = 64):
    """(S [B,H,D,d_v] bfloat16, T [B,H,D] float32) views of a bfloat16-state buffer."""
    D = state_width(d, n)
    ns = B * H * D * d_v * 2
    S = state_bf16[:ns].view(torch.bfloat16).view(B, H, D, d_v)
    T = state_bf16[ns: ns + B * H * D * 4].view(torch.float32).view(B, H, D)
    return S, T


def decode_bf16state(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, state_bf16: torch.Tensor,
                     win_k: torch.Tensor, win_v: torch.Tensor, step: int, n: int, a: float,
                     out_dtype: torch.dtype | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """One decode step against a bfloat16 state with a window of win_k.shape[2] tokens;
    ``step`` = tokens in the window since the last fold (folds when it reaches K - 1)."""
    B, H, d = q.shape
    d_v = v.shape[-1]
    K = win_k.shape[2]
    _check_tensor("q", q, (B, H, d))
    _check_tensor("k", k, (B, H, d), q.dtype)
    _check_tensor("v", v, (B, H, d_v), q.dtype)
    _check_tensor("state_bf16", state_bf16, (B * H * state_bf16_bytes(d, d_v, n),), torch.uint8)
    _check_tensor("win_k", win_k, (B, H, K, d), q.dtype)
    _check_tensor("win_v", win_v, (B, H, K, d_v), q.dtype)
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((B, H, d_v), dtype=out_dtype, device=q.device)
    _check_tensor("out", out, (B, H, d_v), out_dtype)
    _check(_lib.taylor_attn_decode_bf16state(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(state_bf16), _ptr(win_k),
                                             _ptr(win_v), int(step), K, B, H, d, d_v, n, float(a),
                                             _dtype_code(q.dtype), _dtype_code(out_dtype), _stream_ptr(q.device)))
    return out


# ---- eviction-fed hybrid: softmax window + Taylor state for the evicted tokens --
def hybrid_fill_window(k: torch.Tensor, v: torch.Tensor, win_k: torch.Tensor, win_v: torch.Tensor) -> None:
    """Put the last min(N, W) tokens of a context k [B,H,N,d], v [B,H,N,d_v] into
    their ring slots (position i in slot i % W)."""
    B, H, N, d = k.shape
    d_v = v.shape[-1]
    W = win_k.shape[2]
    _check_tensor("k", k, (B, H, N, d))
    _check_tensor("v", v, (B, H, N, d_v), k.dtype)
    _check_tensor("win_k", win_k, (B, H, W, d), k.dtype)
    _check_tensor("win_v", win_v, (B, H, W, d_v), k.dtype)
    _check(_lib.taylor_hybrid_fill_window(_ptr(k), _ptr(v), _ptr(win_k), _ptr(win_v), B, H, N, W, d, d_v,
                                          _dtype_code(k.dtype), _stream_ptr(k.device)))


def hybrid_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, state: torch.Tensor, win_k: torch.Tensor,
                  win_v: torch.Tensor, pos: int, n: int, a: float, out_dtype: torch.dtype | None = None,
                  out: torch.Tensor | None = None) -> torch.Tensor:
    """One hybrid decode step at position ``pos`` (window W = win_k.shape[2])."""
    B, H, d = q.shape
    d_v = v.shape[-1]
    W = win_k.shape[2]
    _check_tensor("q", q, (B, H, d))
    _check_tensor("k", k, (B, H, d), q.dtype)
    _check_tensor("v", v, (B, H, d_v), q.dtype)
    _check_tensor("state", state, (B * H * state_numel(d, d_v, n),), torch.float32)
    _check_tensor("win_k", win_k, (B, H, W, d), q.dtype)
    _check_tensor("win_v", win_v, (B, H, W, d_v), q.dtype)
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((B, H, d_v), dtype=out_dtype, device=q.device)
    _check_tensor("out", out, (B, H, d_v), out_dtype)
    _check(_lib.taylor_hybrid_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(state), _ptr(win_k), _ptr(win_v),
                                     int(pos), W, B, H, d, d_v, n, float(a), _dtype_code(q.dtype),
                                     _dtype_code(out_dtype), _stream_ptr(q.device)))
    return out
