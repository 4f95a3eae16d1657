"""ctypes binding of libgdn.so (argument marshalling only).

Every step of the recurrence runs in the library's HIP kernels; this module
only checks tensor metadata, allocates outputs with PyTorch (device memory and
streams are PyTorch's), and passes raw device pointers plus the current
stream to the C ABI declared in include/gdn.h.  If the library is not built,
importing this module raises ImportError: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch  # loaded first so libgdn binds to the HIP runtime torch uses

_HERE = os.path.dirname(os.path.abspath(__file__))
# GDN_LIB_PATH overrides the library (the host-sanitized build of the tests)
LIB_PATH = os.environ.get("GDN_LIB_PATH") or os.path.join(_HERE, "libgdn.so")

GDN_OK, GDN_EINVAL, GDN_ESHAPE, GDN_EWORKSPACE, GDN_EHIP = range(5)
GDN_F32, GDN_BF16 = 0, 1
_DTYPE_CODE = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16}

_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t

# name -> (restype, argtypes); the single source of the ABI on this side
SIGNATURES = {
    "gdn_status_str": (ctypes.c_char_p, [_i]),
    "gdn_version": (ctypes.c_char_p, []),
    "gdn_prefill_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "gdn_prefill_segments": (_i, [_i, _i, _i, _i, _i, _i, _i, _vp]),
    "gdn_prefill": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                         _i, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "gdn_prefill_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _i, _i, _i, _i, _i, _i, _i, _vp]),
    "gdn_prefill_prepare": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i,
                                 _vp, _sz, _vp]),
    "gdn_prefill_scan": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i,
                              _i, _i, _i, _vp, _sz, _vp]),
    "gdn_decode_step": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                             _i, _i, _i, _i, _i, _i, _vp]),
    "gdn_prefill_qk_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "gdn_prefill_qk": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                            _i, _i, _i, _i, _i, _i, _vp, _i, ctypes.c_float,
                            _i, _i, _vp, _sz, _vp]),
    "gdn_decode_step_qk": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                _i, _i, _i, _i, _i, _vp, _i, ctypes.c_float,
                                _i, _i, _vp]),
    "gdn_gated_recurrent": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _i, _i, _i, _i, _i, _i, _i, _vp]),
    "gdn_gated_prefill_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "gdn_gated_prefill": (_i, [_vp] * 9 + [_i] * 7 + [_vp, _sz, _vp]),
    "gdn_drrqr_select": (_i, [_vp, _i, _i, _i, ctypes.c_double, _i, _vp, _vp, _vp]),
    "gdn_backward_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "gdn_backward": (_i, [_vp] * 14 + [_i] * 6 + [_vp, _sz, _vp]),
    "gdn_truncate_workspace_bytes": (_sz, [_i, _i, _i]),
    "gdn_truncate_rank": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, _sz, _vp]),
}


class GdnError(RuntimeError):
    """A non-zero status returned by libgdn."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)}")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run "
            "`python -m gated_deltanet_recurrent_delta_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def status_str(status: int) -> str:
    return lib.gdn_status_str(status).decode()


def version() -> str:
    return lib.gdn_version().decode()


def _check(status: int, where: str) -> None:
    if status != GDN_OK:
        raise GdnError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(t: torch.Tensor, stream=None):
    s = torch.cuda.current_stream(t.device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev_tensor(t: torch.Tensor, name: str, dtypes, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    return t


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------

def prefill_workspace_bytes(B: int, T: int, H: int, dk: int, dv: int) -> int:
    return int(lib.gdn_prefill_workspace_bytes(B, T, H, dk, dv))


def prefill_segments(B: int, T: int, H: int, dk: int, dv: int,
                     in_dtype=torch.bfloat16, out_dtype=torch.bfloat16):
    """(segments per head, chunks per segment) gdn_prefill will use."""
    sc = ctypes.c_int(0)
    n = lib.gdn_prefill_segments(B, T, H, dk, dv, _DTYPE_CODE[in_dtype],
                                 _DTYPE_CODE[out_dtype], ctypes.byref(sc))
    if n == 0:
        raise ValueError("invalid prefill sizes or dtypes")
    return n, sc.value


def _prefill_args(q, k, v, alpha, beta, S0):
    _dev_tensor(q, "q", _DTYPE_CODE)
    B, T, H, dk = q.shape
    _dev_tensor(k, "k", (q.dtype,), q.shape)
    _dev_tensor(v, "v", (q.dtype,))
    if tuple(v.shape[:3]) != (B, T, H) or v.dim() != 4:
        raise ValueError(f"v: shape {tuple(v.shape)} incompatible with q")
    dv = v.shape[3]
    _dev_tensor(alpha, "alpha", (torch.float32,), (B, T, H))
    _dev_tensor(beta, "beta", (torch.float32,), (B, T, H))
    if S0 is not None:
        _dev_tensor(S0, "S0", (torch.float32,), (B, H, dv, dk))
    return B, T, H, dk, dv


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
            alpha: torch.Tensor, beta: torch.Tensor,
            S0: Optional[torch.Tensor] = None, *,
            out_dtype: Optional[torch.dtype] = None,
            o: Optional[torch.Tensor] = None,
            ST: Optional[torch.Tensor] = None,
            final_state: bool = True,
            workspace: Optional[torch.Tensor] = None,
            stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Gated delta rule over whole sequences.

    q, k [B, T, H, dk], v [B, T, H, dv] (float32 or bfloat16, same dtype);
    alpha, beta [B, T, H] float32; S0 [B, H, dv, dk] float32 or None.
    Returns (o [B, T, H, dv] in out_dtype (default: q's dtype), S_T or None).
    ST may be S0 (in-place update).  `workspace`: optional uint8 GPU tensor
    of at least prefill_workspace_bytes(...) bytes.
    """
    B, T, H, dk, dv = _prefill_args(q, k, v, alpha, beta, S0)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=out_dtype, device=q.device)
    _dev_tensor(o, "o", (out_dtype,), (B, T, H, dv))
    if ST is None and final_state:
        ST = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    if ST is not None:
        _dev_tensor(ST, "ST", (torch.float32,), (B, H, dv, dk))
    need = prefill_workspace_bytes(B, T, H, dk, dv)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = lib.gdn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                         _ptr(S0), _ptr(o), _ptr(ST), B, T, H, dk, dv,
                         _DTYPE_CODE[q.dtype], _DTYPE_CODE[out_dtype],
                         _ptr(workspace), workspace.numel(),
                         _stream_handle(q, stream))
    _check(st, "gdn_prefill")
    return o, ST


NOALLOC_SCRATCH_BYTES = 256 << 20      # GDN_NOALLOC_SCRATCH_BYTES in include/gdn.h


def prefill_noalloc(q, k, v, alpha, beta, S0, o, ST, stream=None) -> None:
    """gdn_prefill_noalloc: prefill into the caller's o and ST (ST may be S0
    or None), its workspace in the library's static device scratch; the
    binding allocates nothing either.  Calls that overlap on one device
    race on that scratch; see include/gdn.h."""
    B, T, H, dk, dv = _prefill_args(q, k, v, alpha, beta, S0)
    if o.dtype not in _DTYPE_CODE:
        raise ValueError(f"o: dtype {o.dtype} not in {tuple(_DTYPE_CODE)}")
    _dev_tensor(o, "o", (o.dtype,), (B, T, H, dv))
    if ST is not None:
        _dev_tensor(ST, "ST", (torch.float32,), (B, H, dv, dk))
    st = lib.gdn_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                 _ptr(S0), _ptr(o), _ptr(ST), B, T, H, dk, dv,
                                 _DTYPE_CODE[q.dtype], _DTYPE_CODE[o.dtype],
                                 _stream_handle(q, stream))
    _check(st, "gdn_prefill_noalloc")


def prefill_prepare(q, k, alpha, beta, dv: int, workspace: torch.Tensor,
                    out_dtype=None, stream=None) -> None:
    """First phase of prefill (chunk-local, state independent) into
    `workspace`, for a scan whose outputs have `out_dtype` (default: q's
    dtype); see include/gdn.h."""
    _dev_tensor(q, "q", _DTYPE_CODE)
    B, T, H, dk = q.shape
    _dev_tensor(k, "k", (q.dtype,), q.shape)
    _dev_tensor(alpha, "alpha", (torch.float32,), (B, T, H))
    _dev_tensor(beta, "beta", (torch.float32,), (B, T, H))
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out_dtype not in _DTYPE_CODE:
        raise ValueError(f"out_dtype {out_dtype} not in {tuple(_DTYPE_CODE)}")
    st = lib.gdn_prefill_prepare(_ptr(q), _ptr(k), _ptr(alpha), _ptr(beta),
                                 B, T, H, dk, dv, _DTYPE_CODE[q.dtype],
                                 _DTYPE_CODE[out_dtype],
                                 _ptr(workspace), workspace.numel(),
                                 _stream_handle(q, stream))
    _check(st, "gdn_prefill_prepare")


def prefill_scan(q, k, v, S0, o, ST, workspace: torch.Tensor,
                 stream=None) -> None:
    """Second phase of prefill (sequential over chunks) reading the
    workspace written by prefill_prepare; see include/gdn.h."""
    _dev_tensor(q, "q", _DTYPE_CODE)
    B, T, H, dk = q.shape
    dv = v.shape[3]
    _dev_tensor(o, "o", _DTYPE_CODE, (B, T, H, dv))
    st = lib.gdn_prefill_scan(_ptr(q), _ptr(k), _ptr(v), _ptr(S0), _ptr(o),
                              _ptr(ST), B, T, H, dk, dv, _DTYPE_CODE[q.dtype],
                              _DTYPE_CODE[o.dtype], _ptr(workspace),
                              workspace.numel(), _stream_handle(q, stream))
    _check(st, "gdn_prefill_scan")


# ---------------------------------------------------------------------------
# the input path fused into the kernels (channel subset, L2 norm, q scale)
# ---------------------------------------------------------------------------

def _channels_arg(channels, H: int, dk_in: int, dev, validate: bool):
    """(channels tensor or None, kept width)."""
    if channels is None:
        return None, dk_in
    _dev_tensor(channels, "channels", (torch.int32,))
    if channels.dim() != 2 or channels.shape[0] != H:
        raise ValueError(f"channels: shape {tuple(channels.shape)} is not [H={H}, dk]")
    if channels.device != dev:
        raise ValueError("channels must be on the same device as q")
    if validate and channels.numel() and (int(channels.min()) < 0 or
                                          int(channels.max()) >= dk_in):
        raise ValueError(f"channels: indices must lie in [0, {dk_in})")
    return channels, channels.shape[1]


def prefill_qk_workspace_bytes(B: int, T: int, H: int, dk: int, dv: int,
                               in_dtype=torch.bfloat16, gather: bool = False) -> int:
    return int(lib.gdn_prefill_qk_workspace_bytes(B, T, H, dk, dv,
                                                  _DTYPE_CODE[in_dtype], int(gather)))


def prefill_qk(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
               alpha: torch.Tensor, beta: torch.Tensor,
               S0: Optional[torch.Tensor] = None, *,
               channels: Optional[torch.Tensor] = None,
               l2norm: bool = True, q_scale: float = 1.0,
               out_dtype: Optional[torch.dtype] = None,
               o: Optional[torch.Tensor] = None,
               ST: Optional[torch.Tensor] = None,
               final_state: bool = True,
               workspace: Optional[torch.Tensor] = None,
               validate: bool = True,
               stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Prefill from the raw projection output: q, k [B, T, H, dk_in] are
    reduced to the channels `channels[h]` of each head h (int32 [H, dk],
    dk in {64, 128}; None keeps all dk_in = dk channels), normalised over
    the kept channels (if l2norm) and q is multiplied by q_scale, all inside
    the kernels.  Other arguments as prefill().  `validate` checks the
    channel indices on the host (one device sync); the library does not."""
    _dev_tensor(q, "q", _DTYPE_CODE)
    B, T, H, dk_in = q.shape
    _dev_tensor(k, "k", (q.dtype,), q.shape)
    channels, dk = _channels_arg(channels, H, dk_in, q.device, validate)
    _dev_tensor(v, "v", (q.dtype,))
    if tuple(v.shape[:3]) != (B, T, H) or v.dim() != 4:
        raise ValueError(f"v: shape {tuple(v.shape)} incompatible with q")
    dv = v.shape[3]
    _dev_tensor(alpha, "alpha", (torch.float32,), (B, T, H))
    _dev_tensor(beta, "beta", (torch.float32,), (B, T, H))
    if S0 is not None:
        _dev_tensor(S0, "S0", (torch.float32,), (B, H, dv, dk))
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=out_dtype, device=q.device)
    _dev_tensor(o, "o", (out_dtype,), (B, T, H, dv))
    if ST is None and final_state:
        ST = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    if ST is not None:
        _dev_tensor(ST, "ST", (torch.float32,), (B, H, dv, dk))
    need = prefill_qk_workspace_bytes(B, T, H, dk, dv, q.dtype, channels is not None)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = lib.gdn_prefill_qk(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                            _ptr(S0), _ptr(o), _ptr(ST), B, T, H, dk, dv, dk_in,
                            _ptr(channels), int(l2norm), float(q_scale),
                            _DTYPE_CODE[q.dtype], _DTYPE_CODE[out_dtype],
                            _ptr(workspace), workspace.numel(),
                            _stream_handle(q, stream))
    _check(st, "gdn_prefill_qk")
    return o, ST


def decode_step_qk(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                   alpha: torch.Tensor, beta: torch.Tensor, S: torch.Tensor, *,
                   channels: Optional[torch.Tensor] = None,
                   l2norm: bool = True, q_scale: float = 1.0,
                   S_out: Optional[torch.Tensor] = None,
                   o: Optional[torch.Tensor] = None,
                   out_dtype: Optional[torch.dtype] = None,
                   validate: bool = True,
                   stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """One decode token from the raw projection output q, k [B, H, dk_in];
    the input path as in prefill_qk, the rest as decode_step()."""
    _dev_tensor(q, "q", _DTYPE_CODE)
    B, H, dk_in = q.shape
    _dev_tensor(k, "k", (q.dtype,), q.shape)
    channels, dk = _channels_arg(channels, H, dk_in, q.device, validate)
    _dev_tensor(v, "v", (q.dtype,))
    if v.dim() != 3 or tuple(v.shape[:2]) != (B, H):
        raise ValueError(f"v: shape {tuple(v.shape)} incompatible with q")
    dv = v.shape[2]
    _dev_tensor(alpha, "alpha", (torch.float32,), (B, H))
    _dev_tensor(beta, "beta", (torch.float32,), (B, H))
    _dev_tensor(S, "S", (torch.float32,), (B, H, dv, dk))
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((B, H, dv), dtype=out_dtype, device=q.device)
    _dev_tensor(o, "o", (out_dtype,), (B, H, dv))
    if S_out is None:
        S_out = torch.empty_like(S)
    _dev_tensor(S_out, "S_out", (torch.float32,), (B, H, dv, dk))
    st = lib.gdn_decode_step_qk(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                _ptr(beta), _ptr(S), _ptr(S_out), _ptr(o),
                                B, H, dk, dv, dk_in, _ptr(channels), int(l2norm),
                                float(q_scale), _DTYPE_CODE[q.dtype],
                                _DTYPE_CODE[out_dtype], _stream_handle(q, stream))
    _check(st, "gdn_decode_step_qk")
    return o, S_out


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                alpha: torch.Tensor, beta: torch.Tensor, S: torch.Tensor, *,
                S_out: Optional[torch.Tensor] = None,
                o: Optional[torch.Tensor] = None,
                out_dtype: Optional[torch.dtype] = None,
                stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """One token for a batch of carried states.

    q, k [B, H, dk], v [B, H, dv] (float32 or bfloat16); alpha, beta [B, H]
    float32; S [B, H, dv, dk] float32.  S_out may be S (in place; the
    default allocates a new state).  Returns (o [B, H, dv], S_out).
    """
    _dev_tensor(q, "q", _DTYPE_CODE)
    B, H, dk = q.shape
    _dev_tensor(k, "k", (q.dtype,), q.shape)
    _dev_tensor(v, "v", (q.dtype,))
    if v.dim() != 3 or tuple(v.shape[:2]) != (B, H):
        raise ValueError(f"v: shape {tuple(v.shape)} incompatible with q")
    dv = v.shape[2]
    _dev_tensor(alpha, "alpha", (torch.float32,), (B, H))
    _dev_tensor(beta, "beta", (torch.float32,), (B, H))
    _dev_tensor(S, "S", (torch.float32,), (B, H, dv, dk))
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((B, H, dv), dtype=out_dtype, device=q.device)
    _dev_tensor(o, "o", (out_dtype,), (B, H, dv))
    if S_out is None:
        S_out = torch.empty_like(S)
    _dev_tensor(S_out, "S_out", (torch.float32,), (B, H, dv, dk))
    st = lib.gdn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                             _ptr(beta), _ptr(S), _ptr(S_out), _ptr(o),
                             B, H, dk, dv, _DTYPE_CODE[q.dtype],
                             _DTYPE_CODE[out_dtype], _stream_handle(q, stream))
    _check(st, "gdn_decode_step")
    return o, S_out


# ---------------------------------------------------------------------------
# generalised gates (per-key-channel retention, split erase / write gates)
# ---------------------------------------------------------------------------

def gated_recurrent(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    alpha: torch.Tensor, b: torch.Tensor, w: torch.Tensor,
                    S0: Optional[torch.Tensor] = None, *,
                    out_dtype: Optional[torch.dtype] = None,
                    o: Optional[torch.Tensor] = None,
                    ST: Optional[torch.Tensor] = None,
                    final_state: bool = True,
                    stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """S_t = S_{t-1} diag(alpha_t) (I - (b_t*k_t) k_t^T) + (w_t*v_t) k_t^T,
    o_t = S_t q_t, token by token (see include/gdn.h).  q, k [B, T, H, dk],
    v [B, T, H, dv] (float32 or bfloat16); alpha, b [B, T, H, dk] and w
    [B, T, H, dv] float32; S0 [B, H, dv, dk] float32 or None.  T == 1 is a
    decode step.  Returns (o, S_T)."""
    _dev_tensor(q, "q", _DTYPE_CODE)
    B, T, H, dk = q.shape
    _dev_tensor(k, "k", (q.dtype,), q.shape)
    _dev_tensor(v, "v", (q.dtype,))
    if tuple(v.shape[:3]) != (B, T, H) or v.dim() != 4:
        raise ValueError(f"v: shape {tuple(v.shape)} incompatible with q")
    dv = v.shape[3]
    _dev_tensor(alpha, "alpha", (torch.float32,), (B, T, H, dk))
    _dev_tensor(b, "b", (torch.float32,), (B, T, H, dk))
    _dev_tensor(w, "w", (torch.float32,), (B, T, H, dv))
    if S0 is not None:
        _dev_tensor(S0, "S0", (torch.float32,), (B, H, dv, dk))
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=out_dtype, device=q.device)
    _dev_tensor(o, "o", (out_dtype,), (B, T, H, dv))
    if ST is None and final_state:
        ST = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    if ST is not None:
        _dev_tensor(ST, "ST", (torch.float32,), (B, H, dv, dk))
    st = lib.gdn_gated_recurrent(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b),
                                 _ptr(w), _ptr(S0), _ptr(o), _ptr(ST), B, T, H, dk, dv,
                                 _DTYPE_CODE[q.dtype], _DTYPE_CODE[out_dtype],
                                 _stream_handle(q, stream))
    _check(st, "gdn_gated_recurrent")
    return o, ST


def gated_prefill_workspace_bytes(B: int, T: int, H: int, dk: int, dv: int,
                                  in_dtype=torch.bfloat16) -> int:
    return int(lib.gdn_gated_prefill_workspace_bytes(B, T, H, dk, dv, _DTYPE_CODE[in_dtype]))


def gated_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  alpha: torch.Tensor, b: torch.Tensor, w: torch.Tensor,
                  S0: Optional[torch.Tensor] = None, *,
                  out_dtype: Optional[torch.dtype] = None,
                  o: Optional[torch.Tensor] = None,
                  ST: Optional[torch.Tensor] = None,
                  final_state: bool = True,
                  workspace: Optional[torch.Tensor] = None,
                  stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """The generalised gates over whole sequences in chunked form (bf16
    inputs; fp32 inputs run the recurrent form); arguments as
    gated_recurrent, plus an optional uint8 `workspace` of at least
    gated_prefill_workspace_bytes(...) bytes."""
    _dev_tensor(q, "q", _DTYPE_CODE)
    B, T, H, dk = q.shape
    _dev_tensor(k, "k", (q.dtype,), q.shape)
    _dev_tensor(v, "v", (q.dtype,))
    if tuple(v.shape[:3]) != (B, T, H) or v.dim() != 4:
        raise ValueError(f"v: shape {tuple(v.shape)} incompatible with q")
    dv = v.shape[3]
    _dev_tensor(alpha, "alpha", (torch.float32,), (B, T, H, dk))
    _dev_tensor(b, "b", (torch.float32,), (B, T, H, dk))
    _dev_tensor(w, "w", (torch.float32,), (B, T, H, dv))
    if S0 is not None:
        _dev_tensor(S0, "S0", (torch.float32,), (B, H, dv, dk))
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=out_dtype, device=q.device)
    _dev_tensor(o, "o", (out_dtype,), (B, T, H, dv))
    if ST is None and final_state:
        ST = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    if ST is not None:
        _dev_tensor(ST, "ST", (torch.float32,), (B, H, dv, dk))
    need = gated_prefill_workspace_bytes(B, T, H, dk, dv, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = lib.gdn_gated_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w),
                               _ptr(S0), _ptr(o), _ptr(ST), B, T, H, dk, dv,
                               _DTYPE_CODE[q.dtype], _DTYPE_CODE[out_dtype],
                               _ptr(workspace), workspace.numel(), _stream_handle(q, stream))
    _check(st, "gdn_gated_prefill")
    return o, ST


# ---------------------------------------------------------------------------
# backward pass
# ---------------------------------------------------------------------------

def backward_workspace_bytes(B: int, T: int, H: int, dk: int, dv: int,
                             in_dtype=torch.bfloat16) -> int:
    return int(lib.gdn_backward_workspace_bytes(B, T, H, dk, dv, _DTYPE_CODE[in_dtype]))


def backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
             alpha: torch.Tensor, beta: torch.Tensor, S0: Optional[torch.Tensor],
             d_o: torch.Tensor, dST: Optional[torch.Tensor] = None, *,
             want_dS0: bool = True, out: Optional[dict] = None,
             workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Gradients of sum <d_o, o> + <dST, S_T> through prefill's recurrence
    (see include/gdn.h): q, k [B, T, H, dk], v, d_o [B, T, H, dv] (float32
    or bfloat16, one dtype); alpha, beta [B, T, H] float32; S0, dST
    [B, H, dv, dk] float32 or None.  Returns a dict of float32 tensors dq,
    dk, dv, dalpha, dbeta and dS0 (None unless want_dS0).  `out`: optional
    dict of preallocated outputs under the same keys."""
    _dev_tensor(q, "q", _DTYPE_CODE)
    B, T, H, dk = q.shape
    _dev_tensor(k, "k", (q.dtype,), q.shape)
    _dev_tensor(v, "v", (q.dtype,))
    if tuple(v.shape[:3]) != (B, T, H) or v.dim() != 4:
        raise ValueError(f"v: shape {tuple(v.shape)} incompatible with q")
    dv = v.shape[3]
    _dev_tensor(d_o, "d_o", (q.dtype,), (B, T, H, dv))
    _dev_tensor(alpha, "alpha", (torch.float32,), (B, T, H))
    _dev_tensor(beta, "beta", (torch.float32,), (B, T, H))
    if S0 is not None:
        _dev_tensor(S0, "S0", (torch.float32,), (B, H, dv, dk))
    if dST is not None:
        _dev_tensor(dST, "dST", (torch.float32,), (B, H, dv, dk))
    shapes = {"dq": (B, T, H, dk), "dk": (B, T, H, dk), "dv": (B, T, H, dv),
              "dalpha": (B, T, H), "dbeta": (B, T, H), "dS0": (B, H, dv, dk)}
    res = dict(out or {})
    for name, shp in shapes.items():
        if name == "dS0" and not want_dS0:
            res[name] = None
            continue
        if res.get(name) is None:
            res[name] = torch.empty(shp, dtype=torch.float32, device=q.device)
        _dev_tensor(res[name], name, (torch.float32,), shp)
    need = backward_workspace_bytes(B, T, H, dk, dv, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = lib.gdn_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S0),
                          _ptr(d_o), _ptr(dST), _ptr(res["dq"]), _ptr(res["dk"]),
                          _ptr(res["dv"]), _ptr(res["dalpha"]), _ptr(res["dbeta"]),
                          _ptr(res["dS0"]), B, T, H, dk, dv, _DTYPE_CODE[q.dtype],
                          _ptr(workspace), workspace.numel(), _stream_handle(q, stream))
    _check(st, "gdn_backward")
    return res


# ---------------------------------------------------------------------------
# DRRQR channel selection (host)
# ---------------------------------------------------------------------------

def drrqr_select(M, k: int, f: float = 2.0, max_swaps: int = 10000):
    """Kept channels of one head from calibration samples M [rows, n] (a
    numpy array or CPU tensor; samples as rows, K and Q samples stacked),
    by the library's host DRRQR (see include/gdn.h).  Returns (int32 array
    of the k kept channels, swaps made, final max rho)."""
    import numpy as np
    if isinstance(M, torch.Tensor):
        if M.is_cuda:
            raise ValueError("M must be in host memory")
        M = M.numpy()
    M = np.ascontiguousarray(M, dtype=np.float64)
    if M.ndim != 2:
        raise ValueError("M must be [rows, n]")
    rows, n = M.shape
    sel = np.empty(max(int(k), 1), dtype=np.int32)
    sw = ctypes.c_int(0)
    rho = ctypes.c_double(0.0)
    st = lib.gdn_drrqr_select(M.ctypes.data_as(ctypes.c_void_p), rows, n, int(k),
                              float(f), int(max_swaps),
                              sel.ctypes.data_as(ctypes.c_void_p), ctypes.byref(sw),
                              ctypes.byref(rho))
    _check(st, "gdn_drrqr_select")
    return sel[:k], sw.value, rho.value


# ---------------------------------------------------------------------------
# rank-r truncation
# ---------------------------------------------------------------------------

def truncate_workspace_bytes(BH: int, dv: int, dk: int) -> int:
    return int(lib.gdn_truncate_workspace_bytes(BH, dv, dk))


def truncate_rank(S: torch.Tensor, r: int, *, stable_rank: bool = True,
                  workspace: Optional[torch.Tensor] = None,
                  stream=None) -> Optional[torch.Tensor]:
    """Project every state in S [..., dv, dk] (float32, updated in place)
    onto its top-r left singular directions; r >= min(dv, dk) leaves S
    unchanged.  Returns the stable rank of each result (float32, shape
    S.shape[:-2]; NaN for a zero state) if `stable_rank`, else None."""
    _dev_tensor(S, "S", (torch.float32,))
    if S.dim() < 2:
        raise ValueError("S must be [..., dv, dk]")
    dv, dk = S.shape[-2:]
    BH = S.numel() // (dv * dk) if S.numel() else 0
    er = (torch.empty(S.shape[:-2], dtype=torch.float32, device=S.device)
          if stable_rank else None)
    if BH == 0:
        return er
    need = truncate_workspace_bytes(BH, dv, dk) if r < min(dv, dk) else 0
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=S.device)
    st = lib.gdn_truncate_rank(_ptr(S), BH, dv, dk, int(r), _ptr(er),
                               _ptr(workspace),
                               0 if workspace is None else workspace.numel(),
                               _stream_handle(S, stream))
    _check(st, "gdn_truncate_rank")
    return er


def prefill_truncated(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                      alpha: torch.Tensor, beta: torch.Tensor, r: int,
                      S0: Optional[torch.Tensor] = None, *,
                      segment: int = 256,
                      out_dtype: Optional[torch.dtype] = None,
                      stream=None):
    """Segment-truncated prefill: the recurrence runs over `segment`-token
    pieces, and between pieces every carried state is replaced by its
    rank-r truncation (never after the last token).  Returns (o, S_T,
    stable rank of S_T).  Each piece is one gdn_prefill call on a
    contiguous slice (one call per batch row when B > 1), each boundary one
    gdn_truncate_rank call; all of it is enqueued on one stream."""
    B, T, H, dk, dv = _prefill_args(q, k, v, alpha, beta, S0)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    o = torch.empty((B, T, H, dv), dtype=out_dtype, device=q.device)
    S = (torch.zeros((B, H, dv, dk), dtype=torch.float32, device=q.device)
         if S0 is None else S0.clone())
    lengths = {min(segment, T - t0) for t0 in range(0, T, segment)}
    seg_ws = torch.empty(max([16] + [prefill_workspace_bytes(1, n, H, dk, dv)
                                     for n in lengths]),
                         dtype=torch.uint8, device=q.device)
    tr_ws = torch.empty(max(truncate_workspace_bytes(B * H, dv, dk), 16),
                        dtype=torch.uint8, device=q.device)
    for t0 in range(0, T, segment):
        t1 = min(T, t0 + segment)
        for b in range(B):
            sl = (slice(b, b + 1), slice(t0, t1))
            prefill(q[sl], k[sl], v[sl], alpha[sl], beta[sl], S[b:b + 1],
                    out_dtype=out_dtype, o=o[sl], ST=S[b:b + 1],
                    workspace=seg_ws, stream=stream)
        if t1 < T:
            truncate_rank(S, r, stable_rank=False, workspace=tr_ws,
                          stream=stream)
    er = truncate_rank(S, min(dv, dk), stable_rank=True, stream=stream)
    return o, S, er
