"""Thin Python binding over libflux_attn.so (the C ABI in include/flux_attn.h).

Argument marshalling only: every step of the attention path runs in the HIP
kernels behind the C ABI.  torch is used for device memory and streams
(``tensor.data_ptr()``, ``torch.cuda.current_stream().cuda_stream``).  There is
no fallback: if the library is not built, importing this package raises.

Function names match the C entry points.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

__all__ = [
    "FluxError", "lib", "status_string", "last_error_detail", "flux_version",
    "flux_build_block_mask", "flux_attn_prefill", "flux_attn_prefill_layers", "flux_attn_prefill_layers_routed",
    "flux_decode_workspace_size", "flux_attn_decode", "flux_attn_decode_noalloc", "flux_window_cache_rows",
    "flux_decode_step", "flux_decode_step_layers", "flux_route_workspace_size", "flux_route_layers",
    "flux_route_soft_weights", "flux_prefill_soft_workspace_size", "flux_attn_prefill_soft",
    "flux_attn_backward_workspace_size", "flux_attn_backward", "FLUX_DECODE_SCRATCH_BYTES",
    "FLUX_OK", "FLUX_ERR_INVALID_ARG", "FLUX_ERR_UNSUPPORTED", "FLUX_ERR_CAPACITY", "FLUX_ERR_WORKSPACE",
    "FLUX_ERR_HIP", "FLUX_DTYPE_BF16", "FLUX_DTYPE_F32", "FLUX_MODE_DENSE", "FLUX_MODE_SPARSE", "FLUX_KV_FULL",
    "FLUX_KV_WINDOW",
    "EXPORTED_SYMBOLS",
]

FLUX_OK, FLUX_ERR_INVALID_ARG, FLUX_ERR_UNSUPPORTED, FLUX_ERR_CAPACITY, FLUX_ERR_WORKSPACE, FLUX_ERR_HIP = range(6)
FLUX_DTYPE_BF16, FLUX_DTYPE_F32 = 0, 1
FLUX_MODE_DENSE, FLUX_MODE_SPARSE = 0, 1
FLUX_KV_FULL, FLUX_KV_WINDOW = 0, 1
FLUX_DECODE_SCRATCH_BYTES = 16 << 20

EXPORTED_SYMBOLS = (
    "flux_status_string", "flux_last_error_detail", "flux_version", "flux_build_block_mask",
    "flux_attn_prefill", "flux_attn_prefill_layers", "flux_attn_prefill_layers_routed",
    "flux_decode_workspace_size", "flux_attn_decode", "flux_attn_decode_noalloc", "flux_window_cache_rows",
    "flux_decode_step", "flux_decode_step_layers", "flux_route_workspace_size", "flux_route_layers", "flux_route_soft_weights",
    "flux_prefill_soft_workspace_size", "flux_attn_prefill_soft", "flux_attn_backward_workspace_size",
    "flux_attn_backward",
)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libflux_attn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python long_context_attention_tiled_amd/build.py` "
        "(hipcc for gfx950).  There is no CPU fallback.")

# torch first: its HIP runtime (same soname as the system one) is then the one this library binds to, so
# tensors, streams and our launches share one runtime whichever module the caller imported first.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)
_i32, _i64, _f32, _vp, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
_pp = ctypes.POINTER(ctypes.c_void_p)

_lib.flux_status_string.argtypes = [ctypes.c_int]
_lib.flux_status_string.restype = ctypes.c_char_p
_lib.flux_last_error_detail.argtypes = []
_lib.flux_last_error_detail.restype = ctypes.c_char_p
_lib.flux_version.argtypes = []
_lib.flux_version.restype = ctypes.c_int
_lib.flux_build_block_mask.argtypes = [_i64, _i64, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _i64,
                                       ctypes.POINTER(_i64)]
_lib.flux_build_block_mask.restype = ctypes.c_int
_lib.flux_attn_prefill.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i64, _i64, _i32, _i32, _i32, _f32, _i32,
                                   _i32, _i32, _i32, _i32, _vp, _vp, _i64, _vp]
_lib.flux_attn_prefill.restype = ctypes.c_int
_lib.flux_attn_prefill_layers.argtypes = [_i32, _vp, _pp, _pp, _pp, _pp, _pp, _i32, _i32, _i64, _i64, _i32, _i32,
                                          _i32, _f32, _i32, _i32, _i32, _vp, _vp, _i64, _vp]
_lib.flux_attn_prefill_layers.restype = ctypes.c_int
_lib.flux_attn_prefill_layers_routed.argtypes = [_i32, _vp, _pp, _pp, _pp, _pp, _pp, _i32, _i32, _i64, _i64, _i32,
                                                 _i32, _i32, _f32, _i32, _i32, _i32, _vp, _vp, _i64, _vp]
_lib.flux_attn_prefill_layers_routed.restype = ctypes.c_int
_lib.flux_decode_workspace_size.argtypes = [_i64, _i32, _i32, _i64, _i32, _i32, _i32, _i32, _i32, _i32]
_lib.flux_decode_workspace_size.restype = _sz
_lib.flux_attn_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i64, _i64, _i64, _i32, _i32, _i32, _f32,
                                  _i32, _i32, _i32, _i32, _i32, _vp, _sz, _vp]
_lib.flux_attn_decode.restype = ctypes.c_int
_lib.flux_attn_decode_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i64, _i64, _i64, _i32, _i32, _i32,
                                          _f32, _i32, _i32, _i32, _i32, _i32, _vp]
_lib.flux_attn_decode_noalloc.restype = ctypes.c_int
_lib.flux_window_cache_rows.argtypes = [_i32, _i32, _i32]
_lib.flux_window_cache_rows.restype = _i64
_lib.flux_decode_step.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _i32, _i32, _i32, _i32,
                                  _f32, _i32, _i32, _i32, _i32, _i32, _vp, _sz, _vp]
_lib.flux_decode_step.restype = ctypes.c_int
_lib.flux_decode_step_layers.argtypes = [_i32, _vp, _pp, _pp, _pp, _pp, _pp, _pp, _pp, _i32, _i64, _i64, _i64, _i32,
                                         _i32, _i32, _f32, _i32, _i32, _i32, _vp, _sz, _vp]
_lib.flux_decode_step_layers.restype = ctypes.c_int
_lib.flux_route_soft_weights.argtypes = [_vp, _vp, _f32, _i32, _vp, _vp]
_lib.flux_route_soft_weights.restype = ctypes.c_int
_lib.flux_prefill_soft_workspace_size.argtypes = [_i64, _i64, _i32, _i32]
_lib.flux_prefill_soft_workspace_size.restype = _sz
_lib.flux_attn_prefill_soft.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32, _i64, _i64, _i32, _i32, _i32, _f32, _i32, _i32,
                                        _i32, _vp, _vp, _i64, _vp, _vp, _sz, _vp]
_lib.flux_attn_prefill_soft.restype = ctypes.c_int
_lib.flux_attn_backward_workspace_size.argtypes = [_i64, _i64, _i32, _i32, _i32, _i32, _i32, _i32]
_lib.flux_attn_backward_workspace_size.restype = _sz
_lib.flux_attn_backward.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i64, _i64, _i32, _i32, _i32,
                                    _f32, _i32, _i32, _i32, _i32, _i32, _vp, _sz, _vp]
_lib.flux_attn_backward.restype = ctypes.c_int
_lib.flux_route_workspace_size.argtypes = [_i32, _i32, _i32, _i32]
_lib.flux_route_workspace_size.restype = _sz
_lib.flux_route_layers.argtypes = [_pp, _i32, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp,
                                   _sz, _vp]
_lib.flux_route_layers.restype = ctypes.c_int


def lib():
    """The loaded ctypes library (for callers that marshal raw pointers themselves)."""
    return _lib


class FluxError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({last_error_detail()})")


def status_string(status: int) -> str:
    return _lib.flux_status_string(int(status)).decode()


def last_error_detail() -> str:
    return _lib.flux_last_error_detail().decode()


def flux_version() -> int:
    return int(_lib.flux_version())


def _check(status: int, where: str):
    if status != FLUX_OK:
        raise FluxError(status, where)


# ------------------------------------------------------------------ helpers
def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return FLUX_DTYPE_BF16
    if t.dtype == torch.float32:
        return FLUX_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _dev(t, name, shape=None, dtypes=None, like=None):
    """Check a tensor argument before its pointer crosses the C ABI, which cannot tell a host pointer or a
    short buffer from a good one: a contiguous GPU tensor, on the same device as `like`, of the given
    shape and dtype(s)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (it is on {t.device})")
    if like is not None and t.device != like.device:
        raise ValueError(f"{name} is on {t.device}, the other tensors on {like.device}")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {tuple(str(x) for x in dtypes)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _float_types():
    import torch
    return (torch.bfloat16, torch.float32)


def _check_csr(rp, ci, seq, block, like):
    """Device CSR from flux_build_block_mask(seq, seq, block, ...): row_ptr int32 [ceil(seq/block)+1]."""
    import torch
    if rp is None or ci is None:
        return
    _dev(rp, "blk_row_ptr", (-(-seq // block) + 1,), (torch.int32,), like)
    _dev(ci, "blk_col_idx", None, (torch.int32,), like)
    if ci.dim() != 1:
        raise ValueError("blk_col_idx must be one-dimensional")


def _check_attention(q, k, v, o, lse, like=None):
    """q [B,S,Hq,d], k/v [B,S,Hkv,d] of q's dtype, o [B,S,Hq,d] bf16/fp32, lse [B,Hq,S] fp32 or None."""
    import torch
    for name, t in (("q", q), ("k", k)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [batch, seq, heads, head_dim]")
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    like = q if like is None else like
    _dev(q, "q", None, _float_types(), like)
    _dev(k, "k", (B, S, Hkv, d), (q.dtype,), like)
    _dev(v, "v", (B, S, Hkv, d), (q.dtype,), like)
    _dev(o, "o", (B, S, Hq, d), _float_types(), like)
    if lse is not None:
        _dev(lse, "lse", (B, Hq, S), (torch.float32,), like)
    return B, S, Hq, Hkv, d


def _check_workspace(ws, like):
    import torch
    if ws is not None:
        _dev(ws, "workspace", None, None, like)
        if ws.dtype != torch.uint8:
            raise TypeError("workspace must be a uint8 tensor")


# ------------------------------------------------------------------ entry points
def flux_build_block_mask(seq_q: int, seq_k: int, block: int = 64, sink_tokens: int = 128, window_tokens: int = 2048,
                          causal: int = 1, mode: int = FLUX_MODE_SPARSE):
    """Host CSR of the active key blocks: (row_ptr int32 [nbq+1], col_idx int32 [nnz])."""
    nnz = _i64(0)
    _check(_lib.flux_build_block_mask(seq_q, seq_k, block, sink_tokens, window_tokens, causal, mode, None, None, 0,
                                      ctypes.byref(nnz)), "flux_build_block_mask")
    nbq = -(-seq_q // block)
    row_ptr = np.zeros(nbq + 1, np.int32)
    col_idx = np.zeros(max(1, nnz.value), np.int32)
    _check(_lib.flux_build_block_mask(seq_q, seq_k, block, sink_tokens, window_tokens, causal, mode,
                                      row_ptr.ctypes.data_as(_vp), col_idx.ctypes.data_as(_vp), col_idx.size,
                                      ctypes.byref(nnz)), "flux_build_block_mask")
    return row_ptr, col_idx[:nnz.value]


def flux_attn_prefill(q, k, v, o, lse=None, *, causal: int = 1, mode: int = FLUX_MODE_DENSE, block: int = 64,
                      sink_tokens: int = 128, window_tokens: int = 2048, blk_row_ptr=None, blk_col_idx=None,
                      scale: float | None = None, stream=None):
    """q [B,S,Hq,d], k/v [B,S,Hkv,d], o [B,S,Hq,d] (device tensors); lse [B,Hq,S] float32 or None.

    blk_row_ptr / blk_col_idx: device int32 tensors from flux_build_block_mask (sparse mode)."""
    B, S, Hq, Hkv, d = _check_attention(q, k, v, o, lse)
    _check_csr(blk_row_ptr, blk_col_idx, S, block, q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nnz = int(blk_col_idx.numel()) if blk_col_idx is not None else 0
    _check(_lib.flux_attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _dtype_code(q), _dtype_code(o), B, S,
                                  Hq, Hkv, d, scale, causal, mode, block, sink_tokens, window_tokens,
                                  _ptr(blk_row_ptr), _ptr(blk_col_idx), nnz, _stream(stream)), "flux_attn_prefill")


def _ptr_array(ts):
    arr = (ctypes.c_void_p * len(ts))(*[(t.data_ptr() if t is not None else None) for t in ts])
    return ctypes.cast(arr, _pp), arr


def _check_layers(qs, ks, vs, os_, lses):
    L = len(qs)
    if L < 1 or not (len(ks) == len(vs) == len(os_) == L) or (lses is not None and len(lses) != L):
        raise ValueError("qs, ks, vs, os_ (and lses) must hold one tensor per layer")
    dims = _check_attention(qs[0], ks[0], vs[0], os_[0], None if lses is None else lses[0])
    for l in range(1, L):
        _check_attention(qs[l], ks[l], vs[l], os_[l], None if lses is None else lses[l], like=qs[0])
        if tuple(qs[l].shape) != tuple(qs[0].shape) or tuple(ks[l].shape) != tuple(ks[0].shape) or \
                qs[l].dtype != qs[0].dtype or os_[l].dtype != os_[0].dtype:
            raise ValueError(f"layer {l} differs in shape or dtype from layer 0")
    return dims


def flux_attn_prefill_layers(modes_host, qs, ks, vs, os_, lses=None, *, block: int = 64, sink_tokens: int = 128,
                             window_tokens: int = 2048, blk_row_ptr=None, blk_col_idx=None,
                             scale: float | None = None, stream=None):
    """Per-layer dispatch: layer l runs dense or block-sparse prefill per modes_host[l] (host int32)."""
    L = len(qs)
    modes = np.ascontiguousarray(np.asarray(modes_host, dtype=np.int32))
    if modes.shape != (L,):
        raise ValueError(f"modes_host must hold one mode per layer ({L})")
    B, S, Hq, Hkv, d = _check_layers(qs, ks, vs, os_, lses)
    _check_csr(blk_row_ptr, blk_col_idx, S, block, qs[0])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    pq, _a = _ptr_array(qs)
    pk, _b = _ptr_array(ks)
    pv, _c = _ptr_array(vs)
    po, _d = _ptr_array(os_)
    pl, _e = _ptr_array(lses) if lses is not None else (None, None)
    nnz = int(blk_col_idx.numel()) if blk_col_idx is not None else 0
    _check(_lib.flux_attn_prefill_layers(L, modes.ctypes.data_as(_vp), pq, pk, pv, po, pl, _dtype_code(qs[0]),
                                         _dtype_code(os_[0]), B, S, Hq, Hkv, d, scale, block, sink_tokens,
                                         window_tokens, _ptr(blk_row_ptr), _ptr(blk_col_idx), nnz, _stream(stream)),
           "flux_attn_prefill_layers")


def flux_attn_prefill_layers_routed(modes_dev, qs, ks, vs, os_, lses=None, *, block: int = 64,
                                    sink_tokens: int = 128, window_tokens: int = 2048, blk_row_ptr=None,
                                    blk_col_idx=None, scale: float | None = None, stream=None):
    """Per-layer dispatch with the modes left on the device (int32 tensor of len(qs) entries, e.g. the
    modes_out of flux_route_layers): the kernels read layer l's mode themselves, no host round trip.
    The block-sparse CSR is required."""
    L = len(qs)
    import torch
    B, S, Hq, Hkv, d = _check_layers(qs, ks, vs, os_, lses)
    _dev(modes_dev, "modes_dev", None, (torch.int32,), qs[0])
    if modes_dev.numel() != L:
        raise ValueError("modes_dev must be a contiguous int32 device tensor with one entry per layer")
    _check_csr(blk_row_ptr, blk_col_idx, S, block, qs[0])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    pq, _a = _ptr_array(qs)
    pk, _b = _ptr_array(ks)
    pv, _c = _ptr_array(vs)
    po, _d = _ptr_array(os_)
    pl, _e = _ptr_array(lses) if lses is not None else (None, None)
    nnz = int(blk_col_idx.numel()) if blk_col_idx is not None else 0
    _check(_lib.flux_attn_prefill_layers_routed(L, _ptr(modes_dev), pq, pk, pv, po, pl, _dtype_code(qs[0]),
                                                _dtype_code(os_[0]), B, S, Hq, Hkv, d, scale, block, sink_tokens,
                                                window_tokens, _ptr(blk_row_ptr), _ptr(blk_col_idx), nnz,
                                                _stream(stream)),
           "flux_attn_prefill_layers_routed")


def flux_decode_workspace_size(batch, hq, hkv, kv_len, head_dim, mode=FLUX_MODE_DENSE, block=64, sink_tokens=128,
                               window_tokens=2048, num_splits=0) -> int:
    return int(_lib.flux_decode_workspace_size(batch, hq, hkv, kv_len, head_dim, mode, block, sink_tokens,
                                               window_tokens, num_splits))


def flux_attn_decode(q, k_cache, v_cache, o, lse=None, *, kv_len: int | None = None, mode: int = FLUX_MODE_DENSE,
                     block: int = 64, sink_tokens: int = 128, window_tokens: int = 2048, num_splits: int = 0,
                     workspace=None, scale: float | None = None, stream=None):
    """q [B,Hq,d], caches [B,cap,Hkv,d] bf16, o [B,Hq,d]; workspace: a uint8 device tensor."""
    import torch
    _dev(q, "q", None, (torch.bfloat16,))
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [batch, q_heads, head_dim] and the caches [batch, rows, kv_heads, head_dim]")
    B, Hq, d = q.shape
    cap, Hkv = k_cache.shape[1], k_cache.shape[2]
    _dev(k_cache, "k_cache", (B, cap, Hkv, d), (torch.bfloat16,), q)
    _dev(v_cache, "v_cache", (B, cap, Hkv, d), (torch.bfloat16,), q)
    _dev(o, "o", (B, Hq, d), _float_types(), q)
    if lse is not None:
        _dev(lse, "lse", (B, Hq), (torch.float32,), q)
    _check_workspace(workspace, q)
    if kv_len is None:
        kv_len = cap
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.flux_attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse), _dtype_code(q),
                                 _dtype_code(o), B, kv_len, cap, Hq, Hkv, d, scale, mode, block, sink_tokens,
                                 window_tokens, num_splits, _ptr(workspace), ws_bytes, _stream(stream)),
           "flux_attn_decode")


def flux_attn_decode_noalloc(q, k_cache, v_cache, o, lse=None, *, kv_len: int | None = None,
                             mode: int = FLUX_MODE_DENSE, block: int = 64, sink_tokens: int = 128,
                             window_tokens: int = 2048, num_splits: int = 0, scale: float | None = None, stream=None):
    """flux_attn_decode without a workspace: the partials go to the library's fixed per-device scratch of
    FLUX_DECODE_SCRATCH_BYTES (calls that may overlap on one GPU race; calls in order on one stream do not)."""
    import torch
    _dev(q, "q", None, (torch.bfloat16,))
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [batch, q_heads, head_dim] and the caches [batch, rows, kv_heads, head_dim]")
    B, Hq, d = q.shape
    cap, Hkv = k_cache.shape[1], k_cache.shape[2]
    _dev(k_cache, "k_cache", (B, cap, Hkv, d), (torch.bfloat16,), q)
    _dev(v_cache, "v_cache", (B, cap, Hkv, d), (torch.bfloat16,), q)
    _dev(o, "o", (B, Hq, d), _float_types(), q)
    if lse is not None:
        _dev(lse, "lse", (B, Hq), (torch.float32,), q)
    if kv_len is None:
        kv_len = cap
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check(_lib.flux_attn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse), _dtype_code(q),
                                         _dtype_code(o), B, kv_len, cap, Hq, Hkv, d, scale, mode, block, sink_tokens,
                                         window_tokens, num_splits, _stream(stream)),
           "flux_attn_decode_noalloc")


def flux_window_cache_rows(block: int = 64, sink_tokens: int = 128, window_tokens: int = 2048) -> int:
    return int(_lib.flux_window_cache_rows(block, sink_tokens, window_tokens))


def _check_step_layer(q, k_new, v_new, k_cache, v_cache, o, lse, B, Hq, Hkv, d, rows, tag):
    import torch
    _dev(q, "q" + tag, (B, Hq, d), (torch.bfloat16,))
    _dev(k_new, "k_new" + tag, (B, Hkv, d), (torch.bfloat16,), q)
    _dev(v_new, "v_new" + tag, (B, Hkv, d), (torch.bfloat16,), q)
    _dev(k_cache, "k_cache" + tag, (B, rows, Hkv, d), (torch.bfloat16,), q)
    _dev(v_cache, "v_cache" + tag, (B, rows, Hkv, d), (torch.bfloat16,), q)
    _dev(o, "o" + tag, (B, Hq, d), _float_types(), q)
    if lse is not None:
        _dev(lse, "lse" + tag, (B, Hq), (torch.float32,), q)


def flux_decode_step(q, k_new, v_new, k_cache, v_cache, o, lse=None, *, pos: int, layout: int = FLUX_KV_FULL,
                     mode: int = FLUX_MODE_DENSE, block: int = 64, sink_tokens: int = 128, window_tokens: int = 2048,
                     num_splits: int = 0, workspace=None, scale: float | None = None, stream=None):
    """Append token `pos` (k_new/v_new [B,Hkv,d] bf16) to the cache [B,rows,Hkv,d] and attend from q [B,Hq,d]."""
    import torch
    _dev(q, "q", None, (torch.bfloat16,))
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [batch, q_heads, head_dim] and the caches [batch, rows, kv_heads, head_dim]")
    B, Hq, d = q.shape
    rows, Hkv = k_cache.shape[1], k_cache.shape[2]
    _check_step_layer(q, k_new, v_new, k_cache, v_cache, o, lse, B, Hq, Hkv, d, rows, "")
    _check_workspace(workspace, q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.flux_decode_step(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse),
                                 _dtype_code(o), B, pos, rows, layout, Hq, Hkv, d, scale, mode, block, sink_tokens,
                                 window_tokens, num_splits, _ptr(workspace), ws_bytes, _stream(stream)),
           "flux_decode_step")


def flux_decode_step_layers(modes_host, qs, k_news, v_news, k_caches, v_caches, os_, lses=None, *, pos: int,
                            dense_cache_rows: int, block: int = 64, sink_tokens: int = 128,
                            window_tokens: int = 2048, workspace=None, scale: float | None = None, stream=None):
    """One decode step over a routed stack: dense layers on full caches, sparse layers on window caches."""
    L = len(qs)
    modes = np.ascontiguousarray(np.asarray(modes_host, dtype=np.int32))
    if modes.shape != (L,):
        raise ValueError(f"modes_host must hold one mode per layer ({L})")
    if not (len(k_news) == len(v_news) == len(k_caches) == len(v_caches) == len(os_) == L) or \
            (lses is not None and len(lses) != L):
        raise ValueError("every per-layer list must hold one tensor per layer")
    if qs[0].dim() != 3 or k_news[0].dim() != 3:
        raise ValueError("q must be [batch, q_heads, head_dim] and k_new [batch, kv_heads, head_dim]")
    B, Hq, d = qs[0].shape
    Hkv = k_news[0].shape[1]
    win_rows = flux_window_cache_rows(block, sink_tokens, window_tokens)
    for l in range(L):
        rows = dense_cache_rows if modes[l] == FLUX_MODE_DENSE else win_rows
        _check_step_layer(qs[l], k_news[l], v_news[l], k_caches[l], v_caches[l], os_[l],
                          None if lses is None else lses[l], B, Hq, Hkv, d, rows, f"[{l}]")
        if qs[l].device != qs[0].device:
            raise ValueError("all layers must be on one device")
    _check_workspace(workspace, qs[0])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    arrs = [_ptr_array(x) for x in (qs, k_news, v_news, k_caches, v_caches, os_)]
    pl, _e = _ptr_array(lses) if lses is not None else (None, None)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.flux_decode_step_layers(L, modes.ctypes.data_as(_vp), *[a[0] for a in arrs], pl, _dtype_code(os_[0]),
                                        B, pos, dense_cache_rows, Hq, Hkv, d, scale, block, sink_tokens, window_tokens,
                                        _ptr(workspace), ws_bytes, _stream(stream)),
           "flux_decode_step_layers")


def flux_route_workspace_size(n_layers, hq, head_dim, hidden) -> int:
    return int(_lib.flux_route_workspace_size(n_layers, hq, head_dim, hidden))


def flux_route_layers(q_layers, w_enc, b_enc, w_head, b_head, modes_out, logits_out=None, *, workspace=None,
                      pool_tokens: int = 100, stream=None):
    """q_layers: list of device tensors [S,Hq,d]; weights device float32; modes_out device int32 [L];
    workspace: uint8 device tensor of flux_route_workspace_size(...) bytes (allocated here if None)."""
    import torch
    L = len(q_layers)
    if L < 1 or q_layers[0].dim() != 3:
        raise ValueError("q_layers must be a non-empty list of [seq, q_heads, head_dim] tensors")
    S, Hq, d = q_layers[0].shape
    for l, x in enumerate(q_layers):
        _dev(x, f"q_layers[{l}]", (S, Hq, d), (q_layers[0].dtype,) if l else _float_types(), q_layers[0])
    if w_enc.dim() != 3:
        raise ValueError("w_enc must be [n_layers, hidden, q_heads * head_dim]")
    hidden = w_enc.shape[1]
    f32 = (torch.float32,)
    _dev(w_enc, "w_enc", (L, hidden, Hq * d), f32, q_layers[0])
    _dev(b_enc, "b_enc", (L, hidden), f32, q_layers[0])
    _dev(w_head, "w_head", (L, 2, hidden), f32, q_layers[0])
    _dev(b_head, "b_head", (L, 2), f32, q_layers[0])
    _dev(modes_out, "modes_out", (L,), (torch.int32,), q_layers[0])
    if logits_out is not None:
        _dev(logits_out, "logits_out", (L, 2), f32, q_layers[0])
    _check_workspace(workspace, q_layers[0])
    if workspace is None:
        import torch
        workspace = torch.empty(flux_route_workspace_size(L, Hq, d, hidden), dtype=torch.uint8,
                                device=q_layers[0].device)
    ws_bytes = workspace.numel() * workspace.element_size()
    pq, _keep = _ptr_array(q_layers)
    _check(_lib.flux_route_layers(pq, L, S, Hq, d, _dtype_code(q_layers[0]), pool_tokens, _ptr(w_enc), _ptr(b_enc),
                                  hidden, _ptr(w_head), _ptr(b_head), _ptr(logits_out), _ptr(modes_out),
                                  _ptr(workspace), ws_bytes, _stream(stream)), "flux_route_layers")


def flux_route_soft_weights(logits, uniforms, tau: float, weights_out, stream=None):
    """Gumbel-softmax weights [L,2] (device float32) from logits [L,2] and uniforms [L,2] in (0,1)."""
    import torch
    if logits.dim() != 2 or logits.shape[1] != 2:
        raise ValueError("logits must be [n_layers, 2]")
    L = logits.shape[0]
    f32 = (torch.float32,)
    _dev(logits, "logits", (L, 2), f32)
    _dev(uniforms, "uniforms", (L, 2), f32, logits)
    _dev(weights_out, "weights_out", (L, 2), f32, logits)
    _check(_lib.flux_route_soft_weights(_ptr(logits), _ptr(uniforms), tau, L, _ptr(weights_out), _stream(stream)),
           "flux_route_soft_weights")


def flux_prefill_soft_workspace_size(batch, seq, hq, head_dim) -> int:
    return int(_lib.flux_prefill_soft_workspace_size(batch, seq, hq, head_dim))


def flux_attn_prefill_soft(q, k, v, o, weights_dev, *, block: int = 64, sink_tokens: int = 128,
                           window_tokens: int = 2048, blk_row_ptr=None, blk_col_idx=None, workspace=None,
                           scale: float | None = None, stream=None):
    """o = w[0] * dense-causal attention + w[1] * block-sparse attention; weights_dev: device float32 [2]."""
    import torch
    B, S, Hq, Hkv, d = _check_attention(q, k, v, o, None)
    _dev(weights_dev, "weights_dev", (2,), (torch.float32,), q)
    _check_csr(blk_row_ptr, blk_col_idx, S, block, q)
    _check_workspace(workspace, q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        workspace = torch.empty(flux_prefill_soft_workspace_size(B, S, Hq, d), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    nnz = int(blk_col_idx.numel()) if blk_col_idx is not None else 0
    _check(_lib.flux_attn_prefill_soft(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _dtype_code(q), _dtype_code(o), B, S, Hq,
                                       Hkv, d, scale, block, sink_tokens, window_tokens, _ptr(blk_row_ptr),
                                       _ptr(blk_col_idx), nnz, _ptr(weights_dev), _ptr(workspace), ws_bytes,
                                       _stream(stream)),
           "flux_attn_prefill_soft")


def flux_attn_backward_workspace_size(batch, seq, hq, hkv, head_dim, mode=FLUX_MODE_DENSE, block=64,
                                      sink_tokens=0) -> int:
    return int(_lib.flux_attn_backward_workspace_size(batch, seq, hq, hkv, head_dim, mode, block, sink_tokens))


def flux_attn_backward(q, k, v, o, d_o, lse, dq, dk, dv, *, causal: bool = True, mode: int = FLUX_MODE_DENSE,
                       block: int = 64, sink_tokens: int = 0, window_tokens: int = 0, scale: float | None = None,
                       workspace=None, stream=None):
    """Gradients dq, dk, dv (fp32, written) of attention for output gradient d_o; lse from the forward pass."""
    import torch
    B, S, Hq, Hkv, d = _check_attention(q, k, v, o, lse)
    if lse is None:
        raise ValueError("lse (from the forward pass) is required")
    _dev(d_o, "d_o", (B, S, Hq, d), (q.dtype,), q)
    f32 = (torch.float32,)
    _dev(dq, "dq", (B, S, Hq, d), f32, q)
    _dev(dk, "dk", (B, S, Hkv, d), f32, q)
    _dev(dv, "dv", (B, S, Hkv, d), f32, q)
    _check_workspace(workspace, q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        workspace = torch.empty(max(flux_attn_backward_workspace_size(B, S, Hq, Hkv, d, mode, block, sink_tokens), 1),
                                dtype=torch.uint8,
                                device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.flux_attn_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(lse), _ptr(dq), _ptr(dk),
                                   _ptr(dv), _dtype_code(q), _dtype_code(o), B, S, Hq, Hkv, d, scale, int(causal), mode, block,
                                   sink_tokens, window_tokens, _ptr(workspace), ws_bytes, _stream(stream)),
           "flux_attn_backward")
