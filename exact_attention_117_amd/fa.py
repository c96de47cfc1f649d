"""Python binding of libfa.so: marshals torch tensors into the C ABI declared
in include/fa.h. Tensors may be bfloat16 or float16 (one type per call): the
plain calls take bfloat16, and float16 goes through the *_typed calls. No arithmetic of the method happens here; torch only provides
device memory and the current stream. If libfa.so is missing this module
raises on import: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

# FA_LIBRARY names another build of the library (the timing build,
# libfa_trace.so, for `bench.py --trace-phases`); by default libfa.so here.
_LIB_PATH = os.environ.get("FA_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libfa.so")

if not os.path.exists(_LIB_PATH):
    raise ImportError("libfa.so is not built (run __graft_entry__.build() or "
                      "python -m exact_attention_117_amd.build): " + _LIB_PATH)

lib = ctypes.CDLL(_LIB_PATH)
_vp, _i, _f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
lib.fa_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp]
lib.fa_fwd.restype = _i
lib.fa_fwd_varlen.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp]
lib.fa_fwd_varlen.restype = _i
lib.fa_bwd_workspace_size.argtypes = [_i, _i, _i, _i]
lib.fa_bwd_workspace_size.restype = ctypes.c_size_t
lib.fa_bwd.argtypes = [_vp] * 10 + [_i, _i, _i, _i, _f, _i, _vp]
lib.fa_bwd.restype = _i
lib.fa_bwd_varlen.argtypes = [_vp] * 11 + [_i, _i, _i, _i, _i, _f, _i, _vp]
lib.fa_bwd_varlen.restype = _i
lib.fa_fwd_window.argtypes = lib.fa_fwd.argtypes[:-1] + [_i, _i, _vp]
lib.fa_fwd_window.restype = _i
lib.fa_fwd_varlen_window.argtypes = lib.fa_fwd_varlen.argtypes[:-1] + [_i, _i, _vp]
lib.fa_fwd_varlen_window.restype = _i
lib.fa_bwd_window.argtypes = lib.fa_bwd.argtypes[:-1] + [_i, _i, _vp]
lib.fa_bwd_window.restype = _i
lib.fa_bwd_varlen_window.argtypes = lib.fa_bwd_varlen.argtypes[:-1] + [_i, _i, _vp]
lib.fa_bwd_varlen_window.restype = _i
lib.fa_fwd_kvcache_workspace_size.argtypes = [_i] * 5
lib.fa_fwd_kvcache_workspace_size.restype = ctypes.c_size_t
lib.fa_fwd_kvcache.argtypes = [_vp] * 10 + [_i] * 8 + [_f, _i, _i, _i, _vp]
lib.fa_fwd_kvcache.restype = _i
lib.fa_fwd_typed.argtypes = [_i] + lib.fa_fwd_window.argtypes
lib.fa_fwd_typed.restype = _i
lib.fa_fwd_varlen_typed.argtypes = [_i] + lib.fa_fwd_varlen_window.argtypes
lib.fa_fwd_varlen_typed.restype = _i
lib.fa_bwd_typed.argtypes = [_i] + lib.fa_bwd_window.argtypes
lib.fa_bwd_typed.restype = _i
lib.fa_bwd_varlen_typed.argtypes = [_i] + lib.fa_bwd_varlen_window.argtypes
lib.fa_bwd_varlen_typed.restype = _i
lib.fa_fwd_kvcache_typed.argtypes = [_i] + lib.fa_fwd_kvcache.argtypes
lib.fa_fwd_kvcache_typed.restype = _i
lib.fa_fwd_fp8.argtypes = [_vp] * 5 + [_i] * 4 + [_f] * 4 + [_i, _i, _i, _vp]
lib.fa_fwd_fp8.restype = _i
lib.fa_fwd_varlen_fp8.argtypes = [_vp] * 6 + [_i] * 4 + [_f] * 4 + [_i, _i, _i, _vp]
lib.fa_fwd_varlen_fp8.restype = _i
lib.fa_bwd_noalloc.argtypes = [_i] + [_vp] * 9 + [_i, _i, _i, _i, _f, _i, _i, _i, _vp]
lib.fa_bwd_noalloc.restype = _i
lib.fa_status_string.argtypes = [_i]
lib.fa_status_string.restype = ctypes.c_char_p

EXPORTS = ("fa_fwd", "fa_fwd_varlen", "fa_bwd", "fa_bwd_varlen", "fa_bwd_workspace_size",
           "fa_fwd_window", "fa_fwd_varlen_window", "fa_bwd_window", "fa_bwd_varlen_window",
           "fa_fwd_kvcache", "fa_fwd_kvcache_workspace_size", "fa_fwd_typed",
           "fa_fwd_varlen_typed", "fa_bwd_typed", "fa_bwd_varlen_typed", "fa_fwd_kvcache_typed",
           "fa_bwd_noalloc", "fa_fwd_fp8", "fa_fwd_varlen_fp8", "fa_status_string")

# element types (fa_dtype in include/fa.h)
FA_BF16, FA_FP16, FA_FP8_E4M3 = 0, 1, 2
_DTYPES = {torch.bfloat16: FA_BF16, torch.float16: FA_FP16}


class FaError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__("libfa: %s (status %d)" % (lib.fa_status_string(status).decode(),
                                                    status))


def _check(status: int):
    if status != 0:
        raise FaError(status)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _bf16(name, t, shape=None, dtype=None):
    """Checks a 16-bit device tensor: bfloat16 or float16, equal to `dtype`
    when given (all tensors of a call share one element type)."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a device tensor" % name)
    if t.dtype not in _DTYPES or (dtype is not None and t.dtype != dtype):
        raise TypeError("%s must be %s" % (name, dtype or "bfloat16 or float16"))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def _window_call(window, plain, windowed, args, tail, dtype=torch.bfloat16, typed=None,
                 force_typed=False):
    """Calls the plain (bfloat16) entry point, its *_window variant with the two
    window sides inserted before the stream argument, or for float16 (or when
    asked) the *_typed variant (dtype first, window sides as for *_window)."""
    if dtype != torch.bfloat16 or force_typed:
        wl, wr = (-1, -1) if window is None else (int(x) for x in window)
        return typed(_DTYPES[dtype], *args, *tail[:-1], wl, wr, tail[-1])
    if window is None:
        return plain(*args, *tail)
    wl, wr = (int(x) for x in window)
    return windowed(*args, *tail[:-1], wl, wr, tail[-1])


def fa_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: Optional[float] = None,
           causal: bool = False, o: Optional[torch.Tensor] = None,
           lse: Optional[torch.Tensor] = None, need_lse: bool = True, window=None,
           _typed: bool = False) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """O, LSE = attention(q, k, v) on [B, N, H, d] bf16 device tensors.
    Returns (o [B,N,H,d] bf16, lse [B,H,N] fp32 or None). window =
    (left, right) calls fa_fwd_window instead."""
    _bf16("q", q)
    if q.dim() != 4:
        raise ValueError("q must be [B, N, H, d]")
    B, N, H, d = q.shape
    _bf16("k", k, q.shape, q.dtype)
    _bf16("v", v, q.shape, q.dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty_like(q)
    _bf16("o", o, q.shape, q.dtype)
    if lse is None and need_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N)
                            or not lse.is_contiguous()):
        raise ValueError("lse must be contiguous float32 [B, H, N]")
    _check(_window_call(window, lib.fa_fwd, lib.fa_fwd_window,
                        (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, N, H, d,
                         float(scale)), (int(bool(causal)), _stream(q.device)), q.dtype,
                        lib.fa_fwd_typed, _typed))
    return o, lse


def _fp8(name, t, shape=None):
    """Checks an e4m3 code tensor: torch.float8_e4m3fn (or uint8 codes) on the
    device, contiguous."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a device tensor" % name)
    if t.dtype not in (torch.float8_e4m3fn, torch.uint8):
        raise TypeError("%s must hold e4m3 codes (torch.float8_e4m3fn or uint8)" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def fa_fwd_fp8(q, k, v, q_descale: float = 1.0, k_descale: float = 1.0, v_descale: float = 1.0,
               scale: Optional[float] = None, causal: bool = False, o=None, lse=None,
               need_lse: bool = True, window=None):
    """Forward on FP8 (e4m3) [B, N, H, d] inputs with per-tensor descale
    factors (real values = codes * descale). Returns (o [B,N,H,d] bf16,
    lse [B,H,N] fp32 or None)."""
    _fp8("q", q)
    if q.dim() != 4:
        raise ValueError("q must be [B, N, H, d]")
    B, N, H, d = q.shape
    _fp8("k", k, q.shape)
    _fp8("v", v, q.shape)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    _bf16("o", o, q.shape, torch.bfloat16)
    if lse is None and need_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N)
                            or not lse.is_contiguous()):
        raise ValueError("lse must be contiguous float32 [B, H, N]")
    wl, wr = (-1, -1) if window is None else (int(x) for x in window)
    _check(lib.fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, N, H, d,
                          float(scale), float(q_descale), float(k_descale), float(v_descale),
                          int(bool(causal)), wl, wr, _stream(q.device)))
    return o, lse


def fa_fwd_varlen_fp8(q, k, v, cu_seqlens, max_seqlen: int, q_descale: float = 1.0,
                      k_descale: float = 1.0, v_descale: float = 1.0,
                      scale: Optional[float] = None, causal: bool = False, o=None, lse=None,
                      need_lse: bool = True, window=None):
    """Packed variable-length forward on FP8 [total, H, d] inputs (see
    fa_fwd_fp8 and fa_fwd_varlen). Returns (o [total,H,d] bf16, lse [H,total])."""
    _fp8("q", q)
    if q.dim() != 3:
        raise ValueError("q must be [total, H, d]")
    total, H, d = q.shape
    _fp8("k", k, q.shape)
    _fp8("v", v, q.shape)
    if (not cu_seqlens.is_cuda or cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1
            or not cu_seqlens.is_contiguous()):
        raise ValueError("cu_seqlens must be a contiguous int32 device vector")
    nseq = cu_seqlens.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    _bf16("o", o, q.shape, torch.bfloat16)
    if lse is None and need_lse:
        lse = torch.empty((H, total), dtype=torch.float32, device=q.device)
    wl, wr = (-1, -1) if window is None else (int(x) for x in window)
    _check(lib.fa_fwd_varlen_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens),
                                 nseq, int(max_seqlen), H, d, float(scale), float(q_descale),
                                 float(k_descale), float(v_descale), int(bool(causal)), wl, wr,
                                 _stream(q.device)))
    return o, lse


def fa_fwd_window(q, k, v, window_left: int = -1, window_right: int = -1, **kw):
    """Sliding-window forward: row i sees keys i - window_left .. i +
    window_right (-1: unbounded side). Other arguments as for fa_fwd."""
    return fa_fwd(q, k, v, window=(window_left, window_right), **kw)


def fa_fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  cu_seqlens: torch.Tensor, max_seqlen: int, scale: Optional[float] = None,
                  causal: bool = False, o: Optional[torch.Tensor] = None,
                  lse: Optional[torch.Tensor] = None, need_lse: bool = True, window=None,
                  _typed: bool = False):
    """Packed variable-length forward: q, k, v [total, H, d] bf16, cu_seqlens
    int32 [nseq+1] on the device. Returns (o [total,H,d], lse [H,total]).
    total must equal cu_seqlens[-1] (the kernels index lse with that row
    stride; it is not read back here, which would synchronise)."""
    _bf16("q", q)
    if q.dim() != 3:
        raise ValueError("q must be [total, H, d]")
    total, H, d = q.shape
    _bf16("k", k, q.shape, q.dtype)
    _bf16("v", v, q.shape, q.dtype)
    if (not cu_seqlens.is_cuda or cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1
            or not cu_seqlens.is_contiguous()):
        raise ValueError("cu_seqlens must be a contiguous int32 device vector")
    nseq = cu_seqlens.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty_like(q)
    _bf16("o", o, q.shape, q.dtype)
    if lse is None and need_lse:
        lse = torch.empty((H, total), dtype=torch.float32, device=q.device)
    _check(_window_call(window, lib.fa_fwd_varlen, lib.fa_fwd_varlen_window,
                        (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens),
                         nseq, int(max_seqlen), H, d, float(scale)),
                        (int(bool(causal)), _stream(q.device)), q.dtype,
                        lib.fa_fwd_varlen_typed, _typed))
    return o, lse


def fa_fwd_varlen_window(q, k, v, cu_seqlens, max_seqlen: int, window_left: int = -1,
                         window_right: int = -1, **kw):
    """Sliding-window packed forward (see fa_fwd_window, fa_fwd_varlen)."""
    return fa_fwd_varlen(q, k, v, cu_seqlens, max_seqlen, window=(window_left, window_right),
                         **kw)


def fa_bwd_workspace_size(B: int, N: int, H: int, d: int) -> int:
    return int(lib.fa_bwd_workspace_size(B, N, H, d))


def fa_bwd(q, k, v, o, dout, lse, scale: Optional[float] = None, causal: bool = False,
           dq=None, dk=None, dv=None, workspace=None, window=None, _typed: bool = False):
    """dQ, dK, dV of attention by recomputation from the saved lse."""
    _bf16("q", q)
    B, N, H, d = q.shape
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        _bf16(name, t, q.shape, q.dtype)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H, N]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _bf16(name, t, q.shape, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(fa_bwd_workspace_size(B, N, H, d), 16), dtype=torch.uint8,
                                device=q.device)
    _check(_window_call(window, lib.fa_bwd, lib.fa_bwd_window,
                        (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                         _ptr(dk), _ptr(dv), _ptr(workspace), B, N, H, d, float(scale)),
                        (int(bool(causal)), _stream(q.device)), q.dtype, lib.fa_bwd_typed,
                        _typed))
    return dq, dk, dv


def fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, scale: Optional[float] = None,
                   causal: bool = False, window=None):
    """fa_bwd for callers that cannot allocate: the library's static device
    scratch array replaces the workspace. Every output is passed in; nothing
    is allocated here either. Raises FaError (FA_ERR_SCRATCH) when the
    problem needs more scratch than the array holds."""
    _bf16("q", q)
    B, N, H, d = q.shape
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk),
                    ("dv", dv)):
        _bf16(name, t, q.shape, q.dtype)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H, N]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    wl, wr = (-1, -1) if window is None else (int(x) for x in window)
    _check(lib.fa_bwd_noalloc(_DTYPES[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                              _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), B, N, H, d,
                              float(scale), int(bool(causal)), wl, wr, _stream(q.device)))
    return dq, dk, dv


def fa_bwd_window(q, k, v, o, dout, lse, window_left: int = -1, window_right: int = -1, **kw):
    """Backward of fa_fwd_window (same window)."""
    return fa_bwd(q, k, v, o, dout, lse, window=(window_left, window_right), **kw)


def fa_bwd_varlen(q, k, v, o, dout, lse, cu_seqlens, max_seqlen: int,
                  scale: Optional[float] = None, causal: bool = False, dq=None, dk=None, dv=None,
                  workspace=None, window=None, _typed: bool = False):
    """dQ, dK, dV of fa_fwd_varlen: packed [total, H, d] bf16 tensors, lse
    [H, total] fp32 and the same cu_seqlens / max_seqlen as the forward;
    total must equal cu_seqlens[-1], as for fa_fwd_varlen."""
    _bf16("q", q)
    if q.dim() != 3:
        raise ValueError("q must be [total, H, d]")
    total, H, d = q.shape
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        _bf16(name, t, q.shape, q.dtype)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (H, total) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [H, total]")
    if (not cu_seqlens.is_cuda or cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1
            or not cu_seqlens.is_contiguous()):
        raise ValueError("cu_seqlens must be a contiguous int32 device vector")
    nseq = cu_seqlens.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _bf16(name, t, q.shape, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(fa_bwd_workspace_size(1, total, H, d), 16),
                                dtype=torch.uint8, device=q.device)
    _check(_window_call(window, lib.fa_bwd_varlen, lib.fa_bwd_varlen_window,
                        (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                         _ptr(dk), _ptr(dv), _ptr(workspace), _ptr(cu_seqlens), nseq,
                         int(max_seqlen), total, H, d, float(scale)),
                        (int(bool(causal)), _stream(q.device)), q.dtype,
                        lib.fa_bwd_varlen_typed, _typed))
    return dq, dk, dv


def fa_bwd_varlen_window(q, k, v, o, dout, lse, cu_seqlens, max_seqlen: int,
                         window_left: int = -1, window_right: int = -1, **kw):
    """Backward of fa_fwd_varlen_window (same window)."""
    return fa_bwd_varlen(q, k, v, o, dout, lse, cu_seqlens, max_seqlen,
                         window=(window_left, window_right), **kw)


def fa_fwd_kvcache_workspace_size(B: int, Nq: int, H: int, d: int, max_seqlen_k: int) -> int:
    return int(lib.fa_fwd_kvcache_workspace_size(B, Nq, H, d, max_seqlen_k))


def _i32_vector(name, t, n=None):
    if (not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.int32
            or not t.is_contiguous() or (n is not None and t.numel() != n)):
        raise ValueError("%s must be a contiguous int32 device tensor%s" % (
            name, "" if n is None else " of %d elements" % n))


def fa_fwd_kvcache(q, k_cache, v_cache, block_table, cache_seqlens, max_seqlen_k: int,
                   k_new=None, v_new=None, scale: Optional[float] = None, causal: bool = True,
                   window=(-1, -1), o=None, lse=None, need_lse: bool = True, workspace=None,
                   _typed: bool = False):
    """Attention of the newest queries against a paged key/value cache.

    q [B, Nq, H, d] bf16; k_cache, v_cache [num_pages, page_size, H, d] bf16;
    block_table [B, max_pages] int32; cache_seqlens [B] int32 (all on the
    device). With k_new / v_new [B, Nq, H, d], they are written into the cache
    at positions cache_seqlens[b] .. + Nq - 1 first (cache_seqlens is not
    updated). Returns (o [B, Nq, H, d], lse [B, H, Nq] or None)."""
    _bf16("q", q)
    if q.dim() != 4:
        raise ValueError("q must be [B, Nq, H, d]")
    B, Nq, H, d = q.shape
    _bf16("k_cache", k_cache, None, q.dtype)
    if k_cache.dim() != 4 or tuple(k_cache.shape[2:]) != (H, d):
        raise ValueError("k_cache must be [num_pages, page_size, H, d]")
    _bf16("v_cache", v_cache, k_cache.shape, q.dtype)
    num_pages, page_size = k_cache.shape[:2]
    _i32_vector("block_table", block_table)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages]")
    _i32_vector("cache_seqlens", cache_seqlens, B)
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None:
        _bf16("k_new", k_new, q.shape, q.dtype)
        _bf16("v_new", v_new, q.shape, q.dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q) if o is None else o
    _bf16("o", o, q.shape, q.dtype)
    if lse is None and need_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(
            max(fa_fwd_kvcache_workspace_size(B, Nq, H, d, int(max_seqlen_k)), 16),
            dtype=torch.uint8, device=q.device)
    wl, wr = (int(x) for x in window)
    args = (_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
            _ptr(cache_seqlens), _ptr(o), _ptr(lse), _ptr(workspace), B, Nq, H, d, num_pages,
            page_size, block_table.shape[1], int(max_seqlen_k), float(scale), int(bool(causal)),
            wl, wr, _stream(q.device))
    if q.dtype == torch.bfloat16 and not _typed:
        _check(lib.fa_fwd_kvcache(*args))
    else:
        _check(lib.fa_fwd_kvcache_typed(_DTYPES[q.dtype], *args))
    return o, lse


# The *_typed entry points by name (the element type comes from the tensors).
def fa_fwd_typed(q, k, v, window_left: int = -1, window_right: int = -1, **kw):
    return fa_fwd(q, k, v, window=(window_left, window_right), _typed=True, **kw)


def fa_fwd_varlen_typed(q, k, v, cu_seqlens, max_seqlen, window_left=-1, window_right=-1, **kw):
    return fa_fwd_varlen(q, k, v, cu_seqlens, max_seqlen, window=(window_left, window_right),
                         _typed=True, **kw)


def fa_bwd_typed(q, k, v, o, dout, lse, window_left=-1, window_right=-1, **kw):
    return fa_bwd(q, k, v, o, dout, lse, window=(window_left, window_right), _typed=True, **kw)


def fa_bwd_varlen_typed(q, k, v, o, dout, lse, cu_seqlens, max_seqlen, window_left=-1,
                        window_right=-1, **kw):
    return fa_bwd_varlen(q, k, v, o, dout, lse, cu_seqlens, max_seqlen,
                         window=(window_left, window_right), _typed=True, **kw)


def fa_fwd_kvcache_typed(*a, **kw):
    return fa_fwd_kvcache(*a, _typed=True, **kw)
