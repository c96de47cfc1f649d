"""fp64 CPU oracle for exact attention — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The GPU library never imports, links or calls it, and it
shares no code with that library: the arithmetic lives in ``attn_oracle.c``
(plain C, fp64, OpenMP), and this module only marshals numpy arrays.

What is computed (see the header of ``attn_oracle.c`` for the formulas):

* ``attention_fwd``      — O and LSE of softmax(scale * Q K^T [causal]) V, the
  plain definition from the page "FlashAttention-2" (standard attention
  comparison section), layout [batch, seqlen, heads, headdim] as in that
  page's usage section; optionally restricted to a sliding window of keys
  (the local-attention variant of page "FlashAttention技术深度解析").
* ``attention_fwd_varlen`` — the same definition applied to each sequence of
  a packed batch separately, as the page "FlashAttention-2" describes for its
  variable-length function (cu_seqlens = prefix sums of the lengths).
* ``attention_bwd``      — dQ, dK, dV of a loss L with dL/dO = dout, by the
  calculus of the definition (the pages only say gradients are obtained by
  recomputation: page "Flash Attention V3" section 3.2, page
  "FlashAttention-2" backward section).
* ``attention_bwd_varlen`` — the backward of each sequence of a packed batch
  separately (the same calculus, per sequence).
* ``attention_fwd_kvcache`` — Nq new queries per sequence against keys and
  values held in a paged cache (page "FlashAttention技术深度解析": KV-cache
  decoding and the paged KV cache); query i of sequence b sits at position
  L_b - Nq + i.
* ``kvcache_append`` — writing new keys/values into the paged cache at
  positions cache_seqlens[b] .. cache_seqlens[b] + n - 1 (plain indexing).
* ``e4m3_to_f64`` — exact decoding of 8-bit floating-point (e4m3) codes, the
  inputs of the FP8 forward; FP8 attention is then ``attention_fwd`` on the
  decoded values times their per-tensor descale factors.
* ``online_softmax_merge`` — the running-max / running-sum recurrence from
  page "FlashAttention实战" section 3.1, extended with the rescale of the
  partial output that the recurrence needs to be exact.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile attn_oracle.c with gcc into liboracle.so (next to the source)."""
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-Wall", "-Werror", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class using:
    """Context manager: route the functions below through another build of
    attn_oracle.c (the mutation tests compile deliberately broken copies)."""

    def __init__(self, lib_path: str):
        self.path = lib_path

    def __enter__(self):
        global _lib
        self._saved = _lib
        _lib = _bind(ctypes.CDLL(self.path))
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self._saved
        return False


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _bind(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    lp = ctypes.POINTER(ctypes.c_int64)
    i64, f64, cint = ctypes.c_int64, ctypes.c_double, ctypes.c_int
    lib.oracle_fwd_rows.argtypes = [dp, dp, dp, i64, i64, i64, i64, f64, cint, i64, i64, lp,
                                    i64, dp, dp, cint]
    lib.oracle_bwd_rows.argtypes = [dp, dp, dp, dp, i64, i64, i64, i64, f64, cint, i64, i64,
                                    lp, i64, dp, dp, dp, cint]
    lib.oracle_bwd_cols.argtypes = [dp, dp, dp, dp, i64, i64, i64, i64, f64, cint, i64, i64,
                                    dp, dp, lp, i64, dp, dp, cint]
    lib.oracle_fwd_cache.argtypes = [dp, dp, dp, lp, lp, i64, i64, i64, i64, i64, i64, i64,
                                     f64, cint, i64, i64, dp, dp, cint]
    for f in (lib.oracle_fwd_rows, lib.oracle_bwd_rows, lib.oracle_bwd_cols,
              lib.oracle_fwd_cache):
        f.restype = cint
    lib.oracle_max_threads.restype = cint
    return lib


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16/int16) to float64."""
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3_to_f64(codes) -> np.ndarray:
    """Exact value of 8-bit floating-point codes in the OCP e4m3 format (the
    FP8 format of the FP8 attention on page "Flash Attention V3" section 2.1
    and page "FlashAttention实战" section 7; the pages do not spell it out,
    the bit layout below is the format's published definition): bit 7 sign,
    bits 6..3 exponent E with bias 7, bits 2..0 mantissa M.
      E = 0          : subnormal, (-1)^s * M/8 * 2^(1-7)
      E = 15, M = 7  : NaN (there are no infinities)
      otherwise      : normal, (-1)^s * (1 + M/8) * 2^(E-7)
    Written from those cases, with no library float8 type."""
    c = np.ascontiguousarray(codes).view(np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.ldexp(1.0, (e - 7).astype(np.int64))
    sub = (m / 8.0) * 2.0 ** -6
    v = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, v)


def _f64(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a


def _ptr(a, kind=ctypes.c_double):
    return a.ctypes.data_as(ctypes.POINTER(kind))


def _check_qkv(q, k, v):
    if q.ndim != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, N, H, d] shape")


def _window(window):
    wl, wr = (int(x) for x in window)
    if wl < -1 or wr < -1:
        raise ValueError("window sides are -1 (unbounded) or >= 0")
    return wl, wr


def _all_rows(B, N, H):
    b, h, i = np.meshgrid(np.arange(B), np.arange(H), np.arange(N), indexing="ij")
    return np.stack([b.ravel(), h.ravel(), i.ravel()], axis=1).astype(np.int64)


def attention_fwd(q, k, v, scale, causal, rows=None, threads=None, window=(-1, -1)):
    """Forward on fp64 [B, N, H, d] arrays.

    rows=None: every row; returns (o [B,N,H,d], lse [B,H,N]).
    rows = int array [n,3] of (b, h, i): returns (o_rows [n,d], lse_rows [n]).
    window = (wl, wr): row i sees keys i - wl <= j <= i + wr (-1: unbounded).
    """
    wl, wr = _window(window)
    q, k, v = _f64(q), _f64(k), _f64(v)
    _check_qkv(q, k, v)
    B, N, H, d = q.shape
    sel = _all_rows(B, N, H) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = sel.shape[0]
    o_sel = np.empty((n, d), np.float64)
    lse_sel = np.empty((n,), np.float64)
    rc = _load().oracle_fwd_rows(_ptr(q), _ptr(k), _ptr(v), B, N, H, d, float(scale),
                                 int(bool(causal)), wl, wr, _ptr(sel, ctypes.c_int64), n,
                                 _ptr(o_sel), _ptr(lse_sel), threads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_fwd_rows failed: %d" % rc)
    if rows is not None:
        return o_sel, lse_sel
    o = o_sel.reshape(B, H, N, d).transpose(0, 2, 1, 3).copy()
    lse = lse_sel.reshape(B, H, N)
    return o, lse


def attention_fwd_varlen(q, k, v, cu_seqlens, scale, causal, threads=None, window=(-1, -1)):
    """Forward on a packed batch: q, k, v are fp64 [total, H, d]; sequence s
    occupies rows cu_seqlens[s] .. cu_seqlens[s+1]-1. Each sequence is its own
    attention problem. Returns (o [total,H,d], lse [H,total])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu = [int(x) for x in np.asarray(cu_seqlens).ravel()]
    total, H, d = q.shape
    if cu[0] != 0 or cu[-1] != total or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at total")
    o = np.zeros_like(q)
    lse = np.zeros((H, total), np.float64)
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        if b == a:
            continue
        os_, ls = attention_fwd(q[a:b][None], k[a:b][None], v[a:b][None], scale, causal,
                                threads=threads, window=window)
        o[a:b] = os_[0]
        lse[:, a:b] = ls[0]
    return o, lse


def attention_bwd(q, k, v, dout, scale, causal, threads=None, window=(-1, -1)):
    """Full backward on fp64 [B,N,H,d]. Returns dict with dq, dk, dv
    ([B,N,H,d]) and the per-row lse, D ([B,H,N])."""
    wl, wr = _window(window)
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    _check_qkv(q, k, v)
    B, N, H, d = q.shape
    lib = _load()
    nt = threads or default_threads()
    sel = _all_rows(B, N, H)
    n = sel.shape[0]
    dq_sel = np.empty((n, d))
    lse = np.empty((n,))
    D = np.empty((n,))
    rc = lib.oracle_bwd_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, N, H, d, float(scale),
                             int(bool(causal)), wl, wr, _ptr(sel, ctypes.c_int64), n,
                             _ptr(dq_sel), _ptr(lse), _ptr(D), nt)
    if rc != 0:
        raise RuntimeError("oracle_bwd_rows failed: %d" % rc)
    dk_sel = np.empty((n, d))
    dv_sel = np.empty((n, d))
    rc = lib.oracle_bwd_cols(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, N, H, d, float(scale),
                             int(bool(causal)), wl, wr, _ptr(lse), _ptr(D),
                             _ptr(sel, ctypes.c_int64), n, _ptr(dk_sel), _ptr(dv_sel), nt)
    if rc != 0:
        raise RuntimeError("oracle_bwd_cols failed: %d" % rc)

    def to_bnhd(x):
        return x.reshape(B, H, N, d).transpose(0, 2, 1, 3).copy()

    return {"dq": to_bnhd(dq_sel), "dk": to_bnhd(dk_sel), "dv": to_bnhd(dv_sel),
            "lse": lse.reshape(B, H, N), "D": D.reshape(B, H, N)}


def attention_bwd_varlen(q, k, v, dout, cu_seqlens, scale, causal, threads=None,
                         window=(-1, -1)):
    """Backward on a packed batch: fp64 [total, H, d] arrays, sequence s in
    rows cu_seqlens[s] .. cu_seqlens[s+1]-1, each its own attention problem.
    Returns dict with dq, dk, dv ([total,H,d]) and lse, D ([H,total])."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    cu = [int(x) for x in np.asarray(cu_seqlens).ravel()]
    total, H, d = q.shape
    if cu[0] != 0 or cu[-1] != total or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at total")
    out = {n: np.zeros_like(q) for n in ("dq", "dk", "dv")}
    out["lse"] = np.zeros((H, total))
    out["D"] = np.zeros((H, total))
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        if b == a:
            continue
        g = attention_bwd(q[a:b][None], k[a:b][None], v[a:b][None], dout[a:b][None], scale,
                          causal, threads=threads, window=window)
        for n in ("dq", "dk", "dv"):
            out[n][a:b] = g[n][0]
        out["lse"][:, a:b] = g["lse"][0]
        out["D"][:, a:b] = g["D"][0]
    return out


def attention_bwd_sampled(q, k, v, dout, scale, causal, heads, q_rows=None, k_rows=None,
                          threads=None, window=(-1, -1)):
    """Backward on sampled outputs of full-size inputs.

    heads: list of (b, h). For each head, dq for rows q_rows (default: all)
    and dk/dv for keys k_rows (default: all). Per-row lse and D are computed
    for every row of the head first, since dk_j and dv_j sum over all rows.
    Returns {(b,h): {"rows", "dq", "keys", "dk", "dv", "lse", "D"}}.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    _check_qkv(q, k, v)
    wl, wr = _window(window)
    B, N, H, d = q.shape
    lib = _load()
    nt = threads or default_threads()
    out = {}
    lse_all = np.zeros((B, H, N))
    D_all = np.zeros((B, H, N))
    for (b, h) in heads:
        sel = np.stack([np.full(N, b), np.full(N, h), np.arange(N)], 1).astype(np.int64)
        dq = np.empty((N, d))
        lse = np.empty((N,))
        D = np.empty((N,))
        rc = lib.oracle_bwd_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, N, H, d,
                                 float(scale), int(bool(causal)), wl, wr,
                                 _ptr(sel, ctypes.c_int64), N, _ptr(dq), _ptr(lse), _ptr(D), nt)
        if rc != 0:
            raise RuntimeError("oracle_bwd_rows failed: %d" % rc)
        lse_all[b, h] = lse
        D_all[b, h] = D
        rows = np.arange(N) if q_rows is None else np.asarray(q_rows, dtype=np.int64)
        keys = np.arange(N) if k_rows is None else np.asarray(k_rows, dtype=np.int64)
        ksel = np.stack([np.full(len(keys), b), np.full(len(keys), h), keys],
                        1).astype(np.int64)
        dk = np.empty((len(keys), d))
        dv = np.empty((len(keys), d))
        rc = lib.oracle_bwd_cols(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, N, H, d,
                                 float(scale), int(bool(causal)), wl, wr, _ptr(lse_all),
                                 _ptr(D_all), _ptr(ksel, ctypes.c_int64), len(keys), _ptr(dk),
                                 _ptr(dv), nt)
        if rc != 0:
            raise RuntimeError("oracle_bwd_cols failed: %d" % rc)
        out[(b, h)] = {"rows": rows, "dq": dq[rows], "keys": keys, "dk": dk, "dv": dv,
                       "lse": lse, "D": D}
    return out


def attention_fwd_kvcache(q, k_cache, v_cache, block_table, seqlens, scale, causal,
                          window=(-1, -1), threads=None):
    """Forward of new queries against a paged key/value cache.

    q: [B, Nq, H, d]; k_cache, v_cache: [num_pages, page, H, d]; block_table:
    [B, max_pages] integer page ids; seqlens: [B] keys held per sequence
    (the new ones included). Query i of sequence b sits at position
    seqlens[b] - Nq + i. Returns (o [B, Nq, H, d], lse [B, H, Nq]); a query
    that sees no key gets o = 0 and lse = -inf.
    """
    q, kc, vc = _f64(q), _f64(k_cache), _f64(v_cache)
    if q.ndim != 4 or kc.ndim != 4 or vc.shape != kc.shape or kc.shape[2:] != q.shape[2:]:
        raise ValueError("q [B,Nq,H,d] and caches [num_pages,page,H,d] must share H, d")
    B, Nq, H, d = q.shape
    num_pages, page = kc.shape[:2]
    bt = np.ascontiguousarray(block_table, dtype=np.int64)
    sl = np.ascontiguousarray(seqlens, dtype=np.int64)
    if bt.ndim != 2 or bt.shape[0] != B or sl.shape != (B,):
        raise ValueError("block_table [B, max_pages] and seqlens [B]")
    wl, wr = _window(window)
    o = np.empty((B, Nq, H, d))
    lse = np.empty((B, H, Nq))
    rc = _load().oracle_fwd_cache(_ptr(q), _ptr(kc), _ptr(vc), _ptr(bt, ctypes.c_int64),
                                  _ptr(sl, ctypes.c_int64), B, Nq, H, d, page, bt.shape[1],
                                  num_pages, float(scale), int(bool(causal)), wl, wr, _ptr(o),
                                  _ptr(lse), threads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_fwd_cache failed: %d" % rc)
    return o, lse


def kvcache_append(k_cache, v_cache, k_new, v_new, block_table, cache_seqlens):
    """Copies of the caches with row t of k_new[b] / v_new[b] written at
    logical position cache_seqlens[b] + t of sequence b (page
    block_table[b][pos // page], slot pos % page). Works on any dtype: it
    moves values and does no arithmetic on them."""
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    page = kc.shape[1]
    for b in range(k_new.shape[0]):
        for t in range(k_new.shape[1]):
            pos = int(cache_seqlens[b]) + t
            blk = int(block_table[b][pos // page])
            kc[blk, pos % page] = k_new[b, t]
            vc[blk, pos % page] = v_new[b, t]
    return kc, vc


def online_softmax_merge(scores_row, values, tile_bounds):
    """The tiled recurrence for ONE score row, in the notation of page
    "FlashAttention实战" section 3.1 (m: running max, l: running sum of
    exponentials), plus the un-normalised output accumulator that the
    recurrence must rescale by exp(m_prev - m) whenever m changes.

    scores_row: fp64 [n] already-scaled scores of the visible keys.
    values:     fp64 [n, d] the matching value rows.
    tile_bounds: increasing cut points 0 = t0 < t1 < ... < tk = n.
    Returns (o, lse) with o = acc / l and lse = m + ln l.
    """
    m_prev, l_prev = -np.inf, 0.0
    acc = np.zeros(values.shape[1])
    for a, b in zip(tile_bounds[:-1], tile_bounds[1:]):
        x = scores_row[a:b]
        m_cur = np.max(x)
        l_cur = np.sum(np.exp(x - m_cur))
        acc_cur = np.exp(x - m_cur) @ values[a:b]
        m_new = max(m_prev, m_cur)
        a_prev = 0.0 if m_prev == -np.inf else np.exp(m_prev - m_new)
        a_cur = np.exp(m_cur - m_new)
        l_prev = a_prev * l_prev + a_cur * l_cur
        acc = a_prev * acc + a_cur * acc_cur
        m_prev = m_new
    return acc / l_prev, m_prev + np.log(l_prev)
