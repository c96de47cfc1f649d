"""Seeded synthetic inputs for attention (shared by tests, smoke and bench).

This module holds no attention arithmetic: it only draws N(0,1) tensors from a
seeded CPU generator and rounds them to bfloat16 (round-to-nearest-even, what
``Tensor.to(torch.bfloat16)`` does), so the GPU library and the CPU checker see
bit-identical values.

The shapes follow the workloads on the pages: page "FlashAttention实战"
section 6 (batch 8, 16 heads, head dim 64, sequence 1024/2048/4096), page
"FlashAttention-2" usage and benchmark sections (batch 2 or 4, 32 heads, head
dim 128, sequence 2048..16384; packed lengths 128/256/512 with cu_seqlens), all
in the [batch, seqlen, heads, headdim] layout those sections use. The pages draw
their inputs with randn as well. The sliding-window workloads (page
"FlashAttention技术深度解析", attention variants) reuse the page-4 shape
with a causal window of 4096 keys to the left. The decoding workload (page
"FlashAttention技术深度解析": KV-cache incremental decoding, paged KV cache)
keeps 16 sequences of 4096..16384 keys in 64-key pages of a shuffled pool and
decodes one new query per sequence, with the page-4 heads and head dim. The
fp16 workloads repeat the headline and backward shapes in float16, the type
the page "FlashAttention-2" uses in its usage examples. The fp8 workloads
repeat forward shapes with the same fp32 draws turned into e4m3 codes and one
descale factor per tensor (page "Flash Attention V3" section 2.1: FP8
attention).

Seed convention: 1000 * workload_group + index of the shape within the group.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import torch


@dataclass
class Workload:
    name: str
    group: int          # workload group (1..5), part of the seed
    index: int          # index of the shape within its group, part of the seed
    B: int
    N: int
    H: int
    d: int
    causal: bool
    kind: str = "fwd"   # "fwd" | "varlen" | "bwd" | "bwd_varlen" | "decode"
    lengths: Optional[List[int]] = None   # varlen: fixed lengths (None = drawn)
    nseq_random: int = 0                  # varlen: number of lengths to draw
    len_lo: int = 64
    len_hi: int = 4096
    window: Optional[Tuple[int, int]] = None  # (left, right); None = no window
    page: int = 0                         # decode: keys per cache page
    nq: int = 1                           # decode: new queries per sequence
    dtype: str = "bf16"                   # element type: "bf16" or "fp16"
    scale: float = field(default=0.0)

    def __post_init__(self):
        if self.scale == 0.0:
            self.scale = 1.0 / math.sqrt(self.d)

    @property
    def seed(self) -> int:
        return 1000 * self.group + self.index


def _wl(*a, **kw) -> Workload:
    return Workload(*a, **kw)


WORKLOADS = {}
for w in (
    _wl("tiny", 1, 0, 1, 128, 2, 64, False),
    _wl("p1_n1024", 2, 0, 8, 1024, 16, 64, True),
    _wl("p1_n2048", 2, 1, 8, 2048, 16, 64, True),
    _wl("p1_n4096", 2, 2, 8, 4096, 16, 64, True),
    _wl("p4_n2048", 3, 0, 2, 2048, 32, 128, True),
    _wl("p4_n4096", 3, 1, 2, 4096, 32, 128, True),
    _wl("p4_n8192", 3, 2, 2, 8192, 32, 128, True),
    _wl("p4_n16384", 3, 3, 2, 16384, 32, 128, True),
    _wl("p4_n2048_nc", 3, 0, 2, 2048, 32, 128, False),
    _wl("p4_n4096_nc", 3, 1, 2, 4096, 32, 128, False),
    _wl("p4_n8192_nc", 3, 2, 2, 8192, 32, 128, False),
    _wl("p4_n16384_nc", 3, 3, 2, 16384, 32, 128, False),
    _wl("headline", 3, 4, 4, 4096, 32, 128, True),
    _wl("varlen3", 4, 0, 3, 512, 32, 128, True, kind="varlen", lengths=[128, 256, 512]),
    _wl("varlen64", 4, 1, 64, 4096, 32, 128, True, kind="varlen", nseq_random=64),
    _wl("bwd_n8192", 5, 0, 2, 8192, 32, 128, True, kind="bwd"),
    _wl("bwd_varlen64", 5, 1, 64, 4096, 32, 128, True, kind="bwd_varlen", nseq_random=64),
    _wl("window_n16384", 6, 0, 2, 16384, 32, 128, True, window=(4096, 0)),
    _wl("window_bwd_n16384", 6, 0, 2, 16384, 32, 128, True, kind="bwd", window=(4096, 0)),
    _wl("decode_b16", 7, 0, 16, 16384, 32, 128, True, kind="decode", nseq_random=16,
        len_lo=4096, len_hi=16384, page=64, nq=1),
    _wl("headline_fp16", 3, 4, 4, 4096, 32, 128, True, dtype="fp16"),
    _wl("bwd_n8192_fp16", 5, 0, 2, 8192, 32, 128, True, kind="bwd", dtype="fp16"),
    _wl("d256_n8192", 8, 0, 2, 8192, 16, 256, True),
    _wl("bwd_d256_n8192", 8, 0, 2, 8192, 16, 256, True, kind="bwd"),
    _wl("bwd_p1_n4096", 2, 2, 8, 4096, 16, 64, True, kind="bwd"),
    _wl("decode_b16_d256", 8, 1, 16, 16384, 16, 256, True, kind="decode", nseq_random=16,
        len_lo=4096, len_hi=16384, page=64, nq=1),
    _wl("headline_fp8", 3, 4, 4, 4096, 32, 128, True, dtype="fp8"),
    _wl("p4_n8192_fp8", 3, 2, 2, 8192, 32, 128, True, dtype="fp8"),
    _wl("p4_n8192_nc_fp8", 3, 2, 2, 8192, 32, 128, False, dtype="fp8"),
    _wl("d256_n8192_fp8", 8, 0, 2, 8192, 16, 256, True, dtype="fp8"),
    _wl("varlen64_fp8", 4, 1, 64, 4096, 32, 128, True, kind="varlen", nseq_random=64,
        dtype="fp8"),
):
    WORKLOADS[w.name] = w


def qkv(shape, seed: int, n: int = 3, generator: Optional[torch.Generator] = None,
        dtype=torch.bfloat16):
    """Draw ``n`` fp32 N(0,1) CPU tensors of ``shape`` in order (q, k, v[, dout])
    from a generator seeded with ``seed``; return (fp32 list, list rounded to
    ``dtype``: bfloat16 or float16, nearest even)."""
    g = generator if generator is not None else torch.Generator().manual_seed(seed)
    f32 = [torch.randn(shape, generator=g, dtype=torch.float32) for _ in range(n)]
    return f32, [t.to(dtype) for t in f32]


def device_qkv(shape, seed: int, n: int = 3, device="cuda", dtype=torch.bfloat16):
    """Draw ``n`` N(0,1) tensors of ``shape`` directly on ``device`` (q, k,
    v[, dout] in order) from a generator of that device seeded with ``seed``,
    each drawn in fp32 and rounded to ``dtype`` (nearest even). For sizes whose
    host-side draw would not fit in memory; a checker copies the heads it needs
    back to the host."""
    g = torch.Generator(device=device).manual_seed(seed)
    out = []
    for _ in range(n):
        t = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
        out.append(t.to(dtype))
        del t
    return out


def varlen_lengths(w: Workload, g: torch.Generator) -> List[int]:
    if w.lengths is not None:
        return list(w.lengths)
    return [int(x) for x in torch.randint(w.len_lo, w.len_hi + 1, (w.nseq_random,),
                                          generator=g)]


def torch_dtype(w: Workload):
    return {"bf16": torch.bfloat16, "fp16": torch.float16, "fp8": torch.float8_e4m3fn}[w.dtype]


def fp8_codes(t: torch.Tensor):
    """FP8 (e4m3) codes and a per-tensor descale factor for an fp32 tensor:
    descale = max|t| / 384 (so every code stays below the format's largest
    finite value, 448) and codes = t / descale rounded to e4m3 (nearest
    even, the ``Tensor.to(torch.float8_e4m3fn)`` rounding). The real input
    of the attention is then codes * descale."""
    amax = float(t.abs().max()) if t.numel() else 1.0
    descale = (amax / 384.0) if amax > 0 else 1.0
    return (t / descale).to(torch.float8_e4m3fn), descale


def make(w: Workload, with_dout: Optional[bool] = None):
    """Inputs of a named workload as CPU tensors.

    Returns a dict with "f32" and "bf16" lists (q, k, v[, dout]; the second
    list holds the workload's element type, bfloat16 unless it says fp16); varlen
    workloads also carry "lengths", "cu_seqlens" (int32) and "max_seqlen", and
    their tensors are packed [total, H, d].
    """
    if w.kind == "decode":
        g = torch.Generator().manual_seed(w.seed)
        out = make_kvcache(varlen_lengths(w, g), w.H, w.d, w.page, w.nq, w.seed, generator=g)
        out["workload"] = w
        return out
    g = torch.Generator().manual_seed(w.seed)
    n = 4 if (w.kind.startswith("bwd") if with_dout is None else with_dout) else 3
    out = {"workload": w}
    if w.dtype == "fp8":
        # fp32 draws as for the 16-bit workloads, then e4m3 codes with one
        # descale factor per tensor (out["descale"] = [q, k, v])
        shape = (w.B, w.N, w.H, w.d)
        if w.kind == "varlen":
            lens = varlen_lengths(w, g)
            cu = [0]
            for L in lens:
                cu.append(cu[-1] + L)
            shape = (sum(lens), w.H, w.d)
            out.update(lengths=lens, cu_seqlens=torch.tensor(cu, dtype=torch.int32),
                       max_seqlen=max(lens) if lens else 0)
        f32 = [torch.randn(shape, generator=g, dtype=torch.float32) for _ in range(n)]
        codes = [fp8_codes(t) for t in f32]
        out["f32"], out["bf16"] = f32, [c for c, _ in codes]
        out["descale"] = [d for _, d in codes]
        return out
    if w.kind in ("varlen", "bwd_varlen"):
        lens = varlen_lengths(w, g)
        total = sum(lens)
        f32, b16 = qkv((total, w.H, w.d), w.seed, n, generator=g, dtype=torch_dtype(w))
        cu = [0]
        for L in lens:
            cu.append(cu[-1] + L)
        out.update(lengths=lens, cu_seqlens=torch.tensor(cu, dtype=torch.int32),
                   max_seqlen=max(lens) if lens else 0)
    else:
        f32, b16 = qkv((w.B, w.N, w.H, w.d), w.seed, n, generator=g, dtype=torch_dtype(w))
    out["f32"], out["bf16"] = f32, b16
    return out


def random_varlen(lengths: List[int], H: int, d: int, seed: int, n: int = 3):
    """Packed inputs for explicit lengths (edge cases: zero and ragged lengths)."""
    total = sum(lengths)
    f32, b16 = qkv((total, H, d), seed, n)
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + L)
    return f32, b16, torch.tensor(cu, dtype=torch.int32)


def bf16_bits(t: torch.Tensor):
    """numpy uint16 view of a bf16 CPU tensor's bit patterns."""
    return t.contiguous().view(torch.int16).numpy().view("uint16")


def make_kvcache(cache_lens: List[int], H: int, d: int, page: int, nq: int, seed: int,
                 spare_pages: int = 3, generator: Optional[torch.Generator] = None):
    """A paged key/value cache holding sequences of the given lengths plus room
    for nq new keys each, in pages handed out in a shuffled order (spare pages
    mixed in), and the new queries / keys / values.

    Returns CPU tensors: q, k_new, v_new [B, nq, H, d] bf16; k_cache, v_cache
    [num_pages, page, H, d] bf16; block_table [B, max_pages] int32 (-1 where
    a sequence has no page); cache_seqlens [B] int32 (= cache_lens)."""
    g = generator if generator is not None else torch.Generator().manual_seed(seed)
    B = len(cache_lens)
    need = [(L + nq + page - 1) // page for L in cache_lens]
    max_pages = max(need + [1])
    num_pages = sum(need) + spare_pages
    order = torch.randperm(num_pages, generator=g)
    table = torch.full((B, max_pages), -1, dtype=torch.int32)
    k = 0
    for b, n in enumerate(need):
        table[b, :n] = order[k:k + n].to(torch.int32)
        k += n
    shape_c = (num_pages, page, H, d)
    kc, vc = (torch.randn(shape_c, generator=g).to(torch.bfloat16) for _ in range(2))
    q, kn, vn = (torch.randn((B, nq, H, d), generator=g).to(torch.bfloat16) for _ in range(3))
    return {"q": q, "k_new": kn, "v_new": vn, "k_cache": kc, "v_cache": vc,
            "block_table": table, "cache_seqlens": torch.tensor(cache_lens, dtype=torch.int32),
            "lengths": list(cache_lens), "page": page, "nq": nq}