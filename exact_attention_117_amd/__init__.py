"""Exact attention (forward, packed variable-length forward, backward by
recomputation, each also with a sliding window, and decoding against a paged
key/value cache) for AMD Instinct MI355X (gfx950).

The compute lives in ``libfa.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/fa.h``); ``exact_attention_117_amd.fa`` marshals torch
tensors into that ABI. Importing this package does not load the library; the
first call into ``fa`` does, and raises if it is missing.
"""
__all__ = ["fa_fwd", "fa_fwd_varlen", "fa_bwd", "fa_bwd_varlen", "fa_bwd_workspace_size",
           "fa_fwd_window", "fa_fwd_varlen_window", "fa_bwd_window", "fa_bwd_varlen_window",
           "fa_fwd_kvcache", "fa_fwd_kvcache_workspace_size", "fa_fwd_typed",
           "fa_fwd_varlen_typed", "fa_bwd_typed", "fa_bwd_varlen_typed", "fa_fwd_kvcache_typed",
           "fa_bwd_noalloc", "fa_fwd_fp8", "fa_fwd_varlen_fp8"]


def __getattr__(name):
    if name in __all__:
        from . import fa
        return getattr(fa, name)
    raise AttributeError(name)
