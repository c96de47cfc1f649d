/*
 * fa.h — exact attention on AMD Instinct MI355X (gfx950), C ABI of libfa.so.
 *
 * The operation is exact scaled-dot-product attention,
 *     O = softmax(scale * Q K^T [+ causal mask]) V,
 * as defined on the page "FlashAttention-2" (standard-attention comparison
 * section), computed tile by tile with the running-max / running-sum
 * recurrence of page "FlashAttention实战" section 3.1 so that the N x N score
 * matrix never reaches device memory. With causal != 0, query row i attends
 * to keys j <= i (queries and keys have the same length, so the top-left and
 * bottom-right alignments coincide). The *_window calls add the sliding
 * (local) window of page "FlashAttention技术深度解析" (attention variants):
 * row i attends to keys j with i - window_left <= j <= i + window_right.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are device pointers to contiguous bfloat16 arrays in the
 *    [batch, seqlen, heads, headdim] layout the pages use for their library
 *    calls (page "FlashAttention实战" section 4.1; page "FlashAttention-2",
 *    usage section). Row stride is H*d elements.
 *  - d (head dimension) must be 64, 128 or 256 (256 is the largest head
 *    dimension the page "FlashAttention技术深度解析" lists: cross-platform
 *    section, CUDA backend feature table). Other values return
 *    FA_ERR_UNSUPPORTED.
 *  - lse is float32, natural-log units of the scaled scores:
 *    lse[b][h][i] = log(sum_j exp(scale * <q_i, k_j>)) over visible keys j.
 *  - The caller owns every buffer. The library allocates nothing, keeps no
 *    state between calls (beyond a cache of each device's compute-unit
 *    count, which sizes the forward's persistent launches) and may be
 *    called from several host threads.
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = the null
 *    stream) and the call returns without waiting. Faults during execution
 *    surface at the caller's next synchronisation.
 *  - Arguments are checked on the host before anything is enqueued: on any
 *    error the call returns a non-zero status, launches nothing and leaves
 *    every output untouched. An empty problem (B, N, H or nseq equal to 0)
 *    returns FA_OK and launches nothing; pointers are then not inspected.
 *  - Pointers to 16-bit tensors must be 16-byte aligned, float and int32
 *    pointers 4-byte aligned (FA_ERR_MISALIGNED otherwise).
 *  - No exception crosses this boundary and the library never aborts.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v, o, dout, dq, dk, dv and the KV cache. The plain
 * calls take bfloat16; the *_typed calls take this as their first argument
 * (the page "FlashAttention-2" runs its usage examples in float16).
 * FA_FP8_E4M3: q, k and v hold 8-bit floating-point codes in the OCP e4m3
 * format (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
 * infinities; 0x7f and 0xff are NaN), the format the pages' FP8 attention
 * (page "Flash Attention V3" section 2.1, page "FlashAttention实战" section
 * 7) runs its matrix products in; o is bfloat16. Forward calls only
 * (fa_fwd_typed, fa_fwd_varlen_typed with descale factors of 1; fa_fwd_fp8,
 * fa_fwd_varlen_fp8 with explicit ones); the other calls return
 * FA_ERR_UNSUPPORTED for it. */
typedef enum { FA_BF16 = 0, FA_FP16 = 1, FA_FP8_E4M3 = 2 } fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1, /* null pointer, negative size, size overflow */
  FA_ERR_UNSUPPORTED = 2, /* head dimension other than 64, 128 or 256; FP8
                             inputs outside the forward or with d = 64 */
  FA_ERR_MISALIGNED = 3,  /* pointer alignment below what the kernels load */
  FA_ERR_LAUNCH = 4,      /* the HIP runtime refused a kernel launch */
  FA_ERR_SCRATCH = 5      /* fa_bwd_noalloc: the problem needs more scratch
                             memory than the library's static array holds */
} fa_status;

/*
 * Forward attention on a batch of equal-length sequences.
 *
 * q, k, v : [B, N, H, d] bf16, read only.
 * o       : [B, N, H, d] bf16, written (rounded to nearest even).
 * lse     : [B, H, N] float32, written; may be NULL when the caller needs no
 *           backward (the log-sum-exp is then not stored).
 * scale   : multiplier of the scores, finite and > 0 (FA_ERR_INVALID_ARG
 *           otherwise); the pages use 1/sqrt(d).
 * causal  : 0 = every key visible, non-zero = keys j <= i only.
 * Limits  : N*H*d < 2^31 elements per batch entry (one sequence of one
 *           tensor below 4 GiB); FA_ERR_INVALID_ARG otherwise.
 */
fa_status fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                 int N, int H, int d, float scale, int causal, void *stream);

/*
 * Forward attention on a packed batch of variable-length sequences, as the
 * page "FlashAttention-2" describes for its variable-length call: nseq
 * sequences stored back to back without padding.
 *
 * q, k, v    : [total, H, d] bf16, total = cu_seqlens[nseq].
 * o          : [total, H, d] bf16, written.
 * lse        : [H, total] float32, written (may be NULL).
 * cu_seqlens : device int32 [nseq + 1], exclusive prefix sums of the lengths
 *              (cu_seqlens[0] = 0, non-decreasing). Sequence s occupies rows
 *              cu_seqlens[s] .. cu_seqlens[s+1]-1 and is its own attention
 *              problem (queries and keys share these bounds). Zero-length
 *              sequences are allowed. The host never reads this array;
 *              contents that break the rules above are undefined behaviour.
 * max_seqlen : an upper bound of every length; it sizes the launch. A
 *              sequence longer than max_seqlen is taken as its first
 *              max_seqlen rows: those rows attend to those keys only, and its
 *              rows from index max_seqlen on are not written. No access then
 *              leaves the first max_seqlen rows of a sequence.
 * Limits     : max_seqlen*H*d < 2^31 elements (one sequence of one tensor
 *              below 4 GiB); FA_ERR_INVALID_ARG otherwise. The packed batch
 *              as a whole may be larger.
 * lse layout : element (h, r) at h * cu_seqlens[nseq] + r (row stride read on
 *              the device), so the packed tensors should hold exactly
 *              cu_seqlens[nseq] rows.
 */
fa_status fa_fwd_varlen(const void *q, const void *k, const void *v, void *o, float *lse,
                        const int32_t *cu_seqlens, int nseq, int max_seqlen, int H, int d,
                        float scale, int causal, void *stream);

/*
 * Sliding-window (local) forward: fa_fwd / fa_fwd_varlen where query row i
 * sees only keys j with
 *     i - window_left <= j <= i + window_right   (and j <= i if causal),
 * inside its own sequence (page "FlashAttention技术深度解析", attention
 * variants: local attention). A side given as -1 is unbounded, so
 * (-1, -1) is the plain call; causal != 0 makes window_right irrelevant.
 * Every row sees at least its own key, so every lse is finite.
 * Errors: window_left or window_right below -1 -> FA_ERR_INVALID_ARG; the
 * other arguments are checked as for fa_fwd / fa_fwd_varlen.
 */
fa_status fa_fwd_window(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                        int N, int H, int d, float scale, int causal, int window_left,
                        int window_right, void *stream);
fa_status fa_fwd_varlen_window(const void *q, const void *k, const void *v, void *o, float *lse,
                               const int32_t *cu_seqlens, int nseq, int max_seqlen, int H, int d,
                               float scale, int causal, int window_left, int window_right,
                               void *stream);

/*
 * Bytes of device workspace fa_bwd needs for these sizes: the per-row
 * -D_i = -rowsum(dO_i * O_i) and lse_i * log2(e), float32 each (2 * B*H*N
 * values), plus padding. For fa_bwd_varlen pass B = 1 and N = total.
 * Returns 0 when a size is negative or the product overflows.
 */
size_t fa_bwd_workspace_size(int B, int N, int H, int d);

/*
 * Backward of fa_fwd by recomputation (page "Flash Attention V3" section 3.2;
 * page "FlashAttention-2", backward section): the score tiles are rebuilt
 * from q, k and the saved lse, never stored.
 *
 * q, k, v, o : [B, N, H, d] bf16 — the forward's inputs and output.
 * dout       : [B, N, H, d] bf16 — dL/dO.
 * lse        : [B, H, N] float32 — the forward's saved log-sum-exp.
 * dq, dk, dv : [B, N, H, d] bf16, written (each element exactly once; the
 *              result is bit-reproducible from run to run).
 * workspace  : device memory of at least fa_bwd_workspace_size(B, N, H, d)
 *              bytes, 16-byte aligned; its contents on entry do not matter
 *              and are overwritten. Calls that share one workspace must not
 *              overlap in time.
 * scale, causal : as passed to fa_fwd.
 * Limits     : as for fa_fwd (N*H*d < 2^31 elements per batch entry).
 */
fa_status fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
                 const float *lse, void *dq, void *dk, void *dv, void *workspace, int B, int N,
                 int H, int d, float scale, int causal, void *stream);

/*
 * Backward of fa_fwd_varlen: the same gradients for a packed batch of
 * variable-length sequences (page "FlashAttention-2", variable-length and
 * backward sections), each sequence its own attention problem.
 *
 * q, k, v, o, dout : [total, H, d] bf16.
 * lse        : [H, total] float32, as fa_fwd_varlen wrote it.
 * dq, dk, dv : [total, H, d] bf16, written.
 * workspace  : at least fa_bwd_workspace_size(1, total, H, d) bytes.
 * cu_seqlens, nseq, max_seqlen : as for fa_fwd_varlen (device array, never
 *              read by the host; a sequence longer than max_seqlen is taken
 *              as its first max_seqlen rows, the gradients of its other rows
 *              are not written).
 * total      : the number of packed rows, cu_seqlens[nseq]. It sizes the
 *              workspace pass; lse and the workspace are indexed with the row
 *              stride cu_seqlens[nseq] read on the device, exactly as
 *              fa_fwd_varlen writes lse, and rows past cu_seqlens[nseq] are
 *              skipped.
 * Limits     : as for fa_fwd_varlen (max_seqlen*H*d < 2^31 elements), and
 *              total*H < 2^31.
 */
fa_status fa_bwd_varlen(const void *q, const void *k, const void *v, const void *o,
                        const void *dout, const float *lse, void *dq, void *dk, void *dv,
                        void *workspace, const int32_t *cu_seqlens, int nseq, int max_seqlen,
                        int total, int H, int d, float scale, int causal, void *stream);

/*
 * Backward of fa_fwd_window / fa_fwd_varlen_window: arguments as for
 * fa_bwd / fa_bwd_varlen plus the forward's causal, window_left and
 * window_right (same meaning, same checks). The workspace size is the same.
 */
fa_status fa_bwd_window(const void *q, const void *k, const void *v, const void *o,
                        const void *dout, const float *lse, void *dq, void *dk, void *dv,
                        void *workspace, int B, int N, int H, int d, float scale, int causal,
                        int window_left, int window_right, void *stream);
fa_status fa_bwd_varlen_window(const void *q, const void *k, const void *v, const void *o,
                               const void *dout, const float *lse, void *dq, void *dk,
                               void *dv, void *workspace, const int32_t *cu_seqlens, int nseq,
                               int max_seqlen, int total, int H, int d, float scale, int causal,
                               int window_left, int window_right, void *stream);

/*
 * Decoding against a paged key/value cache (page "FlashAttention技术深度解析":
 * causal attention with KV-cache incremental decoding; the paged KV cache
 * among its inference optimisations). Each of B sequences holds its keys and
 * values in fixed-size pages of a shared pool; its Nq newest queries attend
 * over them.
 *
 * q          : [B, Nq, H, d] bf16, the new queries.
 * k_new, v_new : [B, Nq, H, d] bf16, or both NULL. When given, they are first
 *              written into the cache at logical positions cache_seqlens[b]
 *              .. cache_seqlens[b] + Nq - 1 (their pages must already be in
 *              the block table), and the attention covers
 *              L_b = cache_seqlens[b] + Nq keys; otherwise L_b =
 *              cache_seqlens[b]. cache_seqlens itself is not changed.
 * k_cache, v_cache : [num_pages, page_size, H, d] bf16, device; written only
 *              by the append above.
 * block_table: device int32 [B, max_pages]: logical key j of sequence b is
 *              slot j % page_size of page block_table[b][j / page_size].
 *              Entries past a sequence's last page are never read. A key
 *              whose page id is outside [0, num_pages) is treated as absent.
 * cache_seqlens : device int32 [B].
 * o          : [B, Nq, H, d] bf16, written. lse : [B, H, Nq] float32 or NULL.
 * Query i of sequence b sits at position L_b - Nq + i; causal, window_left
 * and window_right apply to that position exactly as in fa_fwd_window. A
 * query that sees no key (L_b = 0, or causal with L_b < Nq) gets o = 0 and
 * lse = -inf.
 * workspace  : device memory of fa_fwd_kvcache_workspace_size(B, Nq, H, d,
 *              max_seqlen_k) bytes, 16-byte aligned, contents irrelevant;
 *              calls sharing it must not overlap in time.
 * max_seqlen_k : an upper bound of every L_b (appended keys included), at
 *              most max_pages * page_size; it sizes the launch. Keys of a
 *              longer sequence past it are not attended to.
 * Limits     : page_size a power of two; d 64, 128 or 256; scale > 0. The device
 *              arrays are not read by the host: contents that break these
 *              rules are undefined behaviour, except that out-of-range page
 *              ids and keys beyond the block table are never dereferenced.
 * Work per call: 1-4 queries are handled per workgroup on the vector ALUs
 * (the cache stream is HBM-bound); larger Nq repeats the stream per group of
 * four queries, so prefill-sized Nq belongs to fa_fwd_varlen.
 */
size_t fa_fwd_kvcache_workspace_size(int B, int Nq, int H, int d, int max_seqlen_k);
fa_status fa_fwd_kvcache(const void *q, const void *k_new, const void *v_new, void *k_cache,
                         void *v_cache, const int32_t *block_table,
                         const int32_t *cache_seqlens, void *o, float *lse, void *workspace,
                         int B, int Nq, int H, int d, int num_pages, int page_size,
                         int max_pages, int max_seqlen_k, float scale, int causal,
                         int window_left, int window_right, void *stream);

/*
 * The same calls for either element type: fa_fwd_typed, fa_fwd_varlen_typed,
 * fa_bwd_typed and fa_bwd_varlen_typed take the arguments of fa_fwd_window,
 * fa_fwd_varlen_window, fa_bwd_window and fa_bwd_varlen_window (pass -1, -1
 * for no window), fa_fwd_kvcache_typed those of fa_fwd_kvcache, each after a
 * leading dtype. Every 16-bit tensor of a call has that type; lse, the
 * workspaces and all arithmetic stay float32, and P is rounded to the
 * tensors' type where the bfloat16 path rounds it to bfloat16 (float16 keeps
 * 11 significant bits instead of 8, over a narrower range). An unknown dtype
 * returns FA_ERR_INVALID_ARG. The plain calls are the FA_BF16 case.
 * FA_FP8_E4M3 is accepted by fa_fwd_typed and fa_fwd_varlen_typed only
 * (q, k, v e4m3 codes, o bfloat16, descale factors 1: see fa_fwd_fp8); the
 * backward and decoding calls return FA_ERR_UNSUPPORTED for it.
 */
fa_status fa_fwd_typed(fa_dtype dtype, const void *q, const void *k, const void *v, void *o,
                       float *lse, int B, int N, int H, int d, float scale, int causal,
                       int window_left, int window_right, void *stream);
fa_status fa_fwd_varlen_typed(fa_dtype dtype, const void *q, const void *k, const void *v,
                              void *o, float *lse, const int32_t *cu_seqlens, int nseq,
                              int max_seqlen, int H, int d, float scale, int causal,
                              int window_left, int window_right, void *stream);
fa_status fa_bwd_typed(fa_dtype dtype, const void *q, const void *k, const void *v,
                       const void *o, const void *dout, const float *lse, void *dq, void *dk,
                       void *dv, void *workspace, int B, int N, int H, int d, float scale,
                       int causal, int window_left, int window_right, void *stream);
fa_status fa_bwd_varlen_typed(fa_dtype dtype, const void *q, const void *k, const void *v,
                              const void *o, const void *dout, const float *lse, void *dq,
                              void *dk, void *dv, void *workspace, const int32_t *cu_seqlens,
                              int nseq, int max_seqlen, int total, int H, int d, float scale,
                              int causal, int window_left, int window_right, void *stream);
fa_status fa_fwd_kvcache_typed(fa_dtype dtype, const void *q, const void *k_new,
                               const void *v_new, void *k_cache, void *v_cache,
                               const int32_t *block_table, const int32_t *cache_seqlens, void *o,
                               float *lse, void *workspace, int B, int Nq, int H, int d,
                               int num_pages, int page_size, int max_pages, int max_seqlen_k,
                               float scale, int causal, int window_left, int window_right,
                               void *stream);

/*
 * fa_bwd_typed for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments minus `workspace`. The D and lse*log2(e) rows that the
 * workspace holds in fa_bwd go to a static device array of the library, 16
 * MiB per GPU (each GPU the library runs on holds it until the process
 * ends). The call allocates nothing; the caller still passes every input
 * and output. Sizes whose fa_bwd_workspace_size(B, N, H, d) exceeds 16 MiB
 * (B*H*N above about 2 million rows) return FA_ERR_SCRATCH; other errors
 * as for fa_bwd_typed. Every call on one GPU shares that array, which keeps
 * the last call's contents (every entry a call reads it has written first):
 * calls that overlap in time on one GPU (two streams, two host threads)
 * race and must be serialised by the caller. The device is the current one
 * (hipGetDevice) at the call, which must own `stream`.
 */
fa_status fa_bwd_noalloc(fa_dtype dtype, const void *q, const void *k, const void *v,
                         const void *o, const void *dout, const float *lse, void *dq, void *dk,
                         void *dv, int B, int N, int H, int d, float scale, int causal,
                         int window_left, int window_right, void *stream);

/*
 * Forward attention on FP8 (OCP e4m3) inputs with per-tensor descale
 * factors: the real inputs are q_descale * q, k_descale * k and
 * v_descale * v (elementwise, on the decoded codes), so
 *     O = softmax(scale * q_descale * k_descale * Qc Kc^T [+ mask]) Vc * v_descale
 * with Qc, Kc, Vc the decoded codes. The pages give FP8 attention's speed
 * (page "FlashAttention实战" section 7; page "Flash Attention V3" sections
 * 2.1 and 4.2) but no scaling recipe; per-tensor factors passed by the caller
 * are the plainest one. The products Qc Kc^T run on the FP8 matrix cores
 * with float32 accumulation (exact products); V is widened exactly to
 * bfloat16 and P rounded to bfloat16 for the P.V product, as in the 16-bit
 * path; lse is float32 in the units of the real scores, o is bfloat16.
 *
 * q, k, v    : [B, N, H, d] (fa_fwd_fp8) or [total, H, d] (fa_fwd_varlen_fp8)
 *              e4m3 codes, one byte each, 16-byte aligned.
 * o, lse     : as for fa_fwd / fa_fwd_varlen (bfloat16 o; lse may be NULL).
 * d          : 128 or 256 (FA_ERR_UNSUPPORTED otherwise).
 * q_descale, k_descale, v_descale : finite and > 0 (FA_ERR_INVALID_ARG).
 * The other arguments, limits and errors are those of fa_fwd_window and
 * fa_fwd_varlen_window (window sides -1 for no window). Codes 0x7f / 0xff
 * (NaN) give NaN outputs where they are seen.
 */
fa_status fa_fwd_fp8(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                     int N, int H, int d, float scale, float q_descale, float k_descale,
                     float v_descale, int causal, int window_left, int window_right,
                     void *stream);
fa_status fa_fwd_varlen_fp8(const void *q, const void *k, const void *v, void *o, float *lse,
                            const int32_t *cu_seqlens, int nseq, int max_seqlen, int H, int d,
                            float scale, float q_descale, float k_descale, float v_descale,
                            int causal, int window_left, int window_right, void *stream);

/* Static, human-readable text for a status code. */
const char *fa_status_string(fa_status s);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
