// Host-side launch interface between the C ABI layer (fa_api.cpp) and the
// kernel translation units. Arguments are validated before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Which keys a query row sees. kMaskLocal is the sliding window: row i sees
// keys j with i - wl <= j <= i + wr (a causal window has wr = 0); FwdArgs /
// BwdArgs carry wl and wr, INT_MAX for an unbounded side.
enum MaskKind : int { kMaskNone = 0, kMaskCausal = 1, kMaskLocal = 2 };

// Tensors are passed as raw 16-bit element arrays; the element type is a
// template argument of the kernels (ElemBF16 / ElemF16 in fa_device.h).
// kElemFP8 (forward only): q, k, v hold OCP e4m3 codes, o is bf16.
enum ElemKind : int { kElemBF16 = 0, kElemF16 = 1, kElemFP8 = 2 };

struct FwdArgs {
  const void *q, *k, *v;
  void *o;
  float *lse;               // may be null
  const int32_t *cu_seqlens;  // varlen only
  int N;                    // fixed-length: sequence length
  int H;
  int nseq;                 // varlen: number of sequences (total = cu_seqlens[nseq])
  int n_qtiles;             // query tiles per (sequence, head)
  int wl, wr;               // kMaskLocal: window sides (>= 0, INT_MAX = unbounded)
  float scale_log2;         // scale * log2(e) (FP8: times the q and k descale factors)
  float v_descale;          // FP8: v's descale factor, applied to O
};

struct BwdArgs {
  const void *q, *k, *v, *o, *dout;
  const float *lse;
  void *dq, *dk, *dv;
  float *delta;               // workspace: -D_i = -rowsum(dO_i * O_i), laid out like lse
  float *lse2;                // workspace: lse_i * log2(e), laid out like lse
  const int32_t *cu_seqlens;  // varlen only
  int N;                      // fixed-length: sequence length; varlen: max_seqlen
  int H;
  int nseq;                   // fixed-length: B; varlen: number of sequences
  int total;                  // rows of the [rows, H, d] tensors (B*N when fixed-length)
  int n_tiles;                // 128-row tiles per (sequence, head)
  int wl, wr;                 // kMaskLocal: window sides (>= 0, INT_MAX = unbounded)
  float scale;
  float scale_log2;
};

// Decoding against a paged key/value cache (split over the keys, then merged).
struct DecodeArgs {
  const void *q;                     // [B, Nq, H, d]
  const void *k_new, *v_new;         // [B, Nq, H, d] or null
  void *k_cache, *v_cache;           // [num_pages, page, H, d]
  const int32_t *block_table;        // [B, max_pages]
  const int32_t *cache_seqlens;      // [B]
  void *o;                           // [B, Nq, H, d]
  float *lse;                        // [B, H, Nq] or null
  float *part_o;                     // workspace: [B, Nq, nsplit, H, d]
  float *part_ml;                    // workspace: [B, Nq, nsplit, H, 2] (max * c, sum)
  int B, Nq, H;
  int num_pages, page, page_shift, max_pages;
  int n_new;                         // keys appended before attending (0 or Nq)
  int split_len, nsplit, nqc;        // keys per split, splits, query chunks
  int wl, wr;                        // window sides (INT_MAX unbounded; causal: wr = 0)
  float scale_log2;
};

int fwd_block_m(int d);  // query rows per forward workgroup
hipError_t launch_fwd(const FwdArgs &a, int n_seq, int d, MaskKind mask, bool varlen,
                      ElemKind elem, hipStream_t stream);
// The fixed-length bf16 / fp16 forward without a window (called by
// launch_fwd; defined in the FA_FWD_PLAIN compilation of fa_fwd.hip).
hipError_t launch_fwd_plain(const FwdArgs &a, int n_seq, int d, MaskKind mask, ElemKind elem,
                            hipStream_t stream);
int bwd_block();
// Size of the static device scratch array of the no-allocation backward,
// and its address on the current device (looked up once per device).
constexpr size_t kNoallocScratchBytes = size_t(16) << 20;
hipError_t noalloc_scratch(void **ptr);
hipError_t launch_bwd(const BwdArgs &a, int d, MaskKind mask, bool varlen, ElemKind elem,
                      hipStream_t stream);
int decode_queries_per_chunk();
hipError_t launch_decode(const DecodeArgs &a, int d, ElemKind elem, hipStream_t stream);

}  // namespace fa
