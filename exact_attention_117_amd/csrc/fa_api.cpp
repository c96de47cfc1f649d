// C ABI of libfa.so: argument checks, launch sizing and dispatch to the
// kernels. Every check runs on the host before anything is enqueued; a
// failed check returns its status and touches no output.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "../../include/fa.h"
#include "fa_launch.h"

namespace {

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// The kernels track the maximum of the raw scores and fold scale * log2(e)
// into the exponent, which orders the scores correctly only for scale > 0.
bool valid_scale(float scale) { return std::isfinite(scale) && scale > 0.f; }

// The kernels address the rows of one sequence of one head through buffer
// resources with 32-bit byte offsets from that (sequence, head)'s first
// element, so one sequence of a [rows, H, d] tensor must stay below 4 GiB:
// len * H * d < 2^31 16-bit elements.
bool seq_span_ok(long long len, int H, int d) { return len * H * (long long)d < (1LL << 31); }

// Head dimensions with kernels: 64, 128 and 256.
fa_status check_head_dim(int d) {
  if (d <= 0) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128 && d != 256) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// Shared size checks for the fixed-length calls. Sets *empty for a no-op.
fa_status check_sizes(int B, int N, int H, int d, float scale, bool *empty) {
  if (B < 0 || N < 0 || H < 0) return FA_ERR_INVALID_ARG;
  fa_status s = check_head_dim(d);
  if (s != FA_OK) return s;
  if (!valid_scale(scale)) return FA_ERR_INVALID_ARG;
  *empty = (B == 0 || N == 0 || H == 0);
  if (*empty) return FA_OK;
  // row indices (b*N + i) and per-row element offsets stay within int range
  if ((long long)B * N > INT_MAX || (long long)H * d > INT_MAX) return FA_ERR_INVALID_ARG;
  if (!seq_span_ok(N, H, d)) return FA_ERR_INVALID_ARG;
  const long long tiles = (N + fa::fwd_block_m(d) - 1) / fa::fwd_block_m(d);
  if ((long long)B * H * tiles > INT_MAX) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

fa_status from_hip(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH; }

// Mask kind and kernel window sides for (causal, window_left, window_right):
// -1 leaves a side unbounded; causal caps the right side at the row itself.
struct Mask {
  fa::MaskKind kind;
  int wl, wr;
};
fa_status make_mask(int causal, int window_left, int window_right, Mask *m) {
  if (window_left < -1 || window_right < -1) return FA_ERR_INVALID_ARG;
  const bool left = window_left >= 0, right = window_right >= 0 && causal == 0;
  m->wl = m->wr = INT_MAX;
  if (!left && !right) {
    m->kind = causal ? fa::kMaskCausal : fa::kMaskNone;
    return FA_OK;
  }
  m->kind = fa::kMaskLocal;
  if (left) m->wl = window_left;
  m->wr = causal ? 0 : (right ? window_right : INT_MAX);
  return FA_OK;
}

// Element kind for a dtype argument (FA_ERR_INVALID_ARG for an unknown one).
// FP8 inputs have forward kernels only; the other calls reject them.
fa_status elem_kind(int dtype, fa::ElemKind *e) {
  if (dtype == FA_BF16) {
    *e = fa::kElemBF16;
    return FA_OK;
  }
  if (dtype == FA_FP16) {
    *e = fa::kElemF16;
    return FA_OK;
  }
  if (dtype == FA_FP8_E4M3) {
    *e = fa::kElemFP8;
    return FA_OK;
  }
  return FA_ERR_INVALID_ARG;
}
fa_status elem_kind_16(int dtype, fa::ElemKind *e) {
  fa_status s = elem_kind(dtype, e);
  if (s == FA_OK && *e == fa::kElemFP8) return FA_ERR_UNSUPPORTED;
  return s;
}

// FP8 inputs: head dimensions 128 and 256, descale factors finite and > 0.
// Scores are scale * q_descale * k_descale * <q_codes, k_codes>; the output
// is multiplied by v_descale.
struct Descale {
  float q = 1.f, k = 1.f, v = 1.f;
};
fa_status check_fp8(fa::ElemKind elem, int d, const Descale &ds) {
  if (elem != fa::kElemFP8) return FA_OK;
  if (!valid_scale(ds.q) || !valid_scale(ds.k) || !valid_scale(ds.v)) return FA_ERR_INVALID_ARG;
  if (d != 128 && d != 256) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

fa_status fwd_fixed(int dtype, const void *q, const void *k, const void *v, void *o, float *lse,
                    int B, int N, int H, int d, float scale, int causal, int wl, int wr,
                    void *stream, Descale ds = Descale()) {
  fa::ElemKind elem;
  if (elem_kind(dtype, &elem) != FA_OK) return FA_ERR_INVALID_ARG;
  Mask m;
  fa_status s = make_mask(causal, wl, wr, &m);
  if (s != FA_OK) return s;
  bool empty = false;
  s = check_sizes(B, N, H, d, scale, &empty);
  if (s == FA_OK) s = check_fp8(elem, d, ds);
  if (s != FA_OK || empty) return s;
  if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4))
    return FA_ERR_MISALIGNED;
  fa::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.cu_seqlens = nullptr;
  a.N = N;
  a.H = H;
  a.nseq = B;
  a.n_qtiles = (N + fa::fwd_block_m(d) - 1) / fa::fwd_block_m(d);
  a.wl = m.wl;
  a.wr = m.wr;
  a.scale_log2 = scale * ds.q * ds.k * 1.4426950408889634f;
  a.v_descale = ds.v;
  return from_hip(fa::launch_fwd(a, B, d, m.kind, false, elem, static_cast<hipStream_t>(stream)));
}

fa_status fwd_packed(int dtype, const void *q, const void *k, const void *v, void *o,
                     float *lse, const int32_t *cu_seqlens, int nseq, int max_seqlen, int H,
                     int d, float scale, int causal, int wl, int wr, void *stream,
                     Descale ds = Descale()) {
  fa::ElemKind elem;
  if (elem_kind(dtype, &elem) != FA_OK) return FA_ERR_INVALID_ARG;
  Mask m;
  fa_status s = make_mask(causal, wl, wr, &m);
  if (s != FA_OK) return s;
  if (nseq < 0 || max_seqlen < 0 || H < 0) return FA_ERR_INVALID_ARG;
  s = check_head_dim(d);
  if (s != FA_OK) return s;
  if (!valid_scale(scale)) return FA_ERR_INVALID_ARG;
  s = check_fp8(elem, d, ds);
  if (s != FA_OK) return s;
  if (nseq == 0 || max_seqlen == 0 || H == 0) return FA_OK;
  if (!q || !k || !v || !o || !cu_seqlens) return FA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4) || !aligned(cu_seqlens, 4))
    return FA_ERR_MISALIGNED;
  if ((long long)H * d > INT_MAX || !seq_span_ok(max_seqlen, H, d)) return FA_ERR_INVALID_ARG;
  const long long tiles = (max_seqlen + fa::fwd_block_m(d) - 1) / fa::fwd_block_m(d);
  if ((long long)nseq * H * tiles > INT_MAX) return FA_ERR_INVALID_ARG;
  fa::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.cu_seqlens = cu_seqlens;
  a.N = max_seqlen;
  a.H = H;
  a.nseq = nseq;
  a.n_qtiles = (int)tiles;
  a.wl = m.wl;
  a.wr = m.wr;
  a.scale_log2 = scale * ds.q * ds.k * 1.4426950408889634f;
  a.v_descale = ds.v;
  return from_hip(fa::launch_fwd(a, nseq, d, m.kind, true, elem, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

const char *fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument (null pointer, negative or overflowing size, scale not finite and positive)";
    case FA_ERR_UNSUPPORTED:
      return "unsupported head dimension or element type (64, 128 and 256 are supported; FP8 "
             "inputs: forward only, head dimension 128 or 256)";
    case FA_ERR_MISALIGNED: return "misaligned pointer (tensors need 16 bytes, float and int arrays 4)";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_SCRATCH:
      return "problem needs more scratch memory than the no-allocation entry point holds "
             "(16 MiB: 2 * B * H * N float32 values plus padding)";
  }
  return "unknown status";
}

fa_status fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int N,
                 int H, int d, float scale, int causal, void *stream) {
  return fwd_fixed(FA_BF16, q, k, v, o, lse, B, N, H, d, scale, causal, -1, -1, stream);
}

fa_status fa_fwd_window(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                        int N, int H, int d, float scale, int causal, int window_left,
                        int window_right, void *stream) {
  return fwd_fixed(FA_BF16, q, k, v, o, lse, B, N, H, d, scale, causal, window_left,
                   window_right, stream);
}

fa_status fa_fwd_varlen(const void *q, const void *k, const void *v, void *o, float *lse,
                        const int32_t *cu_seqlens, int nseq, int max_seqlen, int H, int d,
                        float scale, int causal, void *stream) {
  return fwd_packed(FA_BF16, q, k, v, o, lse, cu_seqlens, nseq, max_seqlen, H, d, scale, causal,
                    -1, -1, stream);
}

fa_status fa_fwd_varlen_window(const void *q, const void *k, const void *v, void *o, float *lse,
                               const int32_t *cu_seqlens, int nseq, int max_seqlen, int H, int d,
                               float scale, int causal, int window_left, int window_right,
                               void *stream) {
  return fwd_packed(FA_BF16, q, k, v, o, lse, cu_seqlens, nseq, max_seqlen, H, d, scale, causal,
                    window_left, window_right, stream);
}

size_t fa_bwd_workspace_size(int B, int N, int H, int d) {
  (void)d;
  if (B < 0 || N < 0 || H < 0) return 0;
  const unsigned long long rows = (unsigned long long)B * H * N;
  if (rows > (1ull << 58)) return 0;
  // D and lse * log2(e), float32 each, in two 256-byte aligned halves
  const unsigned long long half = (rows * 4 + 255) / 256 * 256;
  return (size_t)(2 * half + 256);
}

}  // extern "C"

namespace {

fa_status bwd_pointers(const void *q, const void *k, const void *v, const void *o,
                       const void *dout, const float *lse, void *dq, void *dk, void *dv,
                       void *workspace) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace)
    return FA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(workspace, 16) || !aligned(lse, 4))
    return FA_ERR_MISALIGNED;
  return FA_OK;
}

void fill_bwd(fa::BwdArgs *a, const void *q, const void *k, const void *v, const void *o,
              const void *dout, const float *lse, void *dq, void *dk, void *dv, void *workspace,
              long long stat_rows, float scale) {
  a->q = q;
  a->k = k;
  a->v = v;
  a->o = o;
  a->dout = dout;
  a->lse = lse;
  a->dq = dq;
  a->dk = dk;
  a->dv = dv;
  const size_t half = ((size_t)stat_rows * 4 + 255) / 256 * 256;
  a->delta = static_cast<float *>(workspace);
  a->lse2 = reinterpret_cast<float *>(static_cast<char *>(workspace) + half);
  a->scale = scale;
  a->scale_log2 = scale * 1.4426950408889634f;
}

fa_status bwd_fixed(int dtype, const void *q, const void *k, const void *v, const void *o,
                    const void *dout, const float *lse, void *dq, void *dk, void *dv,
                    void *workspace, int B, int N, int H, int d, float scale, int causal, int wl,
                    int wr, void *stream) {
  fa::ElemKind elem;
  {
    const fa_status es = elem_kind_16(dtype, &elem);  // FP8 has forward kernels only
    if (es != FA_OK) return es;
  }
  Mask m;
  fa_status s = make_mask(causal, wl, wr, &m);
  if (s != FA_OK) return s;
  bool empty = false;
  s = check_sizes(B, N, H, d, scale, &empty);
  if (s != FA_OK || empty) return s;
  s = bwd_pointers(q, k, v, o, dout, lse, dq, dk, dv, workspace);
  if (s != FA_OK) return s;
  fa::BwdArgs a{};
  fill_bwd(&a, q, k, v, o, dout, lse, dq, dk, dv, workspace, (long long)B * H * N, scale);
  a.cu_seqlens = nullptr;
  a.N = N;
  a.H = H;
  a.nseq = B;
  a.total = B * N;
  a.n_tiles = (N + fa::bwd_block() - 1) / fa::bwd_block();
  a.wl = m.wl;
  a.wr = m.wr;
  return from_hip(fa::launch_bwd(a, d, m.kind, false, elem, static_cast<hipStream_t>(stream)));
}

fa_status bwd_packed(int dtype, const void *q, const void *k, const void *v, const void *o,
                     const void *dout, const float *lse, void *dq, void *dk, void *dv,
                     void *workspace, const int32_t *cu_seqlens, int nseq, int max_seqlen,
                     int total, int H, int d, float scale, int causal, int wl, int wr,
                     void *stream) {
  fa::ElemKind elem;
  {
    const fa_status es = elem_kind_16(dtype, &elem);  // FP8 has forward kernels only
    if (es != FA_OK) return es;
  }
  Mask m;
  fa_status s = make_mask(causal, wl, wr, &m);
  if (s != FA_OK) return s;
  if (nseq < 0 || max_seqlen < 0 || total < 0 || H < 0) return FA_ERR_INVALID_ARG;
  s = check_head_dim(d);
  if (s != FA_OK) return s;
  if (!valid_scale(scale)) return FA_ERR_INVALID_ARG;
  if (nseq == 0 || max_seqlen == 0 || total == 0 || H == 0) return FA_OK;
  s = bwd_pointers(q, k, v, o, dout, lse, dq, dk, dv, workspace);
  if (s != FA_OK) return s;
  if (!cu_seqlens) return FA_ERR_INVALID_ARG;
  if (!aligned(cu_seqlens, 4)) return FA_ERR_MISALIGNED;
  if ((long long)H * d > INT_MAX || (long long)total * H > INT_MAX) return FA_ERR_INVALID_ARG;
  if (!seq_span_ok(max_seqlen, H, d)) return FA_ERR_INVALID_ARG;
  const long long tiles = (max_seqlen + fa::bwd_block() - 1) / fa::bwd_block();
  if ((long long)nseq * H * tiles > INT_MAX) return FA_ERR_INVALID_ARG;
  fa::BwdArgs a{};
  fill_bwd(&a, q, k, v, o, dout, lse, dq, dk, dv, workspace, (long long)H * total, scale);
  a.cu_seqlens = cu_seqlens;
  a.N = max_seqlen;
  a.H = H;
  a.nseq = nseq;
  a.total = total;
  a.n_tiles = (int)tiles;
  a.wl = m.wl;
  a.wr = m.wr;
  return from_hip(fa::launch_bwd(a, d, m.kind, true, elem, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

fa_status fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
                 const float *lse, void *dq, void *dk, void *dv, void *workspace, int B, int N,
                 int H, int d, float scale, int causal, void *stream) {
  return bwd_fixed(FA_BF16, q, k, v, o, dout, lse, dq, dk, dv, workspace, B, N, H, d, scale,
                   causal, -1, -1, stream);
}

fa_status fa_bwd_window(const void *q, const void *k, const void *v, const void *o,
                        const void *dout, const float *lse, void *dq, void *dk, void *dv,
                        void *workspace, int B, int N, int H, int d, float scale, int causal,
                        int window_left, int window_right, void *stream) {
  return bwd_fixed(FA_BF16, q, k, v, o, dout, lse, dq, dk, dv, workspace, B, N, H, d, scale,
                   causal, window_left, window_right, stream);
}

fa_status fa_bwd_varlen(const void *q, const void *k, const void *v, const void *o,
                        const void *dout, const float *lse, void *dq, void *dk, void *dv,
                        void *workspace, const int32_t *cu_seqlens, int nseq, int max_seqlen,
                        int total, int H, int d, float scale, int causal, void *stream) {
  return bwd_packed(FA_BF16, q, k, v, o, dout, lse, dq, dk, dv, workspace, cu_seqlens, nseq,
                    max_seqlen, total, H, d, scale, causal, -1, -1, stream);
}

fa_status fa_bwd_varlen_window(const void *q, const void *k, const void *v, const void *o,
                               const void *dout, const float *lse, void *dq, void *dk,
                               void *dv, void *workspace, const int32_t *cu_seqlens, int nseq,
                               int max_seqlen, int total, int H, int d, float scale, int causal,
                               int window_left, int window_right, void *stream) {
  return bwd_packed(FA_BF16, q, k, v, o, dout, lse, dq, dk, dv, workspace, cu_seqlens, nseq,
                    max_seqlen, total, H, d, scale, causal, window_left, window_right, stream);
}

// ---------------------------------------------------------------------------
// Decoding against a paged key/value cache.

fa_status fa_fwd_typed(fa_dtype dtype, const void *q, const void *k, const void *v, void *o,
                       float *lse, int B, int N, int H, int d, float scale, int causal,
                       int window_left, int window_right, void *stream) {
  return fwd_fixed(dtype, q, k, v, o, lse, B, N, H, d, scale, causal, window_left, window_right,
                   stream);
}

fa_status fa_fwd_varlen_typed(fa_dtype dtype, const void *q, const void *k, const void *v,
                              void *o, float *lse, const int32_t *cu_seqlens, int nseq,
                              int max_seqlen, int H, int d, float scale, int causal,
                              int window_left, int window_right, void *stream) {
  return fwd_packed(dtype, q, k, v, o, lse, cu_seqlens, nseq, max_seqlen, H, d, scale, causal,
                    window_left, window_right, stream);
}

fa_status fa_fwd_fp8(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                     int N, int H, int d, float scale, float q_descale, float k_descale,
                     float v_descale, int causal, int window_left, int window_right,
                     void *stream) {
  Descale ds;
  ds.q = q_descale;
  ds.k = k_descale;
  ds.v = v_descale;
  return fwd_fixed(FA_FP8_E4M3, q, k, v, o, lse, B, N, H, d, scale, causal, window_left,
                   window_right, stream, ds);
}

fa_status fa_fwd_varlen_fp8(const void *q, const void *k, const void *v, void *o, float *lse,
                            const int32_t *cu_seqlens, int nseq, int max_seqlen, int H, int d,
                            float scale, float q_descale, float k_descale, float v_descale,
                            int causal, int window_left, int window_right, void *stream) {
  Descale ds;
  ds.q = q_descale;
  ds.k = k_descale;
  ds.v = v_descale;
  return fwd_packed(FA_FP8_E4M3, q, k, v, o, lse, cu_seqlens, nseq, max_seqlen, H, d, scale,
                    causal, window_left, window_right, stream, ds);
}

fa_status fa_bwd_typed(fa_dtype dtype, const void *q, const void *k, const void *v,
                       const void *o, const void *dout, const float *lse, void *dq, void *dk,
                       void *dv, void *workspace, int B, int N, int H, int d, float scale,
                       int causal, int window_left, int window_right, void *stream) {
  return bwd_fixed(dtype, q, k, v, o, dout, lse, dq, dk, dv, workspace, B, N, H, d, scale,
                   causal, window_left, window_right, stream);
}

fa_status fa_bwd_varlen_typed(fa_dtype dtype, const void *q, const void *k, const void *v,
                              const void *o, const void *dout, const float *lse, void *dq,
                              void *dk, void *dv, void *workspace, const int32_t *cu_seqlens,
                              int nseq, int max_seqlen, int total, int H, int d, float scale,
                              int causal, int window_left, int window_right, void *stream) {
  return bwd_packed(dtype, q, k, v, o, dout, lse, dq, dk, dv, workspace, cu_seqlens, nseq,
                    max_seqlen, total, H, d, scale, causal, window_left, window_right, stream);
}

// fa_bwd_typed without a workspace argument: the D / lse*log2(e) rows go to
// the library's static device scratch array instead. Allocates nothing.
fa_status fa_bwd_noalloc(fa_dtype dtype, const void *q, const void *k, const void *v,
                         const void *o, const void *dout, const float *lse, void *dq, void *dk,
                         void *dv, int B, int N, int H, int d, float scale, int causal,
                         int window_left, int window_right, void *stream) {
  fa::ElemKind elem;
  {
    const fa_status es = elem_kind_16(dtype, &elem);  // FP8 has forward kernels only
    if (es != FA_OK) return es;
  }
  Mask m;
  fa_status s = make_mask(causal, window_left, window_right, &m);
  if (s != FA_OK) return s;
  bool empty = false;
  s = check_sizes(B, N, H, d, scale, &empty);
  if (s != FA_OK || empty) return s;
  const size_t need = fa_bwd_workspace_size(B, N, H, d);
  if (need == 0 || need > fa::kNoallocScratchBytes) return FA_ERR_SCRATCH;
  void *ws = nullptr;
  if (fa::noalloc_scratch(&ws) != hipSuccess) return FA_ERR_LAUNCH;
  return bwd_fixed(dtype, q, k, v, o, dout, lse, dq, dk, dv, ws, B, N, H, d, scale, causal,
                   window_left, window_right, stream);
}

}  // extern "C"

namespace {

// Keys per split of the decode launch: enough splits that the launch has
// about 2048 workgroups (8 per CU; 1024 at d = 256), at least 64 keys each.
// Timed on 16 sequences of 4-16 K keys: at d = 128, 1024 to 4096 workgroups
// were level to 3.5% slower than 2048; at d = 256, 1024 ran 6% faster than
// 2048 (512 +5%, 768 -8%, 1536 level).
void decode_split(int B, int Nq, int H, int d, int max_seqlen_k, int *split_len, int *nsplit) {
  const int hpw = 256 / (d / 8);
  const long long units =
      (long long)B * ((H + hpw - 1) / hpw) *
      ((Nq + fa::decode_queries_per_chunk() - 1) / fa::decode_queries_per_chunk());
  const long long target = d >= 256 ? 1024 : 2048;
  const long long want = units >= target ? 1 : (target + units - 1) / units;
  long long len = ((long long)max_seqlen_k + want - 1) / want;
  len = (len + 63) / 64 * 64;
  if (len < 64) len = 64;
  *split_len = (int)len;
  *nsplit = max_seqlen_k <= 0 ? 1 : (int)(((long long)max_seqlen_k + len - 1) / len);
}

bool decode_sizes_ok(int B, int Nq, int H, int d, int max_seqlen_k) {
  return B >= 0 && Nq >= 0 && H >= 0 && max_seqlen_k >= 0 && (d == 64 || d == 128 || d == 256);
}

}  // namespace

extern "C" {

size_t fa_fwd_kvcache_workspace_size(int B, int Nq, int H, int d, int max_seqlen_k) {
  if (!decode_sizes_ok(B, Nq, H, d, max_seqlen_k)) return 0;
  int split_len, nsplit;
  decode_split(B, Nq, H, d, max_seqlen_k, &split_len, &nsplit);
  const unsigned long long rows = (unsigned long long)B * Nq * nsplit * H;
  if (rows > (1ull << 50)) return 0;
  // partial outputs (d floats per row), then (max, sum) per row
  const unsigned long long o_bytes = (rows * d * 4 + 255) / 256 * 256;
  return (size_t)(o_bytes + rows * 8 + 256);
}

fa_status fa_fwd_kvcache_typed(fa_dtype dtype, const void *q, const void *k_new,
                               const void *v_new, void *k_cache, void *v_cache,
                               const int32_t *block_table, const int32_t *cache_seqlens, void *o,
                               float *lse, void *workspace, int B, int Nq, int H, int d,
                               int num_pages, int page_size, int max_pages, int max_seqlen_k,
                               float scale, int causal, int window_left, int window_right,
                               void *stream) {
  fa::ElemKind elem;
  {
    const fa_status es = elem_kind_16(dtype, &elem);  // FP8 has forward kernels only
    if (es != FA_OK) return es;
  }
  Mask m;
  fa_status s = make_mask(causal, window_left, window_right, &m);
  if (s != FA_OK) return s;
  if (B < 0 || Nq < 0 || H < 0 || max_seqlen_k < 0 || num_pages < 0 || max_pages < 0)
    return FA_ERR_INVALID_ARG;
  s = check_head_dim(d);
  if (s != FA_OK) return s;
  if (!valid_scale(scale)) return FA_ERR_INVALID_ARG;
  if (page_size < 1 || (page_size & (page_size - 1)) != 0) return FA_ERR_INVALID_ARG;
  if (B == 0 || Nq == 0 || H == 0) return FA_OK;
  if (num_pages < 1 || max_pages < 1) return FA_ERR_INVALID_ARG;
  if ((long long)max_pages * page_size > INT_MAX || max_seqlen_k > max_pages * page_size)
    return FA_ERR_INVALID_ARG;
  if ((long long)H * d > INT_MAX || (long long)B * Nq > INT_MAX) return FA_ERR_INVALID_ARG;
  if (!q || !k_cache || !v_cache || !block_table || !cache_seqlens || !o || !workspace)
    return FA_ERR_INVALID_ARG;
  if ((k_new == nullptr) != (v_new == nullptr)) return FA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16) ||
      !aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(workspace, 16) ||
      !aligned(lse, 4) || !aligned(block_table, 4) || !aligned(cache_seqlens, 4))
    return FA_ERR_MISALIGNED;
  fa::DecodeArgs a{};
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.cache_seqlens = cache_seqlens;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.Nq = Nq;
  a.H = H;
  a.num_pages = num_pages;
  a.page = page_size;
  a.page_shift = 0;
  while ((1 << a.page_shift) < page_size) ++a.page_shift;
  a.max_pages = max_pages;
  a.n_new = k_new ? Nq : 0;
  decode_split(B, Nq, H, d, max_seqlen_k, &a.split_len, &a.nsplit);
  const int qpc = fa::decode_queries_per_chunk();
  a.nqc = (Nq + qpc - 1) / qpc;
  a.wl = m.wl;
  a.wr = m.kind == fa::kMaskCausal ? 0 : m.wr;
  a.scale_log2 = scale * 1.4426950408889634f;
  const unsigned long long rows = (unsigned long long)B * Nq * a.nsplit * H;
  const size_t o_bytes = (size_t)((rows * d * 4 + 255) / 256 * 256);
  a.part_o = static_cast<float *>(workspace);
  a.part_ml = reinterpret_cast<float *>(static_cast<char *>(workspace) + o_bytes);
  return from_hip(fa::launch_decode(a, d, elem, static_cast<hipStream_t>(stream)));
}

fa_status fa_fwd_kvcache(const void *q, const void *k_new, const void *v_new, void *k_cache,
                         void *v_cache, const int32_t *block_table,
                         const int32_t *cache_seqlens, void *o, float *lse, void *workspace,
                         int B, int Nq, int H, int d, int num_pages, int page_size,
                         int max_pages, int max_seqlen_k, float scale, int causal,
                         int window_left, int window_right, void *stream) {
  return fa_fwd_kvcache_typed(FA_BF16, q, k_new, v_new, k_cache, v_cache, block_table,
                              cache_seqlens, o, lse, workspace, B, Nq, H, d, num_pages,
                              page_size, max_pages, max_seqlen_k, scale, causal, window_left,
                              window_right, stream);
}

}  // extern "C"
