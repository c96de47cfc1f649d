// Forward attention kernel for gfx950.
//
// Method: the tiled exact attention of page "FlashAttention实战" (section 2
// tiling loop, section 3.1 running statistics) with the work split of page
// "FlashAttention-2" (design section: parallel over the sequence, each
// workgroup owns one block of query rows, the output is normalised once at
// the end). The running statistics per query row are the max m and the sum
// l of exponentials; the un-normalised output accumulator is multiplied by
// exp(m_old - m_new) whenever m grows, which keeps the result exact.
//
// Mapping to CDNA4:
//  * one workgroup = 4 wavefronts = BM (128) query rows of one (batch, head);
//    each wavefront owns 32 rows, so row statistics never cross wavefronts.
//  * scores are computed transposed, S^T = K Q^T, on 32x32x16 bf16 MFMA: the
//    accumulator column is the query row, so each lane holds 16 scores of one
//    row and the row max / sum need one exchange with lane l^32 only.
//  * Q stays in VGPRs (B operand) for the whole kernel; K and V tiles of BN
//    keys go through LDS, V stored transposed so that the P.V product
//    O^T = V^T P^T reads its A operand with 128-bit LDS loads and takes P
//    straight from the score accumulators (no LDS round trip for P).
//  * the key order inside a 32-key score block is permuted (bits 2 and 3 of
//    the row index swapped) so that each lane's 8 probabilities of one MFMA
//    k-step are 8 consecutive keys.
//  * softmax uses exp2 with scale*log2(e) folded into one FMA per score.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kBM = 128;  // query rows per workgroup
constexpr int kBN = 64;   // keys per iteration
constexpr int kThreads = 256;

template <int D>
struct FwdTile {
  static constexpr int KP = D + 8;    // K row pitch in LDS (bf16), padded
  static constexpr int VP = kBN + 8;  // V^T row pitch in LDS (bf16), padded
  static constexpr int CPT = kBN * D / 8 / kThreads;  // 16-byte chunks per thread
  static constexpr int TPR = D / 8;                   // threads per K/V row
};

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kThreads, 2) void fwd_kernel(FwdArgs a) {
  using T = FwdTile<D>;
  __shared__ __attribute__((aligned(16))) bf16 sK[kBN * T::KP];
  __shared__ __attribute__((aligned(16))) bf16 sV[D * T::VP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hf = lane >> 5;
  const int ln = lane & 31;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / a.n_qtiles;
  const int t = logical - bh * a.n_qtiles;
  // causal: the heaviest query tiles (most keys) are started first
  const int qt = CAUSAL ? a.n_qtiles - 1 - t : t;
  const int b = bh / a.H;
  const int h = bh - b * a.H;

  int seq0, len;
  if (VARLEN) {
    seq0 = a.cu_seqlens[b];
    len = a.cu_seqlens[b + 1] - seq0;
  } else {
    seq0 = b * a.N;
    len = a.N;
  }
  if (qt * kBM >= len) return;

  const int rs = a.H * D;  // row stride (elements)
  const size_t base = (size_t)seq0 * rs + (size_t)h * D;
  const bf16 *qg = a.q + base;
  const bf16 *kg = a.k + base;
  const bf16 *vg = a.v + base;

  // ---- Q block of this wavefront -> B operands (column = query row) ----
  const int qrow = qt * kBM + wave * 32 + ln;
  bf16x8 qr[D / 16];
  if (qrow < len) {
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc)
      qr[kc] = as_bf16x8(ld128(qg + (size_t)qrow * rs + 16 * kc + 8 * hf));
  } else {
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) qr[kc] = as_bf16x8(u32x4{0, 0, 0, 0});
  }

  const float c = a.scale_log2;  // scale * log2(e)
  float m = -INFINITY;           // running max of raw scores of this row
  float l = 0.f;                 // this lane's share of the running sum
  float lr = 0.f;                // the same sum over P rounded to bf16
  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};

  const int kv_end = CAUSAL ? min(len, (qt + 1) * kBM) : len;
  const int ntiles = (kv_end + kBN - 1) / kBN;

  // global -> register staging of one K/V tile: thread owns CPT consecutive
  // keys and one 8-element column chunk
  const int ccol = 8 * (tid % T::TPR);
  const int ckey = T::CPT * (tid / T::TPR);
  u32x4 kreg[T::CPT], vreg[T::CPT];

  auto load_tile = [&](int j) {
#pragma unroll
    for (int r = 0; r < T::CPT; ++r) {
      const int key = j * kBN + ckey + r;
      if (key < kv_end) {
        kreg[r] = ld128(kg + (size_t)key * rs + ccol);
        vreg[r] = ld128(vg + (size_t)key * rs + ccol);
      } else {
        kreg[r] = u32x4{0, 0, 0, 0};
        vreg[r] = u32x4{0, 0, 0, 0};
      }
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int r = 0; r < T::CPT; ++r) st128(&sK[(ckey + r) * T::KP + ccol], kreg[r]);
    store_transposed<T::CPT>(sV, T::VP, ccol, ckey, vreg);  // sV[col][key]
  };

  load_tile(0);
  const int krow0 = perm_row32(ln);

  for (int j = 0; j < ntiles; ++j) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (j + 1 < ntiles) load_tile(j + 1);

    // ---- S^T = K Q^T for 64 keys (two 32-key blocks) ----
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const bf16 *kp = &sK[(32 * kb + krow0) * T::KP + 8 * hf];
#pragma unroll
      for (int kc = 0; kc < D / 16; ++kc)
        s[kb] = mfma32x32x16(as_bf16x8(ld128(kp + 16 * kc)), qr[kc], s[kb]);
    }

    // ---- mask: keys past the sequence end, and keys after the row (causal)
    const int kv0 = j * kBN;
    const bool need_mask = (kv0 + kBN > len) || (CAUSAL && kv0 + kBN - 1 > qt * kBM);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kv0 + 32 * kb + perm_row32(8 * (e >> 2) + 4 * hf + (e & 3));
          if (key >= len || (CAUSAL && key > qrow)) s[kb][e] = -INFINITY;
        }
    }

    // ---- online softmax statistics ----
    float mx = s[0][0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, s[0][e]);
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[1][e]);
    mx = fmaxf(mx, swap_halves(mx));
    const float m_new = fmaxf(m, mx);
    const float ms = (m_new == -INFINITY) ? 0.f : m_new * c;
    const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m * c - ms);
    m = m_new;

    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        s[kb][e] = fast_exp2(fmaf(s[kb][e], c, -ms));
        psum += s[kb][e];
      }

    // P rounded to bf16 is the MFMA operand. Its row sum lr (of the rounded
    // values) normalises O, so the weights applied to V sum to one and the
    // rounding error of P scales with |v_j - o_i|; the sum l of the exact
    // values gives the log-sum-exp.
    bf16x8 pb[4];
    float rsum = 0.f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const f32x16 &sv = s[kk >> 1];
      const int o = 8 * (kk & 1);
      const float pv[8] = {sv[o], sv[o + 1], sv[o + 2], sv[o + 3],
                           sv[o + 4], sv[o + 5], sv[o + 6], sv[o + 7]};
      pb[kk] = pack_bf16x8_sum(pv, &rsum);
    }
    l = fmaf(l, alpha, psum);
    lr = fmaf(lr, alpha, rsum);
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc[i] *= alpha;

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) {
      const bf16 *vp = &sV[(32 * cb + ln) * T::VP + 8 * hf];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        acc[cb] = mfma32x32x16(as_bf16x8(ld128(vp + 16 * kk)), pb[kk], acc[cb]);
    }
  }

  // ---- epilogue: normalise once, store O (bf16) and the log-sum-exp ----
  const float lt = l + swap_halves(l);
  const float lrt = lr + swap_halves(lr);
  if (qrow < len) {
    const float inv = 1.f / lrt;
    bf16 *og = a.o + base + (size_t)qrow * rs;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w = {pack_bf16x2(acc[cb][4 * g] * inv, acc[cb][4 * g + 1] * inv),
                   pack_bf16x2(acc[cb][4 * g + 2] * inv, acc[cb][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2 *>(og + 32 * cb + 8 * g + 4 * hf) = w;
      }
    if (a.lse != nullptr && hf == 0) {
      const float ms = m * c;
      const size_t li = VARLEN ? (size_t)h * a.cu_seqlens[a.nseq] + seq0 + qrow
                               : ((size_t)b * a.H + h) * a.N + qrow;
      a.lse[li] = (ms + fast_log2(lt)) * kLn2;
    }
  }
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch(const FwdArgs &a, int n_seq, hipStream_t stream) {
  const long long grid = (long long)n_seq * a.H * a.n_qtiles;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  FwdArgs arg = a;
  void *params[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void *>(&fwd_kernel<D, CAUSAL, VARLEN>),
                         dim3((unsigned)grid), dim3(kThreads), params, 0, stream);
}

}  // namespace

int fwd_block_m() { return kBM; }

hipError_t launch_fwd(const FwdArgs &a, int n_seq, int d, bool causal, bool varlen,
                      hipStream_t stream) {
#define FA_CASE(DD, CC, VV) \
  if (d == DD && causal == CC && varlen == VV) return launch<DD, CC, VV>(a, n_seq, stream);
  FA_CASE(64, false, false)
  FA_CASE(64, true, false)
  FA_CASE(64, false, true)
  FA_CASE(64, true, true)
  FA_CASE(128, false, false)
  FA_CASE(128, true, false)
  FA_CASE(128, false, true)
  FA_CASE(128, true, true)
#undef FA_CASE
  return hipErrorInvalidValue;
}

}  // namespace fa
