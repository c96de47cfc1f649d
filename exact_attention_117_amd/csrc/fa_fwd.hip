// Forward attention kernel for gfx950.
//
// Method: the tiled exact attention of page "FlashAttention实战" (section 2
// tiling loop, section 3.1 running statistics) with the work split of page
// "FlashAttention-2" (design section: parallel over the sequence, each
// workgroup owns one block of query rows, the output is normalised once at
// the end). Per query row the kernel keeps a running max m and a running sum
// l of exponentials; the un-normalised output accumulator is multiplied by
// exp(m_old - m_new) when m is raised, which keeps the result exact.
//
// Mapping to CDNA4:
//  * one workgroup = 4 wavefronts = BM (128) query rows of one (batch, head);
//    each wavefront owns 32 rows, so row statistics never cross wavefronts.
//  * scores are computed transposed, S^T = K Q^T, on 32x32x16 bf16 MFMA: the
//    accumulator column is the query row, so a lane holds 16 scores of one row
//    per 32-key block and row reductions need one exchange with lane l^32.
//  * Q stays in VGPRs (B operand) for the whole kernel. K and V tiles of BN
//    keys are copied row-major into LDS by direct global-to-LDS loads, double
//    buffered (one barrier per tile); the copy of tile j+1 overlaps the math
//    of tile j. The P.V product O^T = V^T P^T reads its A operand with the
//    transposing LDS read and takes P straight from the score accumulators.
//  * the key order inside a 32-key score block is permuted (perm_row32) so a
//    lane's 8 probabilities of one MFMA k-step are 8 consecutive keys.
//  * softmax uses exp2 with scale*log2(e) folded into one FMA per score. The
//    running max used for the exponentials is only raised when the true max
//    exceeds it by more than 2^8 (in exp2 units 8): until then P may reach
//    256, which bf16 and the fp32 sums hold as well as values below 1, and
//    the O rescale (one multiply per accumulator) is skipped. The result is
//    the same up to rounding.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kBM = 128;  // query rows per workgroup
constexpr int kBN = 64;   // keys per iteration
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kRescaleLog2 = 8.f;  // lazy rescale threshold (exp2 units)

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kThreads, 2) void fwd_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(1024))) bf16 sK[2][kBN * D];
  __shared__ __attribute__((aligned(1024))) bf16 sV[2][kBN * D];

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
  const int row0 = qt * kBM + wave * 32;  // first row of this wavefront
  const int qrow = row0 + ln;
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
  float m = -INFINITY;           // max of raw scores the exponentials are taken against
  float l = 0.f;                 // this lane's share of the sum of exponentials
  float lr = 0.f;                // the same sum over P rounded to bf16
  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};

  const int kv_end = CAUSAL ? min(len, (qt + 1) * kBM) : len;
  const int ntiles = (kv_end + kBN - 1) / kBN;
  const bool wave_live = row0 < len;

  load_tile_to_lds<D, kBN, kWaves>(sK[0], kg, rs, 0, kv_end - 1, wave, lane);
  load_tile_to_lds<D, kBN, kWaves>(sV[0], vg, rs, 0, kv_end - 1, wave, lane);

  const int krow = perm_row32(ln);
  // transposing-read coordinates of this lane (see the V^T operand below)
  const int tg = lane >> 4, ts = lane & 15;
  const int tr_row = 8 * (tg >> 1) + (ts >> 2);
  const int tr_col = 16 * (tg & 1) + 4 * (ts & 3);

  for (int j = 0; j < ntiles; ++j) {
    wait_vmem();
    __syncthreads();  // tile j is in LDS; every wavefront is done with tile j-1
    if (j + 1 < ntiles) {
      load_tile_to_lds<D, kBN, kWaves>(sK[(j + 1) & 1], kg, rs, (j + 1) * kBN, kv_end - 1,
                                       wave, lane);
      load_tile_to_lds<D, kBN, kWaves>(sV[(j + 1) & 1], vg, rs, (j + 1) * kBN, kv_end - 1,
                                       wave, lane);
    }
    const int kv0 = j * kBN;
    // a wavefront skips tiles whose keys all lie after its last row (causal)
    if (!wave_live || (CAUSAL && kv0 > row0 + 31)) continue;
    const bf16 *tK = sK[j & 1];
    const bf16 *tV = sV[j & 1];

    // ---- S^T = K Q^T for 64 keys (two 32-key blocks) ----
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int kc = 0; kc < D / 16; ++kc)
        s[kb] = mfma32x32x16(
            as_bf16x8(ld128(&tK[tile_off<D>(32 * kb + krow, 16 * kc + 8 * hf)])), qr[kc],
            s[kb]);
    }

    // ---- mask: keys past the sequence end, and keys after the row (causal)
    const bool need_mask = (kv0 + kBN > len) || (CAUSAL && kv0 + kBN - 1 > row0);
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
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int e = 2; e < 16; e += 2) mx = fmaxf(mx, fmaxf(s[0][e], s[0][e + 1]));
#pragma unroll
    for (int e = 0; e < 16; e += 2) mx = fmaxf(mx, fmaxf(s[1][e], s[1][e + 1]));
    mx = fmaxf(mx, swap_halves(mx));
    const float m_new = fmaxf(m, mx);
    // raise m (and rescale) only when the new max exceeds it by > 2^8; false
    // while the row has seen no visible key (both -inf), true at its first one
    if (__any((m_new - m) * c > kRescaleLog2)) {
      const float alpha = (m == -INFINITY) ? 0.f : fast_exp2((m - m_new) * c);
      l *= alpha;
      lr *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i) acc[i] *= alpha;
      m = m_new;
    }
    const float ms = (m == -INFINITY) ? 0.f : m * c;

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
    // rounding error of P scales with |v_j - o_i|; the sum l of the unrounded
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
    l += psum;
    lr += rsum;

    // ---- O^T += V^T P^T ----
    // A operand of k-step kk, block cb: lane (m = l % 32, h = l / 32) needs
    // V[16kk + 8h + t][32cb + m], t = 0..7: two transposing reads of 4 keys.
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) {
        const int r0 = 16 * kk + tr_row, c0 = 32 * cb + tr_col;
        const u32x2 lo = ds_read_tr16x4(&tV[tile_off<D>(r0, c0)]);
        const u32x2 hi = ds_read_tr16x4(&tV[tile_off<D>(r0 + 4, c0)]);
        acc[cb] = mfma32x32x16(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), pb[kk], acc[cb]);
      }
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
      const size_t li = VARLEN ? (size_t)h * a.cu_seqlens[a.nseq] + seq0 + qrow
                               : ((size_t)b * a.H + h) * a.N + qrow;
      a.lse[li] = (m * c + fast_log2(lt)) * kLn2;
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
