// Backward attention kernels for gfx950: gradients by recomputation.
//
// The pages only state that the backward rebuilds the forward's tiles instead
// of storing the N x N matrix (page "Flash Attention V3" section 3.2; page
// "FlashAttention-2", backward section). The formulas are the calculus of
// O = softmax(scale * Q K^T) V with the saved per-row log-sum-exp:
//     P_ij  = exp(scale * <q_i, k_j> - lse_i)
//     dV_j  = sum_i P_ij dO_i
//     dP_ij = <dO_i, v_j>
//     D_i   = sum_j P_ij dP_ij = <dO_i, O_i>
//     dS_ij = P_ij (dP_ij - D_i)
//     dQ_i  = scale * sum_j dS_ij k_j
//     dK_j  = scale * sum_i dS_ij q_i
//
// Three launches on the caller's stream, no atomics, every output element
// written once (bit-reproducible):
//   pre_kernel  : D_i = <dO_i, O_i> in fp32 (a streaming pass over O and dO);
//   dkdv_kernel : one workgroup per (batch, head, 128 keys); each wavefront
//                 keeps 32 keys' K and V in VGPRs and their dK, dV in MFMA
//                 accumulators, and streams 64-row Q / dO tiles through LDS;
//   dq_kernel   : one workgroup per (batch, head, 128 query rows); each
//                 wavefront keeps 32 rows' Q, dO in VGPRs and dQ in
//                 accumulators, and streams 64-key K / V tiles through LDS.
// Recomputing P in both gradient kernels costs two extra matmuls per tile
// pair (seven instead of five) and removes every cross-workgroup reduction.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// D_i = <dO_i, O_i>, written to delta[b][h][i].
template <int D>
__global__ __launch_bounds__(kThreads) void pre_kernel(const bf16 *__restrict__ o,
                                                       const bf16 *__restrict__ dout,
                                                       float *__restrict__ delta, int N, int H,
                                                       long long nrows) {
  constexpr int TPR = D / 8;  // threads per [b, i, h] row (16-byte chunks)
  const long long t = (long long)blockIdx.x * kThreads + threadIdx.x;
  const long long row = t / TPR;
  const int chunk = (int)(t % TPR);
  float s = 0.f;
  if (row < nrows) {
    const u32x4 x = ld128(o + row * D + chunk * 8);
    const u32x4 y = ld128(dout + row * D + chunk * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      s = fmaf(bf16_lo(x[w]), bf16_lo(y[w]), s);
      s = fmaf(bf16_hi(x[w]), bf16_hi(y[w]), s);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  if (row < nrows && chunk == 0) {
    const int h = (int)(row % H);
    const long long bi = row / H;
    const int i = (int)(bi % N);
    const long long b = bi / N;
    delta[(b * H + h) * N + i] = s;
  }
}

// ---------------------------------------------------------------------------
// dK, dV for 128 keys per workgroup.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void dkdv_kernel(BwdArgs a, int n_ktiles) {
  constexpr int BKV = 128;             // keys per workgroup (4 wavefronts x 32)
  constexpr int BQ = 64;               // query rows per iteration
  constexpr int RP = D + 8;            // row-major tile pitch (bf16)
  constexpr int TP = BQ + 8;           // transposed tile pitch (bf16)
  constexpr int CPT = BQ * D / 8 / kThreads;  // staged rows per thread
  constexpr int TPR = D / 8;
  __shared__ __attribute__((aligned(16))) bf16 sQ[BQ * RP];
  __shared__ __attribute__((aligned(16))) bf16 sdO[BQ * RP];
  __shared__ __attribute__((aligned(16))) bf16 sQt[D * TP];
  __shared__ __attribute__((aligned(16))) bf16 sdOt[D * TP];
  __shared__ __attribute__((aligned(16))) float sL[BQ];   // lse_i * log2(e)
  __shared__ __attribute__((aligned(16))) float sDv[BQ];  // D_i

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, ln = lane & 31;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / n_ktiles;
  const int kt = logical - bh * n_ktiles;  // causal: low kt sees the most rows, runs first
  const int b = bh / a.H, h = bh - b * a.H;
  const int N = a.N, rs = a.H * D;
  const size_t base = (size_t)b * N * rs + (size_t)h * D;
  const float *lse = a.lse + ((size_t)b * a.H + h) * N;
  const float *dlt = a.delta + ((size_t)b * a.H + h) * N;

  // this lane's key: K and V rows as B operands (column = key)
  const int key = kt * BKV + wave * 32 + ln;
  bf16x8 kr[D / 16], vr[D / 16];
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) {
    if (key < N) {
      kr[kc] = as_bf16x8(ld128(a.k + base + (size_t)key * rs + 16 * kc + 8 * hf));
      vr[kc] = as_bf16x8(ld128(a.v + base + (size_t)key * rs + 16 * kc + 8 * hf));
    } else {
      kr[kc] = as_bf16x8(u32x4{0, 0, 0, 0});
      vr[kc] = as_bf16x8(u32x4{0, 0, 0, 0});
    }
  }
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }

  const int n_qt = (N + BQ - 1) / BQ;
  const int qt_begin = CAUSAL ? (kt * BKV) / BQ : 0;
  const float c = a.scale_log2;

  const int ccol = 8 * (tid % TPR), crow = CPT * (tid / TPR);
  u32x4 qreg[CPT], oreg[CPT];
  float lreg = 0.f, dreg = 0.f;
  auto load_tile = [&](int qt) {
#pragma unroll
    for (int r = 0; r < CPT; ++r) {
      const int row = qt * BQ + crow + r;
      if (row < N) {
        qreg[r] = ld128(a.q + base + (size_t)row * rs + ccol);
        oreg[r] = ld128(a.dout + base + (size_t)row * rs + ccol);
      } else {
        qreg[r] = u32x4{0, 0, 0, 0};
        oreg[r] = u32x4{0, 0, 0, 0};
      }
    }
    if (tid < BQ) {
      const int row = qt * BQ + tid;
      // rows past the end get lse = +inf, so their P (and dS) is exactly 0
      lreg = row < N ? lse[row] * kLog2e : INFINITY;
      dreg = row < N ? dlt[row] : 0.f;
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int r = 0; r < CPT; ++r) {
      st128(&sQ[(crow + r) * RP + ccol], qreg[r]);
      st128(&sdO[(crow + r) * RP + ccol], oreg[r]);
    }
    store_transposed<CPT>(sQt, TP, ccol, crow, qreg);
    store_transposed<CPT>(sdOt, TP, ccol, crow, oreg);
    if (tid < BQ) {
      sL[tid] = lreg;
      sDv[tid] = dreg;
    }
  };

  if (qt_begin < n_qt) load_tile(qt_begin);
  const int prow = perm_row32(ln);
  for (int qt = qt_begin; qt < n_qt; ++qt) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (qt + 1 < n_qt) load_tile(qt + 1);
    const int q0 = qt * BQ;

    // S = Q K^T and dP = dO V^T for two 32-row blocks (rows permuted)
    f32x16 s[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      s[qb] = f32x16{};
      dp[qb] = f32x16{};
      const bf16 *qp = &sQ[(32 * qb + prow) * RP + 8 * hf];
      const bf16 *op = &sdO[(32 * qb + prow) * RP + 8 * hf];
#pragma unroll
      for (int kc = 0; kc < D / 16; ++kc) {
        s[qb] = mfma32x32x16(as_bf16x8(ld128(qp + 16 * kc)), kr[kc], s[qb]);
        dp[qb] = mfma32x32x16(as_bf16x8(ld128(op + 16 * kc)), vr[kc], dp[qb]);
      }
    }

    // P = exp(S*scale - lse), dS = P (dP - D); causal: P = 0 for key > row
    const bool need_mask = CAUSAL && (kt * BKV + BKV - 1 > q0);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int rb = 32 * qb + perm_row32(8 * g + 4 * hf);  // 4 consecutive rows
        const f32x4 L = *reinterpret_cast<const f32x4 *>(&sL[rb]);
        const f32x4 Dd = *reinterpret_cast<const f32x4 *>(&sDv[rb]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = 4 * g + r;
          float p = fast_exp2(fmaf(s[qb][e], c, -L[r]));
          if (need_mask && key > q0 + rb + r) p = 0.f;
          s[qb][e] = p;
          dp[qb][e] = p * (dp[qb][e] - Dd[r]);
        }
      }

    // dV^T += dO^T P and dK^T += Q^T dS, 16 rows per k-step
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const f32x16 &sv = s[kk >> 1];
      const f32x16 &dv_ = dp[kk >> 1];
      const int o = 8 * (kk & 1);
      const bf16x8 pb = as_bf16x8(u32x4{pack_bf16x2(sv[o], sv[o + 1]),
                                        pack_bf16x2(sv[o + 2], sv[o + 3]),
                                        pack_bf16x2(sv[o + 4], sv[o + 5]),
                                        pack_bf16x2(sv[o + 6], sv[o + 7])});
      const bf16x8 db = as_bf16x8(u32x4{pack_bf16x2(dv_[o], dv_[o + 1]),
                                        pack_bf16x2(dv_[o + 2], dv_[o + 3]),
                                        pack_bf16x2(dv_[o + 4], dv_[o + 5]),
                                        pack_bf16x2(dv_[o + 6], dv_[o + 7])});
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) {
        dv[cb] = mfma32x32x16(as_bf16x8(ld128(&sdOt[(32 * cb + ln) * TP + 16 * kk + 8 * hf])),
                              pb, dv[cb]);
        dk[cb] = mfma32x32x16(as_bf16x8(ld128(&sQt[(32 * cb + ln) * TP + 16 * kk + 8 * hf])),
                              db, dk[cb]);
      }
    }
  }

  // lane holds dV^T[32cb + 8g + 4h + r][key] -> dV[key][32cb + 8g + 4h .. +3]
  if (key < N) {
    bf16 *dkg = a.dk + base + (size_t)key * rs;
    bf16 *dvg = a.dv + base + (size_t)key * rs;
    const float sc = a.scale;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * cb + 8 * g + 4 * hf;
        *reinterpret_cast<u32x2 *>(dvg + col) =
            u32x2{pack_bf16x2(dv[cb][4 * g], dv[cb][4 * g + 1]),
                  pack_bf16x2(dv[cb][4 * g + 2], dv[cb][4 * g + 3])};
        *reinterpret_cast<u32x2 *>(dkg + col) =
            u32x2{pack_bf16x2(dk[cb][4 * g] * sc, dk[cb][4 * g + 1] * sc),
                  pack_bf16x2(dk[cb][4 * g + 2] * sc, dk[cb][4 * g + 3] * sc)};
      }
  }
}

// ---------------------------------------------------------------------------
// dQ for 128 query rows per workgroup.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void dq_kernel(BwdArgs a, int n_qtiles) {
  constexpr int BM = 128;               // query rows per workgroup
  constexpr int BN = 64;                // keys per iteration
  constexpr int RP = D + 8;
  constexpr int TP = BN + 8;
  constexpr int CPT = BN * D / 8 / kThreads;
  constexpr int TPR = D / 8;
  __shared__ __attribute__((aligned(16))) bf16 sK[BN * RP];
  __shared__ __attribute__((aligned(16))) bf16 sV[BN * RP];
  __shared__ __attribute__((aligned(16))) bf16 sKt[D * TP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, ln = lane & 31;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / n_qtiles;
  const int t = logical - bh * n_qtiles;
  const int qt = CAUSAL ? n_qtiles - 1 - t : t;
  const int b = bh / a.H, h = bh - b * a.H;
  const int N = a.N, rs = a.H * D;
  const size_t base = (size_t)b * N * rs + (size_t)h * D;

  // this lane's query row: Q and dO rows as B operands (column = row)
  const int qrow = qt * BM + wave * 32 + ln;
  bf16x8 qr[D / 16], dor[D / 16];
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) {
    if (qrow < N) {
      qr[kc] = as_bf16x8(ld128(a.q + base + (size_t)qrow * rs + 16 * kc + 8 * hf));
      dor[kc] = as_bf16x8(ld128(a.dout + base + (size_t)qrow * rs + 16 * kc + 8 * hf));
    } else {
      qr[kc] = as_bf16x8(u32x4{0, 0, 0, 0});
      dor[kc] = as_bf16x8(u32x4{0, 0, 0, 0});
    }
  }
  const size_t ri = ((size_t)b * a.H + h) * N + qrow;
  const float l2 = qrow < N ? a.lse[ri] * kLog2e : 0.f;
  const float Dr = qrow < N ? a.delta[ri] : 0.f;
  f32x16 dq[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dq[i] = f32x16{};

  const int kv_end = CAUSAL ? min(N, (qt + 1) * BM) : N;
  const int ntiles = (kv_end + BN - 1) / BN;
  const float c = a.scale_log2;

  const int ccol = 8 * (tid % TPR), ckey = CPT * (tid / TPR);
  u32x4 kreg[CPT], vreg[CPT];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int r = 0; r < CPT; ++r) {
      const int kk = j * BN + ckey + r;
      if (kk < kv_end) {
        kreg[r] = ld128(a.k + base + (size_t)kk * rs + ccol);
        vreg[r] = ld128(a.v + base + (size_t)kk * rs + ccol);
      } else {
        kreg[r] = u32x4{0, 0, 0, 0};
        vreg[r] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int r = 0; r < CPT; ++r) {
      st128(&sK[(ckey + r) * RP + ccol], kreg[r]);
      st128(&sV[(ckey + r) * RP + ccol], vreg[r]);
    }
    store_transposed<CPT>(sKt, TP, ccol, ckey, kreg);
  };

  if (ntiles > 0) load_tile(0);
  const int prow = perm_row32(ln);
  for (int j = 0; j < ntiles; ++j) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (j + 1 < ntiles) load_tile(j + 1);

    // S^T = K Q^T and dP^T = V dO^T (keys permuted within 32-key blocks)
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      dp[kb] = f32x16{};
      const bf16 *kp = &sK[(32 * kb + prow) * RP + 8 * hf];
      const bf16 *vp = &sV[(32 * kb + prow) * RP + 8 * hf];
#pragma unroll
      for (int kc = 0; kc < D / 16; ++kc) {
        s[kb] = mfma32x32x16(as_bf16x8(ld128(kp + 16 * kc)), qr[kc], s[kb]);
        dp[kb] = mfma32x32x16(as_bf16x8(ld128(vp + 16 * kc)), dor[kc], dp[kb]);
      }
    }

    const int kv0 = j * BN;
    const bool need_mask = (kv0 + BN > N) || (CAUSAL && kv0 + BN - 1 > qt * BM);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float p = fast_exp2(fmaf(s[kb][e], c, -l2));
        if (need_mask) {
          const int kk = kv0 + 32 * kb + perm_row32(8 * (e >> 2) + 4 * hf + (e & 3));
          if (kk >= N || (CAUSAL && kk > qrow)) p = 0.f;
        }
        dp[kb][e] = p * (dp[kb][e] - Dr);
      }

    // dQ^T += K^T dS^T, 16 keys per k-step
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const f32x16 &dv_ = dp[kk >> 1];
      const int o = 8 * (kk & 1);
      const bf16x8 db = as_bf16x8(u32x4{pack_bf16x2(dv_[o], dv_[o + 1]),
                                        pack_bf16x2(dv_[o + 2], dv_[o + 3]),
                                        pack_bf16x2(dv_[o + 4], dv_[o + 5]),
                                        pack_bf16x2(dv_[o + 6], dv_[o + 7])});
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb)
        dq[cb] = mfma32x32x16(as_bf16x8(ld128(&sKt[(32 * cb + ln) * TP + 16 * kk + 8 * hf])),
                              db, dq[cb]);
    }
  }

  if (qrow < N) {
    bf16 *dqg = a.dq + base + (size_t)qrow * rs;
    const float sc = a.scale;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<u32x2 *>(dqg + 32 * cb + 8 * g + 4 * hf) =
            u32x2{pack_bf16x2(dq[cb][4 * g] * sc, dq[cb][4 * g + 1] * sc),
                  pack_bf16x2(dq[cb][4 * g + 2] * sc, dq[cb][4 * g + 3] * sc)};
  }
}

template <typename Arg>
hipError_t launch1(const void *fn, long long grid, Arg &arg, int extra, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  void *params[] = {&arg, &extra};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kThreads), params, 0, stream);
}

template <int D, bool CAUSAL>
hipError_t launch_all(const BwdArgs &a0, hipStream_t stream) {
  BwdArgs a = a0;
  const long long nrows = (long long)a.B * a.N * a.H;
  {
    const bf16 *o = a.o, *dout = a.dout;
    float *delta = a.delta;
    int N = a.N, H = a.H;
    long long nr = nrows;
    void *params[] = {&o, &dout, &delta, &N, &H, &nr};
    const long long grid = (nrows * (D / 8) + kThreads - 1) / kThreads;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&pre_kernel<D>),
                                   dim3((unsigned)grid), dim3(kThreads), params, 0, stream);
    if (e != hipSuccess) return e;
  }
  const int n_kt = (a.N + 127) / 128;
  hipError_t e = launch1(reinterpret_cast<const void *>(&dkdv_kernel<D, CAUSAL>),
                         (long long)a.B * a.H * n_kt, a, n_kt, stream);
  if (e != hipSuccess) return e;
  const int n_qt = (a.N + 127) / 128;
  return launch1(reinterpret_cast<const void *>(&dq_kernel<D, CAUSAL>),
                 (long long)a.B * a.H * n_qt, a, n_qt, stream);
}

}  // namespace

hipError_t launch_bwd(const BwdArgs &a, int d, bool causal, hipStream_t stream) {
  if (d == 64) return causal ? launch_all<64, true>(a, stream) : launch_all<64, false>(a, stream);
  if (d == 128)
    return causal ? launch_all<128, true>(a, stream) : launch_all<128, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
