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
//   pre_kernel  : -D_i = -<dO_i, O_i> and lse_i * log2(e), fp32, into the
//                 workspace (a streaming pass over O and dO; -D seeds the
//                 dK/dV kernel's dP accumulators, so dP - D comes out of the
//                 MFMAs);
//   dkdv_kernel : one workgroup per (sequence, head, 128 keys); each
//                 wavefront keeps 32 keys' K and V in VGPRs and their dK, dV
//                 in MFMA accumulators, and streams 32-row Q / dO tiles (with
//                 their lse and D) through LDS. For d = 256 two workgroups
//                 share a key tile, each owning half of dK's and dV's columns
//                 (both recompute S and dP): K, V and the full accumulators
//                 would not fit one lane's 512 registers;
//   dq_kernel   : one workgroup per (sequence, head, 128 query rows); each
//                 wavefront keeps 32 rows' Q and dO in VGPRs and dQ in
//                 accumulators, and streams 64-key K / V tiles (32-key for
//                 d = 256, within the LDS) through LDS. At d = 128 two
//                 wavefronts share each 32-row group, one per half of every
//                 tile, and sum their partial dQ at the end. A window's key
//                 tiles are streamed in a rotated order, so the workgroups of
//                 a head read the same tile at the same time.
// Recomputing P in both gradient kernels costs two extra matmuls per tile
// pair (seven instead of five) and removes every cross-workgroup reduction.
//
// Both gradient kernels follow the forward kernel's layout on CDNA4: tiles
// are copied row-major into 4-slot LDS rings by direct buffer-to-LDS loads,
// started two to three tiles ahead; products over d read row fragments
// (ds_read_b128) and products over the streamed rows read transposed
// fragments (ds_read_b64_tr_b16) of the same tile. Each tile j runs in two
// fenced phases: the score-side products (S, dP) of tile j+1 on the matrix
// cores beside the exponentials and dS of tile j on the vector ALUs, then
// the gradient products of tile j beside packing P and dS to bf16.
#include <mutex>
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

// Timing build (FA_BWD_TRACE, in a separate library; the product library has
// none of this): every wavefront of the first kTraceGroups workgroups of
// each gradient kernel records six shader-clock stamps per iteration for its
// first iterations: loop top, after its copy wait, after the barrier, after
// starting the copies, after phase 1 and after phase 2 (both 0 if it skips
// the tile). Every iteration of every wavefront ends with exactly one store
// instruction (lanes 0..5, one stamp each; to a sink outside the recorded
// range; one more before the loop), which counts in the vector-memory
// counter like the tile copies: the copy waits allow it (kTraceStores), so a
// wavefront never waits for its own record.
#ifdef FA_BWD_TRACE
constexpr int kTraceGroups = 256, kTraceDkdv = 260, kTraceDq = 160, kTraceStores = 1;
__device__ unsigned long long g_dkdv_trace[kTraceGroups * 4 * kTraceDkdv * 6];
__device__ unsigned long long g_dq_trace[kTraceGroups * 8 * kTraceDq * 6];
__device__ unsigned long long g_trace_sink[kTraceGroups * 8 * 6];
__device__ __forceinline__ unsigned long long trace_clock() {
  __builtin_amdgcn_sched_barrier(0);
  const unsigned long long t = __builtin_amdgcn_s_memtime();
  __builtin_amdgcn_sched_barrier(0);
  return t;
}
// one 8-byte store per lane 0..5: a single instruction
__device__ __forceinline__ void trace_store(unsigned long long *g, int lane, unsigned long long a,
                                            unsigned long long b, unsigned long long c,
                                            unsigned long long d, unsigned long long e,
                                            unsigned long long f) {
  const unsigned long long v =
      lane == 0 ? a : lane == 1 ? b : lane == 2 ? c : lane == 3 ? d : lane == 4 ? e : f;
  if (lane < 6) g[lane] = v;
}
#define FA_TRACE_STAMP(v) const unsigned long long v = trace_clock()
#define FA_TRACE_DECL unsigned long long trace_t2 = 0
#define FA_TRACE_MID trace_t2 = trace_clock()
#define FA_TRACE_RECORD(buf, W, IT, j, t0, ta, tb, tc, t3)                             \
  do {                                                                                \
    const size_t slot_ = (size_t)(blockIdx.x % kTraceGroups) * (W) + wave;            \
    trace_store((j) < (IT) && blockIdx.x < kTraceGroups                               \
                    ? (buf) + (slot_ * (IT) + (j)) * 6                                \
                    : g_trace_sink + slot_ * 6,                                       \
                lane, t0, ta, tb, tc, (t3) ? trace_t2 : 0, t3);                       \
    trace_t2 = 0;                                                                     \
  } while (0)
// one record store before the loop, so a copy wait always has exactly one
// record younger than the copies it waits for
#define FA_TRACE_PRIME(W) \
  trace_store(g_trace_sink + ((size_t)(blockIdx.x % kTraceGroups) * (W) + wave) * 6, lane, 0, 0, 0, 0, 0, 0)
#else
constexpr int kTraceStores = 0;
#define FA_TRACE_PRIME(W)
#define FA_TRACE_STAMP(v)
#define FA_TRACE_DECL
#define FA_TRACE_MID
#define FA_TRACE_RECORD(buf, W, IT, j, t0, ta, tb, tc, t3)
#endif

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBR = 128;     // keys (dK/dV) or query rows (dQ) per workgroup
// rows of a streamed K / V tile of the dQ kernel: two 32-key score blocks,
// one for d = 256 (four-slot rings of 64 x 256 would exceed the LDS)
template <int D>
constexpr int dq_blocks() { return D == 256 ? 1 : 2; }
// Wavefronts per SIMD the gradient kernels are compiled for. At d = 64 both
// fit 256 VGPRs, so two workgroups share a CU (their LDS rings take 33 and
// 64 KiB) and each SIMD interleaves two wavefronts: 52% faster than one at
// B4 N4096 H16 causal. At d >= 128 the K, V operands and dK, dV accumulators
// (or Q, dO and dQ) need more than 256 VGPRs: one wavefront per SIMD. (dQ
// with 32-key tiles fits 256 at d = 128 but ran 8% slower.)
template <int D>
constexpr int bwd_waves_per_simd() { return D == 64 ? 2 : 1; }
constexpr int kStages = 4;   // ring slots; iteration j reads tiles j and j+1
// Workgroups per XCD that work_order groups its units for. dK/dV: 256
// (measured on the causal backward: 32, 128, 256, 512 gave 685, 694, 696, 681
// TFLOP/s at B2 N8192 H32 d128 and 407, 436, 438, 438 at B4 N4096 H16 d64;
// 64, i.e. one head per XCD at a time, fetched 1.03 GB instead of 1.48 GB
// but ran 2.5% slower). dQ: 64, one head's query tiles per XCD at a time, so
// they stream the same K / V rows together: 0.83 GB fetched instead of
// 1.49 GB for 0.6% more time (both A/B on one box at B2 N8192 H32 d128).
constexpr int kGroupSlots = 256;
constexpr int kGroupSlotsDq = 64;
constexpr int PF = 3;        // LDS fragment prefetch distance (MFMAs)

// ---------------------------------------------------------------------------
// D_i = <dO_i, O_i> and lse_i * log2(e), both laid out like lse.
template <int D, bool VARLEN, class E>
__global__ __launch_bounds__(kThreads) void pre_kernel(BwdArgs a, long long nrows) {
  using Et = typename E::T;
  constexpr int TPR = D / 8;  // threads per [row, h] (16-byte chunks)
  const long long t = (long long)blockIdx.x * kThreads + threadIdx.x;
  const long long row = t / TPR;  // (packed row, head) pair: row = r * H + h
  const int chunk = (int)(t % TPR);
  float s = 0.f;
  if (row < nrows) {
    const u32x4 x = ld128(static_cast<const Et *>(a.o) + row * D + chunk * 8);
    const u32x4 y = ld128(static_cast<const Et *>(a.dout) + row * D + chunk * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      s = fmaf(E::lo(x[w]), E::lo(y[w]), s);
      s = fmaf(E::hi(x[w]), E::hi(y[w]), s);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  if (row < nrows && chunk == 0) {
    const int h = (int)(row % a.H);
    const long long r = row / a.H;  // packed row
    size_t idx;
    if (VARLEN) {
      const int packed = a.cu_seqlens[a.nseq];  // lse row stride
      if (r >= packed) return;                  // spare rows past the last sequence
      idx = (size_t)h * packed + r;
    } else {
      const long long b = r / a.N, i = r % a.N;
      idx = ((size_t)b * a.H + h) * a.N + i;
    }
    a.delta[idx] = -s;  // -D
    a.lse2[idx] = a.lse[idx] * kLog2e;
  }
}

// Per-(sequence, head) context shared by the gradient kernels.
template <int D, bool VARLEN>
struct Seq {
  int b, h, seq0, len;
  size_t base;   // element offset of (row 0, head h) in the [rows, H, d] tensors
  size_t stat0;  // offset of row 0 of (b, h) in the lse-like arrays
  __device__ Seq(const BwdArgs &a, int bh) {
    b = bh / a.H;
    h = bh - b * a.H;
    if (VARLEN) {
      // a sequence longer than max_seqlen (a.N) is taken as its first a.N
      // rows, as in the forward; lse and the workspace have row stride
      // cu_seqlens[nseq], as the forward writes lse
      seq0 = a.cu_seqlens[b];
      len = min(a.cu_seqlens[b + 1] - seq0, a.N);
      stat0 = (size_t)h * a.cu_seqlens[a.nseq] + seq0;
    } else {
      seq0 = b * a.N;
      len = a.N;
      stat0 = ((size_t)b * a.H + h) * a.N;
    }
    base = (size_t)seq0 * a.H * D + (size_t)h * D;
  }
};

// Copies of ROWS x D tiles of one [rows, H, d] tensor into swizzled LDS
// tiles (the forward's layout): this wavefront's kInsts 16-byte lanes.
template <int D, class E, int ROWS, int NW = kWaves>
struct TileCopier {
  static constexpr int kInsts = ROWS * D / 512 / NW;
  uint32_t goff[kInsts];
  int rs, wave, lane;
  __device__ TileCopier(int rs_, int wave_, int lane_) : rs(rs_), wave(wave_), lane(lane_) {
#pragma unroll
    for (int i = 0; i < kInsts; ++i) {
      const int e = (wave * kInsts + i) * 512 + 8 * lane;
      const int row = e / D;
      const int lch = ((e % D) >> 3) ^ chunk_swizzle<D>(row);
      goff[i] = (uint32_t)(row * rs + 8 * lch) * 2u;
    }
  }
  // rows row0 .. row0+ROWS-1 of the tensor; rows at or past `end` re-read
  // row end-1
  __device__ void issue(typename E::T *lds, u32x4 src, int row0, int end) const {
    const uint32_t soff = (uint32_t)row0 * (uint32_t)rs * 2u;
    const uint32_t dst = lds_address(lds) + (uint32_t)(wave * kInsts * 1024);
    if (row0 + ROWS <= end) {
#pragma unroll
      for (int i = 0; i < kInsts; ++i) load_lds16_at(src, dst + i * 1024, goff[i], soff);
    } else {
#pragma unroll
      for (int i = 0; i < kInsts; ++i) {
        const int e = (wave * kInsts + i) * 512 + 8 * lane;
        const int row = min(e / D, end - 1 - row0);
        const int lch = ((e % D) >> 3) ^ chunk_swizzle<D>(e / D);
        load_lds16_at(src, dst + i * 1024, (uint32_t)(row * rs + 8 * lch) * 2u, soff);
      }
    }
  }
};

// Row fragment (MFMA A operand of a product over d): rows 32*blk + perm(ln),
// d-chunk 16*kc + 8*hf of a swizzled tile.
template <int D, class E>
__device__ __forceinline__ typename E::T8 row_frag(const typename E::T *t, int blk, int kc, int prow,
                                                   int hf) {
  return E::frag(ld128(&t[tile_off<D>(32 * blk + prow, 16 * kc + 8 * hf)]));
}

// Transposed fragment (MFMA A operand of a product over the tile's rows):
// lane (m = l % 32, h = l / 32) gets tile[16kk + 8h + t][32cb + m], t = 0..7,
// with two transposing reads of 4 rows.
template <int D, class E>
__device__ __forceinline__ typename E::T8 tr_frag(const typename E::T *t, int kk, int cb, int tr_row,
                                                  int tr_col) {
  const int r0 = 16 * kk + tr_row, c0 = 32 * cb + tr_col;
  const u32x2 lo = ds_read_tr16x4(&t[tile_off<D>(r0, c0)]);
  const u32x2 hi = ds_read_tr16x4(&t[tile_off<D>(r0 + 4, c0)]);
  return E::frag(u32x4{lo[0], lo[1], hi[0], hi[1]});
}

#define FA_SC(s, e) s[(e) >> 4][(e) & 15]

// ---------------------------------------------------------------------------
// dK, dV for 128 keys per workgroup, streaming 32-row Q / dO tiles (32 rows
// keep S and dP of two tiles within the register budget next to the dK, dV
// accumulators and the K, V operands). The workgroup writes columns
// DG * g .. DG * g + DG - 1 of dK and dV (DG = d, or d / 2 for d = 256).
template <int D, int MASK, bool VARLEN, class E>
__global__ __launch_bounds__(kThreads, bwd_waves_per_simd<D>()) void dkdv_kernel(BwdArgs a) {
  using Et = typename E::T;   // element type of the tensors
  using E8 = typename E::T8;  // MFMA operand: 8 elements
  const Et *Qg = static_cast<const Et *>(a.q), *Kg = static_cast<const Et *>(a.k);
  const Et *Vg = static_cast<const Et *>(a.v), *dOg = static_cast<const Et *>(a.dout);
  constexpr bool CAUSAL = MASK == kMaskCausal;
  constexpr bool LOCAL = MASK == kMaskLocal;  // window a.wl, a.wr (causal: wr = 0)
  constexpr int BQ = 32;  // query rows per streamed tile
  __shared__ __attribute__((aligned(1024))) Et sQ[kStages][BQ * D];
  __shared__ __attribute__((aligned(1024))) Et sO[kStages][BQ * D];  // dO tiles
  __shared__ __attribute__((aligned(256))) float sL[kStages][BQ];      // lse * log2(e)
  __shared__ __attribute__((aligned(256))) float sDl[kStages][BQ];     // D
  constexpr int G = D == 256 ? 2 : 1;            // column groups of dK, dV
  constexpr int DG = D / G;                      // columns per workgroup
  constexpr int CB = DG / 32;                    // 32-column blocks per workgroup
  constexpr int kInsts = BQ * D / 512 / kWaves;  // 16-byte copies per wave per tensor
  constexpr int NSD = D / 16;                    // MFMAs of S (and of dP) per tile
  constexpr int NGR = 2 * CB;                    // MFMAs of dV^T (and of dK^T) per tile
  // elements of tile j per d-chunk: the first half beside its S MFMA, the
  // rest beside its dP MFMA
  constexpr int NE = 16 / NSD, NE_S = (NE + 1) / 2, NE_D = NE - NE_S;
  constexpr int CPG = 4 / CB;                    // P/dS word packs per dV^T MFMA
  static_assert(NE >= 1 && CPG >= 1, "tile shape");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, ln = lane & 31;
  int bhg, kt;
  // causal: key tile 0 sees the most query rows and is started first; the
  // column groups of one (sequence, head) are adjacent units
  work_order(blockIdx.x, a.nseq * a.H * G, a.n_tiles, kGroupSlots, a.H * G, &bhg, &kt);
  const int bh = bhg / G, cb0 = (bhg - bh * G) * CB;  // first column block
  const Seq<D, VARLEN> sq(a, bh);
  const int len = sq.len;
  if (kt * kBR >= len) return;
  const int rs = a.H * D;

  // this lane's key: K and V rows as B operands (column = key)
  const int key = kt * kBR + wave * 32 + ln;
  E8 kr[D / 16], vr[D / 16];
  f32x16 dk[CB], dv[CB];
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }

  // streamed query tiles q0 .. q0 + ntiles - 1 (BQ rows each): the rows
  // that see the workgroup's keys
  int q0 = 0, q_end = len;
  if (CAUSAL) q0 = (kt * kBR) / BQ;
  if (LOCAL) {
    q0 = win_lo(kt * kBR, a.wr) / BQ;
    q_end = win_hi(min(kt * kBR + kBR, len) - 1, a.wl, len);
  }
  const int ntiles = (q_end + BQ - 1) / BQ - q0;
  const int k_lo = kt * kBR + wave * 32;  // first key of this wavefront

  const uint32_t span = (uint32_t)(((size_t)(len - 1) * rs + D) * 2);
  const u32x4 rq = make_rsrc(Qg + sq.base, span);
  const u32x4 ro = make_rsrc(dOg + sq.base, span);
  const u32x4 rl = make_rsrc(a.lse2 + sq.stat0, (uint32_t)len * 4u);
  const u32x4 rd = make_rsrc(a.delta + sq.stat0, (uint32_t)len * 4u);
  // per-lane offsets of this wavefront's 16-byte share of a tile
  uint32_t goff[kInsts];
#pragma unroll
  for (int i = 0; i < kInsts; ++i) {
    const int e = (wave * kInsts + i) * 512 + 8 * lane;
    const int row = e / D;
    goff[i] = (uint32_t)(row * rs + 8 * (((e % D) >> 3) ^ chunk_swizzle<D>(row))) * 2u;
  }
  auto issue = [&](Et *lds, u32x4 src, int row0) {
    const uint32_t soff = (uint32_t)row0 * (uint32_t)rs * 2u;
    // d = 256: formed per call (opaque_sgpr; the hoisted destinations left
    // the loop short of scalar registers); d <= 128 has room for them
    const uint32_t woff = (uint32_t)(wave * kInsts * 1024);
    const uint32_t dst = lds_address(lds) + (D == 256 ? opaque_sgpr(woff) : woff);
    if (row0 + BQ <= len) {
#pragma unroll
      for (int i = 0; i < kInsts; ++i) load_lds16_at(src, dst + i * 1024, goff[i], soff);
    } else {
      // tail tile: rows past the end re-read the last row
#pragma unroll
      for (int i = 0; i < kInsts; ++i) {
        const int e = (wave * kInsts + i) * 512 + 8 * lane;
        const int row = min(e / D, len - 1 - row0);
        const int lch = ((e % D) >> 3) ^ chunk_swizzle<D>(e / D);
        load_lds16_at(src, dst + i * 1024, (uint32_t)(row * rs + 8 * lch) * 2u, soff);
      }
    }
  };
  // copies this wavefront starts per tile: its share of Q and dO (2 kInsts
  // instructions), plus (waves 0 and 1, lanes 0..31) the tile's 32 lse and D
  // values (one more)

  // tile j goes to slot j % kStages; iteration j starts tile j+3
  auto start_tile = [&](auto slot_c, int j) {
    constexpr int S = decltype(slot_c)::value;
    if (j >= ntiles) return;
    const int r0 = (q0 + j) * BQ;
    issue(sQ[S], rq, r0);
    issue(sO[S], ro, r0);
    if (wave < 2 && lane < BQ) {
      const int r = min(r0 + lane, len - 1);
      load_lds4(wave == 0 ? rl : rd, wave == 0 ? sL[S] : sDl[S], (uint32_t)r * 4u, 0u);
    }
  };
  // tile j+1 landed: only the copies of iteration j-1 (tile j+2) may be in
  // flight. Constant counts: a count chosen at run time costs a chain of
  // branches on every iteration.
  auto wait_tile_after = [&](int j) {
    if (j + 2 < ntiles) {
      if (wave < 2) wait_vmem_n<2 * kInsts + 1 + kTraceStores>();
      else wait_vmem_n<2 * kInsts + kTraceStores>();
    } else {
      wait_vmem_n<kTraceStores>();
    }
  };

  const int prow = perm_row32(ln);
  const int tg = lane >> 4, ts = lane & 15;
  const int tr_row = 8 * (tg >> 1) + (ts >> 2);
  const int tr_col = 16 * (tg & 1) + 4 * (ts & 3);
  const float c = a.scale_log2;

  // keys after the row (causal) or outside its window, and rows past the
  // sequence end -> P = 0
  auto need_mask = [&](int j) {
    const int r0 = (q0 + j) * BQ;
    if (LOCAL)
      return (r0 + BQ > len) || (k_lo + 31 - r0 > a.wr) || (r0 + BQ - 1 - k_lo > a.wl);
    return (r0 + BQ > len) || (CAUSAL && r0 < k_lo + 31);
  };

  E8 qf[NSD], of[NSD];  // row fragments of Q and dO, in flight
  FA_TRACE_DECL;
  E8 gq[NGR], go[NGR];  // transposed fragments of Q and dO, in flight

  // -D of this lane's 16 rows of a tile (element e: row perm(8 * (e / 4) +
  // 4 * hf + e % 4)), the initial dP accumulator: the MFMAs then give dP - D
  auto load_nd = [&](const float *td) {
    f32x16 nd;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(&td[perm_row32(8 * g + 4 * hf)]);
#pragma unroll
      for (int k = 0; k < 4; ++k) nd[4 * g + k] = v[k];
    }
    return nd;
  };
  // S and dP - D of one tile (rows permuted) from LDS
  auto sd_products = [&](const Et *tq, const Et *to, const f32x16 &nd, f32x16 &s, f32x16 &dp) {
#pragma unroll
    for (int kc = 0; kc < NSD; ++kc) {
      s = E::mfma32(row_frag<D, E>(tq, 0, kc, prow, hf), kr[kc], kc == 0 ? f32x16{} : s);
      dp = E::mfma32(row_frag<D, E>(to, 0, kc, prow, hf), vr[kc], kc == 0 ? nd : dp);
    }
  };

  // P_e = exp(s_e * scale - lse_row), dS_e = P_e (dP_e - D_row) for element e
  // of this lane (row perm(8 * (e / 4) + 4 * hf + e % 4) of the tile); dp
  // already holds dP - D. The tile's lse values of this lane's rows, and -D
  // of the next tile's, are read from LDS at the start of the step, ahead of
  // the operand prefetch: a read in the middle of the MFMA stream would wait
  // for its result (and, the LDS counter being in order, for every operand
  // fragment read before it) with the matrix core idle.
  f32x4 L4[4];
  auto load_stats = [&](const float *tl) {
#pragma unroll
    for (int g = 0; g < 4; ++g) L4[g] = *reinterpret_cast<const f32x4 *>(&tl[perm_row32(8 * g + 4 * hf)]);
  };
  auto elementwise = [&](f32x16 &s, f32x16 &dp, int e) {
    const float p = fast_exp2(fmaf(s[e], c, -L4[e >> 2][e & 3]));
    dp[e] = p * dp[e];
    s[e] = p;
    pin(s[e]);
    pin(dp[e]);
  };

  // One tile j. On entry s, dp hold S and dP of tile j; on exit s_n, dp_n
  // hold those of tile j+1.
  auto step = [&](auto u_c, int j, f32x16 &s, f32x16 &dp, f32x16 &s_n, f32x16 &dp_n) {
    constexpr int U = decltype(u_c)::value;
    const Et *tq0 = sQ[U], *to0 = sO[U];
    const Et *tq1 = sQ[(U + 1) % kStages], *to1 = sO[(U + 1) % kStages];
    load_stats(sL[U]);
    const f32x16 nd1 = load_nd(sDl[(U + 1) % kStages]);  // -D of tile j+1
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      qf[i] = row_frag<D, E>(tq1, 0, i, prow, hf);
      of[i] = row_frag<D, E>(to1, 0, i, prow, hf);
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- phase 1: S, dP of tile j+1 beside P, dS of tile j ----
#pragma unroll
    for (int kc = 0; kc < NSD; ++kc) {
      if (kc + PF < NSD) {
        qf[kc + PF] = row_frag<D, E>(tq1, 0, kc + PF, prow, hf);
        of[kc + PF] = row_frag<D, E>(to1, 0, kc + PF, prow, hf);
      }
      s_n = E::mfma32(qf[kc], kr[kc], kc == 0 ? f32x16{} : s_n);
#pragma unroll
      for (int u = 0; u < NE_S; ++u) elementwise(s, dp, kc * NE + u);
      __builtin_amdgcn_sched_barrier(0);
      dp_n = E::mfma32(of[kc], vr[kc], kc == 0 ? nd1 : dp_n);
#pragma unroll
      for (int u = 0; u < NE_D; ++u) elementwise(s, dp, kc * NE + NE_S + u);
      __builtin_amdgcn_sched_barrier(0);
    }

    FA_TRACE_MID;
    // ---- mask tile j: P = dS = 0 for keys after the row, rows past the end
    if (need_mask(j)) {
      const int r0 = (q0 + j) * BQ;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = r0 + perm_row32(8 * (e >> 2) + 4 * hf + (e & 3));
        if (row >= len || (CAUSAL && key > row) ||
            (LOCAL && (key - row > a.wr || row - key > a.wl))) {
          s[e] = 0.f;
          dp[e] = 0.f;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      gq[i] = tr_frag<D, E>(tq0, i / CB, cb0 + i % CB, tr_row, tr_col);
      go[i] = tr_frag<D, E>(to0, i / CB, cb0 + i % CB, tr_row, tr_col);
    }
    // P and dS of k-step kk (rows 16kk .. 16kk+15) as bf16 B operands
    uint32_t pw[2][4], dw[2][4];
    auto pack = [&](int kk, int w) {
      const int e = 8 * kk + 2 * w;
      pw[kk][w] = E::pack2(s[e], s[e + 1]);
      dw[kk][w] = E::pack2(dp[e], dp[e + 1]);
    };
#pragma unroll
    for (int w = 0; w < 4; ++w) pack(0, w);
    __builtin_amdgcn_sched_barrier(0);

    // ---- phase 2: dV^T += dO^T P and dK^T += Q^T dS for tile j ----
#pragma unroll
    for (int m = 0; m < NGR; ++m) {
      const int kk = m / CB, cb = m % CB;
      if (m + PF < NGR) {
        gq[m + PF] = tr_frag<D, E>(tq0, (m + PF) / CB, cb0 + (m + PF) % CB, tr_row, tr_col);
        go[m + PF] = tr_frag<D, E>(to0, (m + PF) / CB, cb0 + (m + PF) % CB, tr_row, tr_col);
      }
      const E8 pb = E::frag(u32x4{pw[kk][0], pw[kk][1], pw[kk][2], pw[kk][3]});
      const E8 db = E::frag(u32x4{dw[kk][0], dw[kk][1], dw[kk][2], dw[kk][3]});
      dv[cb] = E::mfma32(go[m], pb, dv[cb]);
      if (kk == 0) {
#pragma unroll
        for (int u = 0; u < CPG; ++u) pack(1, cb * CPG + u);
      }
      __builtin_amdgcn_sched_barrier(0);
      dk[cb] = E::mfma32(gq[m], db, dk[cb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- prologue: tiles 0..2 (as iterations -3..-1 would start them), K and
  // V rows of this lane; everything waited for here ----
  start_tile(std::integral_constant<int, 0>{}, 0);
  start_tile(std::integral_constant<int, 1>{}, 1);
  start_tile(std::integral_constant<int, 2>{}, 2);
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) {
    if (key < len) {
      kr[kc] = E::frag(ld128(Kg + sq.base + (size_t)key * rs + 16 * kc + 8 * hf));
      vr[kc] = E::frag(ld128(Vg + sq.base + (size_t)key * rs + 16 * kc + 8 * hf));
    } else {
      kr[kc] = E::frag(u32x4{0, 0, 0, 0});
      vr[kc] = E::frag(u32x4{0, 0, 0, 0});
    }
  }
  wait_vmem();
  __syncthreads();
  f32x16 sa, pa, sb, pb2;
  sd_products(sQ[0], sO[0], load_nd(sDl[0]), sa, pa);
  FA_TRACE_PRIME(kWaves);

  auto iter = [&](auto u_c, int j, f32x16 &s, f32x16 &dp, f32x16 &s_n, f32x16 &dp_n) {
    constexpr int U = decltype(u_c)::value;
    FA_TRACE_STAMP(t0);
    wait_tile_after(j);
    FA_TRACE_STAMP(ta);
    __syncthreads();
    FA_TRACE_STAMP(tb);
    start_tile(std::integral_constant<int, (U + 3) % kStages>{}, j + 3);
    FA_TRACE_STAMP(tc);
    step(u_c, j, s, dp, s_n, dp_n);
    FA_TRACE_STAMP(t3);
    FA_TRACE_RECORD(g_dkdv_trace, kWaves, kTraceDkdv, j, t0, ta, tb, tc, t3);
  };
  static_assert(kStages == 4, "unroll below");
  for (int j = 0; j < ntiles; j += 4) {
    iter(std::integral_constant<int, 0>{}, j, sa, pa, sb, pb2);
    if (j + 1 < ntiles) iter(std::integral_constant<int, 1>{}, j + 1, sb, pb2, sa, pa);
    if (j + 2 < ntiles) iter(std::integral_constant<int, 2>{}, j + 2, sa, pa, sb, pb2);
    if (j + 3 < ntiles) iter(std::integral_constant<int, 3>{}, j + 3, sb, pb2, sa, pa);
  }

  // lane holds dV^T[32cb + 8g + 4h + r][key] -> dV[key][32cb + 8g + 4h .. +3]
  // (cb counted from the workgroup's first column block)
  if (key < len) {
    Et *dkg = static_cast<Et *>(a.dk) + sq.base + (size_t)key * rs;
    Et *dvg = static_cast<Et *>(a.dv) + sq.base + (size_t)key * rs;
    const float sc = a.scale;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * (cb0 + cb) + 8 * g + 4 * hf;
        *reinterpret_cast<u32x2 *>(dvg + col) =
            u32x2{E::pack2(dv[cb][4 * g], dv[cb][4 * g + 1]),
                  E::pack2(dv[cb][4 * g + 2], dv[cb][4 * g + 3])};
        *reinterpret_cast<u32x2 *>(dkg + col) =
            u32x2{E::pack2(dk[cb][4 * g] * sc, dk[cb][4 * g + 1] * sc),
                  E::pack2(dk[cb][4 * g + 2] * sc, dk[cb][4 * g + 3] * sc)};
      }
  }
}

// ---------------------------------------------------------------------------
// dQ for 128 query rows per workgroup. At d = 128 each 32-row group has two
// wavefronts (8 in all, two per SIMD): wavefront r of a group takes 32-key
// block r of every 64-key tile, and the two partial dQ are summed through LDS
// at the end. Each then needs 256 registers or fewer, and one SIMD interleaves
// two instruction streams (one's exponentials beside the other's MFMAs)
// while the workgroup still copies each K / V tile once.
template <int D>
constexpr int dq_split() { return D == 128 ? 2 : 1; }
template <int D>
constexpr int dq_threads() { return 64 * kWaves * dq_split<D>(); }

template <int D, int MASK, bool VARLEN, class E>
__global__ __launch_bounds__(dq_threads<D>(), bwd_waves_per_simd<D>()) void dq_kernel(BwdArgs a) {
  using Et = typename E::T;
  using E8 = typename E::T8;
  const Et *Qg = static_cast<const Et *>(a.q), *Kg = static_cast<const Et *>(a.k);
  const Et *Vg = static_cast<const Et *>(a.v), *dOg = static_cast<const Et *>(a.dout);
  constexpr bool CAUSAL = MASK == kMaskCausal;
  constexpr bool LOCAL = MASK == kMaskLocal;
  constexpr int SPLIT = dq_split<D>();  // wavefronts per 32-row group
  constexpr int NW = kWaves * SPLIT;    // wavefronts per workgroup
#ifdef FA_BWD_TRACE
  static_assert(NW <= 8, "timing record: 8 wavefront slots per workgroup");
#endif
  constexpr int KB = dq_blocks<D>();    // 32-key score blocks per tile
  constexpr int KBW = KB / SPLIT;       // of them, blocks per wavefront
  static_assert(KBW >= 1 && KBW * SPLIT == KB, "key blocks per wavefront");
  constexpr int kBT = 32 * KB;          // keys per streamed tile
  __shared__ __attribute__((aligned(1024))) Et sK[kStages][kBT * D];
  __shared__ __attribute__((aligned(1024))) Et sV[kStages][kBT * D];
  // Wavefronts that start the tile copies: with two per 32-row group (two
  // per SIMD), the four older ones (role 0), which the matrix cores serve
  // first and which otherwise wait at each barrier for their partners.
  constexpr int CW = SPLIT == 2 ? kWaves : NW;
  constexpr int kInsts = TileCopier<D, E, kBT, CW>::kInsts;
  constexpr int NSD = KBW * (D / 16);  // MFMAs of S^T (and of dP^T) per tile
  constexpr int KS = 2 * KBW;          // 16-key k-steps of dQ^T per tile
  constexpr int NGR = KS * (D / 32);   // MFMAs of dQ^T per tile
  // elements of tile j per phase-1 step: the first half beside its S^T MFMA,
  // the rest beside its dP^T MFMA
  constexpr int NE = 16 * KBW / NSD, NE_S = (NE + 1) / 2, NE_D = NE - NE_S;
  // words of the next k-step packed per phase-2 MFMA (4 per k-step; for
  // d = 256 the first four MFMAs of a k-step pack one each)
  constexpr int CPG = D / 32 <= 4 ? 4 / (D / 32) : 1;
  // LDS fragment prefetch distance: 2 keeps the split form within 256 VGPRs
  constexpr int PF = SPLIT == 2 ? 2 : fa::PF;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave % kWaves;              // 32-row group
  const int role = wave / kWaves;            // which key blocks of a tile
  const int blk0 = role * KBW;               // first key block of this wavefront
  const int hf = lane >> 5, ln = lane & 31;
  int bh, t;
  work_order(blockIdx.x, a.nseq * a.H, a.n_tiles, kGroupSlotsDq, a.H, &bh, &t);
  // causal: the last query tiles see the most keys and are started first
  const int qt = MASK != kMaskNone ? a.n_tiles - 1 - t : t;
  const Seq<D, VARLEN> sq(a, bh);
  const int len = sq.len;
  if (qt * kBR >= len) return;
  const int rs = a.H * D;

  const int row0 = qt * kBR + rg * 32;
  const int qrow = row0 + ln;
  E8 qr[D / 16], dor[D / 16];
  f32x16 dq[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dq[i] = f32x16{};

  // keys the workgroup's rows see: tiles kv_beg + j * kBT, j < ntiles
  const int last_row = min((qt + 1) * kBR, len) - 1;
  int kv_beg = 0, kv_end = len;
  if (CAUSAL) kv_end = last_row + 1;
  if (LOCAL) {
    kv_beg = win_lo(qt * kBR, a.wl) / kBT * kBT;
    kv_end = win_hi(last_row, a.wr, len);
  }
  const int ntiles = (kv_end - kv_beg + kBT - 1) / kBT;
  // Window: iteration j takes tile (j + phase) mod ntiles. The windows of a
  // head's workgroups start kBR keys (two tiles) apart; rotated this way all
  // of them read the key tile whose index is j modulo ntiles in iteration j
  // and share it in the L2, where in key order the 32 workgroups of an XCD
  // would stream about 130 different tiles at once, more than the L2 holds.
  // Other masks: tile j. The phase is 0 when the range starts at key 0, so a
  // window as wide as the sequence sums in the plain kernel's order.
  int phase = 0;
  if constexpr (LOCAL) phase = (ntiles - (kv_beg / kBT) % ntiles) % ntiles;
  auto tile_kv = [&](int j) {  // first key of iteration j's tile, j < ntiles
    int k = j;
    if constexpr (LOCAL) {
      k += phase;
      if (k >= ntiles) k -= ntiles;
    }
    return kv_beg + k * kBT;
  };
  // tiles w_lo .. nt_w-1 hold keys this row group sees
  int w_lo = 0, nt_w = 0;
  if (row0 < len) {
    const int wlast = min(row0 + 31, len - 1);
    const int last_key = CAUSAL ? wlast : LOCAL ? win_hi(wlast, a.wr, len) - 1 : len - 1;
    nt_w = (last_key - kv_beg) / kBT + 1;
    if (LOCAL) w_lo = (win_lo(row0, a.wl) - kv_beg) / kBT;
  }

  const uint32_t span = (uint32_t)(((size_t)(len - 1) * rs + D) * 2);
  const u32x4 rk = make_rsrc(Kg + sq.base, span);
  const u32x4 rv = make_rsrc(Vg + sq.base, span);
  const bool copier = CW == NW || wave < CW;
  const TileCopier<D, E, kBT, CW> cp(rs, copier ? wave : 0, lane);

  auto start_tile = [&](auto slot_c, int j) {
    constexpr int S = decltype(slot_c)::value;
    if (j >= ntiles || !copier) return;
    cp.issue(sK[S], rk, tile_kv(j), kv_end);
    cp.issue(sV[S], rv, tile_kv(j), kv_end);
  };
  auto wait_tile_after = [&](int j) {
    if (!copier) return;  // none of its own copies in flight
    if (j + 2 < ntiles) wait_vmem_n<2 * kInsts + kTraceStores>();
    else wait_vmem_n<kTraceStores>();
  };

  const int krow = perm_row32(ln);
  const int tg = lane >> 4, ts = lane & 15;
  const int tr_row = 8 * (tg >> 1) + (ts >> 2);
  const int tr_col = 16 * (tg & 1) + 4 * (ts & 3);
  const float c = a.scale_log2;
  float L2 = 0.f, nDr = 0.f;  // this row's lse * log2(e) and -D

  // keys of this wavefront's blocks in tile j: kv0 + 32 * blk0 .. + 32 * KBW - 1
  auto need_mask = [&](int j) {
    const int k0 = tile_kv(j) + 32 * blk0, k1 = k0 + 32 * KBW - 1;
    if (LOCAL) return (k1 >= len) || (k1 - row0 > a.wr) || (row0 + 31 - k0 > a.wl);
    return (k1 >= len) || (CAUSAL && k1 > row0);
  };

  E8 kf[NSD], vf[NSD], gk[NGR];
  FA_TRACE_DECL;

  auto sd_products = [&](const Et *tk, const Et *tv, f32x16 (&s)[KBW], f32x16 (&dp)[KBW]) {
#pragma unroll
    for (int m = 0; m < NSD; ++m) {
      const int blk = m % KBW, kc = m / KBW;
      s[blk] = E::mfma32(row_frag<D, E>(tk, blk0 + blk, kc, krow, hf), qr[kc],
                         kc == 0 ? f32x16{} : s[blk]);
      dp[blk] = E::mfma32(row_frag<D, E>(tv, blk0 + blk, kc, krow, hf), dor[kc],
                          kc == 0 ? f32x16{} : dp[blk]);
    }
  };

  // One key tile j. On entry s, dp hold S^T and dP^T of this wavefront's
  // blocks of tile j (keys permuted within 32-key blocks, column = query
  // row); on exit s_n, dp_n hold those of tile j+1.
  auto step = [&](auto u_c, int j, f32x16 (&s)[KBW], f32x16 (&dp)[KBW], f32x16 (&s_n)[KBW],
                  f32x16 (&dp_n)[KBW]) {
    constexpr int U = decltype(u_c)::value;
    const Et *tk0 = sK[U];
    const Et *tk1 = sK[(U + 1) % kStages], *tv1 = sV[(U + 1) % kStages];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      kf[i] = row_frag<D, E>(tk1, blk0 + i % KBW, i / KBW, krow, hf);
      vf[i] = row_frag<D, E>(tv1, blk0 + i % KBW, i / KBW, krow, hf);
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- phase 1: S^T, dP^T of tile j+1 beside P, dS of tile j ----
#pragma unroll
    for (int m = 0; m < NSD; ++m) {
      if (m + PF < NSD) {
        kf[m + PF] = row_frag<D, E>(tk1, blk0 + (m + PF) % KBW, (m + PF) / KBW, krow, hf);
        vf[m + PF] = row_frag<D, E>(tv1, blk0 + (m + PF) % KBW, (m + PF) / KBW, krow, hf);
      }
      const int blk = m % KBW, kc = m / KBW;
      s_n[blk] = E::mfma32(kf[m], qr[kc], kc == 0 ? f32x16{} : s_n[blk]);
#pragma unroll
      for (int u = 0; u < NE_S; ++u) {
        const int e = m * NE + u;
        const float p = fast_exp2(fmaf(FA_SC(s, e), c, -L2));
        FA_SC(dp, e) = p * (FA_SC(dp, e) + nDr);
        pin(FA_SC(dp, e));
      }
      __builtin_amdgcn_sched_barrier(0);
      dp_n[blk] = E::mfma32(vf[m], dor[kc], kc == 0 ? f32x16{} : dp_n[blk]);
#pragma unroll
      for (int u = 0; u < NE_D; ++u) {
        const int e = m * NE + NE_S + u;
        const float p = fast_exp2(fmaf(FA_SC(s, e), c, -L2));
        FA_SC(dp, e) = p * (FA_SC(dp, e) + nDr);
        pin(FA_SC(dp, e));
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    FA_TRACE_MID;
    // ---- mask tile j: dS = 0 for keys past the end, after the row or
    // outside its window ----
    if (need_mask(j)) {
      const int kv0 = tile_kv(j) + 32 * blk0;
#pragma unroll
      for (int e = 0; e < 16 * KBW; ++e) {
        const int k = kv0 + 32 * (e >> 4) + perm_row32(8 * ((e & 15) >> 2) + 4 * hf + (e & 3));
        if (k >= len || (CAUSAL && k > qrow) || (LOCAL && (k - qrow > a.wr || qrow - k > a.wl)))
          FA_SC(dp, e) = 0.f;
      }
    }
    // K^T operand of dQ^T MFMA m: k-step kk of this wavefront's keys
    // (tile k-step 2 * blk0 + kk), d-block cb
#pragma unroll
    for (int i = 0; i < PF; ++i)
      gk[i] = tr_frag<D, E>(tk0, 2 * blk0 + i / (D / 32), i % (D / 32), tr_row, tr_col);
    uint32_t dw[KS][4];
    auto pack = [&](int kk, int w) {
      const int e = 8 * kk + 2 * w;
      dw[kk][w] = E::pack2(FA_SC(dp, e), FA_SC(dp, e + 1));
    };
#pragma unroll
    for (int w = 0; w < 4; ++w) pack(0, w);
    __builtin_amdgcn_sched_barrier(0);

    // ---- phase 2: dQ^T += K^T dS^T for tile j ----
#pragma unroll
    for (int m = 0; m < NGR; ++m) {
      const int kk = m / (D / 32), cb = m % (D / 32);
      if (m + PF < NGR)
        gk[m + PF] = tr_frag<D, E>(tk0, 2 * blk0 + (m + PF) / (D / 32), (m + PF) % (D / 32),
                                   tr_row, tr_col);
      const E8 db = E::frag(u32x4{dw[kk][0], dw[kk][1], dw[kk][2], dw[kk][3]});
      dq[cb] = E::mfma32(gk[m], db, dq[cb]);
      if (kk + 1 < KS && cb * CPG < 4) {
#pragma unroll
        for (int u = 0; u < CPG; ++u) pack(kk + 1, cb * CPG + u);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- prologue ----
  start_tile(std::integral_constant<int, 0>{}, 0);
  start_tile(std::integral_constant<int, 1>{}, 1);
  start_tile(std::integral_constant<int, 2>{}, 2);
  if (qrow < len) {
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      qr[kc] = E::frag(ld128(Qg + sq.base + (size_t)qrow * rs + 16 * kc + 8 * hf));
      dor[kc] = E::frag(ld128(dOg + sq.base + (size_t)qrow * rs + 16 * kc + 8 * hf));
    }
    L2 = a.lse2[sq.stat0 + qrow];
    nDr = a.delta[sq.stat0 + qrow];
  } else {
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      qr[kc] = E::frag(u32x4{0, 0, 0, 0});
      dor[kc] = E::frag(u32x4{0, 0, 0, 0});
    }
  }
  wait_vmem();
  __syncthreads();
  // iteration j's tile holds keys this row group sees
  auto wave_runs = [&](int j) {
    const int k = (tile_kv(j) - kv_beg) / kBT;
    return k >= w_lo && k < nt_w;
  };
  f32x16 sa[KBW], pa[KBW], sb[KBW], pb2[KBW];
  if (wave_runs(0)) sd_products(sK[0], sV[0], sa, pa);
  FA_TRACE_PRIME(8);

  auto iter = [&](auto u_c, int j, f32x16 (&s)[KBW], f32x16 (&dp)[KBW], f32x16 (&s_n)[KBW],
                  f32x16 (&dp_n)[KBW]) {
    constexpr int U = decltype(u_c)::value;
    FA_TRACE_STAMP(t0);
    wait_tile_after(j);
    FA_TRACE_STAMP(ta);
    __syncthreads();
    FA_TRACE_STAMP(tb);
    start_tile(std::integral_constant<int, (U + 3) % kStages>{}, j + 3);
    FA_TRACE_STAMP(tc);
#ifdef FA_BWD_TRACE
    unsigned long long t3 = 0;
#endif
    if (wave_runs(j)) {
      step(u_c, j, s, dp, s_n, dp_n);
#ifdef FA_BWD_TRACE
      t3 = trace_clock();
#endif
    } else if (LOCAL && j + 1 < ntiles && wave_runs(j + 1)) {
      // a window's wavefront may skip iterations (at most two runs of
      // tiles, the key range being rotated): the first S^T, dP^T of a run
      // are computed one iteration ahead, like step's
      sd_products(sK[(U + 1) % kStages], sV[(U + 1) % kStages], s_n, dp_n);
    }
    FA_TRACE_RECORD(g_dq_trace, 8, kTraceDq, j, t0, ta, tb, tc, t3);
  };
  static_assert(kStages == 4, "unroll below");
  for (int j = 0; j < ntiles; j += 4) {
    iter(std::integral_constant<int, 0>{}, j, sa, pa, sb, pb2);
    if (j + 1 < ntiles) iter(std::integral_constant<int, 1>{}, j + 1, sb, pb2, sa, pa);
    if (j + 2 < ntiles) iter(std::integral_constant<int, 2>{}, j + 2, sa, pa, sb, pb2);
    if (j + 3 < ntiles) iter(std::integral_constant<int, 3>{}, j + 3, sb, pb2, sa, pa);
  }

  if constexpr (SPLIT == 2) {
    // sum the two partial dQ of a row group: the second wavefront passes its
    // accumulators through LDS (the K ring, free once every wavefront is past
    // its last tile), element i of lane l at float4 (i, l) of its group's
    // area, so each ds_write_b128 / ds_read_b128 covers consecutive 16 bytes
    static_assert(kWaves * 64 * D / 8 * 16 <= sizeof(sK), "reduction area");
    f32x4 *red = reinterpret_cast<f32x4 *>(&sK[0][0]) + rg * (D / 8) * 64;
    __syncthreads();
    if (role == 1) {
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          red[(cb * 4 + g) * 64 + lane] =
              f32x4{dq[cb][4 * g], dq[cb][4 * g + 1], dq[cb][4 * g + 2], dq[cb][4 * g + 3]};
    }
    __syncthreads();
    if (role == 1) return;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 o = red[(cb * 4 + g) * 64 + lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) dq[cb][4 * g + r] += o[r];
      }
  }

  if (qrow < len) {
    Et *dqg = static_cast<Et *>(a.dq) + sq.base + (size_t)qrow * rs;
    const float sc = a.scale;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<u32x2 *>(dqg + 32 * cb + 8 * g + 4 * hf) =
            u32x2{E::pack2(dq[cb][4 * g] * sc, dq[cb][4 * g + 1] * sc),
                  E::pack2(dq[cb][4 * g + 2] * sc, dq[cb][4 * g + 3] * sc)};
  }
}

#undef FA_SC

template <typename Kernel>
hipError_t launch1(Kernel *fn, long long grid, int threads, const BwdArgs &a0,
                   hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  BwdArgs a = a0;
  void *params[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3((unsigned)grid),
                         dim3(threads), params, 0, stream);
}

template <int D, int MASK, bool VARLEN, class E>
hipError_t launch_all(const BwdArgs &a, hipStream_t stream) {
  {
    const long long nrows = (long long)a.total * a.H;
    const long long grid = (nrows * (D / 8) + kThreads - 1) / kThreads;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    BwdArgs arg = a;
    long long nr = nrows;
    void *params[] = {&arg, &nr};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&pre_kernel<D, VARLEN, E>),
                                   dim3((unsigned)grid), dim3(kThreads), params, 0, stream);
    if (e != hipSuccess) return e;
  }
  const long long grid = (long long)a.nseq * a.H * a.n_tiles;
  constexpr int G = D == 256 ? 2 : 1;  // dK / dV column groups per key tile
  hipError_t e = launch1(&dkdv_kernel<D, MASK, VARLEN, E>, grid * G, kThreads, a, stream);
  if (e != hipSuccess) return e;
  return launch1(&dq_kernel<D, MASK, VARLEN, E>, grid, dq_threads<D>(), a, stream);
}

// Scratch memory of the no-allocation backward: the rows of D and
// lse * log2(e) that the workspace argument carries in the other calls, in a
// static device array. Every GPU the library runs on holds one copy until
// the process ends; calls on one GPU share it.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

}  // namespace

// Device address of this GPU's copy of `scratch`. In host code the array's
// name is only a host-side stand-in, so the address is looked up once per
// device (with that device current) and kept.
hipError_t noalloc_scratch(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

int bwd_block() { return kBR; }

hipError_t launch_bwd(const BwdArgs &a, int d, MaskKind mask, bool varlen, ElemKind elem,
                      hipStream_t stream) {
#define FA_CASE(DD, MM, EE)                                                        \
  if (d == DD && mask == MM)                                                       \
    return varlen ? launch_all<DD, MM, true, EE>(a, stream)                        \
                  : launch_all<DD, MM, false, EE>(a, stream);
#define FA_ELEM(EE)             \
  FA_CASE(64, kMaskNone, EE)    \
  FA_CASE(64, kMaskCausal, EE)  \
  FA_CASE(64, kMaskLocal, EE)   \
  FA_CASE(128, kMaskNone, EE)   \
  FA_CASE(128, kMaskCausal, EE) \
  FA_CASE(128, kMaskLocal, EE)  \
  FA_CASE(256, kMaskNone, EE)   \
  FA_CASE(256, kMaskCausal, EE) \
  FA_CASE(256, kMaskLocal, EE)
  if (elem == kElemBF16) {
    FA_ELEM(ElemBF16)
  } else if (elem == kElemF16) {
    FA_ELEM(ElemF16)
  }
#undef FA_ELEM
#undef FA_CASE
  return hipErrorInvalidValue;
}

#ifdef FA_BWD_TRACE
// Copies the timing build's clock stamps of the dK/dV (kernel 0) or dQ
// (kernel 1) kernel to the host (n values, at most the size of the record);
// returns the hipError_t of the copy.
extern "C" int fa_bwd_trace_read(int kernel, unsigned long long *host, int n) {
  const int cap = kernel == 0 ? kTraceGroups * 4 * kTraceDkdv * 6 : kTraceGroups * 8 * kTraceDq * 6;
  if (kernel < 0 || kernel > 1 || n < 0 || n > cap) return (int)hipErrorInvalidValue;
  const size_t bytes = (size_t)n * sizeof(unsigned long long);
  return kernel == 0
             ? (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_dkdv_trace), bytes, 0,
                                        hipMemcpyDeviceToHost)
             : (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_dq_trace), bytes, 0,
                                        hipMemcpyDeviceToHost);
}
#endif

}  // namespace fa
