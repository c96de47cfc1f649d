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
//  * one work unit = BM (256) query rows of one (batch, head), run by a
//    workgroup of 8 wavefronts, one workgroup per CU (two wavefronts per
//    SIMD); each wavefront owns 32 rows, so row statistics never cross
//    wavefronts. 256 rows per K/V tile copy halve the L2 traffic of 128-row
//    workgroups. Large fixed-length launches are persistent (see fwd_kernel).
//  * scores are computed transposed, S^T = K Q^T, on 32x32x16 bf16 MFMA: the
//    accumulator column is the query row, so a lane holds 16 scores of one row
//    per 32-key block and row reductions need one exchange with lane l^32
//    (v_permlane32_swap, no LDS round trip).
//  * Q stays in VGPRs (B operand) for the whole kernel. K and V tiles of BN
//    keys are copied row-major into LDS by direct global-to-LDS loads (a
//    uniform tile base plus fixed per-lane offsets) into 4-slot rings, started
//    3 tiles ahead of use, with one barrier per tile; a wavefront only waits
//    for the copies it needs next, newer ones stay in flight. With two
//    wavefronts per SIMD (d = 64 and 128) the copies are started by the older
//    wavefront of each pair alone (copy_waves). The P.V
//    product O^T = V^T P^T reads its A operand with the transposing LDS read
//    and takes P straight from the score accumulators.
//  * software pipelining inside each wavefront: while the matrix cores
//    compute the scores of tile j+1, the vector ALUs compute the softmax of
//    tile j; the P.V product of tile j then overlaps the row sums. K runs one
//    tile ahead of V in LDS for this.
//  * the key order inside a 32-key score block is permuted (perm_row32) so a
//    lane's 8 probabilities of one MFMA k-step are 8 consecutive keys.
//  * softmax uses exp2 with scale*log2(e) folded into one FMA per score. The
//    running max used for the exponentials is only raised when the true max
//    exceeds it by more than 2^8 (in exp2 units 8): until then P may reach
//    256, which bf16 and the fp32 sums hold as well as values below 1, and
//    the O rescale (one multiply per accumulator) is skipped. The result is
//    the same up to rounding.
//  * O is normalised by the row sum of P as rounded to bf16 (the weights the
//    MFMA applied then sum to one); that sum comes from a small MFMA of a 0/1
//    matrix with P, since dot-product instructions stall the matrix cores.
//  * a sliding window (kMaskLocal) starts the key loop at the first tile the
//    workgroup's window reaches, in a rotated order that makes the
//    workgroups of a head read the same K/V tile at the same time; a
//    wavefront whose own first tile comes later computes its first scores
//    one iteration ahead of it.
//  * FP8 (e4m3) inputs: S^T on the 32x32x64 FP8 MFMA from byte tiles of K
//    and Q, the descale factors folded into the exp2 constant; V arrives as
//    bytes and is widened exactly to bf16 in LDS one tile ahead, so P.V runs
//    the bf16 path with P in bf16.
#include <atomic>
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

// Tile shape per head dimension. For d <= 128: 8 wavefronts (two per SIMD),
// 256 query rows per workgroup, 64-key tiles (two 32-key score blocks).
// d = 256 needs twice the registers per query row (the Q operands and the
// O accumulator take 64 + 128 VGPRs per lane), so one wavefront per SIMD:
// 4 wavefronts, 128 rows, and 32-key tiles (one score block), which keep the
// four-slot K and V rings at 128 KiB of LDS.
template <int D>
struct FwdShape {
  static constexpr int kWaves = D == 256 ? 4 : 8;  // 32 query rows each
  static constexpr int KB = D == 256 ? 1 : 2;      // 32-key score blocks per tile
  static constexpr int kBN = 32 * KB;              // keys per iteration
  static constexpr int kBM = 32 * kWaves;          // query rows per workgroup
  static constexpr int kThreads = 64 * kWaves;
};

// Wavefronts that start a tile's copies. The copy instructions hold their
// wavefront for about 450 cycles per tile, and the two wavefronts sharing a
// SIMD run about 500 cycles apart (the matrix cores serve the older one
// first, which then waits at each barrier for its partner); so with two per
// SIMD the older four take all the copies, and their partners start their
// MFMAs at once. Timed against every wavefront copying: the fixed-length
// kernels without a window 1-3% faster (d = 64 and 128, bf16, fp16, FP8),
// the windows and packed sequences 2-5.5% (once their key loops were free of
// spill code; before, they spilled with it and ran 10-52% slower).
template <int D>
constexpr int copy_waves() {
  return FwdShape<D>::kWaves == 8 ? 4 : FwdShape<D>::kWaves;
}
constexpr int kStages = 4;   // K and V tiles in LDS (ring buffers)
constexpr int kAhead = kStages - 1;  // tiles a copy is started ahead of use
constexpr float kRescaleLog2 = 8.f;  // lazy rescale threshold (exp2 units)
// Workgroups per XCD that work_order groups its units for: the 32 CUs of an
// MI355X XCD (one workgroup each). Then the K/V of about two heads are live
// per XCD, within its 4 MB L2: the causal B4 N4096 H32 d128 forward fetches
// 1.05x (dispatched) to 1.12x (persistent) its algorithmic bytes. Groups of
// 64 ran 1% faster there but fetched 1.35x (re-reads from outside the L2).
constexpr int kGroupSlots = 32;

// Timing build (FA_FWD_TRACE, compiled into the plain kernels' object of a
// separate library; the product library has none of this): every wavefront
// of the first kTraceGroups workgroups records six shader-clock stamps per
// key iteration, for its first kTraceIters iterations (over all its units):
// loop top, after its copy wait, after the barrier, after starting the
// copies, after phase 1 and after phase 2 (both 0 if it skips the tile). The
// stamps cost about 4% of the run time. Every iteration of every wavefront
// ends with exactly one store instruction (lanes 0..5, one stamp each; to a
// sink outside the recorded range; one more before the loop), which counts
// in the vector-memory counter like the tile copies: the copy waits allow it
// (kTraceStores), so a wavefront never waits for its own record.
#ifdef FA_FWD_TRACE
constexpr int kTraceGroups = 256, kTraceIters = 320, kTraceStores = 1;
__device__ unsigned long long g_fwd_trace[kTraceGroups * 8 * kTraceIters * 6];
__device__ unsigned long long g_fwd_trace_sink[kTraceGroups * 8 * 6];
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
#define FA_TRACE_PARAM , int &trace_it
#define FA_TRACE_ARG , trace_it
#define FA_TRACE_STAMP(v) const unsigned long long v = trace_clock()
#define FA_TRACE_VARS(a, b) unsigned long long a = 0, b = 0
#define FA_TRACE_SET(v) v = trace_clock()
#define FA_TRACE_RECORD(t0, ta, tb, tc, t2, t3)                                          \
  do {                                                                                  \
    const size_t slot_ = (size_t)(blockIdx.x % kTraceGroups) * 8 + wave;                \
    trace_store(trace_it < kTraceIters && blockIdx.x < kTraceGroups                     \
                    ? g_fwd_trace + (slot_ * kTraceIters + trace_it) * 6                \
                    : g_fwd_trace_sink + slot_ * 6,                                     \
                lane, t0, ta, tb, tc, t2, t3);                                          \
    ++trace_it;                                                                         \
  } while (0)
// one record store before the loop, so a copy wait always has exactly one
// record younger than the copies it waits for
#define FA_TRACE_PRIME \
  trace_store(g_fwd_trace_sink + ((size_t)(blockIdx.x % kTraceGroups) * 8 + wave) * 6, lane, 0, 0, 0, 0, 0, 0)
#else
constexpr int kTraceStores = 0;
#define FA_TRACE_PRIME
#define FA_TRACE_PARAM
#define FA_TRACE_ARG
#define FA_TRACE_STAMP(v)
#define FA_TRACE_VARS(a, b)
#define FA_TRACE_SET(v)
#define FA_TRACE_RECORD(t0, ta, tb, tc, t2, t3)
#endif

// FP8 (e4m3) inputs: a byte tile of D-byte rows whose 16-byte chunks are
// XOR-permuted by a function of the row, so the S^T operand reads (16
// consecutive rows, one chunk each) touch every LDS bank once.
template <int D>
__device__ __forceinline__ int swz8(int row) {
  static_assert(D == 128 || D == 256, "fp8 head dim");
  if constexpr (D == 128) return (row >> 1) & 7;
  else return row & 15;
}

// Shared memory of one forward workgroup: the K and V rings (elements of
// the inputs' type) and, for FP8 inputs, two V tiles widened to bf16 (the
// P.V product runs on the bf16 MFMA with P in bf16). Each is its own
// __shared__ array, so LDS reads address it from one base register plus an
// immediate offset (a single block of over 64 KiB would not fit the offset
// field).
template <int D, class E, bool F8>
struct FwdLdsT {
  using In = std::conditional_t<F8, uint8_t, typename E::T>;
  typedef In Ring[kStages][FwdShape<D>::kBN * D];
  typedef typename E::T Wide[F8 ? 2 : 1][F8 ? FwdShape<D>::kBN * D : 8];
};

// This wavefront's Q rows as MFMA B operands: 8 elements per k-step of 16
// (16-bit inputs), 32 bytes per k-step of 64 (FP8 on the 32x32x64 MFMA).
template <int D, class E, bool F8>
struct QOps {
  typename E::T8 r[D / 16];
};
template <int D, class E>
struct QOps<D, E, true> {
  i32x8 r[D / 64];
};

// One S^T MFMA: FP8 on the 32x32x64 MFMA, 16-bit inputs on E's 32x32x16.
template <bool F8, class E, class KOp, class QOp>
__device__ __forceinline__ f32x16 score_mfma(KOp k, QOp q, f32x16 c) {
  if constexpr (F8) return mfma_fp8(k, q, c);
  else return E::mfma32(k, q, c);
}

// Even split of n items over m segments: segment i takes items
// [seg_lo(i), seg_lo(i + 1)); seg_of(e) is the segment of item e.
constexpr int seg_lo(int i, int n, int m) { return (i * n + m - 1) / m; }
constexpr int seg_of(int e, int n, int m) { return (e * m) / n; }

// The split exponential schedule of a tile (see fwd_unit) is consistent:
// every later k-step is exponentiated and packed before its first P.V
// MFMA, and every score pair is exponentiated before phase 2 sums it.
constexpr bool exp_schedule_ok(int KS, int KSA, int NPV, int CBN, int PPM, int MPP) {
  const int NSC = 8 * KS, EA = 8 * KSA, EB = NSC - EA, NSEG = NPV - CBN;
  for (int k2 = KSA; k2 < KS; ++k2)
    if (seg_of(8 * k2 + 7 - EA, EB, NSEG) >= k2 * CBN) return false;
  for (int p = 0; p < NSC / 2; ++p) {
    const int e = 2 * p + 1;
    if (e < EA) continue;
    const int used = PPM > 0 ? p / PPM : p * MPP;
    if (seg_of(e - EA, EB, NSEG) > used) return false;
  }
  return true;
}

// Maximum / sum of x over the lane pair (l, l ^ 32), in every lane.
__device__ __forceinline__ float pair_max(float x) {
  const auto r =
      __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r =
      __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Persistent schedule of a fixed-length launch: gridDim.x workgroups, one per
// CU, gridDim.x / 8 per XCD (the hardware deals workgroups to the 8 XCDs
// round-robin by index). XCD x owns the units (b, h) dealt to it in chunks
// of C adjacent heads, as in work_order; its (unit, tile) slots, unit-major
// with each unit's heaviest tile first, are taken W = gridDim.x / 8 at a time
// in rounds, and workgroup i of the XCD takes slot i of even rounds and slot
// W - 1 - i of odd rounds. With causal costs that fall by one tile per tile
// index, two consecutive rounds give every workgroup the same work (a heavy
// tile paired with a light one), and the workgroups of an XCD work on the
// same few heads at a time, which share the L2. Returns false once round r
// has no slot for this workgroup (nor will any later round).
[[maybe_unused]] __device__ __forceinline__ bool persistent_slot(int r, int n_units, int n_tiles,
                                                                int per_seq, int *unit,
                                                                int *tile) {
  constexpr int kXcd = 8;
  const int W = gridDim.x / kXcd, x = blockIdx.x % kXcd, i = blockIdx.x / kXcd;
  const int nu = n_units / kXcd;
  const int s = r * W + ((r & 1) ? W - 1 - i : i);
  if (s >= nu * n_tiles) return false;
  const int j = s / n_tiles;  // this XCD's j-th unit
  const int G = max(1, W / n_tiles);  // units a round covers
  int C = 1;
  if (per_seq % kXcd == 0)
    while (G % (2 * C) == 0 && (per_seq / kXcd) % (2 * C) == 0) C *= 2;
  *unit = ((j / C) * kXcd + x) * C + j % C;
  *tile = s - j * n_tiles;
  return true;
}

// The attention of one work unit: query tile t (0 = the heaviest) of the
// (sequence, head) pair bh, with the K/V rings in sK, sV and this
// wavefront's Q operands in qr. With q_ready, qr already holds the unit's Q
// rows (loaded by the previous unit). With next_q non-null, the rows from
// next_row of the next unit's Q (fixed-length: next_row < N) are loaded into
// qr after the key loop, so their latency overlaps this unit's epilogue.
// F8: q, k, v hold e4m3 codes (one byte each) with per-tensor descale
// factors; S^T runs on the 32x32x64 FP8 MFMA, V is widened to bf16 in LDS one
// tile ahead, and everything after S^T is the 16-bit path (P, O in bf16).
template <int D, int MASK, bool VARLEN, class E, bool F8>
__device__ __forceinline__ void fwd_unit(const FwdArgs &a, int bh, int t,
                                         typename FwdLdsT<D, E, F8>::Ring &sK,
                                         typename FwdLdsT<D, E, F8>::Ring &sV,
                                         typename FwdLdsT<D, E, F8>::Wide &sVb,
                                         QOps<D, E, F8> &qo, bool q_ready,
                                         const void *next_q, int next_row FA_TRACE_PARAM) {
  using Et = typename E::T;   // element type of O, P and the 16-bit inputs
  using E8 = typename E::T8;  // MFMA operand: 8 elements
  using In = std::conditional_t<F8, uint8_t, Et>;  // element type of q, k, v
  using KOp = std::conditional_t<F8, i32x8, E8>;   // S^T MFMA operand
  constexpr int EB = sizeof(In);                   // bytes per input element
  auto &qr = qo.r;
  constexpr int kWaves = FwdShape<D>::kWaves, KB = FwdShape<D>::KB;
  constexpr int kBN = FwdShape<D>::kBN, kBM = FwdShape<D>::kBM;
  constexpr bool CAUSAL = MASK == kMaskCausal;
  constexpr bool LOCAL = MASK == kMaskLocal;  // window a.wl, a.wr (causal: wr = 0)
  // direct-load instructions per copying wavefront per tile (each fills 1 KiB)
  constexpr int kCopyWaves = copy_waves<D>();
  constexpr int kInsts = kBN * D * EB / 1024 / kCopyWaves;
  static_assert(kInsts >= 1 && kInsts * 1024 * kCopyWaves == kBN * D * EB, "copy split");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool copier = kCopyWaves == kWaves || wave < kCopyWaves;  // starts tile copies
  const int cw = copier ? wave : 0;       // its index among the copiers
  const int hf = lane >> 5;
  const int ln = lane & 31;

  // causal: the heaviest query tiles (most keys) are started first
  const int qt = MASK != kMaskNone ? a.n_qtiles - 1 - t : t;
  const int b = bh / a.H;
  const int h = bh - b * a.H;

  int seq0, len;
  if (VARLEN) {
    // a sequence longer than max_seqlen (a.N) is taken as its first a.N
    // rows: every access then stays inside the span the host checked
    seq0 = a.cu_seqlens[b];
    len = min(a.cu_seqlens[b + 1] - seq0, a.N);
  } else {
    seq0 = b * a.N;
    len = a.N;
  }
  if (qt * kBM >= len) return;

  const int rs = a.H * D;  // row stride (elements)
  const size_t base = (size_t)seq0 * rs + (size_t)h * D;
  const In *qg = static_cast<const In *>(a.q) + base;
  const In *kg = static_cast<const In *>(a.k) + base;
  const In *vg = static_cast<const In *>(a.v) + base;

  const int row0 = qt * kBM + wave * 32;  // first row of this wavefront
  const int qrow = row0 + ln;
  // Q rows of a wavefront -> B operands (column = query row); rows past the
  // sequence end are zeros
  auto load_q = [&](const In *q0, int row) {
    if constexpr (F8) {
      // k-step kc of 64: this lane's 32 bytes at 64 kc + 32 hf (the MFMA's A
      // and B operands share one k layout, so any fixed split works)
#pragma unroll
      for (int kc = 0; kc < D / 64; ++kc) {
        const u32x4 lo = row < len ? ld128(q0 + (size_t)row * rs + 64 * kc + 32 * hf) : u32x4{};
        const u32x4 hi =
            row < len ? ld128(q0 + (size_t)row * rs + 64 * kc + 32 * hf + 16) : u32x4{};
        qr[kc] = join8(lo, hi);
      }
    } else if (row < len) {
#pragma unroll
      for (int kc = 0; kc < D / 16; ++kc)
        qr[kc] = E::frag(ld128(q0 + (size_t)row * rs + 16 * kc + 8 * hf));
    } else {
#pragma unroll
      for (int kc = 0; kc < D / 16; ++kc) qr[kc] = E::frag(u32x4{0, 0, 0, 0});
    }
  };

  // keys the workgroup's rows see: tiles kv_beg + j * kBN, j < ntiles
  const int last_row = min((qt + 1) * kBM, len) - 1;
  int kv_beg = 0, kv_end = len;
  if (CAUSAL) kv_end = last_row + 1;
  if (LOCAL) {
    kv_beg = win_lo(qt * kBM, a.wl) / kBN * kBN;
    kv_end = win_hi(last_row, a.wr, len);
  }
  const int ntiles = (kv_end - kv_beg + kBN - 1) / kBN;
  // Window: iteration j takes tile (j + phase) mod ntiles, so that in every
  // iteration the workgroups of a head (whose windows start one query tile,
  // kBM keys, apart) read the key tile whose index is j modulo ntiles: they
  // share that tile in the L2 at the same time, instead of each reading it
  // kBM / kBN iterations after its neighbour. Other masks: tile j.
  int phase = 0;
  if constexpr (LOCAL) phase = (ntiles - (kv_beg / kBN) % ntiles) % ntiles;
  auto tile_of = [&](int j) {  // j < 2 * ntiles
    if constexpr (LOCAL) {
      const int k = j + phase;
      return k >= ntiles ? k - ntiles : k;
    } else {
      return j;
    }
  };
  auto tile_kv = [&](int j) { return kv_beg + tile_of(j) * kBN; };
  // tiles w_lo .. nt_w-1 hold keys this wavefront's rows see
  int w_lo = 0, nt_w = 0;
  if (row0 < len) {
    const int wlast = min(row0 + 31, len - 1);
    const int last_key = CAUSAL ? wlast : LOCAL ? win_hi(wlast, a.wr, len) - 1 : len - 1;
    nt_w = (last_key - kv_beg) / kBN + 1;
    if (LOCAL) w_lo = (win_lo(row0, a.wl) - kv_beg) / kBN;
  }

  // ---- direct global->LDS copies of this wavefront's share of a tile ----
  // Buffer loads: a resource per tensor covering this (sequence, head)'s rows
  // (reads past it return zeros instead of faulting), a scalar tile offset
  // and fixed per-lane offsets. Element e = 512 * (cw * kInsts + i) +
  // 8 * lane of the tile is tile row e / D, chunk (e % D) / 8, stored at LDS
  // chunk chunk ^ swizzle(row).
  const uint32_t span = (uint32_t)(((size_t)(len - 1) * rs + D) * EB);
  const u32x4 rk = make_rsrc(kg, span);
  const u32x4 rv = make_rsrc(vg, span);
  // byte offset in the sequence's rows of the 16-byte chunk that tile byte b
  // (b = 1024 * (cw * kInsts + i) + 16 * lane) holds, for tile row r:
  // chunks are permuted within a row (chunk_swizzle for 16-bit elements, swz8
  // for bytes)
  auto chunk_src = [&](int b, int r) {
    const int row = b / (D * EB), ch = (b % (D * EB)) >> 4;
    int lch;
    if constexpr (F8) lch = ch ^ swz8<D>(row);
    else lch = ch ^ chunk_swizzle<D>(row);
    return (uint32_t)(r * rs * EB + 16 * lch);
  };
  uint32_t goff[kInsts];
#pragma unroll
  for (int i = 0; i < kInsts; ++i) {
    const int b = (cw * kInsts + i) * 1024 + 16 * lane;
    goff[i] = chunk_src(b, b / (D * EB));
  }
  auto issue = [&](In *lds, u32x4 src, int kv0) {
    const uint32_t soff = (uint32_t)kv0 * (uint32_t)rs * EB;
    // formed per call (opaque_sgpr), except in the fixed-length 16-bit d = 256
    // kernels without a window, whose key loop has the scalar registers to
    // hold them and ran 3% slower so
    constexpr bool kHoist = D == 256 && !F8 && !VARLEN && MASK != kMaskLocal;
    const uint32_t woff = (uint32_t)(cw * kInsts * 1024);
    const uint32_t dst = lds_address(lds) + (kHoist ? woff : opaque_sgpr(woff));
    if (kv0 + kBN <= kv_end) {
#pragma unroll
      for (int i = 0; i < kInsts; ++i) load_lds16_at(src, dst + i * 1024, goff[i], soff);
    } else {
      // tail tile: rows past kv_end re-read the last valid row
#pragma unroll
      for (int i = 0; i < kInsts; ++i) {
        const int b = (cw * kInsts + i) * 1024 + 16 * lane;
        const int row = min(b / (D * EB), kv_end - 1 - kv0);
        load_lds16_at(src, dst + i * 1024, chunk_src(b, row), soff);
      }
    }
  };
  // F8: widen the fp8 V tile in ring slot u into bf16 tile vb (all threads
  // of the workgroup, 16 bytes = 16 values each per pass); exact, since
  // every e4m3 value is a bf16 value. In three steps, so the loop can spread
  // them over its MFMAs: widen_read(u, p, w) reads pass p's 16 bytes,
  // widen_cvt(w, k, o) converts word k of them (4 values), widen_store(vb,
  // p, o) writes the 32 bytes.
  constexpr int kWThr = 64 * kWaves, kWPass = F8 ? kBN * D / 16 / kWThr : 1;
  static_assert(!F8 || kWPass * 16 * kWThr == kBN * D, "widen split");
  auto widen_read = [&](int u, int p, u32x4 &w) {
    if constexpr (F8) {
      const int cidx = p * kWThr + tid;
      const int row = cidx / (D / 16), ch = cidx % (D / 16);
      w = ld128(&sV[u][row * D + 16 * (ch ^ swz8<D>(row))]);
    }
  };
  auto widen_cvt = [&](const u32x4 &w, int k, uint32_t (&o)[8]) {
    if constexpr (F8) {
      const auto p0 = __builtin_amdgcn_cvt_pk_f32_fp8(w[k], false);  // bytes 0, 1
      const auto p1 = __builtin_amdgcn_cvt_pk_f32_fp8(w[k], true);   // bytes 2, 3
      o[2 * k] = pack_bf16x2(p0[0], p0[1]);
      o[2 * k + 1] = pack_bf16x2(p1[0], p1[1]);
    }
  };
  auto widen_store = [&](int vb, int p, const uint32_t (&o)[8]) {
    if constexpr (F8) {
      const int cidx = p * kWThr + tid;
      const int row = cidx / (D / 16), ch = cidx % (D / 16);
      // the two 16-byte halves, odd rows high half first
      const int f = row & 1;
      *reinterpret_cast<u32x4 *>(&sVb[vb][tile_off<D>(row, 16 * ch + 8 * f)]) =
          f ? u32x4{o[4], o[5], o[6], o[7]} : u32x4{o[0], o[1], o[2], o[3]};
      *reinterpret_cast<u32x4 *>(&sVb[vb][tile_off<D>(row, 16 * ch + 8 - 8 * f)]) =
          f ? u32x4{o[0], o[1], o[2], o[3]} : u32x4{o[4], o[5], o[6], o[7]};
    }
  };
  auto widen_v = [&](int u, int vb) {
#pragma unroll
    for (int p = 0; p < kWPass; ++p) {
      u32x4 w;
      uint32_t o[8];
      widen_read(u, p, w);
#pragma unroll
      for (int k = 0; k < 4; ++k) widen_cvt(w, k, o);
      widen_store(vb, p, o);
    }
  };
  // V operand tile of iteration j (U = j mod kStages)
  auto v_tile = [&](int u) -> const Et * {
    if constexpr (F8) return sVb[u & 1];
    else return sV[u];
  };

  const float c = a.scale_log2;  // scale * log2(e)
  float m = -INFINITY;           // max of raw scores the exponentials are taken against
  float l = 0.f;                 // this lane's share of the sum of exponentials
  // The sum over P rounded to bf16, accumulated by a 16x16x32 MFMA of
  // a 0/1 matrix with each k-step's P^T operand (a dot-product instruction
  // beside the matrix cores would stall them). Lane g*16 + n of the B
  // operand holds row n + 16 (g % 2) of the tile, so with A[m][k] = 1 when
  // the k-group parity equals (m >= 8), D[m][n] is the row sum of row n for
  // m < 8 and of row n + 16 for m >= 8; lanes 0-15 and 48-63 end up holding
  // their own row's sum and lanes 16-47 their partner's (l ^ 32).
  const uint32_t ones_w = (((lane >> 4) & 1) == ((lane & 15) >> 3)) ? E::kOnes2 : 0u;
  const E8 ones_sel = E::frag(u32x4{ones_w, ones_w, ones_w, ones_w});
  f32x4 lracc = {0.f, 0.f, 0.f, 0.f};
  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};

  const int krow = perm_row32(ln);
  // transposing-read coordinates of this lane (see the V^T operand below)
  const int tg = lane >> 4, ts = lane & 15;
  const int tr_row = 8 * (tg >> 1) + (ts >> 2);
  const int tr_col = 16 * (tg & 1) + 4 * (ts & 3);

  constexpr int NQK = KB * (D / (F8 ? 64 : 16));  // MFMAs of S^T per tile (KB 32-key blocks)
  constexpr int KS = 2 * KB;              // 16-key k-steps of O^T per tile
  constexpr int NPV = KS * (D / 32);      // MFMAs of O^T per tile
#ifndef FA_FWD_PF
#define FA_FWD_PF 3
#endif
  // LDS fragment prefetch distance (MFMAs): 4 in the fixed-length 16-bit
  // d = 256 kernels without a window (1.7% faster; level for FP8, 1.5%
  // slower with a window), else 3 (2 and 4 within 1% at d = 64 and 128)
  constexpr int PF = D == 256 && !F8 && !VARLEN && MASK != kMaskLocal ? 4 : FA_FWD_PF;
  // K operand prefetch distance: FP8 fragments are 32 bytes and feed MFMAs
  // twice as long, so one ahead covers the read (and keeps the registers)
  constexpr int PFK = F8 ? 1 : PF;
  constexpr int NSC = 16 * KB;            // scores per lane per tile
  // Where a tile's exponentials go: k-steps 0 .. KSA-1 (EXA scores) beside
  // the S^T MFMAs of phase 1, the rest beside the first P.V MFMAs of phase 2
  // (before the k-step that needs them is packed). At d = 64 a tile has half
  // the MFMAs per score and the vector ALUs bound the loop, so the split
  // evens their load over both phases (+2.3% at B8 N4096 H16 causal, A/B on
  // one box); at d = 128 the same split was 2-2.5% slower than keeping every
  // exponential in phase 1, so there KSA = KS.
  constexpr int KSA = D == 64 ? (KS + 1) / 2 : KS;  // k-steps exponentiated in phase 1
  constexpr int EXA = 8 * KSA, EXB = NSC - EXA;  // exponentials per phase
  constexpr int CBN = D / 32;             // O^T MFMAs per k-step
  constexpr int NSEG = NPV - CBN;         // phase-2 segments that take exponentials
  static_assert(KS >= 2 && NSEG >= 1, "exponential split");
  // score pairs (summed / maxed) per O^T MFMA, or O^T MFMAs per score pair
  constexpr int PPM = NSC / 2 >= NPV ? NSC / 2 / NPV : 0;
  constexpr int MPP = NSC / 2 >= NPV ? 1 : NPV / (NSC / 2);
  // words of the next k-step packed per O^T MFMA (4 words per k-step, D / 32
  // MFMAs per k-step; for d = 256 the first four MFMAs pack one each)
  constexpr int CPG = D / 32 <= 4 ? 4 / (D / 32) : 1;
  static_assert(exp_schedule_ok(KS, KSA, NPV, CBN, PPM, MPP), "exponential schedule");

  // K operand of S^T MFMA i: key block kb = i % KB, d-chunk kc = i / KB
  // (with two blocks the two accumulation chains alternate). FP8: 32 bytes
  // at 64 kc + 32 hf, the split the Q operand uses.
  auto kfrag = [&](const In *tK, int i) -> KOp {
    const int kc = i / KB, kb = i % KB;
    if constexpr (F8) {
      const int row = 32 * kb + krow, c0 = 4 * kc + 2 * hf;
      const u32x4 lo = ld128(&tK[row * D + 16 * (c0 ^ swz8<D>(row))]);
      const u32x4 hi = ld128(&tK[row * D + 16 * ((c0 + 1) ^ swz8<D>(row))]);
      return join8(lo, hi);
    } else {
      return E::frag(ld128(&tK[tile_off<D>(32 * kb + krow, 16 * kc + 8 * hf)]));
    }
  };

  // V^T operand of O^T MFMA i: k-step kk = i / (D/32), d-block cb = i % (D/32).
  // Lane (m = l % 32, h = l / 32) needs V[16kk + 8h + t][32cb + m], t = 0..7:
  // two transposing reads of 4 keys.
  auto vfrag = [&](const Et *tV, int i) {
    const int kk = i / (D / 32), cb = i % (D / 32);
    const int r0 = 16 * kk + tr_row, c0 = 32 * cb + tr_col;
    const u32x2 lo = ds_read_tr16x4(&tV[tile_off<D>(r0, c0)]);
    const u32x2 hi = ds_read_tr16x4(&tV[tile_off<D>(r0 + 4, c0)]);
    return E::frag(u32x4{lo[0], lo[1], hi[0], hi[1]});
  };
  // keys past the sequence end, after the row (causal) or outside the
  // window -> -inf
  auto need_mask = [&](int kv0) {
    if (LOCAL)
      return (kv0 + kBN > len) || (kv0 + kBN - 1 - row0 > a.wr) || (row0 + 31 - kv0 > a.wl);
    return (kv0 + kBN > len) || (CAUSAL && kv0 + kBN - 1 > row0);
  };
  // Score e of block kb holds key kv0 + 32 kb + perm_row32(8 (e / 4) + 4 hf +
  // e % 4) = kv0 + 8 hf + c with c = 32 kb + perm_row32(8 (e / 4) + e % 4), a
  // constant below 64: two per-lane bounds per tile decide every score, each
  // by one compare with an immediate (key >= len is in the upper bound).
  auto apply_mask = [&](f32x16 (&s)[KB], int kv0) {
    const int base = kv0 + 8 * hf;
    const int hi = opaque_vgpr(
        (LOCAL ? win_hi(qrow, a.wr, len) : CAUSAL ? min(qrow + 1, len) : len) - 1 - base);
    const int lo = LOCAL ? opaque_vgpr(win_lo(qrow, a.wl) - base) : 0;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int c = 32 * kb + perm_row32(8 * (e >> 2) + (e & 3));
        if (c > hi || (LOCAL && c < lo)) s[kb][e] = -INFINITY;
      }
  };
  // score e (0 .. NSC-1) of this lane in a tile: block e / 16, element e % 16
#define FA_SC(s, e) s[(e) >> 4][(e) & 15]

  // One tile j for this wavefront. On entry s holds the masked S^T of tile j
  // and mx its row max; on exit s_next holds the masked S^T of tile j+1
  // (computed on the K tile already resident; unused after the wavefront's
  // last tile) and mx its row max.
  //  phase 1: S^T(j+1) MFMAs, each beside 32/NQK exponentials of tile j;
  //  phase 2: O^T += V^T P^T MFMAs of tile j, each beside packing P to bf16,
  //           the row sums of tile j and the row max of tile j+1.
  // Scheduling fences keep that pairing in the instruction stream; pin()
  // keeps the compiler from sinking the vector work past them.
  // U = j % kStages is a compile-time constant (the loop is unrolled by the
  // ring size), so every LDS address is a lane base plus an immediate.
  // Operand fragments in flight between segments (and, for kf, from the end
  // of one tile into the start of the next).
  KOp kf[NQK];
  E8 vf[NPV];
  float mx = -INFINITY;        // row max of the scores of the next tile to process
  float ms = 0.f;              // m * c of the tile being exponentiated

  // P rounded to bf16 is the MFMA operand. Its row sum lr (of the rounded
  // values) normalises O, so the weights applied to V sum to one and the
  // rounding error of P scales with |v_j - o_i|; the sum l of the unrounded
  // values gives the log-sum-exp. Word w of k-step kk packs this lane's
  // scores 8kk + 2w and 8kk + 2w + 1 (a k-step takes 8 scores per lane).
  uint32_t pw[KS][4];
  // two independent accumulation chains each for the sum and the next
  // tile's max (dependent chains stall the issue)
  float psum[2];
  auto pack = [&](f32x16 (&s)[KB], int kk, int w) {
    const int e = 8 * kk + 2 * w;
    pw[kk][w] = E::pack2(FA_SC(s, e), FA_SC(s, e + 1));
  };

  // First half of tile j: the rescale decision, then phase 1 (S^T(j+1) on
  // the matrix cores beside the exponentials of tile j), then the mask of
  // S^T(j+1).
  auto half_a = [&](auto u_c, int j, f32x16 (&s)[KB], f32x16 (&s_next)[KB]) {
    constexpr int U = decltype(u_c)::value;
    const In *tK = sK[(U + 1) % kStages];   // K(j+1): scores of the next tile
    const Et *tV = v_tile(U % kStages);     // V(j)
    // kf[0 .. PFK-1] (K(j+1)) were read at the end of the previous tile.

    // raise m (and rescale) only when the new max exceeds it by > 2^8;
    // true at a row's first visible key (m = -inf)
    const float m_new = fmaxf(m, mx);
    if (__any((m_new - m) * c > kRescaleLog2)) {
      const float alpha = (m == -INFINITY) ? 0.f : fast_exp2((m - m_new) * c);
      l *= alpha;
      lracc *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i) acc[i] *= alpha;
      m = m_new;
    }
    ms = (m == -INFINITY) ? 0.f : m * c;
    psum[0] = psum[1] = 0.f;
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      if (i + PFK < NQK) kf[i + PFK] = kfrag(tK, i + PFK);
      if (i >= NQK - PF) vf[i - (NQK - PF)] = vfrag(tV, i - (NQK - PF));
      const int kb = i % KB, kc = i / KB;
      s_next[kb] = score_mfma<F8, E>(kf[i], qr[kc], kc == 0 ? f32x16{} : s_next[kb]);
#pragma unroll
      for (int e = seg_lo(i, EXA, NQK); e < seg_lo(i + 1, EXA, NQK); ++e) {
        FA_SC(s, e) = fast_exp2(fmaf(FA_SC(s, e), c, -ms));
        pin(FA_SC(s, e));
      }
      // k-step 0 words whose scores are done
#pragma unroll
      for (int w = 0; w < 4; ++w)
        if (seg_of(2 * w + 1, EXA, NQK) == i) pack(s, 0, w);
      __builtin_amdgcn_sched_barrier(0);
    }

    const int kv_next = tile_kv(j + 1);
    if (need_mask(kv_next)) apply_mask(s_next, kv_next);
    __builtin_amdgcn_sched_barrier(0);
  };

  // Second half of tile j: phase 2, O^T += V^T P^T beside packing P, the row
  // sums of tile j and the row max of tile j+1; it ends by reading the first
  // fragments of K(j+2) for tile j+1. F8: it also widens V(j+1) (landed with
  // the copies waited for at the top of iteration j) into the bf16 tile
  // that V(j-1) held: the read beside the first MFMA, a word of conversions
  // beside each of the next ones, the stores after them. In the last
  // iteration that widens a stale ring slot into a tile nothing reads: the
  // slot is not a copy target then and the tile's last reader passed the
  // iteration's barrier.
  constexpr int kW0 = 2;  // first MFMA the conversions sit beside
  static_assert(!F8 || kW0 + 4 * kWPass <= NPV, "widen schedule");
  auto half_b = [&](auto u_c, int j, f32x16 (&s)[KB], f32x16 (&s_next)[KB]) {
    constexpr int U = decltype(u_c)::value;
    const In *tKn = sK[(U + 2) % kStages];  // K(j+2): first fragments for tile j+1
    const Et *tV = v_tile(U % kStages);     // V(j)
    float mxn[2] = {-INFINITY, -INFINITY};
    u32x4 ww[kWPass];
    uint32_t wo[kWPass][8];
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      const int kk = i / (D / 32), cb = i % (D / 32);
      if (i + PF < NPV) vf[i + PF] = vfrag(tV, i + PF);
      if (i >= NPV - PFK) kf[i - (NPV - PFK)] = kfrag(tKn, i - (NPV - PFK));
      const E8 pb = E::frag(u32x4{pw[kk][0], pw[kk][1], pw[kk][2], pw[kk][3]});
      acc[cb] = E::mfma32(vf[i], pb, acc[cb]);
      if (cb == 0) lracc = E::mfma16(ones_sel, pb, lracc);
      if constexpr (F8) {
#pragma unroll
        for (int p = 0; p < kWPass; ++p) {
          if (i == 0) widen_read((U + 1) % kStages, p, ww[p]);
          if (i >= kW0 + 4 * p && i < kW0 + 4 * p + 4) widen_cvt(ww[p], i - kW0 - 4 * p, wo[p]);
          if (i == kW0 + 4 * p + 3) widen_store((U + 1) & 1, p, wo[p]);
        }
      }
      // the exponentials left from phase 1
      if (i < NSEG) {
#pragma unroll
        for (int e = EXA + seg_lo(i, EXB, NSEG); e < EXA + seg_lo(i + 1, EXB, NSEG); ++e) {
          FA_SC(s, e) = fast_exp2(fmaf(FA_SC(s, e), c, -ms));
          pin(FA_SC(s, e));
        }
      }
      // k-steps 1 .. KSA-1 (done in phase 1): packed one k-step ahead of use,
      // spread over the MFMAs; later k-steps: once their last score is done
      if (kk + 1 < KSA && cb * CPG < 4) {
#pragma unroll
        for (int u = 0; u < CPG; ++u) pack(s, kk + 1, cb * CPG + u);
      }
#pragma unroll
      for (int k2 = KSA; k2 < KS; ++k2)
        if (seg_of(8 * k2 + 7 - EXA, EXB, NSEG) == i)
#pragma unroll
          for (int w = 0; w < 4; ++w) pack(s, k2, w);
      auto sum_max = [&](int p) {  // score pair p of tile j (sum) and j+1 (max)
        const int e = 2 * p, h = p & 1;
        psum[h] += FA_SC(s, e) + FA_SC(s, e + 1);
        mxn[h] = fmaxf(mxn[h], fmaxf(FA_SC(s_next, e), FA_SC(s_next, e + 1)));
        pin(psum[h]);
        pin(mxn[h]);
      };
      if constexpr (PPM > 0) {
#pragma unroll
        for (int u = 0; u < PPM; ++u) sum_max(i * PPM + u);
      } else if (i % MPP == 0) {
        sum_max(i / MPP);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    mx = pair_max(fmaxf(mxn[0], mxn[1]));
    l += psum[0] + psum[1];
  };

  // ---- copy schedule ----
  // Iteration j computes S^T(j+1) (needs K(j+1)) and O += P V(j) (needs
  // V(j)), and reads the first fragments of K(j+2) for iteration j+1. After
  // its barrier it starts the copies of K(j+1+kAhead) and V(j+kAhead); their
  // ring slots held K(j) and V(j-1), last read in iteration j-1. Before the
  // barrier a wavefront waits for its own copies of K(j+2) and V(j): the
  // copies of iteration j-1 stay in flight.
  // copies started by iteration i (U = i mod kStages, a compile-time constant)
  auto start_copies = [&](auto u_c, int i) {
    constexpr int U = decltype(u_c)::value;
    if (!copier) return;
    if (i + 1 + kAhead < ntiles)
      issue(sK[(U + 1 + kAhead) % kStages], rk, tile_kv(i + 1 + kAhead));
    if (i + kAhead < ntiles) issue(sV[(U + kAhead) % kStages], rv, tile_kv(i + kAhead));
  };
  // K(j+2) and V(j) landed (this wavefront's share): only the copies of
  // iteration j-1 may still be in flight, kInsts instructions for each of
  // K(j+kAhead) and V(j-1+kAhead) that exists. Each case waits with a
  // constant count (a count chosen at run time costs a chain of branches on
  // every iteration). A wavefront that copies nothing has nothing to wait for.
  auto wait_copies_of = [&](int j) {
    if (!copier) return;
    if (j + kAhead < ntiles) wait_vmem_n<2 * kInsts + kTraceStores>();
    else if (j - 1 + kAhead < ntiles) wait_vmem_n<kInsts + kTraceStores>();
    else wait_vmem_n<kTraceStores>();
  };

  // ---- prologue: K(0) and the copies of iterations -kAhead .. -1, then
  // the Q block of this wavefront -> B operands (column = query row). All
  // of it is waited for here, so no load is outstanding in the loop except
  // the tile copies, which are counted explicitly.
  if (copier) issue(sK[0], rk, tile_kv(0));
  static_assert(kAhead == 3 && kStages == 4, "prologue below starts iterations -3..-1");
  start_copies(std::integral_constant<int, 1>{}, -3);
  start_copies(std::integral_constant<int, 2>{}, -2);
  start_copies(std::integral_constant<int, 3>{}, -1);
  if (!q_ready) load_q(qg, qrow);
  wait_vmem();
  __syncthreads();
  if constexpr (F8) {
    widen_v(0, 0);  // V(0) lands in ring slot 0
    __syncthreads();
  }
  f32x16 sa[KB], sb[KB];
  // The masked S^T of this wavefront's first tile j (K(j) in tK) and its row
  // max, and the first fragments of K(j+1) (in tKn) for iteration j.
  auto first_scores = [&](const In *tK, const In *tKn, int j, f32x16 (&s)[KB]) {
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const int kb = i % KB, kc = i / KB;
      s[kb] = score_mfma<F8, E>(kfrag(tK, i), qr[kc], kc == 0 ? f32x16{} : s[kb]);
    }
    if (need_mask(tile_kv(j))) apply_mask(s, tile_kv(j));
    mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < NSC; e += 2) mx = fmaxf(mx, fmaxf(FA_SC(s, e), FA_SC(s, e + 1)));
    mx = pair_max(mx);
#pragma unroll
    for (int i = 0; i < PFK; ++i) kf[i] = kfrag(tKn, i);
  };
  // iteration j's tile holds keys this wavefront's rows see
  auto wave_runs = [&](int j) {
    const int k = tile_of(j);
    return k >= w_lo && k < nt_w;
  };
  if (wave_runs(0)) first_scores(sK[0], sK[1], 0, sa);
  FA_TRACE_PRIME;

  // ---- main loop, unrolled by the ring size: slot numbers are constants
  // and the score registers alternate ----
  auto iter = [&](auto u_c, int j, f32x16 (&s)[KB], f32x16 (&s_next)[KB]) {
    constexpr int U = decltype(u_c)::value;
    FA_TRACE_STAMP(t0);
    wait_copies_of(j);
    FA_TRACE_STAMP(ta);
    __syncthreads();
    FA_TRACE_STAMP(tb);
    start_copies(u_c, j);
    FA_TRACE_STAMP(tc);
    FA_TRACE_VARS(t2, t3);
    // F8: V(j+1) landed with the copies waited for above; its bf16 tile is
    // published by the next iteration's barrier (the tile it replaces was
    // last read in iteration j-1). half_b widens it beside its MFMAs; a
    // wavefront that skips the tile widens its share here.
    if (wave_runs(j)) {
      half_a(u_c, j, s, s_next);
      FA_TRACE_SET(t2);
      half_b(u_c, j, s, s_next);
      FA_TRACE_SET(t3);
    } else {
      if constexpr (F8)
        if (j + 1 < ntiles) widen_v((U + 1) % kStages, (U + 1) & 1);
      if (LOCAL && j + 1 < ntiles && wave_runs(j + 1)) {
        // a window's wavefront may skip iterations (at most two runs of
        // tiles, the key range being rotated): the first scores of a run
        // are computed one iteration ahead, like phase 1's
        first_scores(sK[(U + 1) % kStages], sK[(U + 2) % kStages], j + 1, s_next);
      }
    }
    FA_TRACE_RECORD(t0, ta, tb, tc, t2, t3);
  };
  static_assert(kStages == 4, "unroll below");
  for (int j = 0; j < ntiles; j += 4) {
    iter(std::integral_constant<int, 0>{}, j, sa, sb);
    if (j + 1 < ntiles) iter(std::integral_constant<int, 1>{}, j + 1, sb, sa);
    if (j + 2 < ntiles) iter(std::integral_constant<int, 2>{}, j + 2, sa, sb);
    if (j + 3 < ntiles) iter(std::integral_constant<int, 3>{}, j + 3, sb, sa);
  }
  if (next_q != nullptr) load_q(static_cast<const In *>(next_q), next_row);  // qr is free now

#undef FA_SC

  // ---- epilogue: normalise once, store O (bf16) and the log-sum-exp ----
  const float lt = pair_sum(l);
  const float lr_other = swap_halves(lracc[0]);
  const int lg = lane >> 4;
  const float lrt = (lg == 1 || lg == 2) ? lr_other : lracc[0];
  if (qrow < len) {
    // F8: O = sum_j P_j v_j with the codes of v, times v's descale factor
    const float inv = (F8 ? a.v_descale : 1.f) / lrt;
    Et *og = static_cast<Et *>(a.o) + base + (size_t)qrow * rs;
    // Lane (ln, hf) holds d = 32 cb + 8 g + 4 hf + 0..3 of row qrow (ln and
    // ln + 32 share the row). Per pair of g the two lanes trade four values,
    // so each stores 16 bytes: hf = 0 the columns 32 cb + 16 p + 0..7, hf = 1
    // the columns 32 cb + 16 p + 8..15 (half the store instructions). One
    // v_permlane32_swap of (g = 2p, g = 2p + 1) per word pair does the trade:
    // the lower lane keeps its g = 2p word and receives its partner's, the
    // upper lane receives its partner's g = 2p + 1 word and keeps its own.
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        uint32_t we[2], wo[2];  // g = 2p and g = 2p + 1, two packed pairs each
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          we[u] = E::pack2(acc[cb][8 * p + 2 * u] * inv, acc[cb][8 * p + 2 * u + 1] * inv);
          wo[u] = E::pack2(acc[cb][8 * p + 4 + 2 * u] * inv,
                           acc[cb][8 * p + 4 + 2 * u + 1] * inv);
        }
        u32x4 w;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const auto r = __builtin_amdgcn_permlane32_swap(we[u], wo[u], false, false);
          w[u] = r[0];
          w[2 + u] = r[1];
        }
        *reinterpret_cast<u32x4 *>(og + 32 * cb + 16 * p + 8 * hf) = w;
      }
    if (a.lse != nullptr && hf == 0) {
      const size_t li = VARLEN ? (size_t)h * a.cu_seqlens[a.nseq] + seq0 + qrow
                               : ((size_t)b * a.H + h) * a.N + qrow;
      a.lse[li] = (m * c + fast_log2(lt)) * kLn2;
    }
  }
}

// One workgroup per CU. Dispatched (PERS false): one work unit per
// workgroup, ordered by work_order. Persistent (PERS true; fixed-length
// calls whose units split evenly over the XCDs): gridDim.x = the CU count
// and each workgroup runs the units persistent_slot gives it back to back,
// which saves the gap between one workgroup's end and the next one's start
// on a CU and balances the CUs' work statically. Separate instantiations
// keep the loop's live state (and its register pressure) out of the
// dispatched kernel.
template <int D, int MASK, bool VARLEN, class E, bool PERS, bool F8>
__global__ __launch_bounds__(FwdShape<D>::kThreads, 1) void fwd_kernel(FwdArgs a) {
  using In = std::conditional_t<F8, uint8_t, typename E::T>;
  __shared__ __attribute__((aligned(1024))) typename FwdLdsT<D, E, F8>::Ring sK;
  __shared__ __attribute__((aligned(1024))) typename FwdLdsT<D, E, F8>::Ring sV;
  __shared__ __attribute__((aligned(1024))) typename FwdLdsT<D, E, F8>::Wide sVb;
  QOps<D, E, F8> qr;
  int bh, t;
#ifdef FA_FWD_TRACE
  int trace_it = 0;
#endif
  if constexpr (PERS) {
    // fixed-length only: unit (b, h) starts at row b * N, head h
    const int n_units = a.nseq * a.H;
    if (!persistent_slot(0, n_units, a.n_qtiles, a.H, &bh, &t)) return;
    const int lrow = (threadIdx.x >> 6) * 32 + (threadIdx.x & 31);  // row in a unit's tile
    for (int r = 0;; ++r) {
      int nbh = 0, nt = 0;
      const bool next = persistent_slot(r + 1, n_units, a.n_qtiles, a.H, &nbh, &nt);
      const In *nq = nullptr;
      int nrow = 0;
      if (next) {
        const int nb = nbh / a.H;
        nq = static_cast<const In *>(a.q) + (size_t)nb * a.N * a.H * D +
             (size_t)(nbh - nb * a.H) * D;
        nrow = (MASK != kMaskNone ? a.n_qtiles - 1 - nt : nt) * FwdShape<D>::kBM + lrow;
      }
      // the previous unit's last LDS reads are done in every wavefront
      // before this unit's copies refill the rings
      if (r > 0) __syncthreads();
      fwd_unit<D, MASK, VARLEN, E, F8>(a, bh, t, sK, sV, sVb, qr, r > 0, nq, nrow FA_TRACE_ARG);
      if (!next) break;
      bh = nbh;
      t = nt;
    }
  } else {
    work_order(blockIdx.x, a.nseq * a.H, a.n_qtiles, kGroupSlots, a.H, &bh, &t);
    fwd_unit<D, MASK, VARLEN, E, F8>(a, bh, t, sK, sV, sVb, qr, false, nullptr, 0 FA_TRACE_ARG);
  }
}

// Compute units of the current device (cached per device; 0 if unknown,
// which keeps launches dispatched). Calls from several host threads may race
// to fill the cache with the same value.
int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int D, int MASK, bool VARLEN, class E, bool F8 = false>
hipError_t launch(const FwdArgs &a, int n_seq, hipStream_t stream) {
  long long grid = (long long)n_seq * a.H * a.n_qtiles;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  FwdArgs arg = a;
  bool pers = false;
  // persistent: fixed-length, no window, units dealt evenly to the 8 XCDs,
  // and at least four work units per CU (with two, a unit's prologue waits
  // for the previous unit's output stores and the dispatched launch, where
  // the next workgroup's loads overlap them, is as fast or faster)
  const int cus = cu_count();
  if (!VARLEN && MASK != kMaskLocal && cus > 0 && cus % 8 == 0 &&
      ((long long)n_seq * a.H) % 8 == 0 && grid >= 4LL * cus) {
    pers = true;
    grid = cus;
  }
  void *params[] = {&arg};
  const void *kern = reinterpret_cast<const void *>(&fwd_kernel<D, MASK, VARLEN, E, false, F8>);
  if constexpr (!VARLEN && MASK != kMaskLocal) {
    if (pers) kern = reinterpret_cast<const void *>(&fwd_kernel<D, MASK, VARLEN, E, true, F8>);
  }
  return hipLaunchKernel(kern, dim3((unsigned)grid), dim3(FwdShape<D>::kThreads), params, 0,
                         stream);
}

}  // namespace

#if defined(FA_FWD_PLAIN) && defined(FA_FWD_TRACE)
// Copies the timing build's clock stamps to the host (n values, at most the
// size of the record); returns the hipError_t of the copy.
extern "C" int fa_fwd_trace_read(unsigned long long *host, int n) {
  if (n < 0 || n > kTraceGroups * 8 * kTraceIters * 6) return (int)hipErrorInvalidValue;
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_fwd_trace), (size_t)n * sizeof(unsigned long long),
                                  0, hipMemcpyDeviceToHost);
}
#endif

#if defined(FA_FWD_PLAIN)
// Fixed-length launches without a window, bf16 or fp16 inputs (the headline
// kernels). This file is compiled once per group of kernels (FA_FWD_PLAIN,
// and without it the rest), each with its own machine-scheduler strategy;
// the build script states which and why.
hipError_t launch_fwd_plain(const FwdArgs &a, int n_seq, int d, MaskKind mask, ElemKind elem,
                            hipStream_t stream) {
#define FA_CASE(DD, MM, EE) \
  if (d == DD && mask == MM) return launch<DD, MM, false, EE>(a, n_seq, stream);
#define FA_ELEM(EE)              \
  FA_CASE(64, kMaskNone, EE)     \
  FA_CASE(64, kMaskCausal, EE)   \
  FA_CASE(128, kMaskNone, EE)    \
  FA_CASE(128, kMaskCausal, EE)  \
  FA_CASE(256, kMaskNone, EE)    \
  FA_CASE(256, kMaskCausal, EE)
  if (elem == kElemBF16) {
    FA_ELEM(ElemBF16)
  } else if (elem == kElemF16) {
    FA_ELEM(ElemF16)
  }
#undef FA_ELEM
#undef FA_CASE
  return hipErrorInvalidValue;
}
#else
// Fixed-length window launches.
template <int D, class E>
hipError_t launch_window(const FwdArgs &a, int n_seq, hipStream_t stream) {
  return launch<D, kMaskLocal, false, E>(a, n_seq, stream);
}

int fwd_block_m(int d) { return d == 256 ? FwdShape<256>::kBM : FwdShape<128>::kBM; }

hipError_t launch_fwd(const FwdArgs &a, int n_seq, int d, MaskKind mask, bool varlen,
                      ElemKind elem, hipStream_t stream) {
  if (!varlen && elem != kElemFP8 && mask != kMaskLocal)
    return launch_fwd_plain(a, n_seq, d, mask, elem, stream);
  // here: packed sequences (every mask), windows, FP8
#define FA_CASE(DD, EE)                                                         \
  if (d == DD && !varlen) return launch_window<DD, EE>(a, n_seq, stream);      \
  if (d == DD && varlen) {                                                      \
    if (mask == kMaskNone) return launch<DD, kMaskNone, true, EE>(a, n_seq, stream);     \
    if (mask == kMaskCausal) return launch<DD, kMaskCausal, true, EE>(a, n_seq, stream); \
    return launch<DD, kMaskLocal, true, EE>(a, n_seq, stream);                  \
  }
#define FA_ELEM(EE) \
  FA_CASE(64, EE)   \
  FA_CASE(128, EE)  \
  FA_CASE(256, EE)
  if (elem == kElemBF16) {
    FA_ELEM(ElemBF16)
  } else if (elem == kElemF16) {
    FA_ELEM(ElemF16)
  } else if (elem == kElemFP8) {
    // e4m3 inputs, bf16 output; head dimensions 128 and 256
#define FA_F8(DD, MM)                                                              \
  if (d == DD && mask == MM)                                                       \
    return varlen ? launch<DD, MM, true, ElemBF16, true>(a, n_seq, stream)         \
                  : launch<DD, MM, false, ElemBF16, true>(a, n_seq, stream);
    FA_F8(128, kMaskNone)
    FA_F8(128, kMaskCausal)
    FA_F8(128, kMaskLocal)
    FA_F8(256, kMaskNone)
    FA_F8(256, kMaskCausal)
    FA_F8(256, kMaskLocal)
#undef FA_F8
  }
#undef FA_ELEM
#undef FA_CASE
  return hipErrorInvalidValue;
}
#endif

}  // namespace fa
