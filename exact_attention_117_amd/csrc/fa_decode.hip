// Decoding against a paged key/value cache, for gfx950.
//
// Method: the attention of the newest queries of each sequence over the keys
// and values held in its cache (page "FlashAttention技术深度解析": causal
// attention with KV-cache incremental decoding, and the paged KV cache among
// its inference optimisations). Logical key j of sequence b lives in page
// block_table[b][j / page], slot j % page; query i of Nq sits at position
// L - Nq + i and the causal / window rules apply to that position. The keys
// are split into chunks whose partial (max, sum, output) are merged with the
// running-statistics rule of page "FlashAttention实战" section 3.1.
//
// With one to four queries per sequence the work is a stream over the cache:
// each key/value byte is used by at most four queries, so the kernel is
// bound by HBM bandwidth, not by the matrix cores, and computes on the
// vector ALUs in fp32 (P is never rounded to bf16 here).
//
// Launches, all on the caller's stream:
//   append_kernel : (optional) writes k_new / v_new into the cache at
//                   positions cache_seqlens[b] .. + Nq - 1;
//   decode_kernel : one workgroup per (sequence, head group, query chunk,
//                   key split). A head's d values are spread over d / 8
//                   lanes (16 bytes each), so a workgroup reads 2 KiB of
//                   consecutive bytes of every key row (the cache's
//                   [page, H, d] layout keeps a row's heads adjacent); the
//                   score of a key is reduced across those lanes with DPP
//                   row operations. Keys are loaded 8 at a time into two
//                   register sets: with one query the next 8 keys' loads are
//                   always in flight while 8 are computed; with more queries
//                   (more registers per key) 16 keys' loads are issued
//                   together and the first 8 computed while the rest land;
//   merge_kernel  : one wavefront per query row combines the splits' (max,
//                   sum, output) and writes O (bf16) and the log-sum-exp.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kKeys = 8;  // keys per step
constexpr int kMaxQ = 4;  // queries per workgroup (query chunk)

// Sum of x over the groups of G (8, 16 or 32) consecutive lanes, in every
// lane of the group (DPP: swap neighbours, swap pairs, mirror within 8,
// mirror within 16; then the two 16-lane rows of a 32-lane group exchange
// their sums with one permlane16 swap).
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));
  if constexpr (G >= 16)
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, true));
  if constexpr (G == 32) {
    // rows (0,1) and (2,3): r[0] holds the even row's value in both rows of
    // a pair, r[1] the odd row's
    const auto r =
        __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return x;
}

__global__ __launch_bounds__(kThreads) void append_kernel(DecodeArgs a, int d) {
  const int cpr = a.H * d / 8;  // 16-byte chunks per row
  const long long idx = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (long long)a.B * a.Nq * cpr) return;
  const int r = (int)(idx / cpr), c = (int)(idx % cpr);
  const int b = r / a.Nq, t = r - b * a.Nq;
  const int pos = a.cache_seqlens[b] + t;
  const int pg = pos >> a.page_shift;
  if (pos < 0 || pg >= a.max_pages) return;  // no such page: nothing written
  const int blk = a.block_table[(size_t)b * a.max_pages + pg];
  if (blk < 0 || blk >= a.num_pages) return;
  const size_t dst = ((size_t)blk * a.page + (pos & (a.page - 1))) * cpr + c;
  const size_t src = (size_t)r * cpr + c;
  reinterpret_cast<u32x4 *>(a.k_cache)[dst] = reinterpret_cast<const u32x4 *>(a.k_new)[src];
  reinterpret_cast<u32x4 *>(a.v_cache)[dst] = reinterpret_cast<const u32x4 *>(a.v_new)[src];
}

template <int D, int NQ, class E>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  using Et = typename E::T;  // element type of the tensors
  const Et *Qg = static_cast<const Et *>(a.q);
  const Et *Kc = static_cast<const Et *>(a.k_cache), *Vc = static_cast<const Et *>(a.v_cache);
  constexpr int LPH = D / 8;             // lanes per head
  constexpr int HPW = kThreads / LPH;    // heads per workgroup
  int w = blockIdx.x;
  const int s = w % a.nsplit;
  w /= a.nsplit;
  const int qc = w % a.nqc;
  w /= a.nqc;
  const int n_hg = (a.H + HPW - 1) / HPW;
  const int hg = w % n_hg;
  const int b = w / n_hg;

  const int tid = threadIdx.x;
  const int h = hg * HPW + tid / LPH;
  const int ch = tid % LPH;  // this lane's 8 values of d
  const bool live = h < a.H;
  const int L = a.cache_seqlens[b] + a.n_new;  // keys held, appended ones included
  const int q0 = qc * NQ;
  const int nq = min(NQ, a.Nq - q0);
  const int pos0 = L - a.Nq + q0;  // position of this chunk's first query

  // keys of this split that any of the chunk's queries sees (and that the
  // block table can address)
  int lo = s * a.split_len, hi = min(min(L, lo + a.split_len), a.max_pages << a.page_shift);
  lo = max(lo, win_lo(pos0, a.wl));
  hi = min(hi, win_hi(pos0 + nq - 1, a.wr, L));

  const float c = a.scale_log2;
  const size_t rs = (size_t)a.H * D;  // elements per cache / query row
  float qv[NQ][8];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    u32x4 w4 = {0, 0, 0, 0};
    if (live && i < nq) w4 = ld128(Qg + ((size_t)b * a.Nq + q0 + i) * rs + (size_t)h * D + 8 * ch);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[i][2 * e] = E::lo(w4[e]);
      qv[i][2 * e + 1] = E::hi(w4[e]);
    }
  }
  float m[NQ], l[NQ], o[NQ][8];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[i][e] = 0.f;
  }

  const int32_t *bt = a.block_table + (size_t)b * a.max_pages;
  // Loads of keys j0 .. j0+7; ok[u]: the key exists and its page id is
  // valid. Every lane loads unconditionally (no branches between the loads,
  // so they issue back to back): absent keys read row 0 of page 0 and dead
  // lanes (h >= H) their row's last head, and are masked out afterwards.
  const size_t lane_off_c = (size_t)min(h, a.H - 1) * D + 8 * ch;
  auto load = [&](int j0, u32x4 (&kr)[kKeys], u32x4 (&vr)[kKeys], bool (&ok)[kKeys]) {
    int blk[kKeys];
#pragma unroll
    for (int u = 0; u < kKeys; ++u) blk[u] = bt[min(j0 + u, hi - 1) >> a.page_shift];
#pragma unroll
    for (int u = 0; u < kKeys; ++u) {
      const int j = j0 + u;
      ok[u] = j < hi && blk[u] >= 0 && blk[u] < a.num_pages;
      const size_t row = ok[u] ? (size_t)blk[u] * a.page + (j & (a.page - 1)) : 0;
      kr[u] = ld128(Kc + row * rs + lane_off_c);
      vr[u] = ld128(Vc + row * rs + lane_off_c);
    }
  };
  // values of absent keys are zeroed before use (their weight is 0, and
  // whatever the substitute row holds must not reach O as 0 * inf)
  auto drop_absent = [&](u32x4 (&vr)[kKeys], const bool (&ok)[kKeys]) {
#pragma unroll
    for (int u = 0; u < kKeys; ++u)
      if (!ok[u]) vr[u] = u32x4{0, 0, 0, 0};
  };
  auto compute = [&](int j0, const u32x4 (&kr)[kKeys], u32x4 (&vr)[kKeys],
                     const bool (&ok)[kKeys]) {
    drop_absent(vr, ok);
    // scores, masked -> -inf
    float sc[NQ][kKeys];
#pragma unroll
    for (int u = 0; u < kKeys; ++u) {
      float kf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[2 * e] = E::lo(kr[u][e]);
        kf[2 * e + 1] = E::hi(kr[u][e]);
      }
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) p = fmaf(qv[i][e], kf[e], p);
        p = group_sum<LPH>(p);
        const int j = j0 + u, pos = pos0 + i;
        const bool vis = ok[u] && j - pos <= a.wr && pos - j <= a.wl;
        sc[i][u] = vis ? p : -INFINITY;
      }
    }
    // online softmax update per query, then O += P V
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      float gm = sc[i][0];
#pragma unroll
      for (int u = 1; u < kKeys; ++u) gm = fmaxf(gm, sc[i][u]);
      const float mn = fmaxf(m[i], gm);
      const float alpha = (m[i] == -INFINITY) ? 0.f : fast_exp2((m[i] - mn) * c);
      const float ms = (mn == -INFINITY) ? 0.f : mn * c;
      m[i] = mn;
      l[i] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[i][e] *= alpha;
#pragma unroll
      for (int u = 0; u < kKeys; ++u) {
        const float p = fast_exp2(fmaf(sc[i][u], c, -ms));
        l[i] += p;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[i][2 * e] = fmaf(p, E::lo(vr[u][e]), o[i][2 * e]);
          o[i][2 * e + 1] = fmaf(p, E::hi(vr[u][e]), o[i][2 * e + 1]);
        }
      }
    }
  };
  if constexpr (NQ == 1) {
    // Two groups of 8 keys in flight at all times: the loads of group g + 1
    // are issued before group g is computed, so the loads never wait for the
    // vector ALUs (two register sets alternate; the loop is unrolled by two
    // to keep their roles fixed). 1.6% faster than the scheme below at one
    // query; with more queries its registers would cost occupancy.
    u32x4 ka[kKeys], va[kKeys], kb[kKeys], vb[kKeys];
    bool oka[kKeys], okb[kKeys];
    if (lo < hi) load(lo, ka, va, oka);
    for (int j0 = lo; j0 < hi; j0 += 2 * kKeys) {
      if (j0 + kKeys < hi) load(j0 + kKeys, kb, vb, okb);
      compute(j0, ka, va, oka);
      if (j0 + kKeys >= hi) break;
      if (j0 + 2 * kKeys < hi) load(j0 + 2 * kKeys, ka, va, oka);
      compute(j0 + kKeys, kb, vb, okb);
    }
  } else {
    // 16 keys per iteration: all 32 loads are issued first, and the first 8
    // keys are computed while the loads of the second 8 are still in flight
    for (int j0 = lo; j0 < hi; j0 += 2 * kKeys) {
      u32x4 ka[kKeys], va[kKeys], kb[kKeys], vb[kKeys];
      bool oka[kKeys], okb[kKeys];
      load(j0, ka, va, oka);
      load(j0 + kKeys, kb, vb, okb);
      compute(j0, ka, va, oka);
      compute(j0 + kKeys, kb, vb, okb);
    }
  }

  // this split's partial results (an empty split writes max -inf, sum 0, O 0)
  if (!live) return;
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    if (i >= nq) break;
    const size_t row = (((size_t)b * a.Nq + q0 + i) * a.nsplit + s) * a.H + h;
    float *po = a.part_o + row * D + 8 * ch;
    *reinterpret_cast<f32x4 *>(po) = f32x4{o[i][0], o[i][1], o[i][2], o[i][3]};
    *reinterpret_cast<f32x4 *>(po + 4) = f32x4{o[i][4], o[i][5], o[i][6], o[i][7]};
    if (ch == 0) {
      a.part_ml[2 * row] = m[i] == -INFINITY ? -INFINITY : m[i] * c;
      a.part_ml[2 * row + 1] = l[i];
    }
  }
}

// One wavefront per (sequence, query, head) row: the lanes first take the
// maximum over the splits, then groups of D / 8 lanes each sum a share of
// the splits' weighted outputs (8 values of d per lane), and the groups'
// sums are added across lanes.
template <int D, class E>
__global__ __launch_bounds__(kThreads) void merge_kernel(DecodeArgs a) {
  using Et = typename E::T;
  constexpr int LPH = D / 8;
  constexpr int G = 64 / LPH;  // split groups per wavefront
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= (long long)a.B * a.Nq * a.H) return;
  const int h = (int)(row % a.H);
  const long long r = row / a.H;  // b * Nq + i
  const size_t base = (size_t)r * a.nsplit * a.H + h;  // split 0 of this row
  const float *ml = a.part_ml;
  float mx = -INFINITY;
  for (int s = lane; s < a.nsplit; s += 64) mx = fmaxf(mx, ml[2 * (base + (size_t)s * a.H)]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));

  const int g = lane / LPH, ch = lane % LPH;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float sum = 0.f;
  if (mx != -INFINITY) {
#pragma unroll 4
    for (int s = g; s < a.nsplit; s += G) {
      const size_t sr = base + (size_t)s * a.H;
      const float wgt = fast_exp2(ml[2 * sr] - mx);  // 0 for an empty split
      sum = fmaf(wgt, ml[2 * sr + 1], sum);
      const f32x4 x0 = *reinterpret_cast<const f32x4 *>(a.part_o + sr * D + 8 * ch);
      const f32x4 x1 = *reinterpret_cast<const f32x4 *>(a.part_o + sr * D + 8 * ch + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] = fmaf(wgt, x0[e], acc[e]);
        acc[4 + e] = fmaf(wgt, x1[e], acc[4 + e]);
      }
    }
  }
#pragma unroll
  for (int off = LPH; off < 64; off <<= 1) {
    sum += __shfl_xor(sum, off, 64);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off, 64);
  }
  if (g != 0) return;
  const float inv = mx == -INFINITY ? 0.f : 1.f / sum;
  const long long b = r / a.Nq, i = r % a.Nq;
  Et *og = static_cast<Et *>(a.o) + ((size_t)r * a.H + h) * D + 8 * ch;
  *reinterpret_cast<u32x4 *>(og) =
      u32x4{E::pack2(acc[0] * inv, acc[1] * inv), E::pack2(acc[2] * inv, acc[3] * inv),
            E::pack2(acc[4] * inv, acc[5] * inv), E::pack2(acc[6] * inv, acc[7] * inv)};
  if (a.lse != nullptr && ch == 0)
    a.lse[((size_t)b * a.H + h) * a.Nq + i] =
        mx == -INFINITY ? -INFINITY : (mx + fast_log2(sum)) * kLn2;
}

template <int D, int NQ, class E>
hipError_t launch_all(const DecodeArgs &a, hipStream_t stream) {
  constexpr int HPW = kThreads / (D / 8);
  if (a.n_new > 0) {
    const long long n = (long long)a.B * a.Nq * a.H * D / 8;
    const long long grid = (n + kThreads - 1) / kThreads;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    DecodeArgs arg = a;
    int d = D;
    void *params[] = {&arg, &d};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&append_kernel),
                                   dim3((unsigned)grid), dim3(kThreads), params, 0, stream);
    if (e != hipSuccess) return e;
  }
  {
    const long long grid =
        (long long)a.B * ((a.H + HPW - 1) / HPW) * a.nqc * a.nsplit;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    DecodeArgs arg = a;
    void *params[] = {&arg};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&decode_kernel<D, NQ, E>),
                                   dim3((unsigned)grid), dim3(kThreads), params, 0, stream);
    if (e != hipSuccess) return e;
  }
  const long long rows = (long long)a.B * a.Nq * a.H;  // one wavefront each
  const long long grid = (rows + kThreads / 64 - 1) / (kThreads / 64);
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  DecodeArgs arg = a;
  void *params[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void *>(&merge_kernel<D, E>), dim3((unsigned)grid),
                         dim3(kThreads), params, 0, stream);
}

}  // namespace

int decode_queries_per_chunk() { return kMaxQ; }

hipError_t launch_decode(const DecodeArgs &a, int d, ElemKind elem, hipStream_t stream) {
  if (a.B == 0 || a.Nq == 0 || a.H == 0) return hipSuccess;
  const int nq = a.nqc > 1 ? kMaxQ : a.Nq;  // queries per chunk (1..4)
#define FA_CASE(DD, EE)                                         \
  if (d == DD) {                                                \
    if (nq == 1) return launch_all<DD, 1, EE>(a, stream);      \
    if (nq == 2) return launch_all<DD, 2, EE>(a, stream);      \
    return launch_all<DD, 4, EE>(a, stream);                   \
  }
  if (elem == kElemBF16) {
    FA_CASE(64, ElemBF16)
    FA_CASE(128, ElemBF16)
    FA_CASE(256, ElemBF16)
  } else if (elem == kElemF16) {
    FA_CASE(64, ElemF16)
    FA_CASE(128, ElemF16)
    FA_CASE(256, ElemF16)
  }
#undef FA_CASE
  return hipErrorInvalidValue;
}

}  // namespace fa
