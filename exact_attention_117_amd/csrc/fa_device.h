// Device-side building blocks shared by the forward and backward kernels:
// vector types for the gfx950 bf16 MFMA operands, 128-bit loads, the
// launch-order remap over the chip's XCDs, and small lane utilities.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(32x32 f32) += A(32x16 bf16) * B(16x32 bf16), one wavefront.
// Operand layout (lane l, half h = l / 32):
//   A: row l % 32, columns 8h .. 8h+7     B: column l % 32, rows 8h .. 8h+7
//   D: column l % 32, rows 8g + 4h + r at element 4g + r (g, r = 0..3)
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(16x16 f32) += A(16x32 bf16) * B(32x16 bf16), one wavefront.
// Lane l supplies A row l % 16 and B column l % 16, 8 values each of the
// k-group l / 16; D: column l % 16, rows 4 (l / 16) .. +3.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D(32x32 f32) += A(32x64 e4m3) * B(64x32 e4m3), one wavefront: the gfx950
// FP8 MFMA (formats 0/0 = OCP e4m3 for both operands, unit block scales
// 2^0). Lane l supplies 32 bytes of row (A) or column (B) l % 32; A and B
// split the 64 k values over the lanes the same way, so loading both with
// one fixed k -> (lane half, byte) map gives the full dot product. D as for
// the 32x32x16 MFMA.
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ u32x4 ld128(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Two 16-byte halves as one 32-byte FP8 MFMA operand.
__device__ __forceinline__ i32x8 join8(u32x4 lo, u32x4 hi) {
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// Round two floats to bf16 (nearest even) and pack them, first in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// Forces x to be computed at this point of the instruction stream (an empty
// asm that reads it); used with scheduling fences to pair vector work with
// matrix-core work.
__device__ __forceinline__ void pin(float x) { asm volatile("" ::"v"(x)); }

// Value of `x` held by lane (l ^ 32). v_permlane32_swap(a, b) trades the
// upper 32 lanes of a with the lower 32 lanes of b; with a = b = x, lane l
// finds its partner's value in the second result (l < 32) or the first.
__device__ __forceinline__ float swap_halves(float x) {
  const auto r =
      __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Row permutation inside a 32-row MFMA block: accumulator row m = 8g + 4h + r
// holds operand row perm_row32(m) (bits 2 and 3 of m swapped). Loading the
// A operand's rows in this order makes the 8 accumulator values a lane later
// feeds as one B operand k-step (rows 8h..8h+7 of a 16-row chunk) correspond
// to 8 consecutive operand rows. It is an involution.
__device__ __forceinline__ int perm_row32(int m) {
  return (m & 3) | ((m & 4) << 1) | ((m & 8) >> 1) | (m & 16);
}

// LDS layout of a row-major [rows][D] bf16 tile with no padding: the 16-byte
// chunks of each row are XOR-permuted by a function of the row. With it, the
// MFMA operand reads (16 consecutive rows, one chunk each, 16 bytes per lane)
// and the transposing reads below (4 consecutive rows, 4 chunks each) touch
// every LDS bank once per 256 bytes.
template <int D>
__device__ __forceinline__ int chunk_swizzle(int row) {
  static_assert(D == 64 || D == 128 || D == 256, "head dim");
  // a 256-element row spans two 256-byte bank cycles; permuting within each
  // half the way 128-element rows are permuted spreads the same accesses
  if constexpr (D >= 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// Element offset of (row, col) in such a tile.
template <int D>
__device__ __forceinline__ int tile_off(int row, int col) {
  return row * D + ((((col >> 3) ^ chunk_swizzle<D>(row))) << 3) + (col & 7);
}

// Buffer resource (4 dwords) over `bytes` bytes from `base`, raw addressing
// with stride 0: reads at offsets past the end return zeros instead of
// faulting. Dword 3 selects the 32-bit data format raw buffer loads expect.
__device__ __forceinline__ u32x4 make_rsrc(const void *base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}

// 16-byte direct buffer-to-LDS load: lane l reads src[voff + soff] and writes
// LDS bytes a + 16l .. a + 16l + 15 (a: a wave-uniform LDS byte address).
// Written as inline asm so the compiler does not track these LDS writes: it
// would otherwise wait for every outstanding copy before any LDS read it
// cannot prove disjoint, which defeats copying several tiles ahead. Callers
// wait with wait_vmem_n() before reading the destination. M0 carries the LDS
// address (one wait state after writing it) and is restored afterwards.
__device__ __forceinline__ void load_lds16_at(u32x4 src, uint32_t a, uint32_t voff, uint32_t soff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(a), "v"(voff), "s"(src), "s"(soff)
      : "memory");
}

// The LDS byte address of p, a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_address(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

// v, passed through an empty asm statement the compiler cannot see through.
// A copy loop forms its LDS destinations from this value plus constants where
// it issues them; otherwise the compiler computes one scalar register per
// ring slot and copy instruction before the main loop and keeps them all
// live, more than the scalar register file holds, and the spills (to lanes
// of vector registers) cost vector instructions in the loop.
__device__ __forceinline__ uint32_t opaque_sgpr(uint32_t v) {
  asm volatile("" : "+s"(v));
  return v;
}

// The same for a per-lane value: a mask formed from it is computed where it
// is applied, not hoisted as one lane mask (a scalar register pair) per
// element out of a loop in which the value does not change.
__device__ __forceinline__ int opaque_vgpr(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// 4-byte direct buffer-to-LDS load: lane l reads src[voff + soff] and writes
// LDS bytes 4l .. 4l+3 from `lds`. Same conventions as load_lds16_at.
__device__ __forceinline__ void load_lds4(u32x4 src, float *lds, uint32_t voff, uint32_t soff) {
  const uint32_t a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) float *)lds;
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(a), "v"(voff), "s"(src), "s"(soff)
      : "memory");
}

// Wait until this wavefront's outstanding vector-memory loads (including
// direct-to-LDS loads) have completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt immediate that waits for at most n outstanding vector-memory
// loads and nothing else (gfx9 encoding: vmcnt bits 3:0 and 15:14).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Wait until at most N of this wavefront's vector-memory loads (and stores)
// are outstanding; they complete in issue order, so the N youngest may still
// be in flight.
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(N));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Transposing LDS read (gfx950): within each group of 16 lanes, lane i gets
// element r (r = 0..3) = element (i & 3) of the 4 consecutive bf16 that lane
// 4r + (i >> 2) of the group addressed.
__device__ __forceinline__ u32x2 ds_read_tr16x4(const void *p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(const_cast<void *>(p)));
  return __builtin_bit_cast(u32x2, v);
}

// Exact bf16 -> fp32 of the low / high half of a packed word.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Element types of the tensors. Every kernel is written once over a traits
// class E: the tensors move as raw 16-bit data, and E gives the MFMA on its
// operands, the fp32 -> element rounding (nearest even) of a packed pair,
// the element -> fp32 widening of each half of a packed word, and two packed
// ones.
struct ElemBF16 {
  typedef __bf16 T;
  typedef bf16x8 T8;
  static constexpr uint32_t kOnes2 = 0x3f803f80u;
  __device__ static T8 frag(u32x4 v) { return __builtin_bit_cast(T8, v); }
  __device__ static f32x16 mfma32(T8 a, T8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static f32x4 mfma16(T8 a, T8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static uint32_t pack2(float lo, float hi) { return pack_bf16x2(lo, hi); }
  __device__ static float lo(uint32_t w) { return bf16_lo(w); }
  __device__ static float hi(uint32_t w) { return bf16_hi(w); }
};

struct ElemF16 {
  typedef _Float16 T;
  typedef f16x8 T8;
  static constexpr uint32_t kOnes2 = 0x3c003c00u;
  __device__ static T8 frag(u32x4 v) { return __builtin_bit_cast(T8, v); }
  __device__ static f32x16 mfma32(T8 a, T8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ static f32x4 mfma16(T8 a, T8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  __device__ static uint32_t pack2(float lo, float hi) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    f16x2 r;
    r[0] = (_Float16)lo;
    r[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, r);
  }
  __device__ static float lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
  }
  __device__ static float hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  }
};

// Sliding-window bounds (the local-attention variant on page
// "FlashAttention技术深度解析", attention variants): row i sees keys
// [win_lo(i, wl), win_hi(i, wr, len)), and key j is seen by rows
// [win_lo(j, wr), win_hi(j, wl, len)). w >= 0, INT_MAX for an unbounded
// side; no intermediate value overflows.
__device__ __forceinline__ int win_lo(int x, int w) { return x > w ? x - w : 0; }
__device__ __forceinline__ int win_hi(int x, int w, int len) {
  return w >= len - x ? len : x + w + 1;
}

// Workgroups are handed to the 8 XCDs round-robin by launch index, and each
// XCD has its own L2. Map launch index -> logical work index so that every
// XCD receives one contiguous range of logical indices (neighbouring tiles of
// one head then share an L2). A bijection on [0, total).
__device__ __forceinline__ int xcd_remap(int wg, int total) {
  constexpr int kXcd = 8;
  const int q = total / kXcd, r = total % kXcd;
  const int x = wg % kXcd, s = wg / kXcd;
  return x * q + (x < r ? x : r) + s;
}

// Work order of a launch of n_units x n_tiles workgroups, where unit u's
// tile 0 is its heaviest, run `slots` workgroups at a time per XCD; units are
// numbered (sequence, head), `per_seq` units per sequence. The hardware hands
// workgroups to the 8 XCDs round-robin (launch index % 8) and each XCD has its
// own L2. When the units split evenly over the XCDs, each XCD runs its units
// in groups of G, G*n_tiles ~ slots; the k-th workgroup of a group takes tile
// k / G of its unit k % G. A group's heaviest tiles start first and the next
// group fills the slots its light tiles free, so few units (and their K/V) are
// live per L2 at a time and the launch does not end on a late heavy tile.
// The units are dealt to the XCDs in chunks of C adjacent heads, round-robin,
// with C dividing per_seq / 8: every XCD then gets the same heads of every
// sequence, so sequences of different lengths load the XCDs evenly, and
// adjacent heads (adjacent in memory, which the L2 serves with fewer fetches
// than heads 8 apart) stay together. If the units do not split evenly over
// the XCDs, each XCD gets a contiguous range of (unit, tile) pairs.
// A bijection.
__device__ __forceinline__ void work_order(int wg, int n_units, int n_tiles, int slots,
                                           int per_seq, int *unit, int *tile) {
  constexpr int kXcd = 8;
  if (n_units % kXcd == 0) {
    const int nu = n_units / kXcd;
    const int x = wg % kXcd, k = wg / kXcd;
    const int G = max(1, min(nu, slots / n_tiles));
    const int g = k / (G * n_tiles), r = k - g * (G * n_tiles);
    const int gsz = min(G, nu - g * G);  // the last group may be smaller
    const int j = g * G + r % gsz;       // this XCD's j-th unit
    // chunk: the largest power of two dividing G and per_seq / 8 (1 if
    // per_seq is not a multiple of 8); it divides nu
    int C = 1;
    if (per_seq % kXcd == 0)
      while (G % (2 * C) == 0 && (per_seq / kXcd) % (2 * C) == 0) C *= 2;
    *unit = ((j / C) * kXcd + x) * C + j % C;
    *tile = r / gsz;
  } else {
    const int logical = xcd_remap(wg, n_units * n_tiles);
    *unit = logical / n_tiles;
    *tile = logical - *unit * n_tiles;
  }
}

}  // namespace fa
