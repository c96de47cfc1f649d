// Device-side building blocks shared by the forward and backward kernels:
// vector types for the gfx950 bf16 MFMA operands, 128-bit loads, the
// launch-order remap over the chip's XCDs, and small lane utilities.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(32x32 f32) += A(32x16 bf16) * B(16x32 bf16), one wavefront.
// Operand layout (lane l, half h = l / 32):
//   A: row l % 32, columns 8h .. 8h+7     B: column l % 32, rows 8h .. 8h+7
//   D: column l % 32, rows 8g + 4h + r at element 4g + r (g, r = 0..3)
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld128(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ void st128(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Round two floats to bf16 (nearest even) and pack them, first in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// acc + the two bf16 values packed in w (exact products with 1.0, fp32 sums).
// Takes the packed word itself: extracting bf16 pairs from a bit-cast bf16x8
// vector has been compiled into reads of the first pair only.
__device__ __forceinline__ float sum_bf16x2(uint32_t w, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = __builtin_bit_cast(bf16x2, 0x3f803f80u);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
}

// Round 8 floats to bf16 and pack them; *sum += the 8 rounded values.
__device__ __forceinline__ bf16x8 pack_bf16x8_sum(const float *a, float *sum) {
  const uint32_t r0 = pack_bf16x2(a[0], a[1]);
  const uint32_t r1 = pack_bf16x2(a[2], a[3]);
  const uint32_t r2 = pack_bf16x2(a[4], a[5]);
  const uint32_t r3 = pack_bf16x2(a[6], a[7]);
  float t = sum_bf16x2(r0, *sum);
  t = sum_bf16x2(r1, t);
  t = sum_bf16x2(r2, t);
  *sum = sum_bf16x2(r3, t);
  return as_bf16x8(u32x4{r0, r1, r2, r3});
}

// Forces x to be computed at this point of the instruction stream (an empty
// asm that reads it); used with scheduling fences to pair vector work with
// matrix-core work.
__device__ __forceinline__ void pin(float x) { asm volatile("" ::"v"(x)); }

// Value of `x` held by lane (l ^ 32).
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32, 64);
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
  static_assert(D == 64 || D == 128, "head dim");
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// Element offset of (row, col) in such a tile.
template <int D>
__device__ __forceinline__ int tile_off(int row, int col) {
  return row * D + ((((col >> 3) ^ chunk_swizzle<D>(row))) << 3) + (col & 7);
}

// Copy `rows` x D bf16 (global row stride `rs` elements, rows clamped to
// [0, last_row]) into an LDS tile laid out as above, with direct
// global-to-LDS loads: each wavefront instruction fills 1 KiB of LDS, lane l
// writing bytes 16l..16l+15. The wavefronts of the workgroup split the tile.
template <int D, int ROWS, int NWAVES>
__device__ __forceinline__ void load_tile_to_lds(bf16 *lds, const bf16 *g, int rs, int row0,
                                                 int last_row, int wave, int lane) {
  constexpr int kPerInst = 512;  // bf16 elements per wavefront instruction
  constexpr int kInsts = ROWS * D / kPerInst / NWAVES;
  static_assert(kInsts * kPerInst * NWAVES == ROWS * D, "tile split");
#pragma unroll
  for (int i = 0; i < kInsts; ++i) {
    const int base = (wave * kInsts + i) * kPerInst;  // element offset of this 1 KiB
    const int e = base + 8 * lane;
    const int row = e / D;
    const int lchunk = ((e % D) >> 3) ^ chunk_swizzle<D>(row);
    const int grow = min(row0 + row, last_row);
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void *)(g + (size_t)grow * rs + 8 * lchunk),
        (__attribute__((address_space(3))) void *)(lds + base), 16, 0, 0);
  }
}

// Buffer resource over `bytes` bytes from `base` (raw addressing, stride 0):
// reads at offsets past the end return zeros instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  constexpr int kRawDword3 = 0x00020000;  // 32-bit data format, as raw buffer loads expect
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kRawDword3);
}

// 16-byte direct buffer-to-LDS load: lane l reads src[voff + soff] and writes
// LDS bytes 16l .. 16l+15 from `lds` (the same LDS address in every lane).
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t src, bf16 *lds, uint32_t voff,
                                           uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void *)lds,
                                           16, voff, soff, 0, 0);
}

// Wait until this wavefront's outstanding vector-memory loads (including
// direct-to-LDS loads) have completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Transposing LDS read (gfx950): within each group of 16 lanes, lane i gets
// element r (r = 0..3) = element (i & 3) of the 4 consecutive bf16 that lane
// 4r + (i >> 2) of the group addressed.
__device__ __forceinline__ u32x2 ds_read_tr16x4(const bf16 *p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Global -> LDS staging of a tile of ROWS x D bf16 by 256 threads: a thread
// holds CPT consecutive rows (crow..) of one 8-element column chunk (ccol).
// Store the chunk transposed, dst[col * pitch + row], CPT rows per store.
template <int CPT>
__device__ __forceinline__ void store_transposed(bf16 *dst, int pitch, int ccol, int crow,
                                                 const u32x4 *reg) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint32_t w[CPT];
#pragma unroll
    for (int r = 0; r < CPT; ++r) w[r] = (reg[r][e >> 1] >> (16 * (e & 1))) & 0xffffu;
    if constexpr (CPT == 4) {
      const u32x2 p = {w[0] | (w[1] << 16), w[2] | (w[3] << 16)};
      *reinterpret_cast<u32x2 *>(&dst[(ccol + e) * pitch + crow]) = p;
    } else {
      static_assert(CPT == 2, "two or four rows per thread");
      *reinterpret_cast<uint32_t *>(&dst[(ccol + e) * pitch + crow]) = w[0] | (w[1] << 16);
    }
  }
}

// Exact bf16 -> fp32 of the low / high half of a packed word.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

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

}  // namespace fa
