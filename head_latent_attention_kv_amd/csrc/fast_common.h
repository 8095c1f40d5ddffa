// Types and helpers shared by the MFMA (gfx950) kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace mla {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// v_mfma_f32_32x32x16_{f16,bf16}: D[32x32] += A[32x16] * B[16x32], one wave.
// Lane l supplies A row (l % 32), k-slots 8*(l/32)..+7, and B column (l % 32),
// the same k-slots. D element (m, n) sits in lane n + 32*((m/4) % 2), register
// 4*(m/8) + m%4.
__device__ __forceinline__ f32x16 mfma_f16(half8 a, half8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
template <typename T> struct MfmaOp;
template <> struct MfmaOp<_Float16> {
  typedef half8 vec;
  static __device__ __forceinline__ f32x16 run(vec a, vec b, f32x16 c) { return mfma_f16(a, b, c); }
};
template <> struct MfmaOp<__bf16> {
  typedef bf16x8 vec;
  static __device__ __forceinline__ f32x16 run(vec a, vec b, f32x16 c) { return mfma_bf16(a, b, c); }
};

// Row (within a 32-row MFMA tile) of the D element held by register r of a
// lane in half `lh` (lh = lane / 32).
__device__ __forceinline__ int d_row(int r, int lh) { return 8 * (r >> 2) + 4 * lh + (r & 3); }

// Row order for an operand whose D output is fed straight back in as the
// k-operand of the next product: loading A (or B) row m from source row
// swap23(m) (bits 2 and 3 of m exchanged) makes D registers 8s..8s+7 of half
// lh cover source rows 16s + 8lh .. 16s + 8lh + 7 in order, which is exactly
// the k-slot layout of the next MFMA. The map is its own inverse.
__device__ __forceinline__ int swap23(int m) {
  return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1);
}

__device__ __forceinline__ half8 bf16x8_to_half8(u32x4 v) {
  half8 h;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t w = v[k];
    h[2 * k] = static_cast<_Float16>(__uint_as_float(w << 16));
    h[2 * k + 1] = static_cast<_Float16>(__uint_as_float(w & 0xffff0000u));
  }
  return h;
}

// MFMA A fragment (32 m x 16 k, 16-bit elements) of the transpose of an LDS
// tile T whose rows are k and whose m run contiguously: lane (l % 32, l / 32)
// gets T[8 (l / 32) + j][l % 32], j = 0..7, from two ds_read_b64_tr_b16. In
// one such read, lane i of each 16-lane group receives element i % 4 of the
// 8-byte pieces fetched by lanes i / 4 + 4e (e = 0..3) of its group; so lane
// p of group g fetches row 8 (g / 2) + p / 4 at columns 16 (g % 2) + 4 (p % 4)
// (tr_lane_offset), and every lane of the group then holds four consecutive
// rows of its own column. `p` is the tile corner (k0, m0) plus that offset.
__device__ __forceinline__ int tr_lane_offset(int lane, int row_bytes) {
  const int g = lane >> 4, p = lane & 15;
  return (8 * (g >> 1) + (p >> 2)) * row_bytes + (16 * (g & 1) + 4 * (p & 3)) * 2;
}
typedef short short4v __attribute__((ext_vector_type(4)));
template <int kRowBytes>
__device__ __forceinline__ half8 frag_tr(const char* p) {
  typedef __attribute__((address_space(3))) short4v lds_short4;
  const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p));
  const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p + 4 * kRowBytes));
  const half4 l = __builtin_bit_cast(half4, lo), h = __builtin_bit_cast(half4, hi);
  return half8{l[0], l[1], l[2], l[3], h[0], h[1], h[2], h[3]};
}

// Swizzled LDS rows for 16-bit tiles read both row-wise (16-byte fragment
// loads) and transposed (ds_read_b64_tr_b16): the 16-byte slot s of row r is
// stored at slot s ^ ((r / 4) % 4). With a row pitch of 448 bytes (192
// elements) or 320 bytes (128 elements), row-wise loads of 16 consecutive
// rows then hit 16 different bank slots, and a transposed load's four rows
// (r / 4 equal) share one permutation.
constexpr int XS_ROW = 448;
__device__ __forceinline__ int xs_slot(int row, int slot) { return slot ^ ((row >> 2) & 3); }
// Row-wise fragment of row `row`, k-slots 16 k + 8 lh .. (logical 16-byte
// slot 2 k + lh): byte offset xs_row_base(row, lh, k & 1) + 64 (k / 2).
template <int kRowBytes = XS_ROW>
__device__ __forceinline__ int xs_row_base(int row, int lh, int kpar) {
  return row * kRowBytes + xs_slot(row, 2 * kpar + lh) * 16;
}
// Transposed fragment (see frag_tr) of rows k0 .. k0 + 15 (k0 a multiple of
// 16) and columns 32 dm ..: the two reads are at xs_tr_base(lane, 0) and
// xs_tr_base(lane, 1), each plus k0 * row pitch + 64 dm.
template <int kRowBytes = XS_ROW>
__device__ __forceinline__ int xs_tr_base(int lane, int h) {
  const int g = lane >> 4, p = lane & 15;
  const int row = 8 * (g >> 1) + 4 * h + (p >> 2);
  return row * kRowBytes + xs_slot(row, 2 * (g & 1) + ((p & 3) >> 1)) * 16 + 8 * (p & 1);
}
__device__ __forceinline__ half8 frag_tr2(const char* p0, const char* p1) {
  typedef __attribute__((address_space(3))) short4v lds_short4;
  const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p0));
  const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p1));
  const half4 l = __builtin_bit_cast(half4, lo), h = __builtin_bit_cast(half4, hi);
  return half8{l[0], l[1], l[2], l[3], h[0], h[1], h[2], h[3]};
}

// One wave instruction of global_load_lds (16 bytes per lane) in its
// scalar-base form: lane l reads base + off_l (base wave-uniform, off_l a
// 32-bit byte offset) and its 16 bytes land at lds_dst + 16 l, so the wave
// fills 1 KiB of LDS contiguously (lds_dst wave-uniform, in M0). It is
// issued through inline asm so that the compiler does not track it: the
// compiler waits for every outstanding LDS DMA before a transposed LDS read
// (ds_read_b64_tr_b16), which would serialise each next-tile prefetch with
// the current tile's products. Callers therefore wait for the DMA
// themselves (s_waitcnt vmcnt, then a barrier) before reading what it wrote.
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t off, char* lds_dst) {
  const uint32_t m0 = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)(lds_dst)));
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(m0) : "memory");
}

// Lanes l and l ^ 32 hold the same MFMA column. v_permlane32_swap of x with
// itself leaves x[l % 32] in the first result and x[l % 32 + 32] in the
// second, in every lane (checked on the device), so each lane gets both
// halves' values on the VALU, without the LDS round trip of a lane shuffle.
// Max and sum are commutative, so every lane gets the same bits as
// x op x[l ^ 32].
__device__ __forceinline__ float wave_max_pair(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_sum_pair(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace mla
