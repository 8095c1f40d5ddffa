// MFMA GEMM and layout conversions for the fast path.
//
// The latent up-projection (LAGA abstract: per-head K/V rebuilt from the
// gathered latent) and the backward's latent and weight gradients are all
// plain GEMMs with K = d_c, n_h*(d_nope+d_v) or the key count. One kernel
// covers them: both operands are read k-contiguous (so a lane's 8 k-values
// are one 16-byte LDS read), 128x128 output tiles, 64-deep k-chunks staged
// through LDS with a register prefetch of the next chunk, and the result is
// staged through LDS so every global store is a full 16-byte row piece.
#include "fast.h"
#include "fast_common.h"

namespace mla {
namespace {

constexpr int kT = 128;        // tile rows / cols
constexpr int kKC = 64;        // k per chunk
constexpr int kLS = kKC + 8;   // LDS row stride (elements): 144 B, conflict-free 16 B reads

template <typename InT, typename OutT>
__global__ void __launch_bounds__(256)
gemm_nt_kernel(const InT* __restrict__ X, int64_t ldx, int64_t R, const InT* __restrict__ Y,
               int64_t ldy, int64_t C, int64_t K, OutT* __restrict__ out, int64_t ldo,
               int64_t rt_stride, int64_t ct_stride, int64_t R_store, int64_t C_store) {
  typedef typename MfmaOp<InT>::vec vec;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2][2][kT * kLS];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5;
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * kT;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kT;
  const int rw = (w & 1) * 64, cw = (w >> 1) * 64;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  u32x4 pre[8];
  auto load = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 8;
      const int64_t gr = r0 + row, gc = c0 + row;
      const u32x4 z = {0u, 0u, 0u, 0u};
      pre[i] = gr < R ? *reinterpret_cast<const u32x4*>(X + gr * ldx + k0 + col) : z;
      pre[4 + i] = gc < C ? *reinterpret_cast<const u32x4*>(Y + gc * ldy + k0 + col) : z;
    }
  };
  auto store = [&](int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 8;
      *reinterpret_cast<u32x4*>(&smem[st][0][row * kLS + col]) = pre[i];
      *reinterpret_cast<u32x4*>(&smem[st][1][row * kLS + col]) = pre[4 + i];
    }
  };

  const int nk = static_cast<int>(K / kKC);
  load(0);
  store(0);
  __syncthreads();
  for (int kc = 0; kc < nk; ++kc) {
    const int st = kc & 1;
    if (kc + 1 < nk) load(static_cast<int64_t>(kc + 1) * kKC);
    const uint16_t* sx = smem[st][0];
    const uint16_t* sy = smem[st][1];
#pragma unroll
    for (int s = 0; s < kKC / 16; ++s) {
      vec a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const vec*>(sy + (cw + 32 * i + lr) * kLS + 16 * s + 8 * lh);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const vec*>(sx + (rw + 32 * j + lr) * kLS + 16 * s + 8 * lh);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = MfmaOp<InT>::run(a[i], b[j], acc[i][j]);
    }
    if (kc + 1 < nk) store(st ^ 1);
    __syncthreads();
  }

  // D[m = c][n = r]: this lane holds output row r, four consecutive columns per group
  constexpr int SS = kT + (sizeof(OutT) == 4 ? 4 : 8);
  OutT* stg = reinterpret_cast<OutT*>(&smem[0][0][0]);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r = rw + 32 * j + lr;
        const int c = cw + 32 * i + 8 * g + 4 * lh;
        if constexpr (sizeof(OutT) == 4) {
          f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                     acc[i][j][4 * g + 3]};
          *reinterpret_cast<f32x4*>(stg + r * SS + c) = v;
        } else {
          half4 v = {static_cast<_Float16>(acc[i][j][4 * g]),
                     static_cast<_Float16>(acc[i][j][4 * g + 1]),
                     static_cast<_Float16>(acc[i][j][4 * g + 2]),
                     static_cast<_Float16>(acc[i][j][4 * g + 3])};
          *reinterpret_cast<half4*>(stg + r * SS + c) = v;
        }
      }
  __syncthreads();
  constexpr int EPC = 16 / sizeof(OutT);   // elements per 16-byte piece
  constexpr int CPR = kT / EPC;            // pieces per row
  OutT* base = out + (r0 / kT) * rt_stride + (c0 / kT) * ct_stride;
  for (int c = tid; c < kT * CPR; c += 256) {
    const int row = c / CPR, cc = (c % CPR) * EPC;
    if (r0 + row >= R_store || c0 + cc >= C_store) continue;
    *reinterpret_cast<u32x4*>(base + row * ldo + cc) =
        *reinterpret_cast<const u32x4*>(stg + row * SS + cc);
  }
}

template <typename OutT>
__device__ __forceinline__ OutT from_bf16(uint16_t b) {
  if constexpr (sizeof(OutT) == 2 && __is_same(OutT, uint16_t)) {
    return b;
  } else {
    return static_cast<OutT>(bf16_to_f32(b));
  }
}

// 64x64 tile transpose through LDS; grid (cols/64, rows/64, batch).
template <typename OutT>
__global__ void __launch_bounds__(256)
transpose_kernel(const uint16_t* __restrict__ in, int64_t ld_in, int64_t in_batch,
                 int64_t rows_valid, int64_t rows, int64_t cols, OutT* __restrict__ out,
                 int64_t ld_out, int64_t out_batch) {
  __shared__ uint16_t t[64][65];
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * 64;
  in += blockIdx.z * in_batch;
  out += blockIdx.z * out_batch;
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int rr = e >> 6, cc = e & 63;
    const int64_t r = r0 + rr, c = c0 + cc;
    t[rr][cc] = (r < rows_valid && c < cols) ? in[r * ld_in + c] : static_cast<uint16_t>(0);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int cc = e >> 6, rr = e & 63;
    const int64_t r = r0 + rr, c = c0 + cc;
    if (r < rows && c < cols) out[c * ld_out + r] = from_bf16<OutT>(t[rr][cc]);
  }
}

template <typename OutT>
__global__ void __launch_bounds__(256)
convert_kernel(const uint16_t* __restrict__ in, int64_t ld_in, int64_t in_batch,
               int64_t rows_valid, int64_t rows, int64_t cols, OutT* __restrict__ out,
               int64_t ld_out, int64_t out_batch) {
  in += blockIdx.z * in_batch;
  out += blockIdx.z * out_batch;
  const int64_t n = rows * cols;
  for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < n;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t r = e / cols, c = e % cols;
    out[r * ld_out + c] =
        r < rows_valid ? from_bf16<OutT>(in[r * ld_in + c]) : static_cast<OutT>(0);
  }
}

// out[b][r][0..cols) = fp16(in[r][0..cols)) for r < rows_valid, 0 for
// rows_valid <= r < rows; b < batch (out advanced by out_batch). 16 bytes per
// thread; cols, ld_in and ld_out multiples of 8.
__global__ void __launch_bounds__(256)
broadcast_rows_f16_kernel(const uint16_t* __restrict__ in, int64_t ld_in, int64_t rows_valid,
                          int64_t rows, int cols, _Float16* __restrict__ out, int64_t ld_out,
                          int64_t out_batch, int batch) {
  const int cpr = cols / 8;
  const int64_t n = static_cast<int64_t>(batch) * rows * cpr;
  for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < n;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int c = static_cast<int>(e % cpr);
    const int64_t r = (e / cpr) % rows;
    const int64_t b = e / (cpr * rows);
    half8 v;
    if (r < rows_valid) {
      v = bf16x8_to_half8(*reinterpret_cast<const u32x4*>(in + r * ld_in + c * 8));
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = static_cast<_Float16>(0.f);
    }
    *reinterpret_cast<half8*>(out + b * out_batch + r * ld_out + c * 8) = v;
  }
}

}  // namespace

mla_status launch_broadcast_rows_f16(const uint16_t* in, int64_t ld_in, int64_t rows_valid,
                                     int64_t rows, int cols, _Float16* out, int64_t ld_out,
                                     int64_t out_batch, int batch, hipStream_t st,
                                     const char* name) {
  if (cols % 8 || ld_in % 8 || ld_out % 8 || out_batch % 8)
    return fail(MLA_ERR_UNSUPPORTED, "%s: widths must be multiples of 8", name);
  int64_t blocks = (static_cast<int64_t>(batch) * rows * (cols / 8) + 255) / 256;
  blocks = blocks < 1 ? 1 : (blocks > 16384 ? 16384 : blocks);
  KernelTimer kt(name, st);
  hipLaunchKernelGGL(broadcast_rows_f16_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     st, in, ld_in, rows_valid, rows, cols, out, ld_out, out_batch, batch);
  return check_launch(name);
}

mla_status launch_transpose(const uint16_t* in, int64_t ld_in, int64_t in_batch, int64_t rows_valid,
                            int64_t rows, int64_t cols, void* out, int64_t ld_out,
                            int64_t out_batch, Elem out_t, int batch, hipStream_t st,
                            const char* name) {
  dim3 grid(static_cast<unsigned>((cols + 63) / 64), static_cast<unsigned>((rows + 63) / 64),
            static_cast<unsigned>(batch));
  KernelTimer kt(name, st);
  if (out_t == Elem::F16)
    hipLaunchKernelGGL(transpose_kernel<_Float16>, grid, dim3(256), 0, st, in, ld_in, in_batch,
                       rows_valid, rows, cols, static_cast<_Float16*>(out), ld_out, out_batch);
  else
    hipLaunchKernelGGL(transpose_kernel<uint16_t>, grid, dim3(256), 0, st, in, ld_in, in_batch,
                       rows_valid, rows, cols, static_cast<uint16_t*>(out), ld_out, out_batch);
  return check_launch(name);
}

mla_status launch_convert(const uint16_t* in, int64_t ld_in, int64_t in_batch, int64_t rows_valid,
                          int64_t rows, int64_t cols, void* out, int64_t ld_out, int64_t out_batch,
                          Elem out_t, int batch, hipStream_t st, const char* name) {
  int64_t blocks = (rows * cols + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  dim3 grid(static_cast<unsigned>(blocks), 1, static_cast<unsigned>(batch));
  KernelTimer kt(name, st);
  if (out_t == Elem::F16)
    hipLaunchKernelGGL(convert_kernel<_Float16>, grid, dim3(256), 0, st, in, ld_in, in_batch,
                       rows_valid, rows, cols, static_cast<_Float16*>(out), ld_out, out_batch);
  else
    hipLaunchKernelGGL(convert_kernel<uint16_t>, grid, dim3(256), 0, st, in, ld_in, in_batch,
                       rows_valid, rows, cols, static_cast<uint16_t*>(out), ld_out, out_batch);
  return check_launch(name);
}

mla_status launch_gemm_nt(const void* X, int64_t ldx, int64_t R, const void* Y, int64_t ldy,
                          int64_t C, int64_t K, void* out, int64_t ldo, int64_t rt_stride,
                          int64_t ct_stride, int64_t R_store, int64_t C_store, Elem in_t,
                          Elem out_t, hipStream_t st, const char* name) {
  if (K % kKC != 0) return fail(MLA_ERR_UNSUPPORTED, "%s: K=%lld not a multiple of 64", name, (long long)K);
  if (C_store % 8 != 0) return fail(MLA_ERR_UNSUPPORTED, "%s: C_store not a multiple of 8", name);
  const int64_t gr = (R_store + kT - 1) / kT, gc = (C_store + kT - 1) / kT;
  if (gr > 65535) return fail(MLA_ERR_UNSUPPORTED, "%s: too many row tiles", name);
  dim3 grid(static_cast<unsigned>(gc), static_cast<unsigned>(gr));
  KernelTimer kt(name, st);
  if (in_t == Elem::BF16 && out_t == Elem::F16)
    hipLaunchKernelGGL((gemm_nt_kernel<__bf16, _Float16>), grid, dim3(256), 0, st,
                       static_cast<const __bf16*>(X), ldx, R, static_cast<const __bf16*>(Y), ldy,
                       C, K, static_cast<_Float16*>(out), ldo, rt_stride, ct_stride, R_store, C_store);
  else if (in_t == Elem::F16 && out_t == Elem::F32)
    hipLaunchKernelGGL((gemm_nt_kernel<_Float16, float>), grid, dim3(256), 0, st,
                       static_cast<const _Float16*>(X), ldx, R, static_cast<const _Float16*>(Y),
                       ldy, C, K, static_cast<float*>(out), ldo, rt_stride, ct_stride, R_store, C_store);
  else if (in_t == Elem::F16 && out_t == Elem::F16)
    hipLaunchKernelGGL((gemm_nt_kernel<_Float16, _Float16>), grid, dim3(256), 0, st,
                       static_cast<const _Float16*>(X), ldx, R, static_cast<const _Float16*>(Y),
                       ldy, C, K, static_cast<_Float16*>(out), ldo, rt_stride, ct_stride, R_store, C_store);
  else
    return fail(MLA_ERR_UNSUPPORTED, "%s: GEMM type combination not built", name);
  return check_launch(name);
}

}  // namespace mla
