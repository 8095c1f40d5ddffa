// Launchers shared by the fast-path forward and backward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace mla {

enum class Elem { BF16, F16, F32 };

// out[c][r] = conv(in[r][c]) for r < rows_valid (0 for rows_valid <= r < rows),
// c < cols; `batch` independent copies, in/out advanced by in_batch/out_batch
// elements. in is bf16; out is bf16 or fp16. cols a multiple of 64, rows of
// 8, leading dimensions and batch strides of 8, both buffers 16-byte aligned
// (MLA_ERR_UNSUPPORTED otherwise, before any launch).
mla_status launch_transpose(const uint16_t* in, int64_t ld_in, int64_t in_batch, int64_t rows_valid,
                            int64_t rows, int64_t cols, void* out, int64_t ld_out,
                            int64_t out_batch, Elem out_t, int batch, hipStream_t st,
                            const char* name);

// out[r][c] = conv(in[r][c]) with the same conventions (no transpose); cols,
// leading dimensions and batch strides multiples of 8, 16-byte aligned.
mla_status launch_convert(const uint16_t* in, int64_t ld_in, int64_t in_batch, int64_t rows_valid,
                          int64_t rows, int64_t cols, void* out, int64_t ld_out, int64_t out_batch,
                          Elem out_t, int batch, hipStream_t st, const char* name);

// out[b][r][0..cols) = fp16(in[r][..]) (bf16 in), rows_valid <= r < rows
// zero-filled, for b < batch copies advanced by out_batch; 16 B per thread.
mla_status launch_broadcast_rows_f16(const uint16_t* in, int64_t ld_in, int64_t rows_valid,
                                     int64_t rows, int cols, _Float16* out, int64_t ld_out,
                                     int64_t out_batch, int batch, hipStream_t st,
                                     const char* name);

// Tiles of a packed call that get a longest-processing-time order.
constexpr int kMaxOrderTiles = 2048;

// qorder[0 .. n_qt) / korder[0 .. n_kt) = query tiles (256 rows) / key tiles
// (128 workspace keys) of a packed call by decreasing number of visible
// (row, key) pairs; korder may be null. n_qt, n_kt <= kMaxOrderTiles.
mla_status launch_tile_order(const int32_t* cu, int n_seqs, int64_t S_loc, const RowMap& rm,
                             int64_t key_lo, int64_t Kn, int n_qt, int n_kt, int* qorder,
                             int* korder, hipStream_t st);

// Out[r][c] = sum_k X[r][k] * Y[c][k] on MFMA, K % 64 == 0. X rows >= R and
// Y rows >= C count as 0. Element (r, c) is stored at
//   out + (r / 128) * rt_stride + (r % 128) * ldo + (c / 128) * ct_stride + c % 128
// for r < R_store and c < C_store (C_store a multiple of 8; R_store and
// C_store may pad R and C up to the 256-row tile that holds their last row).
// A plain row-major matrix has rt_stride = 128 * ldo and ct_stride = 128.
// in_t: BF16 or F16 (both operands); out_t: F16 or F32. An fp32 output with
// few tiles splits K when `part` holds gemm_splitk_bytes() bytes. An fp32
// output is multiplied by *alpha (device memory) when alpha is not null.
// y_kmajor: Y is stored k-major, Y[k][c] at Y + k * ldy + c (fp16 in, fp32
// out, C a multiple of 8), and read transposed in LDS.
mla_status launch_gemm_nt(const void* X, int64_t ldx, int64_t R, const void* Y, int64_t ldy,
                          int64_t C, int64_t K, void* out, int64_t ldo, int64_t rt_stride,
                          int64_t ct_stride, int64_t R_store, int64_t C_store, Elem in_t,
                          Elem out_t, hipStream_t st, const char* name, float* part = nullptr,
                          int64_t part_bytes = 0, const float* alpha = nullptr,
                          bool y_kmajor = false);

}  // namespace mla
