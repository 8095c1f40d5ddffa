// Device helpers shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Local query rows -> global positions. A shard's rows are `n` ascending,
// disjoint, non-empty position blocks laid end to end (one block at
// q_offset for a contiguous shard; two for a zigzag shard): block r holds
// rows row0[r] .. row0[r+1]-1 at positions pos0[r] .. . Positions therefore
// increase with the row index. Passed to kernels by value; every loop
// below is unrolled with constant indices, so the fields stay scalar loads.
constexpr int kMaxRanges = 16;
struct RowMap {
  int n;
  int row0[kMaxRanges + 1];  // row0[0] = 0, row0[n] = S_loc
  int pos0[kMaxRanges];
};

// Global position of local row i (extrapolated past the last row).
__host__ __device__ __forceinline__ int rm_pos(const RowMap& m, int i) {
  int d = m.pos0[0];
#pragma unroll
  for (int r = 1; r < kMaxRanges; ++r)
    if (r < m.n && i >= m.row0[r]) d = m.pos0[r] - m.row0[r];
  return i + d;
}

// Number of local rows whose position is below p: the first row at or past
// position p (S_loc if none).
__host__ __device__ __forceinline__ int rm_rows_below(const RowMap& m, int64_t p) {
  int c = 0;
#pragma unroll
  for (int r = 0; r < kMaxRanges; ++r) {
    if (r < m.n) {
      const int64_t len = m.row0[r + 1] - m.row0[r], k = p - m.pos0[r];
      c += static_cast<int>(k < 0 ? 0 : (k > len ? len : k));
    }
  }
  return c;
}

// bf16 bit pattern -> float (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

template <bool BF16>
__device__ __forceinline__ float load_in(const void* base, int64_t i) {
  if constexpr (BF16) {
    return bf16_to_f32(static_cast<const uint16_t*>(base)[i]);
  } else {
    return static_cast<const float*>(base)[i];
  }
}

// Start of the packed sample holding global position p: the last k with
// cu[k] <= p (so empty samples, equal neighbouring starts, are skipped);
// 0 without packing. Same rule as the host-side plan.
__device__ __forceinline__ int64_t seg_lo_dev(const int32_t* __restrict__ cu, int n_seqs,
                                              int64_t p) {
  if (n_seqs == 0) return 0;
  int lo = 0, hi = n_seqs + 1;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (static_cast<int64_t>(cu[mid]) <= p) lo = mid; else hi = mid;
  }
  return cu[lo];
}

}  // namespace mla
