// Device helpers shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

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
