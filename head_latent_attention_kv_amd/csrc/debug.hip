// Debug mode and the per-row key-window export.
//
// Debug mode (environment variable MLA_LAGA_DEBUG) wraps a call:
//   before: cu_seqlens_dev is copied back and compared with cu_seqlens_host;
//           the workspace's used bytes and every output are filled with
//           all-ones bytes (NaN in fp32, fp16 and bf16), a canary is
//           written into the 256 bytes that follow the used workspace.
//   after:  every output is scanned for NaN (the index of the first one is
//           kept per output), the canary is read back and checked.
// A NaN left in an output means an element the call did not write, or a
// result that read workspace bytes before the call wrote them, or NaN in
// the inputs. All fills are kernels (no memset nodes), the checks wait for
// the stream.
#include <stdlib.h>
#include <string.h>

#include "plan.h"

namespace mla {

namespace {

constexpr uint32_t kCanary = 0x5CA1AB1Eu;
constexpr int kCanaryWords = 32;            // bytes 0 .. 127 of the tail
constexpr int kSlotOffset = 128;            // then one uint64 per output
constexpr int kMaxDebugOutputs = 8;
static_assert(kSlotOffset + 8 * kMaxDebugOutputs <= kDebugTailBytes, "debug tail layout");

__global__ void __launch_bounds__(256)
fill_u32_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n; i += stride)
    p[i] = v;
}

// *first = min(*first, index of the first fp32 NaN in p[0 .. n)); one atomic
// per workgroup.
__global__ void __launch_bounds__(256)
first_nan_kernel(const uint32_t* __restrict__ p, int64_t n, unsigned long long* __restrict__ first) {
  __shared__ unsigned long long red[256];
  unsigned long long m = ~0ull;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n; i += stride)
    if ((p[i] & 0x7fffffffu) > 0x7f800000u) {
      m = static_cast<unsigned long long>(i);
      break;  // later indices of this thread are larger
    }
  red[threadIdx.x] = m;
  __syncthreads();
  for (int s = 128; s >= 1; s >>= 1) {
    if (static_cast<int>(threadIdx.x) < s) red[threadIdx.x] = min(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  if (threadIdx.x == 0 && red[0] != ~0ull) atomicMin(first, red[0]);
}

int grid_of(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return static_cast<int>(b < 4096 ? (b < 1 ? 1 : b) : 4096);
}

mla_status fill_words(void* p, int64_t words, uint32_t v, hipStream_t st) {
  if (words <= 0) return MLA_OK;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_of(words)), dim3(256), 0, st,
                     static_cast<uint32_t*>(p), words, v);
  return check_launch("debug fill");
}

// Local row -> inclusive window [lo, hi] of global key positions it sees,
// from the same row map and sample-start search the attention kernels use.
__global__ void __launch_bounds__(256)
row_window_kernel(const int32_t* __restrict__ cu, int n_seqs, int S_loc, RowMap rm,
                  int64_t* __restrict__ window) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= S_loc) return;
  const int pos = rm_pos(rm, i);
  window[2 * static_cast<int64_t>(i)] = seg_lo_dev(cu, n_seqs, pos);
  window[2 * static_cast<int64_t>(i) + 1] = pos;
}

}  // namespace

bool debug_mode() {
  const char* e = getenv("MLA_LAGA_DEBUG");
  return e != nullptr && e[0] != '\0' && strcmp(e, "0") != 0;
}

mla_status debug_begin(const int32_t* cu_host, const int32_t* cu_dev, int n_cu, char* ws,
                       int64_t ws_used, const DebugOutput* outs, int n_out, hipStream_t st) {
  if (n_out > kMaxDebugOutputs) return fail(MLA_ERR_INVALID_ARG, "debug: too many outputs");
  if (cu_dev != nullptr && cu_host != nullptr && n_cu > 0) {
    int32_t* back = static_cast<int32_t*>(malloc(sizeof(int32_t) * n_cu));
    if (back == nullptr) return fail(MLA_ERR_DEBUG_CHECK, "debug: host allocation failed");
    hipError_t e = hipMemcpyAsync(back, cu_dev, sizeof(int32_t) * n_cu, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) {
      free(back);
      return fail(MLA_ERR_HIP, "debug: reading cu_seqlens_dev: %s", hipGetErrorString(e));
    }
    for (int k = 0; k < n_cu; ++k)
      if (back[k] != cu_host[k]) {
        const int a = back[k], b = cu_host[k];
        free(back);
        return fail(MLA_ERR_DEBUG_CHECK, "debug: cu_seqlens_dev[%d] = %d but cu_seqlens_host[%d] = %d",
                    k, a, k, b);
      }
    free(back);
  }
  char* tail = ws + ws_used;
  mla_status s = fill_words(ws, ws_used / 4, 0xffffffffu, st);
  if (s == MLA_OK) s = fill_words(tail, kCanaryWords, kCanary, st);
  if (s == MLA_OK) s = fill_words(tail + kSlotOffset, 2 * kMaxDebugOutputs, 0xffffffffu, st);
  for (int k = 0; k < n_out && s == MLA_OK; ++k) s = fill_words(outs[k].ptr, outs[k].n, 0xffffffffu, st);
  return s;
}

mla_status debug_end(char* ws, int64_t ws_used, const DebugOutput* outs, int n_out, hipStream_t st) {
  char* tail = ws + ws_used;
  unsigned long long* slots = reinterpret_cast<unsigned long long*>(tail + kSlotOffset);
  for (int k = 0; k < n_out; ++k) {
    if (outs[k].n <= 0) continue;
    hipLaunchKernelGGL(first_nan_kernel, dim3(grid_of(outs[k].n)), dim3(256), 0, st,
                       static_cast<const uint32_t*>(outs[k].ptr), outs[k].n, slots + k);
    if (mla_status s = check_launch("debug scan"); s != MLA_OK) return s;
  }
  uint32_t back[kDebugTailBytes / 4];
  hipError_t e = hipMemcpyAsync(back, tail, kDebugTailBytes, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "debug: reading the checks back: %s", hipGetErrorString(e));
  for (int k = 0; k < kCanaryWords; ++k)
    if (back[k] != kCanary)
      return fail(MLA_ERR_DEBUG_CHECK,
                  "debug: canary word %d past the %lld used workspace bytes was overwritten (0x%08x)",
                  k, (long long)ws_used, back[k]);
  for (int k = 0; k < n_out; ++k) {
    unsigned long long first;
    memcpy(&first, reinterpret_cast<const char*>(back) + kSlotOffset + 8 * k, 8);
    if (first != ~0ull)
      return fail(MLA_ERR_DEBUG_CHECK,
                  "debug: %s[%llu] is NaN after the call (not written, or computed from "
                  "unwritten workspace or from NaN inputs)",
                  outs[k].name, first);
  }
  return MLA_OK;
}

mla_status launch_row_window(const Plan& p, const int32_t* cu_dev, int64_t* window, hipStream_t st) {
  if (p.S_loc == 0) return MLA_OK;
  hipLaunchKernelGGL(row_window_kernel, dim3(static_cast<unsigned>((p.S_loc + 255) / 256)), dim3(256),
                     0, st, cu_dev, p.n_seqs, static_cast<int>(p.S_loc), p.rm, window);
  return check_launch("row window");
}

}  // namespace mla
