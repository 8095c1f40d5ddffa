// Plain fp32 path: simple HIP kernels for any head shape and for fp32 inputs.
//
// Computes the same explicit MLA block as the fast path (LAGA abstract: per-
// head K/V rebuilt from the gathered latent, then causal attention), with
// one online-softmax update per key and fp32 everywhere. Throughput is not
// its purpose: it covers shapes the MFMA kernels do not take.
#include <math.h>

#include "device_common.h"
#include "plan.h"

namespace mla {
namespace {

constexpr int kRows = 32;    // query rows per workgroup
constexpr int kSlices = 4;   // threads per row, each owning a column slice
constexpr int kKeys = 16;    // keys staged per step
constexpr int kMaxSlice = 64;  // columns per slice (so widths up to 256)

// K[h][t][:] = [c_kv[key_lo+t] @ W_UK_h | k_rope[key_lo+t]], V[h][t][:] = c_kv @ W_UV_h
template <bool BF16>
__global__ void g_upproj(const void* __restrict__ c_kv, const void* __restrict__ k_rope,
                         const void* __restrict__ W_UK, const void* __restrict__ W_UV,
                         float* __restrict__ K, float* __restrict__ V, int n_h, int d_c,
                         int d_rope, int d_nope, int d_v, int64_t key_lo, int64_t Kn) {
  const int d_qk = d_nope + d_rope;
  const int width = d_qk + d_v;  // K columns then V columns
  const int64_t total = static_cast<int64_t>(n_h) * Kn * width;
  for (int64_t idx = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int col = static_cast<int>(idx % width);
    const int64_t t = (idx / width) % Kn;
    const int h = static_cast<int>(idx / (static_cast<int64_t>(width) * Kn));
    const int64_t row = key_lo + t;
    if (col < d_nope) {
      float acc = 0.f;
      for (int c = 0; c < d_c; ++c)
        acc += load_in<BF16>(c_kv, row * d_c + c) *
               load_in<BF16>(W_UK, static_cast<int64_t>(c) * n_h * d_nope + h * d_nope + col);
      K[(static_cast<int64_t>(h) * Kn + t) * d_qk + col] = acc;
    } else if (col < d_qk) {
      K[(static_cast<int64_t>(h) * Kn + t) * d_qk + col] =
          load_in<BF16>(k_rope, row * d_rope + (col - d_nope));
    } else {
      const int d = col - d_qk;
      float acc = 0.f;
      for (int c = 0; c < d_c; ++c)
        acc += load_in<BF16>(c_kv, row * d_c + c) *
               load_in<BF16>(W_UV, static_cast<int64_t>(c) * n_h * d_v + h * d_v + d);
      V[(static_cast<int64_t>(h) * Kn + t) * d_v + d] = acc;
    }
  }
}

// Forward: workgroup = (32 query rows, one head); thread = (row, value slice).
template <bool BF16>
__global__ void g_attn_fwd(const void* __restrict__ q, const float* __restrict__ K,
                           const float* __restrict__ V, const int32_t* __restrict__ cu,
                           float* __restrict__ out, float* __restrict__ lse, int n_h, int d_qk,
                           int d_v, int n_seqs, int64_t S_loc, RowMap rm, int64_t key_lo,
                           int64_t Kn, float scale) {
  extern __shared__ float smem[];
  float* sQ = smem;                     // [kRows][d_qk]
  float* sK = sQ + kRows * d_qk;        // [kKeys][d_qk]
  float* sV = sK + kKeys * d_qk;        // [kKeys][d_v]
  const int h = blockIdx.y;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * kRows;
  const int r = threadIdx.x % kRows;
  const int sl = threadIdx.x / kRows;
  const int slice = (d_v + kSlices - 1) / kSlices;
  const int c0 = sl * slice;
  const int c1 = min(d_v, c0 + slice);
  const int64_t i = i0 + r;
  const bool valid = i < S_loc;
  const int64_t p = rm_pos(rm, static_cast<int>(i));
  const int64_t lo = valid ? seg_lo_dev(cu, n_seqs, p) : 0;
  const int64_t hi = valid ? p : -1;  // invalid rows see nothing

  for (int e = threadIdx.x; e < kRows * d_qk; e += blockDim.x) {
    const int64_t ii = i0 + e / d_qk;
    sQ[e] = ii < S_loc ? load_in<BF16>(q, (ii * n_h + h) * d_qk + e % d_qk) : 0.f;
  }
  // key range of the workgroup, in workspace rows
  const int64_t i_last = min(S_loc - 1, i0 + kRows - 1);
  // (positions increase with the row: the ends of the row range bound it)
  const int64_t j_begin = seg_lo_dev(cu, n_seqs, rm_pos(rm, static_cast<int>(i0))) - key_lo;
  const int64_t j_end = rm_pos(rm, static_cast<int>(i_last)) + 1 - key_lo;

  float m = -INFINITY, l = 0.f;
  float o[kMaxSlice];
#pragma unroll
  for (int c = 0; c < kMaxSlice; ++c) o[c] = 0.f;

  for (int64_t jb = j_begin; jb < j_end; jb += kKeys) {
    __syncthreads();
    for (int e = threadIdx.x; e < kKeys * d_qk; e += blockDim.x) {
      const int64_t t = jb + e / d_qk;
      sK[e] = t < Kn ? K[(static_cast<int64_t>(h) * Kn + t) * d_qk + e % d_qk] : 0.f;
    }
    for (int e = threadIdx.x; e < kKeys * d_v; e += blockDim.x) {
      const int64_t t = jb + e / d_v;
      sV[e] = t < Kn ? V[(static_cast<int64_t>(h) * Kn + t) * d_v + e % d_v] : 0.f;
    }
    __syncthreads();
    for (int kk = 0; kk < kKeys; ++kk) {
      const int64_t j = key_lo + jb + kk;  // global key position
      if (j < lo || j > hi) continue;
      float s = 0.f;
      for (int d = 0; d < d_qk; ++d) s += sQ[r * d_qk + d] * sK[kk * d_qk + d];
      s *= scale;
      const float m_new = fmaxf(m, s);
      const float corr = expf(m - m_new);
      const float pj = expf(s - m_new);
      l = l * corr + pj;
#pragma unroll
      for (int c = 0; c < kMaxSlice; ++c)
        if (c0 + c < c1) o[c] = o[c] * corr + pj * sV[kk * d_v + c0 + c];
      m = m_new;
    }
  }
  if (!valid) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int c = 0; c < kMaxSlice; ++c)
    if (c0 + c < c1) out[(i * n_h + h) * d_v + c0 + c] = o[c] * inv;
  if (sl == 0) lse[i * n_h + h] = l > 0.f ? m + logf(l) : -INFINITY;
}

// D[i,h] = dout[i,h,:] . out[i,h,:]
template <bool BF16>
__global__ void g_bwd_pre(const void* __restrict__ dout, const float* __restrict__ out,
                          float* __restrict__ D, int64_t rows, int d_v) {
  const int64_t r = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (r >= rows) return;
  float acc = 0.f;
  for (int d = 0; d < d_v; ++d) acc += load_in<BF16>(dout, r * d_v + d) * out[r * d_v + d];
  D[r] = acc;
}

// dq: workgroup = (32 query rows, head); thread = (row, dq slice).
template <bool BF16>
__global__ void g_attn_bwd_dq(const void* __restrict__ q, const void* __restrict__ dout,
                              const float* __restrict__ K, const float* __restrict__ V,
                              const float* __restrict__ lse, const float* __restrict__ D,
                              const int32_t* __restrict__ cu, float* __restrict__ dq, int n_h,
                              int d_qk, int d_v, int n_seqs, int64_t S_loc, RowMap rm,
                              int64_t key_lo, int64_t Kn, float scale) {
  extern __shared__ float smem[];
  float* sQ = smem;                    // [kRows][d_qk]
  float* sO = sQ + kRows * d_qk;       // [kRows][d_v]  (dout)
  float* sK = sO + kRows * d_v;        // [kKeys][d_qk]
  float* sV = sK + kKeys * d_qk;       // [kKeys][d_v]
  const int h = blockIdx.y;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * kRows;
  const int r = threadIdx.x % kRows;
  const int sl = threadIdx.x / kRows;
  const int slice = (d_qk + kSlices - 1) / kSlices;
  const int c0 = sl * slice;
  const int c1 = min(d_qk, c0 + slice);
  const int64_t i = i0 + r;
  const bool valid = i < S_loc;
  const int64_t p = rm_pos(rm, static_cast<int>(i));
  const int64_t lo = valid ? seg_lo_dev(cu, n_seqs, p) : 0;
  const int64_t hi = valid ? p : -1;
  const float L = valid ? lse[i * n_h + h] : 0.f;
  const float Di = valid ? D[i * n_h + h] : 0.f;

  for (int e = threadIdx.x; e < kRows * d_qk; e += blockDim.x) {
    const int64_t ii = i0 + e / d_qk;
    sQ[e] = ii < S_loc ? load_in<BF16>(q, (ii * n_h + h) * d_qk + e % d_qk) : 0.f;
  }
  for (int e = threadIdx.x; e < kRows * d_v; e += blockDim.x) {
    const int64_t ii = i0 + e / d_v;
    sO[e] = ii < S_loc ? load_in<BF16>(dout, (ii * n_h + h) * d_v + e % d_v) : 0.f;
  }
  const int64_t i_last = min(S_loc - 1, i0 + kRows - 1);
  // (positions increase with the row: the ends of the row range bound it)
  const int64_t j_begin = seg_lo_dev(cu, n_seqs, rm_pos(rm, static_cast<int>(i0))) - key_lo;
  const int64_t j_end = rm_pos(rm, static_cast<int>(i_last)) + 1 - key_lo;

  float g[kMaxSlice];
#pragma unroll
  for (int c = 0; c < kMaxSlice; ++c) g[c] = 0.f;

  for (int64_t jb = j_begin; jb < j_end; jb += kKeys) {
    __syncthreads();
    for (int e = threadIdx.x; e < kKeys * d_qk; e += blockDim.x) {
      const int64_t t = jb + e / d_qk;
      sK[e] = t < Kn ? K[(static_cast<int64_t>(h) * Kn + t) * d_qk + e % d_qk] : 0.f;
    }
    for (int e = threadIdx.x; e < kKeys * d_v; e += blockDim.x) {
      const int64_t t = jb + e / d_v;
      sV[e] = t < Kn ? V[(static_cast<int64_t>(h) * Kn + t) * d_v + e % d_v] : 0.f;
    }
    __syncthreads();
    for (int kk = 0; kk < kKeys; ++kk) {
      const int64_t j = key_lo + jb + kk;
      if (j < lo || j > hi) continue;
      float s = 0.f;
      for (int d = 0; d < d_qk; ++d) s += sQ[r * d_qk + d] * sK[kk * d_qk + d];
      float dp = 0.f;
      for (int d = 0; d < d_v; ++d) dp += sO[r * d_v + d] * sV[kk * d_v + d];
      const float P = expf(s * scale - L);
      const float dS = P * (dp - Di);
#pragma unroll
      for (int c = 0; c < kMaxSlice; ++c)
        if (c0 + c < c1) g[c] += scale * dS * sK[kk * d_qk + c0 + c];
    }
  }
  if (!valid) return;
#pragma unroll
  for (int c = 0; c < kMaxSlice; ++c)
    if (c0 + c < c1) dq[(i * n_h + h) * d_qk + c0 + c] = g[c];
}

// dK, dV: workgroup = (32 keys, head); thread = (key, slice of dK and dV).
template <bool BF16>
__global__ void g_attn_bwd_dkdv(const void* __restrict__ q, const void* __restrict__ dout,
                                const float* __restrict__ K, const float* __restrict__ V,
                                const float* __restrict__ lse, const float* __restrict__ D,
                                const int32_t* __restrict__ cu, float* __restrict__ dK,
                                float* __restrict__ dV, int n_h, int d_qk, int d_v, int n_seqs,
                                int64_t S_loc, RowMap rm, int64_t key_lo, int64_t Kn,
                                float scale) {
  extern __shared__ float smem[];
  constexpr int kQ = 16;                 // query rows staged per step
  float* sK = smem;                      // [kRows][d_qk]
  float* sV = sK + kRows * d_qk;         // [kRows][d_v]
  float* sQ = sV + kRows * d_v;          // [kQ][d_qk]
  float* sO = sQ + kQ * d_qk;            // [kQ][d_v]
  float* sL = sO + kQ * d_v;             // [kQ]
  float* sD = sL + kQ;                   // [kQ]
  int64_t* sLo = reinterpret_cast<int64_t*>(sD + kQ);  // [kQ]
  int64_t* sP = sLo + kQ;                // [kQ] row positions
  const int h = blockIdx.y;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRows;  // workspace row
  const int r = threadIdx.x % kRows;
  const int sl = threadIdx.x / kRows;
  const int sk = (d_qk + kSlices - 1) / kSlices;
  const int sv = (d_v + kSlices - 1) / kSlices;
  const int64_t t = t0 + r;
  const bool valid = t < Kn;
  const int64_t j = key_lo + t;

  for (int e = threadIdx.x; e < kRows * d_qk; e += blockDim.x) {
    const int64_t tt = t0 + e / d_qk;
    sK[e] = tt < Kn ? K[(static_cast<int64_t>(h) * Kn + tt) * d_qk + e % d_qk] : 0.f;
  }
  for (int e = threadIdx.x; e < kRows * d_v; e += blockDim.x) {
    const int64_t tt = t0 + e / d_v;
    sV[e] = tt < Kn ? V[(static_cast<int64_t>(h) * Kn + tt) * d_v + e % d_v] : 0.f;
  }
  float gk[kMaxSlice], gv[kMaxSlice];
#pragma unroll
  for (int c = 0; c < kMaxSlice; ++c) { gk[c] = 0.f; gv[c] = 0.f; }

  // rows whose position is >= the first key of the block; later rows whose
  // sample starts past the block's last key see none of it (seg_lo grows with p)
  const int64_t j_first = key_lo + t0;
  const int64_t j_last = key_lo + min(Kn - 1, t0 + kRows - 1);
  const int64_t i_begin = rm_rows_below(rm, j_first);
  for (int64_t ib = i_begin; ib < S_loc; ib += kQ) {
    __syncthreads();
    if (seg_lo_dev(cu, n_seqs, rm_pos(rm, static_cast<int>(ib))) > j_last) break;  // uniform
    for (int e = threadIdx.x; e < kQ * d_qk; e += blockDim.x) {
      const int64_t ii = ib + e / d_qk;
      sQ[e] = ii < S_loc ? load_in<BF16>(q, (ii * n_h + h) * d_qk + e % d_qk) : 0.f;
    }
    for (int e = threadIdx.x; e < kQ * d_v; e += blockDim.x) {
      const int64_t ii = ib + e / d_v;
      sO[e] = ii < S_loc ? load_in<BF16>(dout, (ii * n_h + h) * d_v + e % d_v) : 0.f;
    }
    if (threadIdx.x < kQ) {
      const int64_t ii = ib + threadIdx.x;
      const bool ok = ii < S_loc;
      sL[threadIdx.x] = ok ? lse[ii * n_h + h] : 0.f;
      sD[threadIdx.x] = ok ? D[ii * n_h + h] : 0.f;
      sLo[threadIdx.x] = ok ? seg_lo_dev(cu, n_seqs, rm_pos(rm, static_cast<int>(ii))) : INT64_MAX;
      sP[threadIdx.x] = ok ? rm_pos(rm, static_cast<int>(ii)) : -1;
    }
    __syncthreads();
    if (!valid) continue;
    for (int qq = 0; qq < kQ; ++qq) {
      const int64_t ii = ib + qq;
      const int64_t p = sP[qq];
      if (ii >= S_loc || j > p || j < sLo[qq]) continue;
      float s = 0.f;
      for (int d = 0; d < d_qk; ++d) s += sQ[qq * d_qk + d] * sK[r * d_qk + d];
      float dp = 0.f;
      for (int d = 0; d < d_v; ++d) dp += sO[qq * d_v + d] * sV[r * d_v + d];
      const float P = expf(s * scale - sL[qq]);
      const float dS = P * (dp - sD[qq]);
#pragma unroll
      for (int c = 0; c < kMaxSlice; ++c) {
        const int ck = sl * sk + c;
        const int cv = sl * sv + c;
        if (c < sk && ck < d_qk) gk[c] += scale * dS * sQ[qq * d_qk + ck];
        if (c < sv && cv < d_v) gv[c] += P * sO[qq * d_v + cv];
      }
    }
  }
  if (!valid) return;
#pragma unroll
  for (int c = 0; c < kMaxSlice; ++c) {
    const int ck = sl * sk + c;
    const int cv = sl * sv + c;
    if (c < sk && ck < d_qk) dK[(static_cast<int64_t>(h) * Kn + t) * d_qk + ck] = gk[c];
    if (c < sv && cv < d_v) dV[(static_cast<int64_t>(h) * Kn + t) * d_v + cv] = gv[c];
  }
}

// dk_rope[j,:] = sum_h dK[h][j-key_lo][d_nope:] and dc_kv[j,c] =
// sum_h (dK_nope[h][t] . W_UK[c, h-block] + dV[h][t] . W_UV[c, h-block]);
// rows outside [key_lo, key_lo+Kn) are written as 0.
template <bool BF16>
__global__ void g_grad_latent(const float* __restrict__ dK, const float* __restrict__ dV,
                              const void* __restrict__ W_UK, const void* __restrict__ W_UV,
                              float* __restrict__ dc_kv, float* __restrict__ dk_rope, int n_h,
                              int d_c, int d_rope, int d_nope, int d_v, int64_t S,
                              int64_t key_lo, int64_t Kn) {
  const int d_qk = d_nope + d_rope;
  const int width = d_c + d_rope;
  const int64_t total = S * width;
  for (int64_t idx = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int col = static_cast<int>(idx % width);
    const int64_t j = idx / width;
    const int64_t t = j - key_lo;
    const bool in = t >= 0 && t < Kn;
    if (col < d_c) {
      float acc = 0.f;
      if (in) {
        for (int h = 0; h < n_h; ++h) {
          const float* gk = dK + (static_cast<int64_t>(h) * Kn + t) * d_qk;
          const float* gv = dV + (static_cast<int64_t>(h) * Kn + t) * d_v;
          for (int d = 0; d < d_nope; ++d)
            acc += gk[d] * load_in<BF16>(W_UK, static_cast<int64_t>(col) * n_h * d_nope +
                                                   h * d_nope + d);
          for (int d = 0; d < d_v; ++d)
            acc += gv[d] *
                   load_in<BF16>(W_UV, static_cast<int64_t>(col) * n_h * d_v + h * d_v + d);
        }
      }
      dc_kv[j * d_c + col] = acc;
    } else {
      const int r = col - d_c;
      float acc = 0.f;
      if (in)
        for (int h = 0; h < n_h; ++h)
          acc += dK[(static_cast<int64_t>(h) * Kn + t) * d_qk + d_nope + r];
      dk_rope[j * d_rope + r] = acc;
    }
  }
}

// dW_UK[c, h*d_nope+d] = sum_t c_kv[key_lo+t, c] dK[h][t][d]; likewise dW_UV with dV.
template <bool BF16>
__global__ void g_grad_w(const void* __restrict__ c_kv, const float* __restrict__ dK,
                         const float* __restrict__ dV, float* __restrict__ dW_UK,
                         float* __restrict__ dW_UV, int n_h, int d_c, int d_rope, int d_nope,
                         int d_v, int64_t key_lo, int64_t Kn) {
  const int d_qk = d_nope + d_rope;
  const int width = n_h * (d_nope + d_v);
  const int64_t total = static_cast<int64_t>(d_c) * width;
  for (int64_t idx = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int col = static_cast<int>(idx % width);
    const int c = static_cast<int>(idx / width);
    float acc = 0.f;
    if (col < n_h * d_nope) {
      const int h = col / d_nope, d = col % d_nope;
      for (int64_t t = 0; t < Kn; ++t)
        acc += load_in<BF16>(c_kv, (key_lo + t) * d_c + c) *
               dK[(static_cast<int64_t>(h) * Kn + t) * d_qk + d];
      dW_UK[static_cast<int64_t>(c) * n_h * d_nope + col] = acc;
    } else {
      const int cc = col - n_h * d_nope;
      const int h = cc / d_v, d = cc % d_v;
      for (int64_t t = 0; t < Kn; ++t)
        acc += load_in<BF16>(c_kv, (key_lo + t) * d_c + c) *
               dV[(static_cast<int64_t>(h) * Kn + t) * d_v + d];
      dW_UV[static_cast<int64_t>(c) * n_h * d_v + cc] = acc;
    }
  }
}

__global__ void k_zero(float* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0.f;
}

// Kernels whose dynamic LDS exceeds the 64 KiB default need the limit raised.
template <typename K>
mla_status allow_lds(K kernel, size_t bytes) {
  if (bytes <= 65536) return MLA_OK;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(bytes));
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "LDS limit: %s", hipGetErrorString(e));
  return MLA_OK;
}

inline unsigned grid_for(int64_t n, int block) {
  int64_t g = (n + block - 1) / block;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return static_cast<unsigned>(g);
}

template <bool BF16>
mla_status generic_fwd_t(const Plan& p, const void* q, const void* c_kv, const void* k_rope,
                         const void* W_UK, const void* W_UV, const int32_t* cu, float* out,
                         float* lse, char* ws, hipStream_t st) {
  const FwdLayout L = fwd_layout(p);
  float* K = reinterpret_cast<float*>(ws + L.K);
  float* V = reinterpret_cast<float*>(ws + L.V);
  const int64_t n_up = static_cast<int64_t>(p.n_h) * p.Kn * (p.d_qk + p.d_v);
  {
    KernelTimer kt("plain_upproj", st);
    hipLaunchKernelGGL(g_upproj<BF16>, dim3(grid_for(n_up, 256)), dim3(256), 0, st, c_kv, k_rope,
                       W_UK, W_UV, K, V, p.n_h, p.d_c, p.d_rope, p.d_nope, p.d_v, p.key_lo, p.Kn);
  }
  if (mla_status s = check_launch("plain up-projection"); s != MLA_OK) return s;
  const size_t lds = sizeof(float) * (kRows * p.d_qk + kKeys * (p.d_qk + p.d_v));
  if (mla_status s = allow_lds(g_attn_fwd<BF16>, lds); s != MLA_OK) return s;
  dim3 grid(static_cast<unsigned>((p.S_loc + kRows - 1) / kRows), p.n_h);
  {
    KernelTimer kt("plain_attn_fwd", st);
    hipLaunchKernelGGL(g_attn_fwd<BF16>, grid, dim3(kRows * kSlices), lds, st, q, K, V, cu, out,
                       lse, p.n_h, p.d_qk, p.d_v, p.n_seqs, p.S_loc, p.rm, p.key_lo, p.Kn,
                       p.scale);
  }
  return check_launch("plain attention forward");
}

template <bool BF16>
mla_status generic_bwd_t(const Plan& p, const void* dout, const void* q, const void* c_kv,
                         const void* k_rope, const void* W_UK, const void* W_UV,
                         const int32_t* cu, const float* out, const float* lse, float* dq,
                         float* dc_kv, float* dk_rope, float* dW_UK, float* dW_UV, char* ws,
                         hipStream_t st) {
  const BwdLayout L = bwd_layout(p);
  float* K = reinterpret_cast<float*>(ws + L.f.K);
  float* V = reinterpret_cast<float*>(ws + L.f.V);
  float* D = reinterpret_cast<float*>(ws + L.D);
  float* dK = reinterpret_cast<float*>(ws + L.dK);
  float* dV = reinterpret_cast<float*>(ws + L.dV);
  const int64_t n_up = static_cast<int64_t>(p.n_h) * p.Kn * (p.d_qk + p.d_v);
  {
    KernelTimer kt("plain_upproj", st);
    hipLaunchKernelGGL(g_upproj<BF16>, dim3(grid_for(n_up, 256)), dim3(256), 0, st, c_kv, k_rope,
                       W_UK, W_UV, K, V, p.n_h, p.d_c, p.d_rope, p.d_nope, p.d_v, p.key_lo, p.Kn);
  }
  if (mla_status s = check_launch("plain up-projection"); s != MLA_OK) return s;
  const int64_t rows = p.S_loc * p.n_h;
  {
    KernelTimer kt("plain_bwd_pre", st);
    hipLaunchKernelGGL(g_bwd_pre<BF16>, dim3(grid_for(rows, 256)), dim3(256), 0, st, dout, out, D,
                       rows, p.d_v);
  }
  if (mla_status s = check_launch("plain backward preprocess"); s != MLA_OK) return s;
  {
    const size_t lds = sizeof(float) * (kRows * (p.d_qk + p.d_v) + kKeys * (p.d_qk + p.d_v));
    if (mla_status s = allow_lds(g_attn_bwd_dq<BF16>, lds); s != MLA_OK) return s;
    dim3 grid(static_cast<unsigned>((p.S_loc + kRows - 1) / kRows), p.n_h);
    {
      KernelTimer kt("plain_attn_bwd_dq", st);
      hipLaunchKernelGGL(g_attn_bwd_dq<BF16>, grid, dim3(kRows * kSlices), lds, st, q, dout, K, V,
                         lse, D, cu, dq, p.n_h, p.d_qk, p.d_v, p.n_seqs, p.S_loc, p.rm,
                         p.key_lo, p.Kn, p.scale);
    }
    if (mla_status s = check_launch("plain backward dq"); s != MLA_OK) return s;
  }
  {
    constexpr int kQ = 16;
    const size_t lds = sizeof(float) * (kRows * (p.d_qk + p.d_v) + kQ * (p.d_qk + p.d_v) +
                                        2 * kQ) + sizeof(int64_t) * 2 * kQ;
    if (mla_status s = allow_lds(g_attn_bwd_dkdv<BF16>, lds); s != MLA_OK) return s;
    dim3 grid(static_cast<unsigned>((p.Kn + kRows - 1) / kRows), p.n_h);
    {
      KernelTimer kt("plain_attn_bwd_dkdv", st);
      hipLaunchKernelGGL(g_attn_bwd_dkdv<BF16>, grid, dim3(kRows * kSlices), lds, st, q, dout, K,
                         V, lse, D, cu, dK, dV, p.n_h, p.d_qk, p.d_v, p.n_seqs, p.S_loc,
                         p.rm, p.key_lo, p.Kn, p.scale);
    }
    if (mla_status s = check_launch("plain backward dK/dV"); s != MLA_OK) return s;
  }
  const int64_t n_lat = p.S * (p.d_c + p.d_rope);
  {
    KernelTimer kt("plain_grad_latent", st);
    hipLaunchKernelGGL(g_grad_latent<BF16>, dim3(grid_for(n_lat, 256)), dim3(256), 0, st, dK, dV,
                       W_UK, W_UV, dc_kv, dk_rope, p.n_h, p.d_c, p.d_rope, p.d_nope, p.d_v, p.S,
                       p.key_lo, p.Kn);
  }
  if (mla_status s = check_launch("plain latent gradient"); s != MLA_OK) return s;
  const int64_t n_w = static_cast<int64_t>(p.d_c) * p.n_h * (p.d_nope + p.d_v);
  {
    KernelTimer kt("plain_grad_w", st);
    hipLaunchKernelGGL(g_grad_w<BF16>, dim3(grid_for(n_w, 256)), dim3(256), 0, st, c_kv, dK, dV,
                       dW_UK, dW_UV, p.n_h, p.d_c, p.d_rope, p.d_nope, p.d_v, p.key_lo, p.Kn);
  }
  return check_launch("plain weight gradient");
}

}  // namespace

mla_status generic_fwd(const Plan& p, const void* q, const void* c_kv, const void* k_rope,
                       const void* W_UK, const void* W_UV, const int32_t* cu_dev, float* out,
                       float* lse, char* ws, hipStream_t st) {
  return p.bf16 ? generic_fwd_t<true>(p, q, c_kv, k_rope, W_UK, W_UV, cu_dev, out, lse, ws, st)
                : generic_fwd_t<false>(p, q, c_kv, k_rope, W_UK, W_UV, cu_dev, out, lse, ws, st);
}

mla_status generic_bwd(const Plan& p, const void* dout, const void* q, const void* c_kv,
                       const void* k_rope, const void* W_UK, const void* W_UV,
                       const int32_t* cu_dev, const float* out, const float* lse, float* dq,
                       float* dc_kv, float* dk_rope, float* dW_UK, float* dW_UV, char* ws,
                       hipStream_t st) {
  return p.bf16 ? generic_bwd_t<true>(p, dout, q, c_kv, k_rope, W_UK, W_UV, cu_dev, out, lse, dq,
                                      dc_kv, dk_rope, dW_UK, dW_UV, ws, st)
                : generic_bwd_t<false>(p, dout, q, c_kv, k_rope, W_UK, W_UV, cu_dev, out, lse,
                                       dq, dc_kv, dk_rope, dW_UK, dW_UV, ws, st);
}

mla_status zero_fill(float* ptr, int64_t n, hipStream_t st) {
  if (n <= 0) return MLA_OK;
  hipLaunchKernelGGL(k_zero, dim3(grid_for(n, 256)), dim3(256), 0, st, ptr, n);
  return check_launch("zero fill");
}

}  // namespace mla
