// Fast backward: gradients of sum(out * dout) through attention and the
// latent up-projection (the training path of the LAGA abstract: K/V are
// rebuilt from the latent, so their gradients flow back into c_kv, k_rope,
// W_UK and W_UV).
//
//   prep      D = rowsum(dout * out); q and dout to fp16, per head, both
//             row-major [row][dim] and column-major [dim][row]
//   rebuild   K_nope and V again (fp16), in the layouts the kernels read
//   dkdv      key-outer: each wave owns 32 keys. S = Q K^T lands with lanes
//             on keys and registers on query rows, so P and dS feed
//             dV^T += dO^T P and dK^T += Q^T dS without leaving registers.
//   dq        query-outer: each wave owns 32 rows; S^T, dP^T per lane = row,
//             dQ^T += K^T dS^T. No atomics: the result is deterministic.
//   GEMMs     dc_kv = [dK_nope | dV] [W_UK | W_UV]^T,  dW = c_kv^T [dK_nope | dV]
//   reduce    dk_rope = sum over heads of the per-head rope-key gradients
//
// Query/key tiles are DMA-filled (global_load_lds) into XOR-swizzled LDS and
// double-buffered, as in the forward.
#include <math.h>

#include "fast.h"
#include "fast_common.h"

namespace mla {
namespace {

constexpr int DQK = 192, DV = 128;
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ void lds_dma16(const void* src, char* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, lds_dst, 16, 0, 0);
}

// Swizzles (16-byte pieces): rows read 8 at a time by consecutive lanes.
// Tiles whose rows are a multiple of 128 B wide, read at rows swap23(lane):
__device__ __forceinline__ int sw_a(int row) { return (row & 3) | ((row >> 1) & 4); }
__device__ __forceinline__ int off_a(int row, int row_bytes, int c) {
  return row * row_bytes + (((c & ~7) | ((c & 7) ^ sw_a(row))) << 4);
}
// 128-byte rows read at consecutive rows:
__device__ __forceinline__ int off_b(int row, int c) { return row * 128 + ((c ^ (row & 7)) << 4); }
// 64-byte rows (4 pieces) read at consecutive rows:
__device__ __forceinline__ int off_c(int row, int c) { return row * 64 + ((c ^ ((row >> 1) & 3)) << 4); }

__device__ __forceinline__ void work_item(int bid, int n_h, int n_t, int* h, int* t) {
  // as in the forward: all tiles of a head on one XCD when n_h % 8 == 0
  if ((n_h & 7) == 0) {
    const int xcd = bid & 7, slot = bid >> 3;
    *h = (slot / n_t) * 8 + xcd;
    *t = slot % n_t;
  } else {
    *h = bid % n_h;
    *t = bid / n_h;
  }
}

// ------------------------------------------------------------------ prep
// grid (ceil(S_loc/64), n_h). D[h][i] = dout[i,h,:] . out[i,h,:]; fp16 copies
// Qn[h][i][192], Qt[h][192][i], dOn[h][i][128], dOt[h][128][i] (rows past
// S_loc are zero).
__global__ void __launch_bounds__(256)
bwd_prep_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ dout,
                const float* __restrict__ out, float* __restrict__ D, _Float16* __restrict__ Qn,
                _Float16* __restrict__ Qt, _Float16* __restrict__ dOn, _Float16* __restrict__ dOt,
                int n_h, int64_t S_loc, int64_t S_pad) {
  constexpr int TS = DQK + 2;  // LDS row stride (halfs)
  __shared__ _Float16 t[64 * TS];
  const int h = blockIdx.y;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // D: each wave 16 rows, each lane 2 columns
  for (int rr = 0; rr < 16; ++rr) {
    const int64_t i = i0 + w * 16 + rr;
    float v = 0.f;
    if (i < S_loc) {
      const int64_t base = (i * n_h + h) * DV + 2 * lane;
      v = bf16_to_f32(dout[base]) * out[base] + bf16_to_f32(dout[base + 1]) * out[base + 1];
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, 64);
    if (lane == 0) D[h * S_pad + i] = v;
  }
  // q then dout: natural rows to global and LDS, then the transpose
  for (int pass = 0; pass < 2; ++pass) {
    const int width = pass == 0 ? DQK : DV;
    const uint16_t* src = pass == 0 ? q : dout;
    _Float16* nat = (pass == 0 ? Qn : dOn) + static_cast<int64_t>(h) * S_pad * width;
    _Float16* tr = (pass == 0 ? Qt : dOt) + static_cast<int64_t>(h) * width * S_pad;
    const int chunks = width / 8;
    __syncthreads();
    for (int e = tid; e < 64 * chunks; e += 256) {
      const int row = e / chunks, ch = e % chunks;
      const int64_t i = i0 + row;
      half8 v;
      if (i < S_loc) {
        v = bf16x8_to_half8(
            *reinterpret_cast<const u32x4*>(src + (i * n_h + h) * width + ch * 8));
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = static_cast<_Float16>(0.f);
      }
      *reinterpret_cast<half8*>(nat + (i0 + row) * width + ch * 8) = v;
#pragma unroll
      for (int k = 0; k < 8; ++k) t[row * TS + ch * 8 + k] = v[k];
    }
    __syncthreads();
    for (int e = tid; e < width * 8; e += 256) {
      const int dim = e / 8, qc = e % 8;
      half8 v;
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = t[(qc * 8 + k) * TS + dim];
      *reinterpret_cast<half8*>(tr + dim * S_pad + i0 + qc * 8) = v;
    }
  }
}

// ------------------------------------------------------------------ dK, dV
constexpr int KB = 128;     // keys per workgroup (4 waves x 32)
constexpr int QB = 32;      // query rows per step
// stage layout (bytes): Qn [32][192] | dOn [32][128] | Qt [192][32] | dOt [128][32] | row info
constexpr int S_QN = 0, S_DON = QB * DQK * 2, S_QT = S_DON + QB * DV * 2,
              S_DOT = S_QT + DQK * QB * 2, S_INFO = S_DOT + DV * QB * 2,
              S_BYTES = S_INFO + 4 * QB * 4;  // lse2, D, lo, p (32 each)

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_bwd_dkdv_kernel(const _Float16* __restrict__ Qn, const _Float16* __restrict__ Qt,
                     const _Float16* __restrict__ dOn, const _Float16* __restrict__ dOt,
                     const float* __restrict__ lse, const float* __restrict__ D,
                     const _Float16* __restrict__ Knope, const _Float16* __restrict__ Krope,
                     const _Float16* __restrict__ Vkm, const int32_t* __restrict__ cu,
                     _Float16* __restrict__ dKV, _Float16* __restrict__ dKVT,
                     float* __restrict__ dKr, int n_h, int n_seqs, int64_t S_loc, int64_t S_pad,
                     int64_t q_offset, int64_t key_lo, int64_t Kn, int64_t Kpad, int n_kt,
                     float scale, float scale_log2) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * S_BYTES];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5;
  int h, kt;
  work_item(blockIdx.x, n_h, n_kt, &h, &kt);
  const int64_t t0 = static_cast<int64_t>(kt) * KB;        // workspace key row
  const int64_t tw = t0 + 32 * w;                           // this wave's first key
  const int64_t gkey = key_lo + tw + lr;                    // this lane's key (global)
  const int64_t gk_min = key_lo + t0, gk_max = key_lo + t0 + KB - 1;
  const int64_t gw_min = key_lo + tw, gw_max = gw_min + 31;

  // K and V rows of this lane's key as MFMA B fragments
  half8 kf[12], vf[8];
  {
    const _Float16* kn = Knope + (static_cast<int64_t>(h) * Kpad + tw + lr) * 128 + 8 * lh;
    const _Float16* kr = Krope + (tw + lr) * 64 + 8 * lh;
    const _Float16* vr = Vkm + (static_cast<int64_t>(h) * Kpad + tw + lr) * 128 + 8 * lh;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) kf[kk] = *reinterpret_cast<const half8*>(kn + 16 * kk);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) kf[8 + kk] = *reinterpret_cast<const half8*>(kr + 16 * kk);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) vf[kk] = *reinterpret_cast<const half8*>(vr + 16 * kk);
  }

  // query rows that see any key of the block: from the first row at or past
  // the block's first key to the last row whose sample starts by its last key
  int64_t i_begin = gk_min - q_offset;
  if (i_begin < 0) i_begin = 0;
  int64_t i_end = S_loc;
  if (n_seqs > 0) {
    // first sample start after gk_max (S if none): rows at or past it see nothing here
    int lo_i = 0, hi_i = n_seqs + 1;
    while (hi_i - lo_i > 1) {
      const int mid = (lo_i + hi_i) >> 1;
      if (cu[mid] <= gk_max) lo_i = mid; else hi_i = mid;
    }
    const int64_t nxt = lo_i + 1 <= n_seqs ? cu[lo_i + 1] : INT64_MAX;
    if (nxt - q_offset < i_end) i_end = nxt - q_offset;
  }
  const int64_t qb_begin = (i_begin / QB) * QB;
  const int nq = i_end > qb_begin ? static_cast<int>((i_end - qb_begin + QB - 1) / QB) : 0;

  // this wave's DMA pieces per stage: 40 KiB in 40 wave instructions, 10
  // each. Piece I holds Qn (I < 12), dOn (< 20), Qt (< 32) or dOt; the
  // per-lane element offsets below are relative to row qb of that tile.
  const _Float16* Qn_h = Qn + static_cast<int64_t>(h) * S_pad * DQK;
  const _Float16* dOn_h = dOn + static_cast<int64_t>(h) * S_pad * DV;
  const _Float16* Qt_h = Qt + static_cast<int64_t>(h) * DQK * S_pad;
  const _Float16* dOt_h = dOt + static_cast<int64_t>(h) * DV * S_pad;
  int dma_off[10];
#pragma unroll
  for (int j = 0; j < 10; ++j) {
    const int o = (w * 10 + j) * 1024 + lane * 16;
    int off;
    if (o < S_DON) {
      const int row = o / 384, pos = (o % 384) >> 4;
      off = row * DQK + ((pos & ~7) | ((pos & 7) ^ sw_a(row))) * 8;
    } else if (o < S_QT) {
      const int oo = o - S_DON, row = oo >> 8, pos = (oo & 255) >> 4;
      off = row * DV + ((pos & ~7) | ((pos & 7) ^ sw_a(row))) * 8;
    } else if (o < S_DOT) {
      const int oo = o - S_QT, row = oo >> 6, pos = (oo & 63) >> 4;
      off = row * static_cast<int>(S_pad) + (pos ^ ((row >> 1) & 3)) * 8;
    } else {
      const int oo = o - S_DOT, row = oo >> 6, pos = (oo & 63) >> 4;
      off = row * static_cast<int>(S_pad) + (pos ^ ((row >> 1) & 3)) * 8;
    }
    dma_off[j] = off;
  }
  auto issue = [&](int64_t qb, int st) {
    char* base = smem + st * S_BYTES;
#pragma unroll
    for (int j = 0; j < 10; ++j) {
      const int I = w * 10 + j;   // wave-uniform: which tile this piece is in
      const _Float16* src = I < 12 ? Qn_h + qb * DQK
                          : I < 20 ? dOn_h + qb * DV
                          : I < 32 ? Qt_h + qb : dOt_h + qb;
      lds_dma16(src + dma_off[j], base + I * 1024);
    }
    if (tid < QB) {
      const int64_t i = qb + tid;
      float* info = reinterpret_cast<float*>(base + S_INFO);
      const bool ok = i < S_loc;
      info[tid] = ok ? lse[i * n_h + h] * kLog2e : 0.f;
      info[QB + tid] = ok ? D[h * S_pad + i] : 0.f;
      int32_t* ii = reinterpret_cast<int32_t*>(info + 2 * QB);
      ii[tid] = ok ? static_cast<int32_t>(seg_lo_dev(cu, n_seqs, q_offset + i)) : INT32_MAX;
      ii[QB + tid] = ok ? static_cast<int32_t>(q_offset + i) : -1;
    }
  };

  f32x16 dk[6], dv[4];
#pragma unroll
  for (int a = 0; a < 6; ++a)
#pragma unroll
    for (int e = 0; e < 16; ++e) dk[a][e] = 0.f;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int e = 0; e < 16; ++e) dv[a][e] = 0.f;

  if (nq > 0) issue(qb_begin, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int b = 0; b < nq; ++b) {
    const int st = b & 1;
    const int64_t qb = qb_begin + static_cast<int64_t>(b) * QB;
    if (b + 1 < nq) issue(qb + QB, st ^ 1);
    const char* base = smem + st * S_BYTES;
    const float* info = reinterpret_cast<const float*>(base + S_INFO);
    const int32_t* iinfo = reinterpret_cast<const int32_t*>(info + 2 * QB);
    // rows qb.. of this step, as global positions: the first is q_offset+qb;
    // rows past S_loc have p = -1
    const int64_t p_first = q_offset + qb;
    const int64_t p_last = q_offset + min(qb + QB, S_loc) - 1;
    const bool skip = p_last < gw_min || iinfo[0] > gw_max;
    if (!skip) {
      const bool full = qb + QB <= S_loc && p_first >= gw_max && iinfo[QB - 1] <= gw_min;
      const int qrow = swap23(lr);   // A-operand row loaded by this lane
      f32x16 s, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) { s[e] = 0.f; dp[e] = 0.f; }
      {
        // 12 S steps then 8 dP steps, A fragments read two steps ahead
        auto frag = [&](int k) {
          return k < 12 ? *reinterpret_cast<const half8*>(base + S_QN + off_a(qrow, 384, 2 * k + lh))
                        : *reinterpret_cast<const half8*>(base + S_DON + off_a(qrow, 256, 2 * (k - 12) + lh));
        };
        half8 fa[3];
        fa[0] = frag(0);
        fa[1] = frag(1);
#pragma unroll
        for (int k = 0; k < 20; ++k) {
          if (k + 2 < 20) fa[(k + 2) % 3] = frag(k + 2);
          if (k < 12) s = mfma_f16(fa[k % 3], kf[k], s);
          else dp = mfma_f16(fa[k % 3], vf[k - 12], dp);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // register r holds row swap23(d_row(r, lh)); groups of 4 are consecutive rows
      half8 pf[2], dsf[2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r0 = swap23(d_row(4 * g, lh));
        const f32x4 L = *reinterpret_cast<const f32x4*>(info + r0);
        const f32x4 Dd = *reinterpret_cast<const f32x4*>(info + QB + r0);
        const u32x4 lo4 = *reinterpret_cast<const u32x4*>(iinfo + r0);
        const u32x4 p4 = *reinterpret_cast<const u32x4*>(iinfo + QB + r0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float pv = __builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, -L[e]));
          if (!full) {
            const int64_t lo_r = static_cast<int32_t>(lo4[e]);
            const int64_t p_r = static_cast<int32_t>(p4[e]);
            if (gkey < lo_r || gkey > p_r) pv = 0.f;
          }
          const float ds = pv * (dp[r] - Dd[e]);
          pf[r >> 3][r & 7] = static_cast<_Float16>(pv);
          dsf[r >> 3][r & 7] = static_cast<_Float16>(ds);
        }
      }
      // dV^T += dO^T P,  dK^T += Q^T dS (the query rows are the k-slots)
      {
        // 20 products: per ks, 4 into dV^T then 6 into dK^T
        auto frag = [&](int k) {
          const int ks = k / 10, j = k % 10;
          return j < 4 ? *reinterpret_cast<const half8*>(base + S_DOT + off_c(32 * j + lr, 2 * ks + lh))
                       : *reinterpret_cast<const half8*>(base + S_QT + off_c(32 * (j - 4) + lr, 2 * ks + lh));
        };
        half8 fa[3];
        fa[0] = frag(0);
        fa[1] = frag(1);
#pragma unroll
        for (int k = 0; k < 20; ++k) {
          if (k + 2 < 20) fa[(k + 2) % 3] = frag(k + 2);
          const int ks = k / 10, j = k % 10;
          if (j < 4) dv[j] = mfma_f16(fa[k % 3], pf[ks], dv[j]);
          else dk[j - 4] = mfma_f16(fa[k % 3], dsf[ks], dk[j - 4]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // write: lane = key t, registers = columns (four consecutive per group)
  const int64_t t = tw + lr;
  const int64_t nk = static_cast<int64_t>(n_h) * 128;
#pragma unroll
  for (int mt = 0; mt < 6; ++mt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * mt + 8 * g + 4 * lh;   // dims d..d+3
      const float v0 = dk[mt][4 * g] * scale, v1 = dk[mt][4 * g + 1] * scale,
                  v2 = dk[mt][4 * g + 2] * scale, v3 = dk[mt][4 * g + 3] * scale;
      if (d < 128) {
        const int64_t col = static_cast<int64_t>(h) * 128 + d;
        const half4 hv = {static_cast<_Float16>(v0), static_cast<_Float16>(v1),
                          static_cast<_Float16>(v2), static_cast<_Float16>(v3)};
        *reinterpret_cast<half4*>(dKV + t * (2 * nk) + col) = hv;
        dKVT[(col + 0) * Kpad + t] = hv[0];
        dKVT[(col + 1) * Kpad + t] = hv[1];
        dKVT[(col + 2) * Kpad + t] = hv[2];
        dKVT[(col + 3) * Kpad + t] = hv[3];
      } else {
        const f32x4 fv = {v0, v1, v2, v3};
        *reinterpret_cast<f32x4*>(dKr + (static_cast<int64_t>(h) * Kpad + t) * 64 + (d - 128)) = fv;
      }
    }
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * dt + 8 * g + 4 * lh;
      const int64_t col = nk + static_cast<int64_t>(h) * 128 + d;
      const half4 hv = {static_cast<_Float16>(dv[dt][4 * g]), static_cast<_Float16>(dv[dt][4 * g + 1]),
                        static_cast<_Float16>(dv[dt][4 * g + 2]), static_cast<_Float16>(dv[dt][4 * g + 3])};
      *reinterpret_cast<half4*>(dKV + t * (2 * nk) + col) = hv;
      dKVT[(col + 0) * Kpad + t] = hv[0];
      dKVT[(col + 1) * Kpad + t] = hv[1];
      dKVT[(col + 2) * Kpad + t] = hv[2];
      dKVT[(col + 3) * Kpad + t] = hv[3];
    }
}

// ------------------------------------------------------------------ dQ
constexpr int QW = 128;     // query rows per workgroup (4 waves x 32)
constexpr int KS = 64;      // keys per step
// stage: K [64][192] | V [64][128] | K^T [192][64]
constexpr int D_K = 0, D_V = KS * DQK * 2, D_KT = D_V + KS * DV * 2,
              D_BYTES = D_KT + DQK * KS * 2;

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_bwd_dq_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ dout,
                   const float* __restrict__ lse, const float* __restrict__ D,
                   const _Float16* __restrict__ Knope, const _Float16* __restrict__ Krope,
                   const _Float16* __restrict__ Vkm, const _Float16* __restrict__ KnopeT,
                   const _Float16* __restrict__ KropeT, const int32_t* __restrict__ cu,
                   float* __restrict__ dq, int n_h, int n_seqs, int64_t S_loc, int64_t S_pad,
                   int64_t q_offset, int64_t key_lo, int64_t Kpad, int n_qt, float scale,
                   float scale_log2) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * D_BYTES];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5;
  int h, qt;
  work_item(blockIdx.x, n_h, n_qt, &h, &qt);
  qt = n_qt - 1 - qt;   // heaviest (latest) rows first
  const int64_t q0 = static_cast<int64_t>(qt) * QW;
  const int64_t wq0 = q0 + 32 * w;
  const int64_t i = wq0 + lr;
  const bool valid = i < S_loc;
  const int64_t p = valid ? q_offset + i : -1;
  const int64_t lo = valid ? seg_lo_dev(cu, n_seqs, q_offset + i) : 0;
  const float L2 = valid ? lse[i * n_h + h] * kLog2e : 0.f;
  const float Di = valid ? D[h * S_pad + i] : 0.f;
  const bool wave_live = wq0 < S_loc;
  const int64_t wp_min = q_offset + wq0, wp_max = q_offset + min(S_loc - 1, wq0 + 31);
  const int64_t wlo_min = wave_live ? seg_lo_dev(cu, n_seqs, wp_min) : 0;
  const int64_t wlo_max = wave_live ? seg_lo_dev(cu, n_seqs, wp_max) : 0;

  half8 qf[12], df[8];
#pragma unroll
  for (int kk = 0; kk < 12; ++kk) {
    if (valid) {
      qf[kk] = bf16x8_to_half8(*reinterpret_cast<const u32x4*>(q + (i * n_h + h) * DQK + 16 * kk + 8 * lh));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[kk][e] = static_cast<_Float16>(0.f);
    }
  }
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    if (valid) {
      df[kk] = bf16x8_to_half8(*reinterpret_cast<const u32x4*>(dout + (i * n_h + h) * DV + 16 * kk + 8 * lh));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) df[kk][e] = static_cast<_Float16>(0.f);
    }
  }

  const int64_t i_last = min(S_loc - 1, q0 + QW - 1);
  const int64_t kb_begin = ((seg_lo_dev(cu, n_seqs, q_offset + q0) - key_lo) / KS) * KS;
  const int64_t kb_end = q_offset + i_last + 1 - key_lo;
  const int nblk = static_cast<int>((kb_end - kb_begin + KS - 1) / KS);

  const _Float16* Kh = Knope + static_cast<int64_t>(h) * Kpad * 128;
  const _Float16* Vh = Vkm + static_cast<int64_t>(h) * Kpad * 128;
  const _Float16* KTh = KnopeT + static_cast<int64_t>(h) * 128 * Kpad;
  // this wave's 16 DMA pieces per stage (64 KiB): piece I is K (I < 24), V
  // (< 40) or K^T; per-lane element offsets relative to key row kb. A K piece
  // mixes no-position columns (K_nope) and rope columns (k_rope) across lanes.
  int dma_off[16];
  uint32_t rope_mask = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int o = (w * 16 + j) * 1024 + lane * 16;
    int off;
    bool rope = false;
    if (o < D_V) {
      const int row = o / 384, pos = (o % 384) >> 4;
      const int c = (pos & ~7) | ((pos & 7) ^ sw_a(row));
      rope = c >= 16;
      off = rope ? row * 64 + (c - 16) * 8 : row * 128 + c * 8;
    } else if (o < D_KT) {
      const int oo = o - D_V, row = oo >> 8, pos = (oo & 255) >> 4;
      off = row * 128 + ((pos & ~7) | ((pos & 7) ^ sw_a(row))) * 8;
    } else {
      const int oo = o - D_KT, row = oo >> 7, pos = (oo & 127) >> 4;
      rope = row >= 128;
      off = (rope ? row - 128 : row) * static_cast<int>(Kpad) + (pos ^ (row & 7)) * 8;
    }
    dma_off[j] = off;
    if (rope) rope_mask |= 1u << j;
  }
  auto issue = [&](int64_t kb, int st) {
    char* base = smem + st * D_BYTES;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int I = w * 16 + j;
      const bool rope = (rope_mask >> j) & 1u;
      const _Float16* src = I < 24 ? (rope ? Krope + kb * 64 : Kh + kb * 128)
                          : I < 40 ? Vh + kb * 128
                          : (rope ? KropeT + kb : KTh + kb);
      lds_dma16(src + dma_off[j], base + I * 1024);
    }
  };

  f32x16 acc[6];
#pragma unroll
  for (int a = 0; a < 6; ++a)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[a][e] = 0.f;

  if (nblk > 0) issue(kb_begin, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int b = 0; b < nblk; ++b) {
    const int st = b & 1;
    const int64_t kb = kb_begin + static_cast<int64_t>(b) * KS;
    if (b + 1 < nblk) issue(kb + KS, st ^ 1);
    const int64_t g0 = key_lo + kb;
    const bool skip = !wave_live || g0 > wp_max || g0 + KS - 1 < wlo_min;
    if (!skip) {
      const bool need_mask = !(g0 >= wlo_max && g0 + KS - 1 <= wp_min);
      const char* base = smem + st * D_BYTES;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int krow = 32 * mt + swap23(lr);
        f32x16 s, dp;
#pragma unroll
        for (int e = 0; e < 16; ++e) { s[e] = 0.f; dp[e] = 0.f; }
        {
          auto frag = [&](int k) {
            return k < 12 ? *reinterpret_cast<const half8*>(base + D_K + off_a(krow, 384, 2 * k + lh))
                          : *reinterpret_cast<const half8*>(base + D_V + off_a(krow, 256, 2 * (k - 12) + lh));
          };
          half8 fa[3];
          fa[0] = frag(0);
          fa[1] = frag(1);
#pragma unroll
          for (int k = 0; k < 20; ++k) {
            if (k + 2 < 20) fa[(k + 2) % 3] = frag(k + 2);
            if (k < 12) s = mfma_f16(fa[k % 3], qf[k], s);
            else dp = mfma_f16(fa[k % 3], df[k - 12], dp);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        half8 dsf[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pv = __builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, -L2));
          if (need_mask) {
            const int64_t key = g0 + 32 * mt + swap23(d_row(r, lh));
            if (key < lo || key > p) pv = 0.f;
          }
          dsf[r >> 3][r & 7] = static_cast<_Float16>(pv * (dp[r] - Di));
        }
        {
          // key piece 4mt + 2ksl + lh holds keys 32mt + 16ksl + 8lh ..
          auto frag = [&](int k) {
            const int ksl = k / 6, dm = k % 6;
            return *reinterpret_cast<const half8*>(base + D_KT + off_b(32 * dm + lr, 4 * mt + 2 * ksl + lh));
          };
          half8 fa[3];
          fa[0] = frag(0);
          fa[1] = frag(1);
#pragma unroll
          for (int k = 0; k < 12; ++k) {
            if (k + 2 < 12) fa[(k + 2) % 3] = frag(k + 2);
            acc[k % 6] = mfma_f16(fa[k % 3], dsf[k / 6], acc[k % 6]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (valid) {
    float* dst = dq + (i * n_h + h) * DQK;
#pragma unroll
    for (int dm = 0; dm < 6; ++dm)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 v = {acc[dm][4 * g] * scale, acc[dm][4 * g + 1] * scale,
                         acc[dm][4 * g + 2] * scale, acc[dm][4 * g + 3] * scale};
        *reinterpret_cast<f32x4*>(dst + 32 * dm + 8 * g + 4 * lh) = v;
      }
  }
}

// dk_rope[key_lo + t][r] = sum_h dKr[h][t][r] for t < Kn; other rows 0.
__global__ void __launch_bounds__(256)
reduce_rope_kernel(const float* __restrict__ dKr, float* __restrict__ dk_rope, int n_h,
                   int64_t S, int64_t key_lo, int64_t Kn, int64_t Kpad) {
  const int64_t n = S * 64;
  for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < n;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t j = e >> 6, r = e & 63, t = j - key_lo;
    float acc = 0.f;
    if (t >= 0 && t < Kn)
      for (int h = 0; h < n_h; ++h) acc += dKr[(static_cast<int64_t>(h) * Kpad + t) * 64 + r];
    dk_rope[e] = acc;
  }
}

__global__ void __launch_bounds__(256)
zero_rows_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < n;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[e] = 0.f;
}

unsigned grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  return static_cast<unsigned>(g < 1 ? 1 : (g > 16384 ? 16384 : g));
}

}  // namespace

mla_status fast_bwd(const Plan& p, const void* dout, const void* q, const void* c_kv,
                    const void* k_rope, const void* W_UK, const void* W_UV,
                    const int32_t* cu_dev, const float* out, const float* lse, float* dq,
                    float* dc_kv, float* dk_rope, float* dW_UK, float* dW_UV, char* ws,
                    hipStream_t st) {
  const BwdLayout L = bwd_layout(p);
  if (p.Kpad * 256 >= (int64_t(1) << 31) || p.S_loc * DQK >= (int64_t(1) << 31))
    return fail(MLA_ERR_UNSUPPORTED, "fast backward takes fewer than 2^23 rows per call");
  const int64_t nk = static_cast<int64_t>(p.n_h) * 128;
  const int64_t S_pad = align_up(p.S_loc, 64);
  auto at = [&](int64_t off) { return ws + off; };
  uint16_t* WT = reinterpret_cast<uint16_t*>(at(L.f.WT));
  _Float16* Knope = reinterpret_cast<_Float16*>(at(L.f.Knope));
  _Float16* Krope = reinterpret_cast<_Float16*>(at(L.f.Krope));
  _Float16* KnopeT = reinterpret_cast<_Float16*>(at(L.KnopeT));
  _Float16* KropeT = reinterpret_cast<_Float16*>(at(L.KropeT));
  _Float16* Vkm = reinterpret_cast<_Float16*>(at(L.Vkm));
  _Float16* W16 = reinterpret_cast<_Float16*>(at(L.W16));
  _Float16* ckvT = reinterpret_cast<_Float16*>(at(L.ckvT));
  _Float16* Qn = reinterpret_cast<_Float16*>(at(L.Qn));
  _Float16* Qt = reinterpret_cast<_Float16*>(at(L.Qt));
  _Float16* dOn = reinterpret_cast<_Float16*>(at(L.dOn));
  _Float16* dOt = reinterpret_cast<_Float16*>(at(L.dOt));
  float* D = reinterpret_cast<float*>(at(L.D));
  _Float16* dKV = reinterpret_cast<_Float16*>(at(L.dK));
  _Float16* dKVT = reinterpret_cast<_Float16*>(at(L.dV));
  float* dKr = reinterpret_cast<float*>(at(L.dKrope));
  mla_status s;

  // K_nope (both layouts), V key-major, rope key (both layouts)
  if ((s = fast_rebuild_kv(p, c_kv, k_rope, W_UK, W_UV, WT, Knope, nullptr, Vkm, Krope, KnopeT,
                           KropeT, st)) != MLA_OK)
    return s;
  // [W_UK | W_UV] rows in fp16 and c_kv^T in fp16 for the gradient GEMMs
  if ((s = launch_convert(static_cast<const uint16_t*>(W_UK), nk, 0, p.d_c, p.d_c, nk, W16, 2 * nk,
                          0, Elem::F16, 1, st, "prep_w16")) != MLA_OK)
    return s;
  if ((s = launch_convert(static_cast<const uint16_t*>(W_UV), nk, 0, p.d_c, p.d_c, nk, W16 + nk,
                          2 * nk, 0, Elem::F16, 1, st, "prep_w16")) != MLA_OK)
    return s;
  if ((s = launch_transpose(static_cast<const uint16_t*>(c_kv) + p.key_lo * p.d_c, p.d_c, 0, p.Kn,
                            p.Kpad, p.d_c, ckvT, p.Kpad, 0, Elem::F16, 1, st, "prep_ckvT")) != MLA_OK)
    return s;
  {
    KernelTimer kt("bwd_prep", st);
    hipLaunchKernelGGL(bwd_prep_kernel, dim3(static_cast<unsigned>(S_pad / 64), p.n_h), dim3(256),
                       0, st, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(dout),
                       out, D, Qn, Qt, dOn, dOt, p.n_h, p.S_loc, S_pad);
  }
  if ((s = check_launch("backward prep")) != MLA_OK) return s;
  const float scale_log2 = p.scale * kLog2e;
  {
    const int n_kt = static_cast<int>(p.Kpad / KB);
    KernelTimer kt("attn_bwd_dkdv", st);
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel, dim3(static_cast<unsigned>(n_kt * p.n_h)), dim3(256),
                       0, st, Qn, Qt, dOn, dOt, lse, D, Knope, Krope, Vkm, cu_dev, dKV, dKVT, dKr,
                       p.n_h, p.n_seqs, p.S_loc, S_pad, p.q_offset, p.key_lo, p.Kn, p.Kpad, n_kt,
                       p.scale, scale_log2);
  }
  if ((s = check_launch("attention backward dK/dV")) != MLA_OK) return s;
  {
    const int n_qt = static_cast<int>((p.S_loc + QW - 1) / QW);
    KernelTimer kt("attn_bwd_dq", st);
    hipLaunchKernelGGL(attn_bwd_dq_kernel, dim3(static_cast<unsigned>(n_qt * p.n_h)), dim3(256),
                       0, st, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(dout),
                       lse, D, Knope, Krope, Vkm, KnopeT, KropeT, cu_dev, dq, p.n_h, p.n_seqs,
                       p.S_loc, S_pad, p.q_offset, p.key_lo, p.Kpad, n_qt, p.scale, scale_log2);
  }
  if ((s = check_launch("attention backward dQ")) != MLA_OK) return s;
  // dc_kv rows [key_lo, key_hi) = [dK_nope | dV] (fp16) . [W_UK | W_UV] rows; others 0
  if ((s = launch_gemm_nt(dKV, 2 * nk, p.Kn, W16, 2 * nk, p.d_c, 2 * nk, dc_kv + p.key_lo * p.d_c,
                          p.d_c, 128, p.Kn, p.d_c, Elem::F16, Elem::F32, st, "grad_latent")) != MLA_OK)
    return s;
  {
    KernelTimer kt("zero_rows", st);
    if (p.key_lo > 0)
      hipLaunchKernelGGL(zero_rows_kernel, dim3(grid_for(p.key_lo * p.d_c)), dim3(256), 0, st,
                         dc_kv, p.key_lo * p.d_c);
    if (p.key_hi < p.S)
      hipLaunchKernelGGL(zero_rows_kernel, dim3(grid_for((p.S - p.key_hi) * p.d_c)), dim3(256), 0,
                         st, dc_kv + p.key_hi * p.d_c, (p.S - p.key_hi) * p.d_c);
  }
  if ((s = check_launch("zero rows")) != MLA_OK) return s;
  // dW_UK = c_kv^T dK_nope, dW_UV = c_kv^T dV (contract over the shard's keys)
  if ((s = launch_gemm_nt(ckvT, p.Kpad, p.d_c, dKVT, p.Kpad, nk, p.Kpad, dW_UK, nk, 128, p.d_c, nk,
                          Elem::F16, Elem::F32, st, "grad_w")) != MLA_OK)
    return s;
  if ((s = launch_gemm_nt(ckvT, p.Kpad, p.d_c, dKVT + nk * p.Kpad, p.Kpad, nk, p.Kpad, dW_UV, nk,
                          128, p.d_c, nk, Elem::F16, Elem::F32, st, "grad_w")) != MLA_OK)
    return s;
  {
    KernelTimer kt("reduce_rope", st);
    hipLaunchKernelGGL(reduce_rope_kernel, dim3(grid_for(p.S * 64)), dim3(256), 0, st, dKr,
                       dk_rope, p.n_h, p.S, p.key_lo, p.Kn, p.Kpad);
  }
  return check_launch("rope-key gradient reduce");
}

}  // namespace mla
