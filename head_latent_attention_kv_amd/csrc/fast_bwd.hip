// Fast backward: gradients of sum(out * dout) through attention and the
// latent up-projection (the training path of the LAGA abstract: K/V are
// rebuilt from the latent, so their gradients flow back into c_kv, k_rope,
// W_UK and W_UV).
//
//   scale     max|dout| -> a power of two 2^e that brings it into [4, 8)
//   prep      D = rowsum(2^e dout * out); q and 2^e dout to fp16, per head,
//             row-major [row][dim]
//   rebuild   K_nope and V again (fp16), in the layouts the kernels read
//   dK, dV    key-outer, one launch of paired waves: a pair owns 32 keys
//             and steps over query rows; S = Q K^T lands with lanes on keys
//             and, with the query rows loaded in swap23 order, P and dS are
//             already the k-operands of dV^T += dO^T P and dK^T += Q^T dS.
//   dq        query-outer: each wave owns 32 rows (two waves per SIMD); S^T,
//             dP^T per lane = row, dQ^T += K^T dS^T. No atomics: the result
//             is deterministic.
//   GEMMs     dc_kv = [dK_nope | dV] [W_UK | W_UV]^T,  dW = c_kv^T [dK_nope | dV]
//   reduce    dk_rope = sum over heads of the per-head rope-key gradients
//
// Every gradient is linear in dout. dout, dP, dS and the [dK_nope | dV] rows
// are held in fp16, whose normal range starts at 2^-14, while the output
// gradients of a training step are often far smaller. So dout enters scaled
// by 2^e (exact: a power of two), every fp16 intermediate carries that
// factor, and the fp32 results leave multiplied by 2^-e (exact again). The
// scaled dout has its largest magnitude in [4, 8), the range of a standard
// normal sample of this size, for any input scale.
//
// Query/key tiles are DMA-filled (global_load_lds) into swizzled LDS rows
// and double-buffered, as in the forward.
#include <math.h>
#include <stdlib.h>

#include <algorithm>
#include <type_traits>

#include "fast.h"
#include "fast_common.h"

namespace mla {
namespace {

constexpr int DQK = 192, DV = 128;
constexpr float kLog2e = 1.44269504088896340736f;
// The row info holds lse log2(e) - kPShift, so that the dK/dV kernel's
// weights come out as P 2^kPShift <= 2^15 (P <= 1): a key's weights among
// many keys (about 1 / keys each) then stay in fp16's normal range down to
// P = 2^-29 in the dV product. The dQ kernel adds the shift back.
constexpr int kPShift = 15;

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

// ------------------------------------------------------------------ dout scale
// part[b] = bits of the largest |dout| element that block b reads (bf16 bit
// patterns without the sign; as unsigned integers they order like the
// magnitudes, and the non-finite ones sit above 0x7f7f). n8 = elements / 8.
__global__ void __launch_bounds__(256)
dout_absmax_kernel(const u32x4* __restrict__ x, int64_t n8, uint32_t* __restrict__ part) {
  __shared__ uint32_t wmax[4];
  uint32_t m = 0;
  for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < n8;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const u32x4 v = x[e];
#pragma unroll
    for (int k = 0; k < 4; ++k) m = max(m, max(v[k] & 0x7fffu, (v[k] >> 16) & 0x7fffu));
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), s, 64)));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
}

// sc[0] = 2^e, sc[1] = 2^-e with 2^e max|dout| in [4, 8): e = 2 - floor(log2
// max|dout|), read off the bf16 exponent (or, for a subnormal maximum, off
// its leading mantissa bit), clamped to [-126, 126] so that both factors
// are normal floats. e = 0 when dout is all zero or holds a non-finite value.
// It also clears hm[0 .. n_hm), the per-head maxima that the row preparation
// (the next kernel on the stream) raises.
__global__ void __launch_bounds__(256)
dout_scale_kernel(const uint32_t* __restrict__ part, int n, float* __restrict__ sc,
                  uint32_t* __restrict__ hm, int n_hm) {
  __shared__ uint32_t wmax[4];
  for (int i = threadIdx.x; i < n_hm; i += blockDim.x) hm[i] = 0u;
  uint32_t m = 0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) m = max(m, part[i]);
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), s, 64)));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    int e = 0;
    if (m != 0 && m < 0x7f80u) {
      const int ex = static_cast<int>(m >> 7);   // biased exponent (sign bit is clear)
      const int fl = ex > 0 ? ex - 127 : (31 - __clz(static_cast<int>(m & 0x7fu))) - 133;
      e = min(126, max(-126, 2 - fl));
    }
    sc[0] = __uint_as_float(static_cast<uint32_t>(e + 127) << 23);
    sc[1] = __uint_as_float(static_cast<uint32_t>(127 - e) << 23);
  }
}

// fp16 of 8 bf16 values times s (a power of two: the product is exact)
__device__ __forceinline__ half8 bf16x8_to_half8_scaled(u32x4 v, float s) {
  half8 h;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t w = v[k];
    h[2 * k] = static_cast<_Float16>(__uint_as_float(w << 16) * s);
    h[2 * k + 1] = static_cast<_Float16>(__uint_as_float(w & 0xffff0000u) * s);
  }
  return h;
}

// ------------------------------------------------------------------ prep
// grid (ceil(S_loc/64), n_h), dout scaled by sc[0] = 2^e throughout.
// D[h][i] = 2^e dout[i,h,:] . out[i,h,:]; fp16 copies Qn[h][i][192] and
// dOn[h][i][128] (2^e dout; rows past S_loc are zero); and per
// 32-row block the row info the dK/dV kernels read:
// info[h][i/32] = {lse*log2(e) - kPShift [32], D [32], sample start [32],
// position [32]}
// (rows past S_loc: start INT32_MAX, position -1, so they see no key).
// hm[2 h] and hm[2 h + 1] are raised (as float bits: non-negative floats
// order like their bit patterns) to the largest |2^e dout[i,h,:]| (2-norm)
// and |D[h][i]| over the rows: with a key's |V| row norm they bound every
// |dP - D| of the key, which sets its dS scale in the dK/dV kernel.
__global__ void __launch_bounds__(256)
bwd_prep_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ dout,
                const float* __restrict__ out, const float* __restrict__ lse,
                const int32_t* __restrict__ cu, const float* __restrict__ sc, float* __restrict__ D,
                _Float16* __restrict__ Qn, _Float16* __restrict__ dOn, uint32_t* __restrict__ info,
                uint32_t* __restrict__ hm, int n_h, int n_seqs, int64_t S_loc, int64_t S_pad,
                RowMap rm) {
  const int h = blockIdx.y;
  const float dsc = sc[0];
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int tid = threadIdx.x;
  // row info except D: one thread per row
  if (tid < 64) {
    const int64_t i = i0 + tid;
    uint32_t* blk = info + (static_cast<int64_t>(h) * (S_pad / 32) + i / 32) * 128;
    const int r = static_cast<int>(i % 32);
    const bool ok = i < S_loc;
    blk[r] = __float_as_uint(ok ? lse[i * n_h + h] * kLog2e - kPShift : 0.f);
    const int pos = rm_pos(rm, static_cast<int>(i));
    blk[64 + r] = ok ? static_cast<uint32_t>(seg_lo_dev(cu, n_seqs, pos)) : 0x7fffffffu;
    blk[96 + r] = ok ? static_cast<uint32_t>(pos) : 0xffffffffu;
  }
  // q to fp16, 16 bytes per thread
  {
    _Float16* nat = Qn + static_cast<int64_t>(h) * S_pad * DQK;
    constexpr int chunks = DQK / 8;
    for (int e = tid; e < 64 * chunks; e += 256) {
      const int row = e / chunks, ch = e % chunks;
      const int64_t i = i0 + row;
      half8 v;
      if (i < S_loc) {
        v = bf16x8_to_half8_scaled(*reinterpret_cast<const u32x4*>(q + (i * n_h + h) * DQK + ch * 8), 1.f);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = static_cast<_Float16>(0.f);
      }
      *reinterpret_cast<half8*>(nat + (i0 + row) * DQK + ch * 8) = v;
    }
  }
  // 2^e dout to fp16 and D in the same pass: the 16 threads of a row each
  // take 8 columns of dout and out (16-byte loads) and sum their products
  // (and the squares of dout) across the 16 lanes
  {
    __shared__ float wred[2][4];
    float nmax = 0.f, dmax = 0.f;   // largest |dout row|^2 and |D| of the thread's rows
    _Float16* nat = dOn + static_cast<int64_t>(h) * S_pad * DV;
    const int ch = tid & 15;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int row = (tid >> 4) + 16 * it;
      const int64_t i = i0 + row;
      half8 v;
      float part = 0.f, sq = 0.f;
      if (i < S_loc) {
        const int64_t base = (i * n_h + h) * DV + ch * 8;
        const u32x4 d = *reinterpret_cast<const u32x4*>(dout + base);
        const f32x4 o0 = *reinterpret_cast<const f32x4*>(out + base);
        const f32x4 o1 = *reinterpret_cast<const f32x4*>(out + base + 4);
        v = bf16x8_to_half8_scaled(d, dsc);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float lo = __uint_as_float(d[k] << 16) * dsc, hi = __uint_as_float(d[k] & 0xffff0000u) * dsc;
          const float olo = k < 2 ? o0[2 * k] : o1[2 * k - 4], ohi = k < 2 ? o0[2 * k + 1] : o1[2 * k - 3];
          part = fmaf(lo, olo, part);
          part = fmaf(hi, ohi, part);
          sq = fmaf(lo, lo, fmaf(hi, hi, sq));
        }
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = static_cast<_Float16>(0.f);
      }
      *reinterpret_cast<half8*>(nat + (i0 + row) * DV + ch * 8) = v;
#pragma unroll
      for (int sft = 8; sft >= 1; sft >>= 1) {
        part += __shfl_xor(part, sft, 16);
        sq += __shfl_xor(sq, sft, 16);
      }
      nmax = fmaxf(nmax, sq);
      dmax = fmaxf(dmax, fabsf(part));
      if (ch == 0) {
        D[h * S_pad + i] = part;
        info[(static_cast<int64_t>(h) * (S_pad / 32) + i / 32) * 128 + 32 + i % 32] = __float_as_uint(part);
      }
    }
    // block maxima (the 16 lanes of a row group agree), one atomic each
    nmax = fmaxf(nmax, __shfl_xor(nmax, 16));
    nmax = fmaxf(nmax, __shfl_xor(nmax, 32));
    dmax = fmaxf(dmax, __shfl_xor(dmax, 16));
    dmax = fmaxf(dmax, __shfl_xor(dmax, 32));
    if ((tid & 63) == 0) {
      wred[0][tid >> 6] = nmax;
      wred[1][tid >> 6] = dmax;
    }
    __syncthreads();
    if (tid == 0) {
      const float n2 = fmaxf(fmaxf(wred[0][0], wred[0][1]), fmaxf(wred[0][2], wred[0][3]));
      const float dm = fmaxf(fmaxf(wred[1][0], wred[1][1]), fmaxf(wred[1][2], wred[1][3]));
      if (n2 > 0.f) atomicMax(hm + 2 * h, __float_as_uint(sqrtf(n2)));
      if (dm > 0.f) atomicMax(hm + 2 * h + 1, __float_as_uint(dm));
    }
  }
}

// ------------------------------------------------------------------ shared by dK/dV and dQ
constexpr int QB = 64;      // query rows per step of the key-outer kernel

// ------------------------------------------------------------------ dK + dV, paired waves
// One launch for dK and dV without computing S twice. A workgroup owns 128
// keys and runs 8 waves as 4 pairs; the pair p owns keys 32 p .. 32 p + 31.
// Wave p ("A") holds the keys' K rows, computes S = Q K^T and P, publishes P
// (fp16) in a 2 KiB LDS slot and accumulates dV^T += dO^T P. Wave p + 4
// ("B") holds the keys' V rows, computes dP = dO V^T, takes P from the slot,
// forms dS = P (dP - D) and accumulates dK^T += Q^T dS. Both carry
// power-of-two factors that keep the fp16 operands in fp16's normal range
// for long sequences (exact, removed at the write-out): P comes as P 2^15
// (the row info's shift), and B's dS as dS 2^ex with ex per key, the largest
// power for which a bound on every |dP - D| of the key (from the per-head
// maxima of the row preparation and the key's |V| row norm) keeps
// |dS 2^ex| < 2^14. B folds 2^(ex - 15) into its V rows and starts each dP
// accumulation at -D 2^(ex - 15), so that (dP - D) 2^(ex - 15) leaves the
// products as one; after the barrier it converts that to fp16 and forms
// dS 2^ex = (P 2^15) (dP - D) 2^(ex - 15) with packed fp16 products. Each
// role does 20 of
// the 40 products of a 32 x 32 sub-block and keeps under 256 registers, so
// two waves share each SIMD. One barrier per 32-row sub-block separates the
// publication of P from its use; the slot is double-buffered, so A writes
// P(t + 2) only after the barrier that follows B's read of P(t).
//
// Tiles: q rows (swizzled 448-byte rows, read row-wise by A and transposed by
// B) and dout rows (swizzled 320-byte rows, read row-wise by B and transposed
// by A), double-buffered per 64-row block and DMA-filled.
constexpr int PW = 128;                        // keys per workgroup
constexpr int PF = 3;                          // fragment reads in flight ahead of the products
constexpr int kExCap = 64;                     // largest power-of-two factor on dS
constexpr int PD_ROW = 320;                    // dout rows (128 elements), swizzled
constexpr int P_QN = 0, P_DON = 28 * 1024, P_INFO = 48 * 1024, P_BYTES = 49 * 1024;
constexpr int P_PIECES = P_BYTES / 1024;       // 49
constexpr int P_NPW = (P_PIECES + 3) / 4;      // 13 per B wave (only B waves issue the DMA)
constexpr int P_XCH = 2 * P_BYTES;             // P slots: [pair][buffer] x 2 KiB
static_assert(P_DON >= QB * XS_ROW && P_INFO - P_DON >= QB * PD_ROW && P_BYTES - P_INFO >= QB * 16,
              "paired dK/dV stage layout");
// Staging tiles after the loop: dKr rows, 128 keys x 64 floats padded to 68
// (272 bytes); then dKV rows, 128 keys x 256 halves padded to 264 (528
// bytes, an odd number of 16-byte slots)
constexpr int R_PITCH = 68, K_PITCH = 264;
static_assert(128 * R_PITCH * 4 <= 2 * P_BYTES + 4 * 2 * 2048 &&
              128 * K_PITCH * 2 <= 2 * P_BYTES + 4 * 2 * 2048, "staging tiles fit the LDS");

__global__ void __launch_bounds__(512)
attn_bwd_dkdv_kernel(const _Float16* __restrict__ Qn, const _Float16* __restrict__ dOn,
                     const uint32_t* __restrict__ info, const _Float16* __restrict__ Kfull,
                     const _Float16* __restrict__ Vkm, const int32_t* __restrict__ cu,
                     const int* __restrict__ korder, _Float16* __restrict__ dKV,
                     float* __restrict__ dKr, _Float16* __restrict__ dS,
                     const uint32_t* __restrict__ hm, int n_h, int h0, int n_hg, int n_seqs,
                     int S_loc, int S_pad, RowMap rm, int key_lo, int Kpad, int n_kt, float scale,
                     float scale_log2) {
  // stages, then P slots [pair][buffer], then dS slots [pair][buffer]
  __shared__ __attribute__((aligned(1024))) char smem[2 * P_BYTES + 2 * 4 * 2 * 2048];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int lr = lane & 31, lh = lane >> 5;
  const bool role_a = w < 4;
  const int pi = w & 3;                       // pair index
  // heads h0 .. h0 + n_hg - 1; dS (when stored) holds those heads only
  int hl, kt;
  work_item(blockIdx.x, n_hg, n_kt, &hl, &kt);
  const int h = h0 + hl;
  if (korder != nullptr) kt = korder[kt];     // packed calls: heaviest key tiles first
  const int t0 = kt * PW;                     // workspace key row of the workgroup
  const int tw = t0 + 32 * pi;                // the pair's first key
  const int gkey = key_lo + tw + lr;          // this lane's key (global)
  const int gk_min = key_lo + t0, gk_max = key_lo + t0 + PW - 1;
  const int gw_min = key_lo + tw, gw_max = gw_min + 31;
  char* const xslot = smem + P_XCH + pi * 4096;   // this pair's two P slots
  char* const dslot = smem + P_XCH + 4 * 4096 + pi * 4096;   // and its two dS slots

  // query rows that see any key of the workgroup: from the first row at or
  // past its first key to the last row whose sample starts by its last key
  const int i_begin = rm_rows_below(rm, gk_min);
  int i_end = S_loc;
  if (n_seqs > 0) {
    // first sample start after gk_max (none: S): rows from there on see nothing here
    int lo_i = 0, hi_i = n_seqs + 1;
    while (hi_i - lo_i > 1) {
      const int mid = (lo_i + hi_i) >> 1;
      if (cu[mid] <= gk_max) lo_i = mid; else hi_i = mid;
    }
    if (lo_i + 1 <= n_seqs) i_end = rm_rows_below(rm, cu[lo_i + 1]);
  }
  const int qb_begin = (i_begin / QB) * QB;
  const int nq = i_end > qb_begin ? (i_end - qb_begin + QB - 1) / QB : 0;

  // DMA: per-lane source offsets (elements) relative to the region's first
  // row qb; a row's pad slots reload its slot 0 and are never read back
  const _Float16* Qn_h = Qn + static_cast<int64_t>(h) * S_pad * DQK;
  const _Float16* dOn_h = dOn + static_cast<int64_t>(h) * S_pad * DV;
  const uint32_t* info_h = info + static_cast<int64_t>(h) * (S_pad / 32) * 128;
  int doff[P_NPW];
#pragma unroll
  for (int j = 0; j < P_NPW; ++j) {
    const int o = ((w & 3) * P_NPW + j) * 1024 + lane * 16;
    int off = 0;
    if (o < P_DON) {
      const int row = min(o / XS_ROW, QB - 1), ph = (o % XS_ROW) >> 4;
      off = row * DQK + (ph < DQK / 8 ? xs_slot(row, ph) : 0) * 8;
    } else if (o < P_INFO) {
      const int oo = o - P_DON, row = min(oo / PD_ROW, QB - 1), ph = (oo % PD_ROW) >> 4;
      off = row * DV + (ph < DV / 8 ? xs_slot(row, ph) : 0) * 8;
    } else {
      off = min((o - P_INFO) >> 2, 2 * 128 - 4);   // 4-byte elements, 128 per 32 rows
    }
    doff[j] = off;
  }
  auto issue = [&](int qb, int st) {
    char* sbase = smem + st * P_BYTES;
#pragma unroll
    for (int j = 0; j < P_NPW; ++j) {
      const int I = (w & 3) * P_NPW + j;   // wave-uniform region choice
      if (I < P_PIECES) {
        // wave-uniform base plus an opaque unsigned 32-bit lane offset in
        // bytes (the scalar-base form of the load)
        uint32_t off = static_cast<uint32_t>(doff[j]) * (I * 1024 >= P_INFO ? 4u : 2u);
        asm volatile("" : "+v"(off));
        const char* ub;
        if (I * 1024 < P_DON) ub = reinterpret_cast<const char*>(Qn_h + static_cast<int64_t>(qb) * DQK);
        else if (I * 1024 < P_INFO) ub = reinterpret_cast<const char*>(dOn_h + static_cast<int64_t>(qb) * DV);
        else ub = reinterpret_cast<const char*>(info_h + (qb / 32) * 128);
        lds_dma16(ub, off, sbase + I * 1024);
      }
    }
  };

  // The two roles run separate copies of the loop, so that the registers of
  // one (K rows, dV^T) and of the other (V rows, dK^T) can share storage;
  // both copies pass the same barriers in the same order.
  auto run = [&](auto role) {
    constexpr bool kA = decltype(role)::value;
    // A: the keys' K rows; B: their V rows (MFMA B fragments)
    half8 kf[kA ? 12 : 1], vf[kA ? 1 : 8];
    if constexpr (kA) {
      const _Float16* kr = Kfull + (static_cast<int64_t>(h) * Kpad + tw + lr) * DQK + 8 * lh;
#pragma unroll
      for (int kk = 0; kk < 12; ++kk) kf[kk] = *reinterpret_cast<const half8*>(kr + 16 * kk);
    } else {
      const _Float16* vr = Vkm + (static_cast<int64_t>(h) * Kpad + tw + lr) * DV + 8 * lh;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) vf[kk] = *reinterpret_cast<const half8*>(vr + 16 * kk);
    }
    // B: the key's dS factor 2^ex. |dP - D| <= |dO row| |V row| + |D| <=
    // m1 |V_k| + m2 < 2^fe gives |dS 2^ex| <= 2^15 2^fe 2^(ex - 15) = 2^14
    // for ex = 14 - fe (m1 is at least 1 so that |V_k 2^(ex - 15)| < 1/2;
    // a key with a zero bound has dS = 0 and takes the cap). fs = 2^(ex - 15)
    // scales the V rows (exactly: no result leaves fp16's range) and D.
    int ex = kExCap;
    float fs = 1.f;
    if constexpr (!kA) {
      float v2 = 0.f;
  #pragma unroll
      for (int kk = 0; kk < 8; ++kk)
  #pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float v = static_cast<float>(vf[kk][j]);
          v2 = fmaf(v, v, v2);
        }
      v2 += __shfl_xor(v2, 32);   // lanes l and l ^ 32 hold the two halves of the row
      const float m1 = fmaxf(__uint_as_float(hm[2 * h]), 1.f), m2 = __uint_as_float(hm[2 * h + 1]);
      const float bnd = fmaf(m1, sqrtf(v2), m2);
      if (bnd > 0.f) {
        int fe;
        (void)frexpf(bnd, &fe);   // bnd in [2^(fe-1), 2^fe)
        ex = min(kExCap, 14 - fe);
      }
  #pragma unroll
      for (int kk = 0; kk < 8; ++kk)
  #pragma unroll
        for (int j = 0; j < 8; ++j) vf[kk][j] = __builtin_amdgcn_ldexph(vf[kk][j], ex - kPShift);
      fs = ldexpf(1.f, ex - kPShift);
    }
    // A: dV^T tiles (4 x 32 dims); B: dK^T tiles (6 x 32 dims)
    f32x16 acc[6];
  #pragma unroll
    for (int a = 0; a < 6; ++a)
  #pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][e] = 0.f;

    const int qrow = swap23(lr);   // row-operand row loaded by this lane
    // A: q rows (S) and dout^T (dV); B: dout rows (dP) and q^T (dK)
    const int a_r0 = kA ? P_QN + xs_row_base<XS_ROW>(qrow, lh, 0) : P_DON + xs_row_base<PD_ROW>(qrow, lh, 0);
    const int a_r1 = kA ? P_QN + xs_row_base<XS_ROW>(qrow, lh, 1) : P_DON + xs_row_base<PD_ROW>(qrow, lh, 1);
    const int a_t0 = kA ? P_DON + xs_tr_base<PD_ROW>(lane, 0) : P_QN + xs_tr_base<XS_ROW>(lane, 0);
    const int a_t1 = kA ? P_DON + xs_tr_base<PD_ROW>(lane, 1) : P_QN + xs_tr_base<XS_ROW>(lane, 1);

    if (!kA && nq > 0) issue(qb_begin, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // A: the 32-row block whose dS waits in the slot (-1: none). The dS
    // block of (key tile, 32-row block) is 8 KiB: [pair][ks][lane] x 16
    // bytes, lane = 32 lh + lr holding key 32 pair + lr and rows 16 ks +
    // 8 lh .. + 7, so each store writes 1 KiB contiguously.
    int ds_q0 = -1;
    auto store_ds = [&](int par) {
      if (ds_q0 >= 0) {
        const half8 v0 = *reinterpret_cast<const half8*>(dslot + par * 2048 + lane * 16);
        const half8 v1 = *reinterpret_cast<const half8*>(dslot + par * 2048 + 1024 + lane * 16);
        _Float16* db = dS + (((static_cast<int64_t>(hl) * n_kt + kt) * (S_pad / 32) + (ds_q0 >> 5)) * 4096 +
                             pi * 1024 + lane * 8);
        // non-temporal: the dS stream then leaves the q/dO tiles in L2
        __builtin_nontemporal_store(v0, reinterpret_cast<half8*>(db));
        __builtin_nontemporal_store(v1, reinterpret_cast<half8*>(db + 512));
      }
    };
    for (int b = 0; b < nq; ++b) {
      const int st = b & 1;
      const int qb = qb_begin + b * QB;
      if (!kA && b + 1 < nq) issue(qb + QB, st ^ 1);
      const char* base = smem + st * P_BYTES;
  #pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int q0 = qb + 32 * mt;
        char* xs = xslot + mt * 2048;          // sub-block parity: buffer mt
        const float* rinfo = reinterpret_cast<const float*>(base + P_INFO + mt * 512);
        const int32_t* iinfo = reinterpret_cast<const int32_t*>(rinfo + 64);
        // first and last position of the sub-block's rows (positions increase
        // with the row; rows past S_loc hold position -1)
        const int p_first = iinfo[32];
        const int p_last = iinfo[31 + max(min(32, S_loc - q0), 1)];
        // the same for both waves of a pair (same keys, same rows)
        const bool skip = q0 >= S_loc || p_last < gw_min || iinfo[0] > gw_max;
        half8 pf[2];
        f32x16 dp;
        // ---- phase 1: A computes S and P and publishes P; B computes dP
        if (!skip) {
          if constexpr (kA) {
            const bool full = q0 + 32 <= S_loc && p_first >= gw_max && iinfo[31] <= gw_min;
            f32x16 s;
  #pragma unroll
            for (int e = 0; e < 16; ++e) s[e] = 0.f;
            auto frag = [&](int k) {
              return *reinterpret_cast<const half8*>(base + ((k & 1) ? a_r1 : a_r0) + mt * 32 * XS_ROW + 64 * (k >> 1));
            };
            half8 fa[PF + 1];
            #pragma unroll
            for (int i = 0; i < PF; ++i) fa[i] = frag(i);
  #pragma unroll
            for (int k = 0; k < 12; ++k) {
              if (k + PF < 12) fa[(k + PF) % (PF + 1)] = frag(k + PF);
              s = mfma_f16(fa[k % (PF + 1)], kf[k], s);
              __builtin_amdgcn_sched_barrier(0);
            }
            if (!full) {
              // rows that do not see this lane's key get weight 0 (score -> -inf)
  #pragma unroll
              for (int g = 0; g < 4; ++g) {
                const int r0 = swap23(d_row(4 * g, lh));
                const u32x4 lo4 = *reinterpret_cast<const u32x4*>(iinfo + r0);
                const u32x4 p4 = *reinterpret_cast<const u32x4*>(iinfo + 32 + r0);
  #pragma unroll
                for (int e = 0; e < 4; ++e)
                  if (gkey < static_cast<int>(lo4[e]) || gkey > static_cast<int>(p4[e])) s[4 * g + e] = -INFINITY;
              }
            }
            // P = exp2(S scale log2e - lse log2e) in fp16; register r holds row
            // swap23(d_row(r, lh)) and groups of 4 are consecutive rows
  #pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x4 L = *reinterpret_cast<const f32x4*>(rinfo + swap23(d_row(4 * g, lh)));
  #pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int r = 4 * g + e;
                pf[r >> 3][r & 7] = static_cast<_Float16>(__builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, -L[e])));
              }
            }
            *reinterpret_cast<half8*>(xs + lane * 16) = pf[0];
            *reinterpret_cast<half8*>(xs + 1024 + lane * 16) = pf[1];
          } else {
            // dp <- (dO V^T - D) 2^(ex - 15): the accumulation starts at -D fs
  #pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x4 Dd = *reinterpret_cast<const f32x4*>(rinfo + 32 + swap23(d_row(4 * g, lh)));
  #pragma unroll
              for (int e = 0; e < 4; ++e) dp[4 * g + e] = -Dd[e] * fs;
            }
            auto frag = [&](int k) {
              return *reinterpret_cast<const half8*>(base + ((k & 1) ? a_r1 : a_r0) + mt * 32 * PD_ROW + 64 * (k >> 1));
            };
            half8 fa[PF + 1];
            #pragma unroll
            for (int i = 0; i < PF; ++i) fa[i] = frag(i);
  #pragma unroll
            for (int k = 0; k < 8; ++k) {
              if (k + PF < 8) fa[(k + PF) % (PF + 1)] = frag(k + PF);
              dp = mfma_f16(fa[k % (PF + 1)], vf[k], dp);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
        // P(t) visible to B; every wave, every sub-block. Only LDS is waited
        // for: the DMA of the next block keeps running (a __syncthreads()
        // would wait for it here).
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        asm volatile("s_barrier" ::: "memory");
        // ---- phase 2: A accumulates dV^T; B forms dS and accumulates dK^T
        if (!skip) {
          if constexpr (kA) {
            // dV^T (dims x keys) += dO^T (dims x rows) . P (rows x keys)
            auto frag = [&](int k) {
              const int ks = k / 4, dt = k % 4;
              const int o = (32 * mt + 16 * ks) * PD_ROW + 64 * dt;
              return frag_tr2(base + a_t0 + o, base + a_t1 + o);
            };
            half8 fa[PF + 1];
            #pragma unroll
            for (int i = 0; i < PF; ++i) fa[i] = frag(i);
  #pragma unroll
            for (int k = 0; k < 8; ++k) {
              if (k + PF < 8) fa[(k + PF) % (PF + 1)] = frag(k + PF);
              acc[k % 4] = mfma_f16(fa[k % (PF + 1)], pf[k / 4], acc[k % 4]);
              __builtin_amdgcn_sched_barrier(0);
            }
          } else {
            pf[0] = *reinterpret_cast<const half8*>(xs + lane * 16);
            pf[1] = *reinterpret_cast<const half8*>(xs + 1024 + lane * 16);
            // dp in fp16 while P is read (|dp| < 1/2 by the choice of ex:
            // fp16 keeps it to 2^-11 relative), then dS with packed products
            half8 dph[2];
  #pragma unroll
            for (int r = 0; r < 16; ++r) dph[r >> 3][r & 7] = static_cast<_Float16>(dp[r]);
            // dS 2^ex = (P 2^15) (dP - D) 2^(ex - 15)
            half8 dsf[2];
            dsf[0] = pf[0] * dph[0];
            dsf[1] = pf[1] * dph[1];
            // dK^T (dims x keys) += Q^T (dims x rows) . dS (rows x keys)
            auto frag = [&](int k) {
              const int ks = k / 6, dm = k % 6;
              const int o = (32 * mt + 16 * ks) * XS_ROW + 64 * dm;
              return frag_tr2(base + a_t0 + o, base + a_t1 + o);
            };
            half8 fa[PF + 1];
            #pragma unroll
            for (int i = 0; i < PF; ++i) fa[i] = frag(i);
  #pragma unroll
            for (int k = 0; k < 12; ++k) {
              if (k + PF < 12) fa[(k + PF) % (PF + 1)] = frag(k + PF);
              acc[k % 6] = mfma_f16(fa[k % (PF + 1)], dsf[k / 6], acc[k % 6]);
              __builtin_amdgcn_sched_barrier(0);
            }
            // dS (without the factor: the dQ kernel reads it as it is) to the
            // pair's slot for this sub-block parity; wave A stores it in the
            // next phase 2, where it has slack
            if (dS != nullptr) {
              half8 du[2];
  #pragma unroll
              for (int r = 0; r < 16; ++r) du[r >> 3][r & 7] = __builtin_amdgcn_ldexph(dsf[r >> 3][r & 7], -ex);
              *reinterpret_cast<half8*>(dslot + mt * 2048 + lane * 16) = du[0];
              *reinterpret_cast<half8*>(dslot + mt * 2048 + 1024 + lane * 16) = du[1];
            }
          }
        }
        if constexpr (kA) {
          // the previous sub-block's dS (slot 1 - mt, written by B before
          // this sub-block's barrier) to HBM, then remember this one
          store_ds(1 - mt);
          ds_q0 = skip || dS == nullptr ? -1 : q0;
        }
      }
      // B waves issued the DMA of the next block and wait for it; A waves
      // wait for their LDS accesses only, so that their dS stores, still
      // in flight, do not hold the barrier
      if constexpr (!kA) __builtin_amdgcn_s_waitcnt(0);
      else __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      asm volatile("s_barrier" ::: "memory");
    }
    if constexpr (kA) store_ds(1);   // the last sub-block (odd parity)

    // write: lane = key t, registers = dims (four consecutive per group).
    // Every output leaves through LDS in whole rows: first the fp32 rope
    // part of dK (dKr: 128 keys x 64 floats, one contiguous 32 KiB block),
    // then dKV row-major (one key, 2 x 256 bytes), which the latent-gradient
    // GEMM reads as it is and the weight-gradient GEMMs read k-major.
    const int64_t nk = static_cast<int64_t>(n_h) * 128;
    const int key = 32 * pi + lr;                           // key within the workgroup
    // A: P carried 2^15; B: dS carried 2^ex (exact powers of two)
    const float sc = kA ? ldexpf(1.f, -kPShift) : scale * ldexpf(1.f, -ex);
    float* rtile = reinterpret_cast<float*>(smem);          // [128 keys][R_PITCH] (free after the loop)
    if constexpr (!kA) {
  #pragma unroll
      for (int mt = 4; mt < 6; ++mt) {
  #pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = 32 * mt + 8 * g + 4 * lh;   // dims d..d+3 of dK's rope part
          const f32x4 fv = {acc[mt][4 * g] * sc, acc[mt][4 * g + 1] * sc, acc[mt][4 * g + 2] * sc,
                            acc[mt][4 * g + 3] * sc};
          *reinterpret_cast<f32x4*>(rtile + key * R_PITCH + (d - 128)) = fv;
        }
      }
    }
    __syncthreads();   // the B waves' rope rows written
    // dKr[h][t0 .. t0+127][64]: contiguous
    float* kr = dKr + (static_cast<int64_t>(h) * Kpad + t0) * 64;
    for (int e = tid; e < 128 * 16; e += 512) {
      const int k = e >> 4, c = e & 15;
      *reinterpret_cast<f32x4*>(kr + k * 64 + 4 * c) = *reinterpret_cast<const f32x4*>(rtile + k * R_PITCH + 4 * c);
    }
    __syncthreads();   // the tiles are read; reuse the space row-major
    _Float16* rows = reinterpret_cast<_Float16*>(smem);     // [128 keys][K_PITCH]: dK_nope | dV
  #pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
  #pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * mt + 8 * g + 4 * lh;
        const half4 hv = {static_cast<_Float16>(acc[mt][4 * g] * sc), static_cast<_Float16>(acc[mt][4 * g + 1] * sc),
                          static_cast<_Float16>(acc[mt][4 * g + 2] * sc), static_cast<_Float16>(acc[mt][4 * g + 3] * sc)};
        *reinterpret_cast<half4*>(rows + key * K_PITCH + (kA ? 128 : 0) + d) = hv;
      }
    }
    __syncthreads();
    // dKV[t0 + k][h*128 ..] (dK_nope) and [nk + h*128 ..] (dV): 2 x 256 bytes per key
    for (int e = tid; e < 128 * 32; e += 512) {
      const int k = e >> 5, c = e & 31;   // c < 16: dK_nope, else dV
      const int64_t col = (c < 16 ? 0 : nk) + static_cast<int64_t>(h) * 128 + 8 * (c & 15);
      *reinterpret_cast<u32x4*>(dKV + (t0 + k) * (2 * nk) + col) =
          *reinterpret_cast<const u32x4*>(rows + k * K_PITCH + 8 * c);
    }
  };
  if (role_a) run(std::true_type());
  else run(std::false_type());
}

// ------------------------------------------------------------------ dQ
constexpr int QW = 256;     // query rows per workgroup (8 waves x 32, two per SIMD)
constexpr int KS = 64;      // keys per step
constexpr int QPF = 4;      // fragment reads in flight ahead of the products
constexpr int K_ROW = XS_ROW, V_ROW = DV * 2 + 16;  // 448 (swizzled), 272
// stage (bytes): K [64 keys][192] | V [64 keys][128]; the K^T fragments of
// dQ^T += K^T dS^T are transposed reads of the K tile
constexpr int D_K = 0, D_V = KS * K_ROW, D_BYTES = D_V + KS * V_ROW;
constexpr int D_PIECES = D_BYTES / 1024;
static_assert(D_V % 1024 == 0 && D_BYTES % 1024 == 0, "dq stage layout");

__global__ void __launch_bounds__(512)
attn_bwd_dq_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ dout,
                   const uint32_t* __restrict__ info, const _Float16* __restrict__ Kfull,
                   const _Float16* __restrict__ Vkm, const int* __restrict__ qorder,
                   const float* __restrict__ sc, float* __restrict__ dq, int n_h, int S_loc,
                   int S_pad, int key_lo, int Kpad, int n_qt, float scale, float scale_log2) {
  constexpr int NP = (D_PIECES + 7) / 8;
  __shared__ __attribute__((aligned(1024))) char smem[2 * D_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int lr = lane & 31, lh = lane >> 5;
  int h, qt;
  work_item(blockIdx.x, n_h, n_qt, &h, &qt);
  // heaviest tiles first: the latest rows, or the packed call's order
  qt = qorder != nullptr ? qorder[qt] : n_qt - 1 - qt;
  const int q0 = qt * QW;
  const int wq0 = q0 + 32 * w;
  const int i = wq0 + lr;
  const bool valid = i < S_loc;
  // the rows' lse*log2(e), D, sample start and position, as the backward
  // prep stored them (the wave's 32 rows are one info block). Positions
  // increase with the row, so a row range's extremes sit at its ends.
  const uint32_t* info_h = info + static_cast<int64_t>(h) * (S_pad / 32) * 128;
  const bool wave_live = wq0 < S_loc;
  const uint32_t* blk = info_h + (wq0 >> 5) * 128;
  const int n_last = wave_live ? min(S_loc - 1 - wq0, 31) : 0;  // the wave's last valid row
  const float L2 = valid ? __uint_as_float(blk[lr]) + kPShift : 0.f;
  const float Di = valid ? __uint_as_float(blk[32 + lr]) : 0.f;
  const int lo = valid ? static_cast<int>(blk[64 + lr]) : 0;
  const int p = valid ? static_cast<int>(blk[96 + lr]) : -1;
  const int wp_min = wave_live ? static_cast<int>(blk[96]) : 0;
  const int wp_max = wave_live ? static_cast<int>(blk[96 + n_last]) : -1;
  const int wlo_min = wave_live ? static_cast<int>(blk[64]) : 0;
  const int wlo_max = wave_live ? static_cast<int>(blk[64 + n_last]) : 0;

  half8 qf[12], df[8];
#pragma unroll
  for (int kk = 0; kk < 12; ++kk) {
    if (valid) {
      qf[kk] = bf16x8_to_half8(*reinterpret_cast<const u32x4*>(
          q + (static_cast<int64_t>(i) * n_h + h) * DQK + 16 * kk + 8 * lh));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[kk][e] = static_cast<_Float16>(0.f);
    }
  }
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    if (valid) {
      df[kk] = bf16x8_to_half8_scaled(*reinterpret_cast<const u32x4*>(
          dout + (static_cast<int64_t>(i) * n_h + h) * DV + 16 * kk + 8 * lh), sc[0]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) df[kk][e] = static_cast<_Float16>(0.f);
    }
  }

  const int i_last = min(S_loc - 1, q0 + QW - 1);
  const int kb_begin = ((static_cast<int>(info_h[(q0 >> 5) * 128 + 64]) - key_lo) / KS) * KS;
  const int kb_end = static_cast<int>(info_h[(i_last >> 5) * 128 + 96 + (i_last & 31)]) + 1 - key_lo;
  const int nblk = (kb_end - kb_begin + KS - 1) / KS;

  const _Float16* Kh = Kfull + static_cast<int64_t>(h) * Kpad * DQK;
  const _Float16* Vh = Vkm + static_cast<int64_t>(h) * Kpad * DV;
  // DMA pieces of this wave (NP of the 69 per stage): per-lane source offsets
  // relative to the region's first key row kb
  int doff[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int o = (w * NP + j) * 1024 + lane * 16;
    int off = 0;
    if (o < D_V) {   // swizzled K rows; pad slots 24..27 reload slot 0
      const int row = o / K_ROW, ph = (o % K_ROW) >> 4;
      off = row * DQK + (ph < DQK / 8 ? xs_slot(row, ph) : 0) * 8;
    } else if (o < D_BYTES) {
      const int oo = o - D_V, row = oo / V_ROW, pc = min((oo % V_ROW) >> 4, DV / 8 - 1);
      off = row * DV + pc * 8;
    }
    doff[j] = off;
  }
  auto issue = [&](int kb, int st) {
    char* base = smem + st * D_BYTES;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int I = w * NP + j;   // wave-uniform
      if (I < D_PIECES) {
        // wave-uniform base plus an opaque unsigned 32-bit lane offset in
        // bytes (the scalar-base form of the load)
        const char* ub = reinterpret_cast<const char*>(I * 1024 < D_V ? Kh + static_cast<int64_t>(kb) * DQK
                                                                      : Vh + static_cast<int64_t>(kb) * DV);
        uint32_t off = static_cast<uint32_t>(doff[j]) * 2u;
        asm volatile("" : "+v"(off));
        lds_dma16(ub, off, base + I * 1024);
      }
    }
  };

  f32x16 acc[6];
#pragma unroll
  for (int a = 0; a < 6; ++a)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[a][e] = 0.f;
  const int a_k0 = D_K + xs_row_base(swap23(lr), lh, 0), a_k1 = D_K + xs_row_base(swap23(lr), lh, 1);
  const int a_v = D_V + swap23(lr) * V_ROW + lh * 16;
  // K^T fragments: transposed reads of the K tile
  const int a_kt0 = D_K + xs_tr_base(lane, 0), a_kt1 = D_K + xs_tr_base(lane, 1);

  if (nblk > 0) issue(kb_begin, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int b = 0; b < nblk; ++b) {
    const int st = b & 1;
    const int kb = kb_begin + b * KS;
    if (b + 1 < nblk) issue(kb + KS, st ^ 1);
    const int g0 = key_lo + kb;
    const bool skip = !wave_live || g0 > wp_max || g0 + KS - 1 < wlo_min;
    if (!skip) {
      const bool need_mask = !(g0 >= wlo_max && g0 + KS - 1 <= wp_min);
      const char* base = smem + st * D_BYTES;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        f32x16 s, dp;
#pragma unroll
        for (int e = 0; e < 16; ++e) { s[e] = 0.f; dp[e] = 0.f; }
        {
          auto frag = [&](int k) {
            return k < 12 ? *reinterpret_cast<const half8*>(base + ((k & 1) ? a_k1 : a_k0) + mt * 32 * K_ROW + 64 * (k >> 1))
                          : *reinterpret_cast<const half8*>(base + a_v + mt * 32 * V_ROW + 32 * (k - 12));
          };
          half8 fa[QPF + 1];
          #pragma unroll
          for (int i = 0; i < QPF; ++i) fa[i] = frag(i);
          // raised priority over the S / dP chain: the SIMD's other wave
          // fills its gaps with its own VALU work
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int k = 0; k < 20; ++k) {
            if (k + QPF < 20) fa[(k + QPF) % (QPF + 1)] = frag(k + QPF);
            if (k < 12) s = mfma_f16(fa[k % (QPF + 1)], qf[k], s);
            else dp = mfma_f16(fa[k % (QPF + 1)], df[k - 12], dp);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        __builtin_amdgcn_s_setprio(0);
        half8 dsf[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pv = __builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, -L2));
          if (need_mask) {
            const int key = g0 + 32 * mt + swap23(d_row(r, lh));
            if (key < lo || key > p) pv = 0.f;
          }
          dsf[r >> 3][r & 7] = static_cast<_Float16>(pv * (dp[r] - Di));
        }
        {
          // K^T fragment: dims 32dm + lr, keys 32mt + 16ksl + 8lh + j (transposed read)
          auto frag = [&](int k) {
            const int ksl = k / 6, dm = k % 6;
            const int o = (32 * mt + 16 * ksl) * K_ROW + 64 * dm;
            return frag_tr2(base + a_kt0 + o, base + a_kt1 + o);
          };
          half8 fa[QPF + 1];
          #pragma unroll
          for (int i = 0; i < QPF; ++i) fa[i] = frag(i);
#pragma unroll
          for (int k = 0; k < 12; ++k) {
            if (k + QPF < 12) fa[(k + QPF) % (QPF + 1)] = frag(k + QPF);
            acc[k % 6] = mfma_f16(fa[k % (QPF + 1)], dsf[k / 6], acc[k % 6]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (valid) {
    // the scores' scale, and 2^-e for the scaled dout (exact)
    const float osc = scale * sc[1];
    float* dst = dq + (static_cast<int64_t>(i) * n_h + h) * DQK;
#pragma unroll
    for (int dm = 0; dm < 6; ++dm)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 v = {acc[dm][4 * g] * osc, acc[dm][4 * g + 1] * osc,
                         acc[dm][4 * g + 2] * osc, acc[dm][4 * g + 3] * osc};
        *reinterpret_cast<f32x4*>(dst + 32 * dm + 8 * g + 4 * lh) = v;
      }
  }
}

// ------------------------------------------------------------------ dQ from the stored dS
// dQ = scale dS K, reading the dS blocks that the dK/dV kernel wrote (per
// key tile and 32-row block, 4 pairs of 32 keys x [row half ks][lane] x 16
// bytes: lane 32 lh + lr holds key lr, rows 16 ks + 8 lh .. + 7) instead of recomputing
// S and dP: 24 products per wave and 64 keys instead of 64. Eight waves of 32
// rows (two per SIMD) as in the recomputing kernel. Per step of 64 keys the
// K tile (swizzled rows, read transposed for K^T; double-buffered, mostly L2
// hits) is shared, and each wave streams its own 64-key x 32-row dS block
// (two pairs, read transposed: lane = row, eight consecutive keys, the B
// operand of dQ^T += K^T dS^T) through a ring of three buffers, two steps ahead:
// dS is the kernel's HBM stream. Pairs that no row sees were never written;
// they are masked to 0 here.
constexpr int E_KST = KS * K_ROW;                     // one K stage (28 KiB)
constexpr int E_DS0 = 2 * E_KST, E_DST = 8 * KS * 64;  // dS stages: 8 waves x 4 KiB
constexpr int E_BYTES = E_DS0 + 3 * E_DST;
constexpr int E_KPIECES = E_KST / 1024;                // 28
static_assert(E_KST % 1024 == 0 && E_BYTES <= 160 * 1024, "dq-from-dS LDS layout");

// s_waitcnt vmcnt(n) (n = 0 or 4) with lgkmcnt(0): the gfx9 encoding
// (vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
__device__ __forceinline__ void wait_vm_lgkm(bool four) {
  if (four) __builtin_amdgcn_s_waitcnt(0x0074);
  else __builtin_amdgcn_s_waitcnt(0x0070);
}

__global__ void __launch_bounds__(512)
attn_bwd_dq_ds_kernel(const uint32_t* __restrict__ info, const _Float16* __restrict__ Kfull,
                      const _Float16* __restrict__ dS, const int* __restrict__ qorder,
                      const float* __restrict__ sc, float* __restrict__ dq, int n_h, int h0,
                      int n_hg, int S_loc, int S_pad, int key_lo, int Kpad, int n_qt, float scale) {
  __shared__ __attribute__((aligned(1024))) char smem[E_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int lr = lane & 31, lh = lane >> 5;
  // heads h0 .. h0 + n_hg - 1; dS holds those heads only
  int hl, qt;
  work_item(blockIdx.x, n_hg, n_qt, &hl, &qt);
  const int h = h0 + hl;
  qt = qorder != nullptr ? qorder[qt] : n_qt - 1 - qt;
  const int q0 = qt * QW;
  const int wq0 = q0 + 32 * w;
  const int i = wq0 + lr;
  const bool valid = i < S_loc;
  const int n_rb = S_pad / 32;
  const uint32_t* info_h = info + static_cast<int64_t>(h) * n_rb * 128;
  const bool wave_live = wq0 < S_loc;
  const uint32_t* blk = info_h + min(wq0 >> 5, n_rb - 1) * 128;
  const int n_last = wave_live ? min(S_loc - 1 - wq0, 31) : 0;  // the wave's last valid row
  const int lo = valid ? static_cast<int>(blk[64 + lr]) : 0;
  const int p = valid ? static_cast<int>(blk[96 + lr]) : -1;
  const int wp_min = wave_live ? static_cast<int>(blk[96]) : 0;
  const int wp_max = wave_live ? static_cast<int>(blk[96 + n_last]) : -1;
  const int wlo_min = wave_live ? static_cast<int>(blk[64]) : 0;
  const int wlo_max = wave_live ? static_cast<int>(blk[64 + n_last]) : 0;

  const int i_last = min(S_loc - 1, q0 + QW - 1);
  const int kb_begin = ((static_cast<int>(info_h[(q0 >> 5) * 128 + 64]) - key_lo) / KS) * KS;
  const int kb_end = static_cast<int>(info_h[(i_last >> 5) * 128 + 96 + (i_last & 31)]) + 1 - key_lo;
  const int nblk = (kb_end - kb_begin + KS - 1) / KS;

  const _Float16* Kh = Kfull + static_cast<int64_t>(h) * Kpad * DQK;
  // this wave's dS^T rows (32-row block, clamped for rows past S_pad)
  const _Float16* dSw = dS + (static_cast<int64_t>(hl) * (Kpad / 128) * n_rb + min((q0 >> 5) + w, n_rb - 1)) * (128 * 32);
  // K pieces of this wave: w, w + 8, w + 16, w + 24 (< 28); per-lane offsets
  // (elements) of the swizzled rows, pad slots reloading slot 0
  int kdoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int o = (w + 8 * j) * 1024 + lane * 16;
    const int row = min(o / K_ROW, KS - 1), ph = (o % K_ROW) >> 4;
    kdoff[j] = row * DQK + (ph < DQK / 8 ? xs_slot(row, ph) : 0) * 8;
  }
  auto issue_k = [&](int kb, int st) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int I = w + 8 * j;   // wave-uniform
      if (I < E_KPIECES) {
        uint32_t off = static_cast<uint32_t>(kdoff[j]) * 2u;
        asm volatile("" : "+v"(off));
        lds_dma16(Kh + static_cast<int64_t>(kb) * DQK, off, smem + st * E_KST + I * 1024);
      }
    }
  };
  // this wave's dS of step kb: pairs (kb % 128) / 32 and the next of key
  // tile kb / 128, 2 KiB each, contiguous (4 pieces). Piece c is row half
  // c % 2 of pair c / 2; LDS chunk (lane half lh, key lr) of it holds the
  // stored chunk of key lr ^ 4 (2 (c % 2) + lh), which spreads the rows one
  // transposed read fetches over all 64 banks.
  auto issue_ds = [&](int kb, int st) {
    const char* src = reinterpret_cast<const char*>(dSw + (static_cast<int64_t>(kb >> 7) * n_rb * 128 + (kb & 127)) * 32);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint32_t off = static_cast<uint32_t>(c * 1024 + (lane ^ (4 * (2 * (c & 1) + (lane >> 5)))) * 16);
      asm volatile("" : "+v"(off));
      lds_dma16(src, off, smem + E_DS0 + st * E_DST + w * 4096 + c * 1024);
    }
  };

  f32x16 acc[6];
#pragma unroll
  for (int a = 0; a < 6; ++a)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[a][e] = 0.f;
  // K^T fragments: transposed reads of the K tile. dS fragments: transposed
  // reads of this wave's block. In a transposed read, lane q of 16-lane group
  // g fetches keys (k) 8 (g / 2) + q / 4 (the second read: 4 keys further)
  // and rows 16 (g % 2) + 4 (q % 4) .. + 3 of a 16-key step; those four rows
  // are 8 contiguous bytes at row half g % 2, lane half (q / 2) % 2, the
  // swizzled key slot, and 8 (q % 2).
  const int a_kt0 = xs_tr_base(lane, 0), a_kt1 = xs_tr_base(lane, 1);
  const int ds_hb = (lane >> 4) & 1, ds_lb = ((lane & 15) >> 1) & 1;
  const int ds_key = 8 * (lane >> 5) + ((lane & 15) >> 2), ds_x = 4 * (2 * ds_hb + ds_lb);
  const int a_ds0 = E_DS0 + w * 4096 + ds_hb * 1024 + ds_lb * 512 + ((ds_key ^ ds_x) * 16) + (lane & 1) * 8;
  const int a_ds1 = E_DS0 + w * 4096 + ds_hb * 1024 + ds_lb * 512 + (((ds_key + 4) ^ ds_x) * 16) + (lane & 1) * 8;

  // Before step b's products: K(b) and dS(b) landed in every wave. A wave's
  // loads complete in issue order, so with dS(b + 1) issued after K(b), at
  // most its 4 pieces may stay outstanding; the barrier then shows the
  // other waves' pieces, and that every wave is done with the stages the
  // next issues refill.
  if (nblk > 0) {
    issue_k(kb_begin, 0);
    issue_ds(kb_begin, 0);
    if (nblk > 1) issue_ds(kb_begin + KS, 1);
    wait_vm_lgkm(nblk > 1);
    asm volatile("s_barrier" ::: "memory");
  }
  int dst_ = 0;   // dS stage of step b
  for (int b = 0; b < nblk; ++b) {
    const int kb = kb_begin + b * KS;
    if (b + 1 < nblk) issue_k(kb + KS, (b + 1) & 1);
    if (b + 2 < nblk) issue_ds(kb + 2 * KS, dst_ == 0 ? 2 : dst_ - 1);
    const int g0 = key_lo + kb;
    const bool skip = !wave_live || g0 > wp_max || g0 + KS - 1 < wlo_min;
    if (!skip) {
      const bool need_mask = !(g0 >= wlo_max && g0 + KS - 1 <= wp_min);
      const char* kbase = smem + (b & 1) * E_KST;
      const char* dbase = smem + dst_ * E_DST;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        // dS fragment of k-step ksl: row lr, keys 32 mt + 16 ksl + 8 lh + j
        // (pair mt of the step, keys 16 ksl .. of the pair)
        half8 dsf[2];
#pragma unroll
        for (int ksl = 0; ksl < 2; ++ksl) {
          dsf[ksl] = frag_tr2(dbase + a_ds0 + mt * 2048 + ksl * 256, dbase + a_ds1 + mt * 2048 + ksl * 256);
          if (need_mask) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int key = g0 + 32 * mt + 16 * ksl + 8 * lh + j;
              if (key < lo || key > p) dsf[ksl][j] = static_cast<_Float16>(0.f);
            }
          }
        }
        // K^T fragment: dims 32dm + lr, keys 32mt + 16ksl + 8lh + j (transposed read)
        auto frag = [&](int k) {
          const int ksl = k / 6, dm = k % 6;
          const int o = (32 * mt + 16 * ksl) * K_ROW + 64 * dm;
          return frag_tr2(kbase + a_kt0 + o, kbase + a_kt1 + o);
        };
        half8 fa[QPF + 1];
#pragma unroll
        for (int ii = 0; ii < QPF; ++ii) fa[ii] = frag(ii);
#pragma unroll
        for (int k = 0; k < 12; ++k) {
          if (k + QPF < 12) fa[(k + QPF) % (QPF + 1)] = frag(k + QPF);
          acc[k % 6] = mfma_f16(fa[k % (QPF + 1)], dsf[k / 6], acc[k % 6]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if (b + 1 < nblk) {
      wait_vm_lgkm(b + 2 < nblk);
      asm volatile("s_barrier" ::: "memory");
    }
    dst_ = dst_ == 2 ? 0 : dst_ + 1;
  }
  if (valid) {
    // the scores' scale, and 2^-e for the scaled dout (exact)
    const float osc = scale * sc[1];
    float* dst = dq + (static_cast<int64_t>(i) * n_h + h) * DQK;
#pragma unroll
    for (int dm = 0; dm < 6; ++dm)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 v = {acc[dm][4 * g] * osc, acc[dm][4 * g + 1] * osc,
                         acc[dm][4 * g + 2] * osc, acc[dm][4 * g + 3] * osc};
        *reinterpret_cast<f32x4*>(dst + 32 * dm + 8 * g + 4 * lh) = v;
      }
  }
}

// dk_rope[key_lo + t][r] = sc[1] sum_h dKr[h][t][r] for t < Kn (sc[1] = 2^-e
// undoes the dout scale); other rows 0. A thread owns four consecutive r
// (16-byte loads and store) and keeps eight heads' loads in flight; the sum
// still runs over h in order, so the result does not depend on the grid.
__global__ void __launch_bounds__(256)
reduce_rope_kernel(const float* __restrict__ dKr, const float* __restrict__ sc,
                   float* __restrict__ dk_rope, int n_h, int64_t S, int64_t key_lo, int64_t Kn,
                   int64_t Kpad) {
  const float inv = sc[1];
  const int64_t n4 = S * 16;          // 16-byte pieces of dk_rope
  const int64_t hstride = Kpad * 16;  // pieces per head of dKr
  const f32x4* src = reinterpret_cast<const f32x4*>(dKr);
  for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < n4;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t j = e >> 4, t = j - key_lo;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (t >= 0 && t < Kn) {
      const f32x4* pt = src + t * 16 + (e & 15);
      int h = 0;
      for (; h + 8 <= n_h; h += 8) {
        f32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = pt[(h + u) * hstride];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += v[u];
      }
      for (; h < n_h; ++h) acc += pt[h * hstride];
    }
    reinterpret_cast<f32x4*>(dk_rope)[e] = acc * inv;
  }
}

// p[0, n) = 0: 16-byte stores (p 16-byte aligned), the last n % 4 one by one
__global__ void __launch_bounds__(256)
zero_rows_kernel(float* __restrict__ p, int64_t n) {
  const int64_t n4 = n / 4;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < n4;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x)
    reinterpret_cast<f32x4*>(p)[e] = z;
  if (blockIdx.x == 0 && threadIdx.x < n - 4 * n4) p[4 * n4 + threadIdx.x] = 0.f;
}

// The side stream's fork, joined back into the caller's stream on every way
// out of the launcher once it has happened: an error return after the fork
// must not leave work on the side stream unordered with the caller's later
// work (or leave a graph capture with a stream that never rejoins it).
unsigned grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  return static_cast<unsigned>(g < 1 ? 1 : (g > 16384 ? 16384 : g));
}

}  // namespace

mla_status fast_bwd_limits(const Plan& p) {
  // positions (S + 256), key-row offsets (Kpad 256) and query-row offsets
  // (S_loc 192) in 32 bits; the GEMMs' operand rows (2 n_h 128 and Kpad
  // elements) below 2^22
  if (p.S + 256 >= (int64_t(1) << 31) || p.S_loc * DQK >= (int64_t(1) << 31) ||
      p.Kpad >= (int64_t(1) << 22) || static_cast<int64_t>(p.n_h) * 256 >= (int64_t(1) << 22))
    return fail(MLA_ERR_UNSUPPORTED,
                "fast backward takes n_h < 16384, fewer than 2^22 needed keys, S_loc below 2^31 / 192 "
                "and S below 2^31 - 256");
  return MLA_OK;
}

mla_status fast_bwd(const Plan& p, const void* dout, const void* q, const void* c_kv,
                    const void* k_rope, const void* W_UK, const void* W_UV,
                    const int32_t* cu_dev, const float* out, const float* lse, float* dq,
                    float* dc_kv, float* dk_rope, float* dW_UK, float* dW_UV, char* ws,
                    hipStream_t st) {
  const BwdLayout L = bwd_layout(p);
  if (mla_status s = fast_bwd_limits(p); s != MLA_OK) return s;
  const int64_t nk = static_cast<int64_t>(p.n_h) * 128;
  const int64_t S_pad = align_up(p.S_loc, 64);
  auto at = [&](int64_t off) { return ws + off; };
  uint16_t* WT = reinterpret_cast<uint16_t*>(at(L.f.WT));
  _Float16* Kfull = reinterpret_cast<_Float16*>(at(L.f.Kfull));
  _Float16* Vkm = reinterpret_cast<_Float16*>(at(L.Vkm));
  _Float16* W16 = reinterpret_cast<_Float16*>(at(L.W16));
  _Float16* ckvT = reinterpret_cast<_Float16*>(at(L.ckvT));
  _Float16* Qn = reinterpret_cast<_Float16*>(at(L.Qn));
  _Float16* dOn = reinterpret_cast<_Float16*>(at(L.dOn));
  float* D = reinterpret_cast<float*>(at(L.D));
  _Float16* dKV = reinterpret_cast<_Float16*>(at(L.dK));
  float* dKr = reinterpret_cast<float*>(at(L.dKrope));
  uint32_t* info = reinterpret_cast<uint32_t*>(at(L.info));
  // stored dS: the dK/dV kernel writes it, the dQ kernel reads it
  _Float16* dS = p.ds_store ? reinterpret_cast<_Float16*>(at(L.dS)) : nullptr;
  // {2^e, 2^-e}: the dout scale and its inverse; then the per-block maxima
  float* dsc = reinterpret_cast<float*>(at(L.dscale));
  uint32_t* dmax = reinterpret_cast<uint32_t*>(at(L.dscale) + 16);
  // per head {largest |2^e dout row|, largest |D|} (float bits)
  uint32_t* hmax = dmax + kScaleBlocks;
  const int S_loc = static_cast<int>(p.S_loc), Sp = static_cast<int>(S_pad),
            key_lo = static_cast<int>(p.key_lo),
            Kpad = static_cast<int>(p.Kpad);
  mla_status s;
  // The layout conversions and the row preparation do not depend on the K/V
  // rebuild, and the dQ kernel not on the gradient GEMMs: each such group
  // runs on a side stream next to the other (HBM-bound work beside
  // MFMA-bound work in the first pair; in the second the GEMMs and then the
  // rope-key reduction run under the longer dQ kernel).
  SideStream side;
  if ((s = side_stream(&side)) != MLA_OK) return s;
  const hipStream_t st2 = side.st;
  SideFork fork(side, st);
  if ((s = fork.fork()) != MLA_OK) return s;

  // rows of dc_kv outside the shard's keys get no gradient; no other kernel
  // writes them
  if (p.key_lo > 0 || p.key_hi < p.S) {
    KernelTimer kt("zero_rows", st2);
    if (p.key_lo > 0)
      hipLaunchKernelGGL(zero_rows_kernel, dim3(grid_for(p.key_lo * p.d_c / 4)), dim3(256), 0, st2,
                         dc_kv, p.key_lo * p.d_c);
    if (p.key_hi < p.S)
      hipLaunchKernelGGL(zero_rows_kernel, dim3(grid_for((p.S - p.key_hi) * p.d_c / 4)), dim3(256), 0,
                         st2, dc_kv + p.key_hi * p.d_c, (p.S - p.key_hi) * p.d_c);
  }
  if ((s = check_launch("zero rows")) != MLA_OK) return s;
  // [W_UK | W_UV] rows in fp16 and c_kv^T in fp16 for the gradient GEMMs
  if ((s = launch_convert(static_cast<const uint16_t*>(W_UK), nk, 0, p.d_c, p.d_c, nk, W16, 2 * nk,
                          0, Elem::F16, 1, st2, "prep_w16")) != MLA_OK)
    return s;
  if ((s = launch_convert(static_cast<const uint16_t*>(W_UV), nk, 0, p.d_c, p.d_c, nk, W16 + nk,
                          2 * nk, 0, Elem::F16, 1, st2, "prep_w16")) != MLA_OK)
    return s;
  if ((s = launch_transpose(static_cast<const uint16_t*>(c_kv) + p.key_lo * p.d_c, p.d_c, 0, p.Kn,
                            p.Kpad, p.d_c, ckvT, p.Kpad, 0, Elem::F16, 1, st2, "prep_ckvT")) != MLA_OK)
    return s;
  {
    // the dout scale (every kernel that reads dout or its products waits for it)
    KernelTimer kt("dout_scale", st2);
    const int64_t n8 = p.S_loc * p.n_h * DV / 8;
    const unsigned nb = static_cast<unsigned>(std::min<int64_t>(kScaleBlocks, (n8 + 255) / 256));
    hipLaunchKernelGGL(dout_absmax_kernel, dim3(nb), dim3(256), 0, st2,
                       static_cast<const u32x4*>(dout), n8, dmax);
    hipLaunchKernelGGL(dout_scale_kernel, dim3(1), dim3(256), 0, st2, dmax, static_cast<int>(nb), dsc,
                       hmax, 2 * p.n_h);
  }
  if ((s = check_launch("dout scale")) != MLA_OK) return s;
  {
    KernelTimer kt("bwd_prep", st2);
    hipLaunchKernelGGL(bwd_prep_kernel, dim3(static_cast<unsigned>(S_pad / 64), p.n_h), dim3(256),
                       0, st2, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(dout),
                       out, lse, cu_dev, dsc, D, Qn, dOn, info, hmax, p.n_h, p.n_seqs, p.S_loc,
                       S_pad, p.rm);
  }
  if ((s = check_launch("backward prep")) != MLA_OK) return s;
  // keys (row-major, with the rope key) and V key-major
  if ((s = fast_rebuild_kv(p, c_kv, k_rope, W_UK, W_UV, WT, Kfull, nullptr, Vkm, st, st2)) != MLA_OK)
    return s;
  if ((s = fork.join()) != MLA_OK) return s;
  const float scale_log2 = p.scale * kLog2e;
  // packed calls: query and key tiles in longest-processing-time order
  int *qorder = nullptr, *korder = nullptr;
  {
    const int n_qt = static_cast<int>((p.S_loc + QW - 1) / QW), n_kt = static_cast<int>(p.Kpad / PW);
    if (p.n_seqs > 0 && n_qt <= kMaxOrderTiles && n_kt <= kMaxOrderTiles) {
      qorder = reinterpret_cast<int*>(at(L.order));
      korder = qorder + n_qt;
      if ((s = launch_tile_order(cu_dev, p.n_seqs, p.S_loc, p.rm, p.key_lo, p.Kn, n_qt, n_kt,
                                 qorder, korder, st)) != MLA_OK)
        return s;
    }
  }
  const int n_kt = static_cast<int>(p.Kpad / PW), n_qt = static_cast<int>((p.S_loc + QW - 1) / QW);
  auto dkdv = [&](int h0, int n_hg, _Float16* dSg) {
    KernelTimer kt("attn_bwd_dkdv", st);
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel, dim3(static_cast<unsigned>(n_kt * n_hg)), dim3(512), 0,
                       st, Qn, dOn, info, Kfull, Vkm, cu_dev, korder, dKV, dKr, dSg, hmax, p.n_h,
                       h0, n_hg, p.n_seqs, S_loc, Sp, p.rm, key_lo, Kpad, n_kt, p.scale,
                       scale_log2);
    return check_launch("attention backward dK/dV");
  };
  if (dS == nullptr) {
    if ((s = dkdv(0, p.n_h, nullptr)) != MLA_OK) return s;
    if ((s = fork.fork()) != MLA_OK) return s;
    {
      KernelTimer kt("attn_bwd_dq", st2);
      hipLaunchKernelGGL(attn_bwd_dq_kernel, dim3(static_cast<unsigned>(n_qt * p.n_h)), dim3(512),
                         0, st2, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(dout),
                         info, Kfull, Vkm, qorder, dsc, dq, p.n_h, S_loc, Sp, key_lo, Kpad, n_qt,
                         p.scale, scale_log2);
    }
    if ((s = check_launch("attention backward dQ")) != MLA_OK) return s;
  } else {
    // Stored dS, ds_heads heads at a time: dK/dV of group g (main stream)
    // fills buffer g % 2, dQ of group g (side stream) reads it while dK/dV of
    // group g + 1 fills the other; dK/dV of group g + 2 waits until dQ of
    // group g has released its buffer.
    const int G = p.ds_heads;
    const int64_t group_elems = static_cast<int64_t>(G) * p.Kpad * S_pad;
    for (int h0 = 0, g = 0; h0 < p.n_h; h0 += G, ++g) {
      const int n_hg = std::min(G, p.n_h - h0);
      _Float16* dSg = dS + (g & 1) * group_elems;
      if (g >= 2 && hipStreamWaitEvent(st, side.buf_free[g & 1], 0) != hipSuccess)
        return fail(MLA_ERR_HIP, "wait for the stored-dS buffer failed");
      if ((s = dkdv(h0, n_hg, dSg)) != MLA_OK) return s;
      if ((s = fork.fork()) != MLA_OK) return s;
      {
        KernelTimer kt("attn_bwd_dq_ds", st2);
        hipLaunchKernelGGL(attn_bwd_dq_ds_kernel, dim3(static_cast<unsigned>(n_qt * n_hg)), dim3(512),
                           0, st2, info, Kfull, dSg, qorder, dsc, dq, p.n_h, h0, n_hg, S_loc, Sp,
                           key_lo, Kpad, n_qt, p.scale);
      }
      if ((s = check_launch("attention backward dQ")) != MLA_OK) return s;
      if (h0 + G < p.n_h && hipEventRecord(side.buf_free[g & 1], st2) != hipSuccess)
        return fail(MLA_ERR_HIP, "stored-dS buffer event failed");
    }
  }
  // dc_kv rows [key_lo, key_hi) = [dK_nope | dV] (fp16) . [W_UK | W_UV] rows; others 0
  float* gpart = reinterpret_cast<float*>(at(L.gpart));
  const int64_t gpart_bytes = std::max(gemm_splitk_bytes(p.Kn, p.d_c, 2 * nk),
                                       gemm_splitk_bytes(p.d_c, nk, p.Kpad));
  if ((s = launch_gemm_nt(dKV, 2 * nk, p.Kn, W16, 2 * nk, p.d_c, 2 * nk, dc_kv + p.key_lo * p.d_c,
                          p.d_c, 128 * p.d_c, 128, p.Kn, p.d_c, Elem::F16, Elem::F32, st,
                          "grad_latent", gpart, gpart_bytes, dsc + 1)) != MLA_OK)
    return s;
  // dW_UK = c_kv^T dK_nope, dW_UV = c_kv^T dV (contract over the shard's
  // keys): the dKV rows are read k-major (key rows, 2 n_h 128 columns)
  if ((s = launch_gemm_nt(ckvT, p.Kpad, p.d_c, dKV, 2 * nk, nk, p.Kpad, dW_UK, nk, 128 * nk, 128,
                          p.d_c, nk, Elem::F16, Elem::F32, st, "grad_w", gpart, gpart_bytes,
                          dsc + 1, true)) != MLA_OK)
    return s;
  if ((s = launch_gemm_nt(ckvT, p.Kpad, p.d_c, dKV + nk, 2 * nk, nk, p.Kpad, dW_UV, nk,
                          128 * nk, 128, p.d_c, nk, Elem::F16, Elem::F32, st, "grad_w", gpart,
                          gpart_bytes, dsc + 1, true)) != MLA_OK)
    return s;
  // dk_rope = sum over heads of the rope-key partials (HBM-bound): after the
  // gradient GEMMs, where it runs under the tail of the dQ kernel (MFMA-bound)
  // on the side stream
  {
    KernelTimer kt("reduce_rope", st);
    hipLaunchKernelGGL(reduce_rope_kernel, dim3(grid_for(p.S * 16)), dim3(256), 0, st, dKr,
                       dsc, dk_rope, p.n_h, p.S, p.key_lo, p.Kn, p.Kpad);
  }
  if ((s = check_launch("rope-key gradient reduce")) != MLA_OK) return s;
  return fork.join();
}

}  // namespace mla
