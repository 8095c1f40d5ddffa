// Decode in the absorbed form over the latent cache (inference only).
//
// The LAGA abstract describes the absorbed MLA form as the one allowed only in
// inference decode: W_UK is folded into the query and attention runs over the
// compressed latent itself, so no per-head K/V is ever built. One query per
// sequence attends to all of that sequence's cached latent rows:
//   q_lat[b,h,:] = W_UK_h q_nope[b,h,:]                (512)
//   s_j          = scale * (q_lat . c_kv[j] + q_rope . k_rope[j])
//   o_lat[b,h,:] = sum_j softmax(s)_j c_kv[j]          (512)
//   out[b,h,:]   = W_UV_h^T o_lat[b,h,:]               (128)
// which equals the explicit form for a query at the sequence's last position.
//
// Kernels (gfx950, fp16/bf16 MFMA with fp32 accumulation):
//   1. head_gemm_kernel: per-head q_lat (bf16 in, fp16 out);
//   2. decode_attn_pair_kernel: split-KV attention. A workgroup of 8 waves
//      owns one sequence, one chunk of its keys, up to 128 heads and all 512
//      output dims. Keys and values are the same 576-wide latent rows: each
//      32-key block is copied raw by LDS DMA two blocks ahead, then
//      converted bf16 -> fp16 into one swizzled LDS tile that serves both
//      S^T = K Q^T (row-wise fragments) and O^T += V^T P^T (transposed
//      reads). Waves w and w + 4 share 32 heads: each holds half of q_lat's
//      latent dims in registers, takes half of the score products, and the
//      two partial scores are added through LDS; each then accumulates half
//      of the output dims;
//   3. decode_combine_kernel: merges the chunks (max, rescaled sums), writes
//      o_lat in fp16 and lse;
//   4. head_gemm_kernel: per-head out = o_lat W_UV_h (fp16 in, fp32 out).
#include <math.h>

#include <mutex>

#include "fast.h"
#include "fast_common.h"

namespace mla {
namespace {

constexpr int DC = 512;            // latent width
constexpr int DR = 64;             // rope width
constexpr int DL = DC + DR;        // key width in the latent space (576)
constexpr int DB = 32;             // keys per block
// LDS row pitch: 72 data slots of 16 bytes + 4 pad slots. 1216 = 448 + 3*256,
// so rows fall on the banks exactly as the 448-byte swizzled rows do: both
// row-wise and transposed 16-bit reads are conflict-free.
constexpr int DROW = 1216;
constexpr int DSTAGE = DB * DROW;
constexpr int QR_ROW = DR * 2 + 16;               // q_rope LDS row pitch (odd slot count)
constexpr float kTauD = 8.f;                      // lazy-rescale threshold, log2 units
constexpr float kLn2D = 0.69314718055994530942f;

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// out[r][h][c] (at out + r*ldo + h*ho + c) = sum_k X[r][h][k] Y[c][h][k] for
// r < R, c < C, with X[r][h][k] at X + r*ldx + h*hx + k and Y likewise.
// One wave per 32 x 32 tile, operands straight from memory (the products
// here are small next to the attention).
template <typename TIn, typename TOut>
__global__ void __launch_bounds__(64)
head_gemm_kernel(const TIn* __restrict__ X, int64_t ldx, int64_t hx, const TIn* __restrict__ Y,
                 int64_t ldy, int64_t hy, TOut* __restrict__ out, int64_t ldo, int64_t ho, int R,
                 int C, int K) {
  typedef typename MfmaOp<TIn>::vec vec;
  const int ct = blockIdx.x, rt = blockIdx.y, h = blockIdx.z;
  const int lane = threadIdx.x, lr = lane & 31, lh = lane >> 5;
  const int r = 32 * rt + lr, c = 32 * ct + lr;
  const TIn* xr = X + static_cast<int64_t>(r) * ldx + static_cast<int64_t>(h) * hx + 8 * lh;
  const TIn* yr = Y + static_cast<int64_t>(c) * ldy + static_cast<int64_t>(h) * hy + 8 * lh;
  f32x16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  vec zero;
#pragma unroll
  for (int e = 0; e < 8; ++e) zero[e] = static_cast<TIn>(0.f);
  for (int k0 = 0; k0 < K; k0 += 16) {
    const vec a = r < R ? *reinterpret_cast<const vec*>(xr + k0) : zero;
    const vec b = c < C ? *reinterpret_cast<const vec*>(yr + k0) : zero;
    acc = MfmaOp<TIn>::run(a, b, acc);
  }
  if (c >= C) return;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int row = 32 * rt + d_row(e, lh);
    if (row < R)
      out[static_cast<int64_t>(row) * ldo + static_cast<int64_t>(h) * ho + c] = static_cast<TOut>(acc[e]);
  }
}

// Split-KV attention: one workgroup of 8 waves owns a chunk of one
// sequence's keys for up to 128 heads and all 512 output dims. Waves w and w + 4 form a pair
// for heads 32 w' .. (w' = w % 4). Wave half kh = w / 4 holds q_lat dims
// 256 kh .. 256 kh + 255 and computes the scores over those dims and rope
// dims 32 kh .. 32 kh + 31 (18 products per 32-key block); the two partial
// score tiles are added through LDS (a + b is the same in either order, so
// both waves hold the same scores and weights), and each wave then
// accumulates its 256 output dims (16 products). A wave holding all of q_lat
// and half of the output dims would need about 400 registers (one wave per
// SIMD) and two workgroups that each recompute the 36 score products per
// block (52 products per wave and block, each cache block staged twice); here
// it is 34, one staging, and two waves per SIMD.
//
// Staging: each 32-key block is copied raw (bf16) by LDS DMA into one of two
// slots, two blocks ahead, so that two blocks of the cache are in flight per
// workgroup without holding registers; all threads then convert the block
// into the one fp16 tile the products read.
constexpr int PDW = 8;                                  // waves
constexpr int PD_RAW = DB * DC * 2 + DB * DR * 2;       // a raw block: c_kv rows, then k_rope rows (36 KiB)
constexpr int PD_TILE = 2 * PD_RAW;                     // the fp16 tile
constexpr int PD_QR = PD_TILE + DSTAGE;                 // q_rope rows of the 128 heads
constexpr int PD_XS = PD_QR + 128 * QR_ROW;             // partial scores: 8 waves x 4 KiB
constexpr int PD_LDS = PD_XS + PDW * 4096;
static_assert(PD_LDS <= 160 * 1024, "paired decode fits the LDS");
static_assert(PD_RAW % 1024 == 0 && DC * 2 == 1024 && 8 * DR * 2 == 1024,
              "a c_kv row, or the k_rope rows of 8 keys, per DMA wave instruction");
constexpr int PD_PIECES = PD_RAW / 1024;                // 36: piece I = w + 8 j
static_assert(4 * PDW * 64 == DB * (DC / 8) && PDW * 64 / 2 == DB * (DR / 8) &&
                  DB * (DL / 8) == 4 * PDW * 64 + DB * (DR / 8),
              "conversion: four c_kv pieces per thread and a k_rope piece for half the threads");

// s_waitcnt vmcnt(n) for n = 0, 4, 5, 9, other counters at their maxima (gfx9
// encoding: vmcnt bits 3:0, expcnt 6:4, lgkmcnt 11:8)
__device__ __forceinline__ void wait_vm_n(int n) {
  if (n == 9) __builtin_amdgcn_s_waitcnt(0x0F79);
  else if (n == 5) __builtin_amdgcn_s_waitcnt(0x0F75);
  else if (n == 4) __builtin_amdgcn_s_waitcnt(0x0F74);
  else __builtin_amdgcn_s_waitcnt(0x0F70);
}
__device__ __forceinline__ const uint16_t* scalar_ptr(const uint16_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const uint16_t*>((static_cast<uint64_t>(hi) << 32) | lo);
}

__global__ void __launch_bounds__(PDW * 64)
decode_attn_pair_kernel(const _Float16* __restrict__ qlat, const uint16_t* __restrict__ q,
                        const uint16_t* __restrict__ c_kv, const uint16_t* __restrict__ k_rope,
                        const int32_t* __restrict__ cu, _Float16* __restrict__ opart,
                        float2* __restrict__ ml, int n_h, int batch, int nch, int chunk,
                        float scale_log2) {
  // two K/V stages, q_rope of the 128 heads (144-byte rows), partial scores
  __shared__ __attribute__((aligned(1024))) char smem[PD_LDS];
  const int item = blockIdx.x;
  const int ch = item % nch, b = (item / nch) % batch, hg = item / (nch * batch);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lh = lane >> 5;
  const int wp = w & 3, kh = w >> 2;
  const int s0 = cu[b], len = cu[b + 1] - s0;
  const int k0 = ch * chunk;
  if (k0 >= len) return;                     // whole workgroup: nothing to do
  const int k1 = min(len, k0 + chunk);
  const int nblk = (k1 - k0 + DB - 1) / DB;
  const int hw = hg * 128 + 32 * wp;         // the pair's first head
  const bool live = hw < n_h;                // n_h is a multiple of 32
  const int h = hw + lr;

  // DMA of block blk into raw slot blk % 2: piece I (< 32) is key I's c_kv
  // row, piece 32 + r the k_rope rows of keys 8 r .. 8 r + 7. The waves of
  // the first contraction halves (0..3) issue all 36 pieces, 9 each, after
  // their score products, where they would otherwise wait for their partners
  // (which finish theirs later); the other waves issue none. A wave always
  // issues its 9 pieces, so that vmcnt counts stay exact: rows past the chunk
  // read the chunk's last row instead, and the conversion writes zeros for
  // them.
  const int n_dma = kh == 0 ? PD_PIECES / 4 : 0;
  auto issue = [&](int blk) {
    if (kh != 0) return;
    const int kb = k0 + blk * DB;
    const int64_t last = static_cast<int64_t>(s0) + k1 - 1;   // the chunk's last row (>= s0)
    char* raw = smem + (blk & 1) * PD_RAW;
#pragma unroll
    for (int j = 0; j < PD_PIECES / 4; ++j) {
      const int I = w + 4 * j;   // wave-uniform
      if (I < DB) {
        const int64_t row = min(static_cast<int64_t>(s0) + kb + I, last);
        lds_dma16(scalar_ptr(c_kv + row * DC), lane * 16u, raw + I * 1024);
      } else if (I < PD_PIECES) {
        // from the sequence's first row: the lane's row, clamped to the chunk
        const int key = min(kb + 8 * (I - DB) + (lane >> 3), k1 - 1);
        uint32_t off = static_cast<uint32_t>(key * DR * 2 + (lane & 7) * 16);
        asm volatile("" : "+v"(off));
        lds_dma16(scalar_ptr(k_rope + static_cast<int64_t>(s0) * DR), off, raw + I * 1024);
      }
    }
  };
  // raw slot blk % 2 -> fp16 tile: thread t converts key t / 64 + 8 p, slot
  // t % 64 of c_kv (p < 4) and, for t < 256, key t / 8, rope slot t % 8; a
  // piece lands in LDS slot xs_slot(key, slot) of its key's row, zeros past
  // the chunk
  auto convert = [&](int blk) {
    const int kb = k0 + blk * DB;
    const char* raw = smem + (blk & 1) * PD_RAW;
    char* tile = smem + PD_TILE;
    // all reads first, then the conversions and writes; rows past the
    // chunk are cleared through a mask on the raw bits (no branch, so the
    // reads overlap)
    u32x4 v[5];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int key = (tid >> 6) + 8 * p, sl = tid & 63;
      v[p] = *reinterpret_cast<const u32x4*>(raw + key * 1024 + sl * 16);
    }
    const int rkey = (tid >> 3) & 31, rs = tid & 7;
    if (tid < 256) v[4] = *reinterpret_cast<const u32x4*>(raw + DB * 1024 + rkey * 128 + rs * 16);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int key = (tid >> 6) + 8 * p, sl = tid & 63;
      const uint32_t msk = kb + key < k1 ? 0xffffffffu : 0u;
#pragma unroll
      for (int k = 0; k < 4; ++k) v[p][k] &= msk;
      *reinterpret_cast<half8*>(tile + key * DROW + xs_slot(key, sl) * 16) = bf16x8_to_half8(v[p]);
    }
    if (tid < 256) {
      const uint32_t msk = kb + rkey < k1 ? 0xffffffffu : 0u;
#pragma unroll
      for (int k = 0; k < 4; ++k) v[4][k] &= msk;
      *reinterpret_cast<half8*>(tile + rkey * DROW + xs_slot(rkey, 64 + rs) * 16) = bf16x8_to_half8(v[4]);
    }
  };

  // this wave's half of q_lat (B operand of S^T = K Q^T); the rope dims of
  // the pair's heads go to LDS (written by the half-0 wave)
  half8 qf[16];
  {
    const _Float16* ql = qlat + (static_cast<int64_t>(b) * n_h + h) * DC + 256 * kh + 8 * lh;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      if (live) {
        qf[kk] = *reinterpret_cast<const half8*>(ql + 16 * kk);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[kk][e] = static_cast<_Float16>(0.f);
      }
    }
    if (kh == 0) {
      const uint16_t* qr = q + (static_cast<int64_t>(b) * n_h + h) * 192 + 128 + 8 * lh;
      char* qrow = smem + PD_QR + (32 * wp + lr) * QR_ROW + 16 * lh;
#pragma unroll
      for (int j = 0; j < DR / 16; ++j) {
        half8 v;
        if (live) {
          v = bf16x8_to_half8(*reinterpret_cast<const u32x4*>(qr + 16 * j));
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = static_cast<_Float16>(0.f);
        }
        *reinterpret_cast<half8*>(qrow + 32 * j) = v;
      }
    }
  }
  const char* qrope = smem + PD_QR + (32 * wp + lr) * QR_ROW + 16 * lh;

  constexpr int NDT = DC / 2 / 32;
  f32x16 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
  float m = -INFINITY, l = 0.f;
  const half2v ones = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
  const int k_r0 = xs_row_base<DROW>(swap23(lr), lh, 0);
  const int k_r1 = xs_row_base<DROW>(swap23(lr), lh, 1);
  const int v_t0 = xs_tr_base<DROW>(lane, 0);
  const int v_t1 = xs_tr_base<DROW>(lane, 1);
  char* const xs_own = smem + PD_XS + w * 4096 + lane * 16;
  const char* const xs_par = smem + PD_XS + (w ^ 4) * 4096 + lane * 16;

  // the q loads above complete here, before any DMA: the compiler's wait
  // model does not see the DMA instructions, and a q load it still counts
  // as pending would make it wait inside the loop until the DMA issued
  // there lands
  __builtin_amdgcn_s_waitcnt(0);
  if (nblk > 0) issue(0);
  if (nblk > 1) issue(1);
  // block 0 landed (loads complete in issue order, and at most block 1's
  // pieces may remain), q_rope written
  wait_vm_n(nblk > 1 ? n_dma : 0);
  __syncthreads();
  for (int bi = 0; bi < nblk; ++bi) {
    convert(bi);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // tile ready, raw slot free
    const char* base = smem + PD_TILE;
    f32x16 s;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.f;
    if (live) {
      // partial S^T over this half's 18 k-steps: latent 16 kh .. 16 kh + 15,
      // rope 32 + 2 kh, 33 + 2 kh (k-steps of 16 dims of the 576-wide row)
      constexpr int PF = 2;
      auto kstep = [&](int i) { return i < 16 ? 16 * kh + i : 32 + 2 * kh + (i - 16); };
      auto frag = [&](int i) {
        const int kk = kstep(i);
        return *reinterpret_cast<const half8*>(base + ((kk & 1) ? k_r1 : k_r0) + 64 * (kk >> 1));
      };
      half8 fa[PF + 1];
#pragma unroll
      for (int i = 0; i < PF; ++i) fa[i] = frag(i);
#pragma unroll
      for (int i = 0; i < 18; ++i) {
        if (i + PF < 18) fa[(i + PF) % (PF + 1)] = frag(i + PF);
        const half8 qb = i < 16 ? qf[i] : *reinterpret_cast<const half8*>(qrope + 32 * (2 * kh + i - 16));
        s = mfma_f16(fa[i % (PF + 1)], qb, s);
      }
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(xs_own + g * 1024) = f32x4{s[4 * g], s[4 * g + 1], s[4 * g + 2], s[4 * g + 3]};
    }
    // the next DMA, from the waves that would wait here for their partners
    if (bi + 2 < nblk) issue(bi + 2);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // partial scores visible
    half8 pb[2];
    if (live) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(xs_par + g * 1024);
#pragma unroll
        for (int e = 0; e < 4; ++e) s[4 * g + e] += v[e];
      }
      const int kb = k0 + bi * DB;
      if (kb + DB > k1) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb + swap23(d_row(r, lh)) >= k1) s[r] = -INFINITY;
      }
      float mx = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mx = wave_max_pair(mx) * scale_log2;
      const bool grow = mx > m + kTauD;
      if (__any(grow)) {
        const float m_new = grow ? mx : m;
        const float alpha = grow ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;
        m = m_new;
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
      }
      float sum = l;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        half2v pr;
        pr[0] = static_cast<_Float16>(__builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, -m)));
        pr[1] = static_cast<_Float16>(__builtin_amdgcn_exp2f(fmaf(s[r + 1], scale_log2, -m)));
        pb[r >> 3][r & 7] = pr[0];
        pb[r >> 3][(r & 7) + 1] = pr[1];
        sum = __builtin_amdgcn_fdot2(pr, ones, sum, false);
      }
      l = sum;
    }
    if (live) {
      // O^T (this half's dims x heads) += V^T P^T
      constexpr int PF = 2, NPV = 2 * NDT;
      auto vfrag = [&](int k) {
        const int off = 16 * (k / NDT) * DROW + 64 * (NDT * kh + k % NDT);
        return frag_tr2(base + v_t0 + off, base + v_t1 + off);
      };
      half8 fv[PF + 1];
#pragma unroll
      for (int i = 0; i < PF; ++i) fv[i] = vfrag(i);
#pragma unroll
      for (int k = 0; k < NPV; ++k) {
        if (k + PF < NPV) fv[(k + PF) % (PF + 1)] = vfrag(k + PF);
        o[k % NDT] = mfma_f16(fv[k % (PF + 1)], pb[k / NDT], o[k % NDT]);
      }
    }
    // block bi + 1 landed (block bi + 2's pieces may stay in flight); every
    // wave is done with the tile
    if (bi + 1 < nblk) wait_vm_n(bi + 2 < nblk ? n_dma : 0);
    __syncthreads();
  }

  if (!live) return;
  const float lt = wave_sum_pair(l);
  const float inv = 1.f / lt;
  const int64_t slot = (static_cast<int64_t>(b) * nch + ch) * n_h + h;
  _Float16* dst = opart + slot * DC + 256 * kh;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      half4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = static_cast<_Float16>(o[dt][4 * g + e] * inv);
      *reinterpret_cast<half4*>(dst + 32 * dt + 8 * g + 4 * lh) = v;
    }
  if (lh == 0 && kh == 0) ml[slot] = make_float2(m, lt);
}

// o_lat[b][h][:] = sum_c w_c opart[b][c][h][:] / sum_c w_c with w_c =
// l_c 2^(m_c - max m); lse[b][h] = ln(sum_c l_c 2^(m_c)) (natural log).
// One workgroup of 128 threads per (head, sequence), four dims per thread.
__global__ void __launch_bounds__(128)
decode_combine_kernel(const _Float16* __restrict__ opart, const float2* __restrict__ ml,
                      const int32_t* __restrict__ cu, _Float16* __restrict__ olat,
                      float* __restrict__ lse, int n_h, int nch, int chunk) {
  const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int len = cu[b + 1] - cu[b];
  const int nc = (len + chunk - 1) / chunk;
  const int64_t base = static_cast<int64_t>(b) * nch * n_h + h;
  float M = -INFINITY;
  for (int c = 0; c < nc; ++c) M = fmaxf(M, ml[base + static_cast<int64_t>(c) * n_h].x);
  float acc[4] = {0.f, 0.f, 0.f, 0.f}, L = 0.f;
  for (int c = 0; c < nc; ++c) {
    const int64_t sl = base + static_cast<int64_t>(c) * n_h;
    const float2 v = ml[sl];
    const float wgt = v.y * __builtin_amdgcn_exp2f(v.x - M);
    L += wgt;
    const half4 x = *reinterpret_cast<const half4*>(opart + sl * DC + 4 * t);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += wgt * static_cast<float>(x[e]);
  }
  const float inv = 1.f / L;
  half4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = static_cast<_Float16>(acc[e] * inv);
  *reinterpret_cast<half4*>(olat + (static_cast<int64_t>(b) * n_h + h) * DC + 4 * t) = r;
  if (t == 0) lse[static_cast<int64_t>(b) * n_h + h] = (M + __log2f(L)) * kLn2D;
}

}  // namespace

// Scratch of mla_laga_decode_noalloc, for callers that cannot allocate
// device memory: a device array of the library's own, which each GPU holds
// from the loading of the code object until the process ends. On the host,
// `scratch` names a host-side stand-in, not the device memory: host code
// uses only the per-device address that hipGetSymbolAddress returns.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_dev[kMaxScratchDevices] = {};
}  // namespace

mla_status decode_scratch(char** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices)
    return fail(MLA_ERR_HIP, "no current device for the static decode scratch");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    // once per device, with that device current: each GPU holds its own
    // copy of the array at its own address
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(MLA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_dev[dev] = static_cast<char*>(p);
  }
  *ptr = g_scratch_dev[dev];
  return MLA_OK;
}

DecodeLayout decode_layout(const DecodePlan& p) {
  DecodeLayout L{};
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    const int64_t o = off;
    off += align_up(bytes, kAlign);
    return o;
  };
  const int64_t nk = static_cast<int64_t>(p.n_h) * 128;
  L.WTv = take(nk * DC * 2);
  L.qlat = take(static_cast<int64_t>(p.batch) * p.n_h * DC * 2);
  L.olat = take(static_cast<int64_t>(p.batch) * p.n_h * DC * 2);
  L.opart = take(static_cast<int64_t>(p.batch) * p.nch * p.n_h * DC * 2);
  L.ml = take(static_cast<int64_t>(p.batch) * p.nch * p.n_h * 8);
  L.total = off;
  return L;
}

mla_status fast_decode(const DecodePlan& p, const void* q, const void* c_kv, const void* k_rope,
                       const void* W_UK, const void* W_UV, const int32_t* cu_dev, float* out,
                       float* lse, char* ws, hipStream_t st) {
  const DecodeLayout L = decode_layout(p);
  _Float16* WTv = reinterpret_cast<_Float16*>(ws + L.WTv);
  _Float16* qlat = reinterpret_cast<_Float16*>(ws + L.qlat);
  _Float16* olat = reinterpret_cast<_Float16*>(ws + L.olat);
  _Float16* opart = reinterpret_cast<_Float16*>(ws + L.opart);
  float2* ml = reinterpret_cast<float2*>(ws + L.ml);
  const int64_t nk = static_cast<int64_t>(p.n_h) * 128;
  const int n_h = p.n_h, B = p.batch;
  const unsigned rtiles = static_cast<unsigned>((B + 31) / 32);
  mla_status s;
  // W_UV^T in fp16: [h*128 + d][c]
  if ((s = launch_transpose(static_cast<const uint16_t*>(W_UV), nk, 0, DC, DC, nk, WTv, DC, 0,
                            Elem::F16, 1, st, "decode_prep_w")) != MLA_OK)
    return s;
  {
    // q_lat[b][h][c] = sum_d q[b][h][d] W_UK[c][h*128 + d]
    KernelTimer kt("decode_absorb", st);
    hipLaunchKernelGGL((head_gemm_kernel<__bf16, _Float16>), dim3(DC / 32, rtiles, n_h), dim3(64),
                       0, st, static_cast<const __bf16*>(q), static_cast<int64_t>(n_h) * 192,
                       int64_t(192), static_cast<const __bf16*>(W_UK), nk, int64_t(128), qlat,
                       static_cast<int64_t>(n_h) * DC, int64_t(DC), B, DC, 128);
  }
  if ((s = check_launch("decode absorb")) != MLA_OK) return s;
  {
    KernelTimer kt("decode_attn", st);
    const int64_t items = static_cast<int64_t>(p.nch) * B * ((n_h + 127) / 128);
    if (items > INT32_MAX) return fail(MLA_ERR_UNSUPPORTED, "decode: too many workgroups");
    hipLaunchKernelGGL(decode_attn_pair_kernel, dim3(static_cast<unsigned>(items)), dim3(PDW * 64), 0,
                       st, qlat, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(c_kv),
                       static_cast<const uint16_t*>(k_rope), cu_dev, opart, ml, n_h, B, p.nch, p.chunk,
                       p.scale * 1.44269504088896340736f);
  }
  if ((s = check_launch("decode attention")) != MLA_OK) return s;
  {
    KernelTimer kt("decode_combine", st);
    hipLaunchKernelGGL(decode_combine_kernel, dim3(n_h, B), dim3(128), 0, st, opart, ml, cu_dev,
                       olat, lse, n_h, p.nch, p.chunk);
  }
  if ((s = check_launch("decode combine")) != MLA_OK) return s;
  {
    // out[b][h][d] = sum_c o_lat[b][h][c] W_UV[c][h*128 + d]
    KernelTimer kt("decode_outproj", st);
    hipLaunchKernelGGL((head_gemm_kernel<_Float16, float>), dim3(128 / 32, rtiles, n_h), dim3(64), 0,
                       st, olat, static_cast<int64_t>(n_h) * DC, int64_t(DC), WTv, int64_t(DC),
                       int64_t(128) * DC, out, static_cast<int64_t>(n_h) * 128, int64_t(128), B, 128,
                       DC);
  }
  return check_launch("decode output projection");
}

}  // namespace mla
