// Fast forward: rebuild K/V from the latent with the MFMA GEMM, then a
// flash-style causal attention kernel on gfx950 MFMA.
//
// The method (LAGA abstract) rebuilds each head's keys and values from the
// gathered latent and runs attention under a fused kernel. Here:
//   1. W_UK/W_UV are transposed once (k-contiguous GEMM operand), k_rope is
//      converted to fp16;
//   2. K_nope = c_kv W_UK_h is written key-major [h][key][128] and V
//      d-major [h][128][key], both fp16, for the keys this shard needs;
//   3. attention: each workgroup owns 256 query rows of one head (8 waves x
//      32 rows, two waves per SIMD); 64-key K and V^T tiles go straight from memory into LDS
//      (global_load_lds, double-buffered, the next tile in flight while the
//      current one is used). Each wave computes S^T = K Q^T so
//      a lane owns one query column: the row max and sum stay in the lane,
//      plus one exchange with the lane 32 away. Scores and the online
//      softmax are fp32; P goes to fp16 and straight into O^T += V^T P^T.
//      The two 32-key halves of a block are scored as two independent MFMA
//      chains, the running max is taken once per block, and the second
//      half's weights are formed on the VALU while the first half's PV
//      products run. The running max is only moved when a block's max
//      exceeds it by more than 2^8 (so P <= 256), which skips almost every
//      rescale of O.
#include <math.h>
#include <stdlib.h>

#include "fast.h"
#include "fast_common.h"

namespace mla {
namespace {

constexpr int FQ = 256;             // query rows per workgroup
constexpr int FK = 64;              // keys per step
constexpr int DQK = 192;
// LDS tiles carry a 16-byte pad per row: a wave's 16-lane groups then hit 16
// different 16-byte slots of the 64 banks for every read pattern used here
// (row stride 25 or 9 slots, both odd), and each fragment address is a
// per-lane base plus a compile-time offset.
constexpr int K_ROW_B = DQK * 2 + 16;    // 400 B
constexpr int V_ROW_B = FK * 2 + 16;     // 144 B
constexpr int K_TILE_B = FK * K_ROW_B;   // 25 KiB: 64 keys x 192 dims
constexpr int V_TILE_B = 128 * V_ROW_B;  // 18 KiB: V^T, 128 dims x 64 keys
constexpr int STAGE_B = K_TILE_B + V_TILE_B;
constexpr int STAGE_PIECES = STAGE_B / 1024;  // 43 DMA wave instructions
constexpr float kTau = 8.f;         // lazy-rescale threshold, log2 units
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ void work_item(int bid, int n_h, int n_qt, const int* order, int* h,
                                          int* qt) {
  // consecutive workgroups land on different XCDs (round robin over 8); with
  // n_h % 8 == 0 all query tiles of a head run on one XCD and share its L2.
  // Within a head the heaviest query tile goes first: the latest one for a
  // single causal sample, the first of `order` (tiles by decreasing
  // visible pairs) for a packed call.
  int r;
  if ((n_h & 7) == 0) {
    const int xcd = bid & 7, slot = bid >> 3;
    *h = (slot / n_qt) * 8 + xcd;
    r = slot % n_qt;
  } else {
    *h = bid % n_h;
    r = bid / n_h;
  }
  *qt = order != nullptr ? order[r] : n_qt - 1 - r;
}

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// NT: 32-row query tiles per wave; NW: waves per workgroup (NT*NW*32 = 256).
// Only NT = 1, NW = 8 is built: two waves per SIMD let one wave's softmax run
// while the other's MFMAs do. NT = 2 (64 rows per wave, half the LDS reads
// per MFMA, one wave per SIMD) measured slower.
template <int NT, int NW>
__global__ void __launch_bounds__(NW * 64)
attn_fwd_kernel(const uint16_t* __restrict__ q, const _Float16* __restrict__ Kfull,
                const _Float16* __restrict__ Vt, const int32_t* __restrict__ cu,
                const int* __restrict__ order, float* __restrict__ out, float* __restrict__ lse,
                int n_h, int n_seqs, int S_loc, RowMap rm, int key_lo, int Kpad, int n_qt,
                float scale_log2) {
  static_assert(NT * NW * 32 == FQ, "workgroup covers 256 query rows");
  static_assert(NT == 1, "only the 32-row-per-wave form is built");
  constexpr int NP = (STAGE_PIECES + NW - 1) / NW;  // DMA pieces per wave and stage
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE_B];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int lr = lane & 31, lh = lane >> 5;
  int h, qt;
  work_item(blockIdx.x, n_h, n_qt, order, &h, &qt);
  const int q0 = qt * FQ;
  const int wq0 = q0 + NT * 32 * w;

  // this lane's query columns; rows past S_loc see nothing. Positions
  // increase with the row, so a row range's extreme positions and sample
  // starts sit at its ends.
  int p[NT], lo[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int i = wq0 + 32 * nt + lr;
    p[nt] = i < S_loc ? rm_pos(rm, i) : -1;
    lo[nt] = i < S_loc ? static_cast<int>(seg_lo_dev(cu, n_seqs, p[nt])) : 0;
  }
  const bool wave_live = wq0 < S_loc;
  const int wi_last = min(S_loc - 1, wq0 + NT * 32 - 1);
  const int wp_min = rm_pos(rm, wq0), wp_max = rm_pos(rm, wi_last);
  const int wlo_min = wave_live ? static_cast<int>(seg_lo_dev(cu, n_seqs, wp_min)) : 0;
  const int wlo_max = wave_live ? static_cast<int>(seg_lo_dev(cu, n_seqs, wp_max)) : 0;

  // key blocks (workspace rows) the workgroup's rows can see
  const int i_last = min(S_loc - 1, q0 + FQ - 1);
  const int kb_begin = ((static_cast<int>(seg_lo_dev(cu, n_seqs, rm_pos(rm, q0))) - key_lo) / FK) * FK;
  const int kb_end = rm_pos(rm, i_last) + 1 - key_lo;
  const int nblk = (kb_end - kb_begin + FK - 1) / FK;

  // DMA: piece I (wave instruction) fills stage bytes [1024 I, 1024 I + 1024),
  // lane l the 16 bytes at +16 l. Per-lane source offsets (elements) relative
  // to the block's first key row; the 16-byte pad slot of a row reloads that
  // row's last piece (never read back).
  int dsrc[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int o = (w * NP + j) * 1024 + lane * 16;
    int off = 0;
    if (o < K_TILE_B) {
      const int row = o / K_ROW_B, pc = min((o % K_ROW_B) >> 4, DQK / 8 - 1);
      off = row * DQK + pc * 8;
    } else if (o < STAGE_B) {
      const int oo = o - K_TILE_B, d = oo / V_ROW_B, pc = min((oo % V_ROW_B) >> 4, FK / 8 - 1);
      off = d * Kpad + pc * 8;
    }
    dsrc[j] = off;
  }
  const _Float16* Kh = Kfull + static_cast<int64_t>(h) * Kpad * DQK;
  const _Float16* Vh = Vt + static_cast<int64_t>(h) * 128 * Kpad;
  auto issue = [&](int kb, int st) {
    char* dst = smem + st * STAGE_B;
    const _Float16* kbase = Kh + static_cast<int64_t>(kb) * DQK;
    const _Float16* vbase = Vh + kb;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int I = w * NP + j;   // wave-uniform
      if (I < STAGE_PIECES) {
        // wave-uniform base plus an opaque unsigned 32-bit lane offset in
        // bytes (the scalar-base form of the load)
        uint32_t off = static_cast<uint32_t>(dsrc[j]) * 2u;
        asm volatile("" : "+v"(off));
        lds_dma16(I * 1024 < K_TILE_B ? kbase : vbase, off, dst + I * 1024);
      }
    }
  };

  half8 qf[NT][12];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int i = wq0 + 32 * nt + lr;
    const uint16_t* src = q + (static_cast<int64_t>(i) * n_h + h) * DQK + 8 * lh;
#pragma unroll
    for (int kk = 0; kk < 12; ++kk) {
      if (i < S_loc) {
        qf[nt][kk] = bf16x8_to_half8(*reinterpret_cast<const u32x4*>(src + 16 * kk));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[nt][kk][e] = static_cast<_Float16>(0.f);
      }
    }
  }

  f32x16 o[NT][4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[nt][dt][e] = 0.f;
  float m[NT], l[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m[nt] = -INFINITY;
    l[nt] = 0.f;
  }
  const half2v ones = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
  // per-lane fragment bases: K rows swap23(lr) (+32 per key tile), V^T rows lr
  const int k_lane = swap23(lr) * K_ROW_B + lh * 16;
  const int v_lane = lr * V_ROW_B + lh * 16;

  if (nblk > 0) issue(kb_begin, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int b = 0; b < nblk; ++b) {
    const int st = b & 1;
    const int kb = kb_begin + b * FK;
    if (b + 1 < nblk) issue(kb + FK, st ^ 1);
    const int g0 = key_lo + kb;  // global position of the block's first key
    const bool skip = !wave_live || g0 > wp_max || g0 + FK - 1 < wlo_min;
    if (!skip) {
      const bool need_mask = !(g0 >= wlo_max && g0 + FK - 1 <= wp_min);
      const char* sk = smem + st * STAGE_B + k_lane;
      const char* sv = smem + st * STAGE_B + K_TILE_B + v_lane;
      // S^T of both 32-key halves of the block (rows: keys 32 mt +
      // swap23(lr)) as two independent chains issued alternately, K
      // fragment reads FPF products ahead of each chain
      f32x16 s[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[mt][e] = 0.f;
      constexpr int FPF = 3;
      half8 fa[2][FPF + 1];
#pragma unroll
      for (int i = 0; i < FPF; ++i)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          fa[mt][i] = *reinterpret_cast<const half8*>(sk + mt * 32 * K_ROW_B + 32 * i);
      // the score products run at raised wave priority, so that the SIMD's
      // other wave fills the gaps of these chains with its softmax
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kk = 0; kk < 12; ++kk) {
        if (kk + FPF < 12)
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
            fa[mt][(kk + FPF) % (FPF + 1)] =
                *reinterpret_cast<const half8*>(sk + mt * 32 * K_ROW_B + 32 * (kk + FPF));
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) s[mt] = mfma_f16(fa[mt][kk % (FPF + 1)], qf[0][kk], s[mt]);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
      if (need_mask) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = g0 + 32 * mt + swap23(d_row(r, lh));
            if (key < lo[0] || key > p[0]) s[mt][r] = -INFINITY;
          }
      }
      // one running-max update per 64-key block
      float mx = s[0][0];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mt][r]);
      mx = wave_max_pair(mx) * scale_log2;
      const bool grow = mx > m[0] + kTau;
      if (__any(grow)) {
        const float m_new = grow ? mx : m[0];
        const float alpha = grow ? __builtin_amdgcn_exp2f(m[0] - m_new) : 1.f;
        m[0] = m_new;
        l[0] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[0][dt][e] *= alpha;
      }
      const float mu = m[0] == -INFINITY ? 0.f : m[0];
      float sum = l[0];
      // the weights of one half, then its PV products; the second half's
      // weights are formed on the VALU while the first half's products run
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        half8 pb[2];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          half2v pr;
          pr[0] = static_cast<_Float16>(__builtin_amdgcn_exp2f(fmaf(s[mt][r], scale_log2, -mu)));
          pr[1] = static_cast<_Float16>(__builtin_amdgcn_exp2f(fmaf(s[mt][r + 1], scale_log2, -mu)));
          pb[r >> 3][r & 7] = pr[0];
          pb[r >> 3][(r & 7) + 1] = pr[1];
          sum = __builtin_amdgcn_fdot2(pr, ones, sum, false);   // sum of the fp16 weights
        }
#pragma unroll
        for (int ksl = 0; ksl < 2; ++ksl) {
          const int ks = 2 * mt + ksl;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const half8 a = *reinterpret_cast<const half8*>(sv + dt * 32 * V_ROW_B + ks * 32);
            o[0][dt] = mfma_f16(a, pb[ksl], o[0][dt]);
          }
        }
      }
      l[0] = sum;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float lt = wave_sum_pair(l[nt]);
    const int i = wq0 + 32 * nt + lr;
    if (i < S_loc) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      float* dst = out + (static_cast<int64_t>(i) * n_h + h) * 128;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 v = {o[nt][dt][4 * g] * inv, o[nt][dt][4 * g + 1] * inv,
                           o[nt][dt][4 * g + 2] * inv, o[nt][dt][4 * g + 3] * inv};
          *reinterpret_cast<f32x4*>(dst + 32 * dt + 8 * g + 4 * lh) = v;
        }
      if (lh == 0)
        lse[static_cast<int64_t>(i) * n_h + h] = lt > 0.f ? (m[nt] + __log2f(lt)) * kLn2 : -INFINITY;
    }
  }
}

}  // namespace

// Rebuild per-head keys and values from the latent (MFMA GEMMs), in the
// layouts the attention kernels read; null outputs are skipped.
//   Kfull  [n_h][Kpad][192]  key rows: K_nope | k_rope       (forward, backward)
//   Vt     [n_h][128][Kpad]  V transposed                     (forward)
//   Vkm    [n_h][Kpad][128]  V key rows                       (backward)
// WT receives [W_UK | W_UV] transposed (bf16 [2*n_h*128][d_c]). The rope
// key's copy into Kfull (its own 128-byte lines of each key row) goes to
// `side` when given, beside the GEMMs.
mla_status fast_rebuild_kv(const Plan& p, const void* c_kv, const void* k_rope, const void* W_UK,
                           const void* W_UV, uint16_t* WT, _Float16* Kfull, _Float16* Vt,
                           _Float16* Vkm, hipStream_t st, hipStream_t side, const SideStream* vside) {
  const int64_t nk = static_cast<int64_t>(p.n_h) * 128;
  const uint16_t* ckv = static_cast<const uint16_t*>(c_kv) + p.key_lo * p.d_c;
  const uint16_t* kr = static_cast<const uint16_t*>(k_rope) + p.key_lo * 64;
  const uint16_t* WTv = WT + nk * p.d_c;
  mla_status s;
  if (Kfull &&
      (s = launch_broadcast_rows_f16(kr, 64, p.Kn, p.Kpad, 64, Kfull + 128, 192, p.Kpad * 192, p.n_h,
                                     side != nullptr ? side : st, "prep_rope")) != MLA_OK)
    return s;
  // with vside, W_UV's transpose runs on that stream beside the K GEMM and is
  // joined back before the V GEMM
  if ((s = launch_transpose(static_cast<const uint16_t*>(W_UV), nk, 0, p.d_c, p.d_c, nk,
                            WT + nk * p.d_c, p.d_c, 0, Elem::BF16, 1, vside ? vside->st : st,
                            "prep_w")) != MLA_OK)
    return s;
  if ((s = launch_transpose(static_cast<const uint16_t*>(W_UK), nk, 0, p.d_c, p.d_c, nk, WT, p.d_c,
                            0, Elem::BF16, 1, st, "prep_w")) != MLA_OK) return s;
  if (Kfull) {
    // Out[key][h*128 + d] = c_kv[key] . WT[h*128 + d] -> Kfull[h][key][d]
    if ((s = launch_gemm_nt(ckv, p.d_c, p.Kn, WT, p.d_c, nk, p.d_c, Kfull, 192, 128 * 192,
                            p.Kpad * 192, p.Kpad, nk, Elem::BF16, Elem::F16, st, "upproj")) != MLA_OK)
      return s;
  }
  if (vside && (s = side_join(*vside, st)) != MLA_OK) return s;
  if (Vt &&
      (s = launch_gemm_nt(WTv, p.d_c, nk, ckv, p.d_c, p.Kn, p.d_c, Vt, p.Kpad, 128 * p.Kpad, 128, nk,
                          p.Kpad, Elem::BF16, Elem::F16, st, "upproj")) != MLA_OK)
    return s;
  if (Vkm &&
      (s = launch_gemm_nt(ckv, p.d_c, p.Kn, WTv, p.d_c, nk, p.d_c, Vkm, 128, 128 * 128, p.Kpad * 128,
                          p.Kpad, nk, Elem::BF16, Elem::F16, st, "upproj")) != MLA_OK)
    return s;
  return MLA_OK;
}

mla_status fast_fwd_limits(const Plan& p) {
  // positions (S + 256) and key-row offsets (Kpad 192) in 32 bits; the
  // up-projection GEMM's operand rows (n_h 128 and Kpad elements) below 2^22
  if (p.S + 256 >= (int64_t(1) << 31) || p.Kpad >= (int64_t(1) << 22) ||
      static_cast<int64_t>(p.n_h) * 128 >= (int64_t(1) << 22))
    return fail(MLA_ERR_UNSUPPORTED,
                "fast forward takes n_h < 32768, fewer than 2^22 needed keys and S below 2^31 - 256");
  return MLA_OK;
}

mla_status fast_fwd(const Plan& p, const void* q, const void* c_kv, const void* k_rope,
                    const void* W_UK, const void* W_UV, const int32_t* cu_dev, float* out,
                    float* lse, char* ws, hipStream_t st) {
  const FwdLayout L = fwd_layout(p);
  if (mla_status s = fast_fwd_limits(p); s != MLA_OK) return s;
  uint16_t* WT = reinterpret_cast<uint16_t*>(ws + L.WT);
  _Float16* Kfull = reinterpret_cast<_Float16*>(ws + L.Kfull);
  _Float16* Vt = reinterpret_cast<_Float16*>(ws + L.Vt);
  // the rope-key copy runs on a side stream beside the GEMMs, joined back
  // before the attention reads Kfull
  SideStream side;
  mla_status s = side_stream(&side);
  if (s != MLA_OK) return s;
  {
    SideFork fork(side, st);
    if ((s = fork.fork()) != MLA_OK) return s;
    if ((s = fast_rebuild_kv(p, c_kv, k_rope, W_UK, W_UV, WT, Kfull, Vt, nullptr, st, side.st, &side)) != MLA_OK)
      return s;
    if ((s = fork.join()) != MLA_OK) return s;
  }
  const int n_qt = static_cast<int>((p.S_loc + FQ - 1) / FQ);
  const int64_t blocks = static_cast<int64_t>(n_qt) * p.n_h;
  if (blocks > INT32_MAX) return fail(MLA_ERR_UNSUPPORTED, "too many attention workgroups");
  const float scale_log2 = p.scale * 1.44269504088896340736f;
  // packed calls: query tiles in longest-processing-time order
  int* order = nullptr;
  if (p.n_seqs > 0 && n_qt <= kMaxOrderTiles) {
    order = reinterpret_cast<int*>(ws + L.order);
    if ((s = launch_tile_order(cu_dev, p.n_seqs, p.S_loc, p.rm, p.key_lo, p.Kn, n_qt, 0,
                               order, nullptr, st)) != MLA_OK)
      return s;
  }
  const int S_loc = static_cast<int>(p.S_loc), key_lo = static_cast<int>(p.key_lo), Kpad = static_cast<int>(p.Kpad);
  {
    KernelTimer kt("attn_fwd", st);
    hipLaunchKernelGGL((attn_fwd_kernel<1, 8>), dim3(static_cast<unsigned>(blocks)), dim3(512), 0,
                       st, static_cast<const uint16_t*>(q), Kfull, Vt, cu_dev, order, out, lse, p.n_h,
                       p.n_seqs, S_loc, p.rm, key_lo, Kpad, n_qt, scale_log2);
  }
  return check_launch("attention forward");
}

}  // namespace mla
