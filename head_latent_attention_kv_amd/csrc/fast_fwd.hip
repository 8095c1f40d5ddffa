// Fast forward: rebuild K/V from the latent with the MFMA GEMM, then a
// flash-style causal attention kernel on gfx950 MFMA.
//
// The method (LAGA abstract) rebuilds each head's keys and values from the
// gathered latent and runs attention under a fused kernel. Here:
//   1. W_UK/W_UV are transposed once (k-contiguous GEMM operand), k_rope is
//      converted to fp16;
//   2. K_nope = c_kv W_UK_h is written key-major [h][key][128] and V
//      d-major [h][128][key], both fp16, for the keys this shard needs;
//   3. attention: each workgroup owns 256 query rows of one head (4 waves x
//      64 rows); 64-key K and V^T tiles go straight from memory into LDS
//      (global_load_lds, double-buffered, the next tile in flight while the
//      current one is used). Each wave computes S^T = K Q^T so
//      a lane owns one query column: the row max and sum stay in the lane,
//      plus one exchange with the lane 32 away. Scores and the online
//      softmax are fp32; P goes to fp16 and straight into O^T += V^T P^T.
//      The running max is only moved when a block's max exceeds it by more
//      than 2^8 (so P <= 256), which skips almost every rescale of O.
#include <math.h>

#include "fast.h"
#include "fast_common.h"

namespace mla {
namespace {

constexpr int FQ = 256;             // query rows per workgroup
constexpr int FK = 64;              // keys per step
constexpr int DQK = 192;
constexpr int K_ROW_B = DQK * 2;    // bytes per key row in LDS: nope 256 + rope 128
constexpr int K_TILE_B = FK * K_ROW_B;   // 24 KiB
constexpr int V_TILE_B = 128 * FK * 2;   // 16 KiB: V^T, 128 rows of 64 keys
constexpr int STAGE_B = K_TILE_B + V_TILE_B;
constexpr float kTau = 8.f;         // lazy-rescale threshold, log2 units
constexpr float kLn2 = 0.69314718055994530942f;

// LDS tiles are unpadded and XOR-swizzled in 16-byte pieces so that they can
// be filled by global_load_lds (each wave instruction writes 1 KiB
// contiguously, lane l at +16*l) and read back conflict-free: the 8 lanes
// served together read 8 different key rows at the same logical piece, and
// the swizzle spreads those over all 32 banks.
__device__ __forceinline__ int kswz(int row) { return (row & 3) | ((row >> 1) & 4); }
__device__ __forceinline__ int k_off(int row, int c) {
  return row * K_ROW_B + (((c & ~7) | ((c & 7) ^ kswz(row))) << 4);
}
__device__ __forceinline__ int v_off(int d, int c) { return d * (FK * 2) + ((c ^ (d & 7)) << 4); }

__device__ __forceinline__ void work_item(int bid, int n_h, int n_qt, int* h, int* qt) {
  // consecutive workgroups land on different XCDs (round robin over 8); with
  // n_h % 8 == 0 all query tiles of a head run on one XCD and share its L2.
  // Within a head the heaviest (latest) query tile goes first.
  if ((n_h & 7) == 0) {
    const int xcd = bid & 7, slot = bid >> 3;
    *h = (slot / n_qt) * 8 + xcd;
    *qt = n_qt - 1 - slot % n_qt;
  } else {
    *h = bid % n_h;
    *qt = n_qt - 1 - bid / n_h;
  }
}

__device__ __forceinline__ void lds_dma16(const void* src, char* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, lds_dst, 16, 0, 0);
}

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_fwd_kernel(const uint16_t* __restrict__ q, const _Float16* __restrict__ Knope,
                const _Float16* __restrict__ Krope, const _Float16* __restrict__ Vt,
                const int32_t* __restrict__ cu, float* __restrict__ out, float* __restrict__ lse,
                int n_h, int n_seqs, int64_t S_loc, int64_t q_offset, int64_t key_lo, int64_t Kpad,
                int n_qt, float scale_log2) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE_B];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5;
  int h, qt;
  work_item(blockIdx.x, n_h, n_qt, &h, &qt);
  const int64_t q0 = static_cast<int64_t>(qt) * FQ;
  const int64_t wq0 = q0 + 64 * w;

  // this lane's two query columns (nt = 0, 1); rows past S_loc see nothing
  int64_t p[2], lo[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int64_t i = wq0 + 32 * nt + lr;
    p[nt] = i < S_loc ? q_offset + i : -1;
    lo[nt] = i < S_loc ? seg_lo_dev(cu, n_seqs, q_offset + i) : 0;
  }
  const bool wave_live = wq0 < S_loc;
  const int64_t wi_last = min(S_loc - 1, wq0 + 63);
  const int64_t wp_min = q_offset + wq0, wp_max = q_offset + wi_last;
  const int64_t wlo_min = wave_live ? seg_lo_dev(cu, n_seqs, wp_min) : 0;
  const int64_t wlo_max = wave_live ? seg_lo_dev(cu, n_seqs, wp_max) : 0;

  // key blocks (workspace rows) the workgroup's rows can see
  const int64_t i_last = min(S_loc - 1, q0 + FQ - 1);
  const int64_t kb_begin = ((seg_lo_dev(cu, n_seqs, q_offset + q0) - key_lo) / FK) * FK;
  const int64_t kb_end = q_offset + i_last + 1 - key_lo;
  const int nblk = static_cast<int>((kb_end - kb_begin + FK - 1) / FK);

  // per-lane sources of this wave's DMA pieces: 6 of the 24 K-tile KiB and
  // 4 of the 16 V-tile KiB (offsets in elements relative to key block kb)
  int k_src[6];
  bool k_rope[6];
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    const int o = (w * 6 + j) * 1024 + lane * 16;
    const int row = o / K_ROW_B, pos = (o % K_ROW_B) >> 4;
    const int c = (pos & ~7) | ((pos & 7) ^ kswz(row));
    k_rope[j] = c >= 16;
    k_src[j] = c < 16 ? row * 128 + c * 8 : row * 64 + (c - 16) * 8;
  }
  int v_src[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int o = (w * 4 + j) * 1024 + lane * 16;
    const int d = o >> 7, pos = (o & 127) >> 4;
    v_src[j] = d * static_cast<int>(Kpad) + ((pos ^ (d & 7)) << 3);
  }
  const _Float16* Kh = Knope + static_cast<int64_t>(h) * Kpad * 128;
  const _Float16* Vh = Vt + static_cast<int64_t>(h) * 128 * Kpad;
  auto issue = [&](int64_t kb, int st) {
    char* kdst = smem + st * STAGE_B;
    const _Float16* kn = Kh + kb * 128;
    const _Float16* kr = Krope + kb * 64;
#pragma unroll
    for (int j = 0; j < 6; ++j)
      lds_dma16((k_rope[j] ? kr : kn) + k_src[j], kdst + (w * 6 + j) * 1024);
    const _Float16* vb = Vh + kb;
#pragma unroll
    for (int j = 0; j < 4; ++j) lds_dma16(vb + v_src[j], kdst + K_TILE_B + (w * 4 + j) * 1024);
  };

  half8 qf[2][12];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int64_t i = wq0 + 32 * nt + lr;
    const uint16_t* src = q + (i * n_h + h) * DQK + 8 * lh;
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

  f32x16 o[2][4];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[nt][dt][e] = 0.f;
  float m[2] = {-INFINITY, -INFINITY};
  float l[2] = {0.f, 0.f};

  if (nblk > 0) issue(kb_begin, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int b = 0; b < nblk; ++b) {
    const int st = b & 1;
    const int64_t kb = kb_begin + static_cast<int64_t>(b) * FK;
    if (b + 1 < nblk) issue(kb + FK, st ^ 1);
    const int64_t g0 = key_lo + kb;  // global position of the block's first key
    const bool skip = !wave_live || g0 > wp_max || g0 + FK - 1 < wlo_min;
    if (!skip) {
      const bool need_mask = !(g0 >= wlo_max && g0 + FK - 1 <= wp_min);
      const char* sk = smem + st * STAGE_B;
      const char* sv = sk + K_TILE_B;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        // S^T rows: keys 32mt + swap23(lr) of the block
        const int krow = 32 * mt + swap23(lr);
        f32x16 s[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int e = 0; e < 16; ++e) s[nt][e] = 0.f;
        half8 fa[3];
        fa[0] = *reinterpret_cast<const half8*>(sk + k_off(krow, lh));
        fa[1] = *reinterpret_cast<const half8*>(sk + k_off(krow, 2 + lh));
#pragma unroll
        for (int kk = 0; kk < 12; ++kk) {
          if (kk + 2 < 12)
            fa[(kk + 2) % 3] = *reinterpret_cast<const half8*>(sk + k_off(krow, 2 * (kk + 2) + lh));
          s[0] = mfma_f16(fa[kk % 3], qf[0][kk], s[0]);
          s[1] = mfma_f16(fa[kk % 3], qf[1][kk], s[1]);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (need_mask) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t key = g0 + 32 * mt + swap23(d_row(r, lh));
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
              if (key < lo[nt] || key > p[nt]) s[nt][r] = -INFINITY;
          }
        }
        half8 pb[2][2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          float mx = s[nt][0];
#pragma unroll
          for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[nt][r]);
          mx = wave_max_pair(mx) * scale_log2;
          const bool grow = mx > m[nt] + kTau;
          if (__any(grow)) {
            const float m_new = grow ? mx : m[nt];
            const float alpha = grow ? __builtin_amdgcn_exp2f(m[nt] - m_new) : 1.f;
            m[nt] = m_new;
            l[nt] *= alpha;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
              for (int e = 0; e < 16; ++e) o[nt][dt][e] *= alpha;
          }
          const float mu = m[nt] == -INFINITY ? 0.f : m[nt];
          float sum = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pv = __builtin_amdgcn_exp2f(fmaf(s[nt][r], scale_log2, -mu));
            sum += pv;
            pb[nt][r >> 3][r & 7] = static_cast<_Float16>(pv);
          }
          l[nt] += sum;
        }
#pragma unroll
        for (int ksl = 0; ksl < 2; ++ksl) {
          const int ks = 2 * mt + ksl;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const half8 a = *reinterpret_cast<const half8*>(sv + v_off(32 * dt + lr, 2 * ks + lh));
            o[0][dt] = mfma_f16(a, pb[0][ksl], o[0][dt]);
            o[1][dt] = mfma_f16(a, pb[1][ksl], o[1][dt]);
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float lt = l[nt] + __shfl_xor(l[nt], 32, 64);
    const int64_t i = wq0 + 32 * nt + lr;
    if (i < S_loc) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      float* dst = out + (i * n_h + h) * 128;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 v = {o[nt][dt][4 * g] * inv, o[nt][dt][4 * g + 1] * inv,
                           o[nt][dt][4 * g + 2] * inv, o[nt][dt][4 * g + 3] * inv};
          *reinterpret_cast<f32x4*>(dst + 32 * dt + 8 * g + 4 * lh) = v;
        }
      if (lh == 0) lse[i * n_h + h] = lt > 0.f ? (m[nt] + __log2f(lt)) * kLn2 : -INFINITY;
    }
  }
}

}  // namespace

// Up-projection into the forward layouts (shared with the backward, which
// asks for other layouts through the same GEMM).
mla_status fast_rebuild_kv(const Plan& p, const void* c_kv, const void* k_rope, const void* W_UK,
                           const void* W_UV, uint16_t* WT, _Float16* Knope, _Float16* Vt,
                           _Float16* Vkm, _Float16* Krope, _Float16* KnopeT, _Float16* KropeT,
                           hipStream_t st) {
  const int64_t nk = static_cast<int64_t>(p.n_h) * 128;
  const uint16_t* ckv = static_cast<const uint16_t*>(c_kv) + p.key_lo * p.d_c;
  const uint16_t* kr = static_cast<const uint16_t*>(k_rope) + p.key_lo * 64;
  mla_status s;
  // WT[n][c]: rows 0..nk-1 from W_UK, nk..2nk-1 from W_UV
  if ((s = launch_transpose(static_cast<const uint16_t*>(W_UK), nk, 0, p.d_c, p.d_c, nk, WT, p.d_c,
                            0, Elem::BF16, 1, st, "prep_w")) != MLA_OK) return s;
  if ((s = launch_transpose(static_cast<const uint16_t*>(W_UV), nk, 0, p.d_c, p.d_c, nk,
                            WT + nk * p.d_c, p.d_c, 0, Elem::BF16, 1, st, "prep_w")) != MLA_OK)
    return s;
  if (Krope &&
      (s = launch_convert(kr, 64, 0, p.Kn, p.Kpad, 64, Krope, 64, 0, Elem::F16, 1, st,
                          "prep_rope")) != MLA_OK)
    return s;
  if (KropeT &&
      (s = launch_transpose(kr, 64, 0, p.Kn, p.Kpad, 64, KropeT, p.Kpad, 0, Elem::F16, 1, st,
                            "prep_rope")) != MLA_OK)
    return s;
  // K_nope key-major: Out[key][h*128 + d] = c_kv[key] . WT[h*128 + d]
  if (Knope &&
      (s = launch_gemm_nt(ckv, p.d_c, p.Kn, WT, p.d_c, nk, p.d_c, Knope, 128, p.Kpad * 128, p.Kpad,
                          nk, Elem::BF16, Elem::F16, st, "upproj")) != MLA_OK)
    return s;
  // K_nope d-major: Out[h*128 + d][key]
  if (KnopeT &&
      (s = launch_gemm_nt(WT, p.d_c, nk, ckv, p.d_c, p.Kn, p.d_c, KnopeT, p.Kpad, 128, nk, p.Kpad,
                          Elem::BF16, Elem::F16, st, "upproj")) != MLA_OK)
    return s;
  // V d-major (V^T): Out[h*128 + d][key]
  if (Vt &&
      (s = launch_gemm_nt(WT + nk * p.d_c, p.d_c, nk, ckv, p.d_c, p.Kn, p.d_c, Vt, p.Kpad, 128, nk,
                          p.Kpad, Elem::BF16, Elem::F16, st, "upproj")) != MLA_OK)
    return s;
  // V key-major: Out[key][h*128 + d]
  if (Vkm &&
      (s = launch_gemm_nt(ckv, p.d_c, p.Kn, WT + nk * p.d_c, p.d_c, nk, p.d_c, Vkm, 128,
                          p.Kpad * 128, p.Kpad, nk, Elem::BF16, Elem::F16, st, "upproj")) != MLA_OK)
    return s;
  return MLA_OK;
}

mla_status fast_fwd(const Plan& p, const void* q, const void* c_kv, const void* k_rope,
                    const void* W_UK, const void* W_UV, const int32_t* cu_dev, float* out,
                    float* lse, char* ws, hipStream_t st) {
  const FwdLayout L = fwd_layout(p);
  uint16_t* WT = reinterpret_cast<uint16_t*>(ws + L.WT);
  _Float16* Knope = reinterpret_cast<_Float16*>(ws + L.Knope);
  _Float16* Vt = reinterpret_cast<_Float16*>(ws + L.Vt);
  _Float16* Krope = reinterpret_cast<_Float16*>(ws + L.Krope);
  mla_status s = fast_rebuild_kv(p, c_kv, k_rope, W_UK, W_UV, WT, Knope, Vt, nullptr, Krope,
                                 nullptr, nullptr, st);
  if (s != MLA_OK) return s;
  if (p.Kpad * 128 >= (int64_t(1) << 31))
    return fail(MLA_ERR_UNSUPPORTED, "fast path takes fewer than 2^24 latent rows per call");
  const int n_qt = static_cast<int>((p.S_loc + FQ - 1) / FQ);
  const int64_t blocks = static_cast<int64_t>(n_qt) * p.n_h;
  if (blocks > INT32_MAX) return fail(MLA_ERR_UNSUPPORTED, "too many attention workgroups");
  const float scale_log2 = p.scale * 1.44269504088896340736f;
  {
    KernelTimer kt("attn_fwd", st);
    hipLaunchKernelGGL(attn_fwd_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                       static_cast<const uint16_t*>(q), Knope, Krope, Vt, cu_dev, out, lse, p.n_h,
                       p.n_seqs, p.S_loc, p.q_offset, p.key_lo, p.Kpad, n_qt, scale_log2);
  }
  return check_launch("attention forward");
}

}  // namespace mla
