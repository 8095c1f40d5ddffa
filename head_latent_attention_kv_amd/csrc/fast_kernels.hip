// MFMA GEMM and layout conversions for the fast path.
//
// The latent up-projection (LAGA abstract: per-head K/V rebuilt from the
// gathered latent) and the backward's latent and weight gradients are all
// plain GEMMs with K = d_c, n_h*(d_nope+d_v) or the key count. One kernel
// covers them: both operands are read k-contiguous (so a lane's 8 k-values
// are one 16-byte LDS read), 256x256 output tiles over eight waves of
// 128x64, and an fp16 result is staged through LDS so every global store is
// a full 16-byte row piece. Thin outputs (the gradients of c_kv and of the
// weights) split K over more workgroups and sum the fp32 partials in a fixed
// order afterwards.
#include <stdlib.h>

#include <algorithm>
#include <type_traits>

#include "fast.h"
#include "fast_common.h"

namespace mla {
namespace {

constexpr int GT = 256;                 // output tile rows and columns
constexpr int GK = 32;                  // k per chunk: one 64-byte LDS row per operand row
constexpr int G_OP = GT * GK * 2;       // one operand's tile (16 KiB)
constexpr int G_STAGE = 2 * G_OP;       // X and Y tiles
constexpr int G_NST = 5;                // stages in the ring: four chunks in flight
constexpr int G_PIECES = 2 * G_OP / 1024;  // DMA wave instructions per chunk: 32
constexpr int G_MIN_BLOCKS = 512;       // split K until the grid has this many workgroups
static_assert(G_NST * G_STAGE <= 160 * 1024, "ring fits the LDS");
static_assert((G_NST - 2) * G_PIECES / 4 <= 63, "outstanding DMA count fits vmcnt");

// Wait until at most n of this wave's vector-memory operations are
// outstanding (n a multiple of 4 up to 24; gfx9 encoding of s_waitcnt:
// vmcnt bits 3:0 and 15:14, expcnt and lgkmcnt left at their maxima).
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
    case 16: __builtin_amdgcn_s_waitcnt(0x4F70); break;
    case 20: __builtin_amdgcn_s_waitcnt(0x4F74); break;
    default: __builtin_amdgcn_s_waitcnt(0x4F78); break;
  }
}

// Tile of workgroup `bid`. Tiles run in groups of 8 tile rows (all columns of
// a group before the next group); when the count divides by 8, XCD x (blocks
// x, x + 8, ...) takes the x-th eighth of that order, so the tiles one XCD
// holds at a time share rows and columns in its L2.
__device__ __forceinline__ void gemm_tile(int bid, int n_tr, int n_tc, int* tr, int* tc) {
  const int n = n_tr * n_tc;
  const int L = (n & 7) == 0 ? (bid & 7) * (n >> 3) + (bid >> 3) : bid;
  constexpr int G = 8;
  const int group = L / (G * n_tc);
  const int first = group * G;
  const int rows = min(G, n_tr - first);
  const int within = L - group * G * n_tc;
  *tr = first + within % rows;
  *tc = within / rows;
}

// Out[r][c] = sum_k X[r][k] Y[c][k] over one K range (blockIdx.y selects it):
// 256x256 tiles, eight waves of 128x64 (8 MFMA accumulators each, two waves
// per SIMD so one wave's loads and stores overlap the other's MFMAs), 32-deep
// k-chunks DMA-filled (global_load_lds) into a ring of five LDS stages, so
// four chunks are in flight while one is consumed: with one workgroup per
// CU, that depth is what covers the latency of the operand reads that miss
// in L2. A 64-byte operand row holds its four 16-byte k-slots in the order
// slot ^ ((row / 4) % 4), so the 16 rows read together by a fragment load
// fall on 16 different slots of the 64 banks. Rows of X past R and of Y past
// C are clamped to the last valid row when loading and their results are
// written as 0. With kPart, the tile goes unmasked to part[blockIdx.y][r][c]
// (fp32) for a split-K reduction; otherwise to `out` in the tiled layout of
// launch_gemm_nt.
//
// kYT: Y is stored k-major instead, Y[k][c] with ldy elements per k row (the
// row-major gradient rows of the backward, contracted over keys). Its tile
// is then 32 k rows of 256 columns (512 bytes each), DMA-filled two rows per
// wave instruction, and each fragment is read transposed (two
// ds_read_b64_tr_b16). A transposed read's 16 lanes fetch 8 bytes of 4
// consecutive rows in one 32-byte column span; storing the 16-byte slot s of
// row k at slot s ^ (2 (k % 4)) puts those 4 spans on 4 different 32-byte
// groups of banks.
template <typename InT, typename OutT, bool kPart, int kW, bool kYT = false>
__global__ void __launch_bounds__(kW * 64)
gemm_nt_kernel(const InT* __restrict__ X, int64_t ldx, int64_t R, const InT* __restrict__ Y,
               int64_t ldy, int64_t C, int64_t k_len, OutT* __restrict__ out, int64_t ldo,
               int64_t rt_stride, int64_t ct_stride, int64_t R_store, int64_t C_store,
               float* __restrict__ part, const float* __restrict__ alpha, int n_tr, int n_tc) {
  typedef typename MfmaOp<InT>::vec vec;
  // kW = 4 (four waves of 128x128) also indexes correctly but measured slower;
  // only the eight-wave form is built.
  static_assert(kW == 8, "eight waves of 128x64");
  constexpr int NI = kW == 8 ? 2 : 4;   // 32-column tiles per wave
  constexpr int NPW = G_PIECES / kW;    // DMA pieces per wave and chunk
  constexpr int HW = kW / 2;            // waves per operand (DMA) and per row half
  // the ring, reused afterwards to stage an fp16 output tile
  __shared__ __attribute__((aligned(1024))) char smem[G_NST * G_STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int lr = lane & 31, lh = lane >> 5;
  int tr, tc;
  gemm_tile(blockIdx.x, n_tr, n_tc, &tr, &tc);
  const int64_t r0 = static_cast<int64_t>(tr) * GT, c0 = static_cast<int64_t>(tc) * GT;
  const int64_t kbeg = static_cast<int64_t>(blockIdx.y) * k_len;
  const int wr = w / HW, wc = w % HW;  // rows 128 wr .., columns 32 NI wc ..
  const bool live = R > 0 && C > 0;

  // the first half of the waves fill the X tile, the second the Y tile
  const bool is_x = w < HW;
  const bool ykm = kYT && !is_x;   // this wave fills a k-major Y tile
  const int64_t ld = is_x ? ldx : ldy;
  const InT* src = live ? (is_x ? X + r0 * ldx + kbeg : (kYT ? Y + kbeg * ldy + c0 : Y + c0 * ldy + kbeg))
                        : nullptr;
  const int last = static_cast<int>((is_x ? R - r0 : C - c0) - 1);   // >= 0 for live tiles
  // piece p of an operand tile = rows 16p .. 16p + 15; lane l fills row
  // 16p + l / 4, physical slot l % 4, which holds k-slot (l % 4) ^ ((row / 4) % 4).
  // k-major Y: piece p = k rows 2p, 2p + 1; lane l fills k row 2p + l / 32,
  // physical slot l % 32, which holds column slot (l % 32) ^ (2 (row % 4))
  // (columns past C reload the last valid 8 columns; never stored)
  int doff[NPW];
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    if (ykm) {
      const int row = 2 * ((w % HW) * NPW + j) + (lane >> 5);
      const int cs = (lane & 31) ^ (2 * (row & 3));
      doff[j] = row * static_cast<int>(ld) + min(8 * cs, last & ~7);
    } else {
      const int row = 16 * ((w % HW) * NPW + j) + (lane >> 2);
      const int slot = (lane & 3) ^ ((row >> 2) & 3);
      doff[j] = min(row, last) * static_cast<int>(ld) + slot * 8;
    }
  }
  auto issue = [&](int c, int st) {
    char* dst = smem + st * G_STAGE + (is_x ? 0 : G_OP) + (w % HW) * NPW * 1024;
    const char* s0 = reinterpret_cast<const char*>(src + static_cast<int64_t>(c) * GK * (ykm ? ld : 1));
#pragma unroll
    for (int j = 0; j < NPW; ++j) {
      // wave-uniform base plus an unsigned 32-bit lane offset in bytes (the
      // scalar-base form of the load), opaque to the optimizer so that no
      // 64-bit address per piece is hoisted
      uint32_t off = static_cast<uint32_t>(doff[j]) * static_cast<uint32_t>(sizeof(InT));
      asm volatile("" : "+v"(off));
      lds_dma16(s0, off, dst + j * 1024);
    }
  };

  f32x16 acc[NI][4];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // fragment rows are wave base + 32 i + lr, so (row / 4) % 4 = (lr / 4) % 4
  const int so0 = ((0 + lh) ^ ((lr >> 2) & 3)) * 16, so1 = ((2 + lh) ^ ((lr >> 2) & 3)) * 16;
  const int nk = live ? static_cast<int>(k_len / GK) : 0;
  // fragments: [k16 step of the chunk][tile]
  vec a[2][NI], b[2][4];
  // k-major Y: lane (g = l / 16, p = l % 16) reads k rows 16 step + 8 (g / 2)
  // + p / 4 (and 4 further), columns 32 (wc NI + i) + 16 (g % 2) + 4 (p % 4)
  // .. + 3 (frag_tr2); the column slot moves by the row's swizzle
  int yt_off[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int g = lane >> 4, p = lane & 15;
    const int cs = 4 * (wc * NI + i) + 2 * (g & 1) + ((p & 3) >> 1);
    yt_off[i] = (8 * (g >> 1) + (p >> 2)) * (GT * 2) + (cs ^ (2 * (p >> 2))) * 16 + 8 * (p & 1);
  }
  auto frags = [&](int kc, int step) {
    const int st = kc % G_NST, so = step ? so1 : so0;
    const char* xa = smem + st * G_STAGE + (wr * 128 + lr) * (GK * 2) + so;
    const char* ya = smem + st * G_STAGE + G_OP + (wc * 32 * NI + lr) * (GK * 2) + so;
    if constexpr (kYT) {
      const char* yt = smem + st * G_STAGE + G_OP + step * 16 * (GT * 2);
#pragma unroll
      for (int i = 0; i < NI; ++i)
        a[step][i] = frag_tr2(yt + yt_off[i], yt + yt_off[i] + 4 * (GT * 2));
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) a[step][i] = *reinterpret_cast<const vec*>(ya + i * 32 * GK * 2);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) b[step][j] = *reinterpret_cast<const vec*>(xa + j * 32 * GK * 2);
  };
  // half 0 / 1: the first / second half of the column tiles
  auto products = [&](int step, int half) {
#pragma unroll
    for (int i = half * NI / 2; i < (half + 1) * NI / 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = MfmaOp<InT>::run(a[step][i], b[step][j], acc[i][j]);
  };
  // Each chunk runs as two steps of 16 products. The wait, the barrier and
  // the next DMA issue sit between the steps, and each step's fragment reads
  // are issued halfway through the step before it: the LDS-DMA loads make
  // the compiler's waits before the products conservative (all LDS reads
  // done), so the reads must have completed by then anyway. Before chunk
  // kc + 1 is read, this wave's pieces of it have landed once at most the
  // later chunks already issued are outstanding, and the barrier makes every
  // wave's pieces visible; it also shows that every wave has read all of
  // chunk kc - 1, whose stage the issue refills.
  for (int c = 0; c < min(nk, G_NST - 1); ++c) issue(c, c);
  if (nk > 0) {
    wait_vm(min(nk - 1, G_NST - 2) * NPW);
    // a bare s_barrier: __syncthreads() would also drain every outstanding
    // load (vmcnt 0) and with it the ring's look-ahead
    asm volatile("s_barrier" ::: "memory");
    frags(0, 0);
  }
  for (int kc = 0; kc < nk; ++kc) {
    products(0, 0);
    __builtin_amdgcn_sched_barrier(0);
    frags(kc, 1);
    __builtin_amdgcn_sched_barrier(0);
    products(0, 1);
    __builtin_amdgcn_sched_barrier(0);
    const bool more = kc + 1 < nk;
    if (more) {
      wait_vm(min(nk - 2 - kc, G_NST - 3) * NPW);
      asm volatile("s_barrier" ::: "memory");
      if (kc + G_NST - 1 < nk) issue(kc + G_NST - 1, (kc + G_NST - 1) % G_NST);
    }
    products(1, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (more) frags(kc + 1, 0);
    __builtin_amdgcn_sched_barrier(0);
    products(1, 1);
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();   // every wave is done with the ring before it holds the output

  // acc[i][j] is D[m = c][n = r]: this lane holds output row
  // r0 + 128 wr + 32 j + lr, columns c0 + 32 NI wc + 32 i + 8 g + 4 lh + e.
  // fp32 results go straight from the accumulators as 16-byte stores; fp16
  // results are staged through LDS so that each global store is a full
  // 16-byte piece of a row. Only tiles on the bottom or right edge mask
  // (a uniform branch). Stores are streaming: the output is not read again
  // here and would otherwise evict operand rows other tiles still need.
  static_assert(sizeof(OutT) == 4 || __is_same(OutT, _Float16), "fp32 or fp16 output");
  constexpr int SH = GT + 8;   // fp16 staging pitch (elements)
  static_assert(GT * SH * 2 <= G_NST * G_STAGE, "output staging fits the ring");
  const int rlim = static_cast<int>(min<int64_t>(R - r0, GT));        // valid rows in the tile
  const int clim = static_cast<int>(min<int64_t>(C - c0, GT));
  const int rstore = static_cast<int>(min<int64_t>(R_store - r0, GT));
  const int cstore = static_cast<int>(min<int64_t>(C_store - c0, GT));
  const bool edge = !kPart && (rlim < GT || clim < GT || rstore < GT || cstore < GT);
  auto tile_val = [&](int i, int j, int g, int rt, int ct, bool masked) {
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = (!masked || (rt < rlim && ct + e < clim)) ? acc[i][j][4 * g + e] : 0.f;
    return v;
  };
  if constexpr (sizeof(OutT) == 4 || kPart) {
    const int64_t PR = static_cast<int64_t>(n_tr) * GT, PC = static_cast<int64_t>(n_tc) * GT;
    // fp32 results times *alpha when given (split-K: in the reduction)
    const float am = !kPart && alpha != nullptr ? alpha[0] : 1.f;
    auto put = [&](bool masked) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int rt = wr * 128 + 32 * j + lr, ct = wc * 32 * NI + 32 * i + 8 * g + 4 * lh;
            const f32x4 v = tile_val(i, j, g, rt, ct, masked) * am;
            const int64_t r = r0 + rt, c = c0 + ct;
            if constexpr (kPart) {
              __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(part + (blockIdx.y * PR + r) * PC + c));
            } else if (rt < rstore && ct < cstore) {
              __builtin_nontemporal_store(
                  v, reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + (r / 128) * rt_stride +
                                              (r % 128) * ldo + (c / 128) * ct_stride + c % 128));
            }
          }
    };
    if (edge) put(true);
    else put(false);
  } else {
    _Float16* sth = reinterpret_cast<_Float16*>(smem);
    auto stage = [&](bool masked) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int rt = wr * 128 + 32 * j + lr, ct = wc * 32 * NI + 32 * i + 8 * g + 4 * lh;
            const f32x4 v = tile_val(i, j, g, rt, ct, masked);
            const half4 hv = {static_cast<_Float16>(v[0]), static_cast<_Float16>(v[1]),
                              static_cast<_Float16>(v[2]), static_cast<_Float16>(v[3])};
            *reinterpret_cast<half4*>(sth + rt * SH + ct) = hv;
          }
    };
    if (edge) stage(true);
    else stage(false);
    __syncthreads();
    // Thread tid copies the 16-byte piece at column ct = 8 (tid % 32) of
    // tile rows rt = tid / 32 + 16 s, s = 0 .. 15. Tiles start at multiples
    // of 256 rows and columns, so in the tiled output layout the column part
    // of the offset is fixed per thread, and the row part is the thread's
    // first row plus a wave-uniform step (rows 128 and on are in the next
    // 128-row block). All pieces are read before the first store.
    constexpr int NS = GT * (GT / 8) / (kW * 64);   // 16 pieces per thread
    static_assert(GT == 256 && GT % 128 == 0 && NS * kW * 64 == GT * (GT / 8) && NS == 16,
                  "copy-out pattern");
    const int ct = (tid & 31) * 8, rt0 = tid >> 5;
    OutT* const lane_out = out + (r0 / 128) * rt_stride + (c0 / 128 + ct / 128) * ct_stride +
                           (ct % 128) + static_cast<int64_t>(rt0) * ldo;
    u32x4 piece[NS];
#pragma unroll
    for (int q = 0; q < NS; ++q) piece[q] = *reinterpret_cast<const u32x4*>(sth + (rt0 + 16 * q) * SH + ct);
#pragma unroll
    for (int q = 0; q < NS; ++q) {
      const int64_t step = (q >= 8 ? rt_stride : 0) + static_cast<int64_t>(16 * (q & 7)) * ldo;
      if (!edge || (rt0 + 16 * q < rstore && ct < cstore))
        __builtin_nontemporal_store(piece[q], reinterpret_cast<u32x4*>(lane_out + step));
    }
  }
}

// Longest-processing-time order of the attention work tiles of a packed
// (varlen) call, one workgroup of 1024 threads. A query tile holds 256 rows;
// its cost is the number of (row, key) pairs its rows see, sum over rows of
// p - seg_lo(p) + 1 (p the row's position). A key tile holds 128 workspace
// keys; its cost is the number of rows that see each key k (global
// key_lo + t): rows with k <= p < end of k's sample.
// qorder / korder receive the tile indices by decreasing cost (ties: later
// query tiles first, earlier key tiles first); korder may be null.
__global__ void __launch_bounds__(1024)
tile_order_kernel(const int32_t* __restrict__ cu, int n_seqs, int S_loc, RowMap rm, int key_lo,
                  int Kn, int n_qt, int n_kt, int* __restrict__ qorder, int* __restrict__ korder) {
  __shared__ unsigned long long cq[kMaxOrderTiles], ck[kMaxOrderTiles];
  const int tid = threadIdx.x;
  for (int t = tid; t < n_qt; t += 1024) cq[t] = 0;
  for (int t = tid; t < n_kt; t += 1024) ck[t] = 0;
  __syncthreads();
  for (int i = tid; i < S_loc; i += 1024) {
    const int pos = rm_pos(rm, i);
    atomicAdd(&cq[i >> 8], static_cast<unsigned long long>(pos - seg_lo_dev(cu, n_seqs, pos) + 1));
  }
  if (korder != nullptr) {
    for (int t = tid; t < Kn; t += 1024) {
      const int k = key_lo + t;
      // end of k's sample: the first sample start after k (the latent end if none)
      int lo_i = 0, hi_i = n_seqs + 1;
      while (hi_i - lo_i > 1) {
        const int mid = (lo_i + hi_i) >> 1;
        if (cu[mid] <= k) lo_i = mid; else hi_i = mid;
      }
      const int end = lo_i + 1 <= n_seqs ? cu[lo_i + 1] : 0x7fffffff;
      const int seen = rm_rows_below(rm, end) - rm_rows_below(rm, k);
      if (seen > 0) atomicAdd(&ck[t >> 7], static_cast<unsigned long long>(seen));
    }
  }
  __syncthreads();
  for (int t = tid; t < n_qt; t += 1024) {
    int r = 0;
    for (int u = 0; u < n_qt; ++u) r += cq[u] > cq[t] || (cq[u] == cq[t] && u > t);
    qorder[r] = t;
  }
  if (korder != nullptr)
    for (int t = tid; t < n_kt; t += 1024) {
      int r = 0;
      for (int u = 0; u < n_kt; ++u) r += ck[u] > ck[t] || (ck[u] == ck[t] && u < t);
      korder[r] = t;
    }
}

// out(r, c) = alpha sum_z part[z][r][c] for r < R_store, c < C_store (0 past
// R or C), in the tiled layout of launch_gemm_nt; four columns per thread,
// the splits summed in order (deterministic). alpha = *alpha_p, or 1 when
// alpha_p is null.
// Grid: x over groups of 1024 columns (256 threads x 4), y over rows with a
// grid-stride loop; a row's place in the tiled layout is worked out once per
// row, a column's once per thread.
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float* __restrict__ part, int splits, int64_t PR, int64_t PC,
                     float* __restrict__ out, int64_t ldo, int64_t rt_stride, int64_t ct_stride,
                     int64_t R, int64_t C, int64_t R_store, int64_t C_store,
                     const float* __restrict__ alpha_p) {
  const float alpha = alpha_p != nullptr ? alpha_p[0] : 1.f;
  const int64_t c = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (c >= C_store) return;
  const int64_t col_off = (c / 128) * ct_stride + c % 128;
  for (int64_t r = blockIdx.y; r < R_store; r += gridDim.y) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int z = 0; z < splits; ++z) acc += *reinterpret_cast<const f32x4*>(part + (z * PR + r) * PC + c);
    acc *= alpha;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (r >= R || c + q >= C) acc[q] = 0.f;
    *reinterpret_cast<f32x4*>(out + (r / 128) * rt_stride + (r % 128) * ldo + col_off) = acc;
  }
}

int gemm_splits(int64_t R_store, int64_t C_store, int64_t K) {
  const int64_t tiles = ((R_store + GT - 1) / GT) * ((C_store + GT - 1) / GT);
  int s = 1;
  while (tiles * s < G_MIN_BLOCKS && s < 8 && K % (2 * s * GK) == 0 && K / (2 * s) >= 8 * GK) s *= 2;
  return s;
}

// Eight bf16 values as OutT (fp16 converted, raw 16-bit copied).
template <typename OutT>
__device__ __forceinline__ u32x4 from_bf16x8(u32x4 v) {
  if constexpr (__is_same(OutT, uint16_t)) {
    return v;
  } else {
    return __builtin_bit_cast(u32x4, bf16x8_to_half8(v));
  }
}

// Transpose through a 64x64 LDS tile (grid: cols / 64, rows / 64, batch)
// with 16-byte accesses: a thread loads 8 consecutive columns of a row, then
// stores 8 consecutive rows of a column, so a wave instruction moves eight
// full 128-byte row segments each way. cols % 64 == 0, rows % 8 == 0, leading
// dimensions and batch strides multiples of 8, 16-byte aligned bases; rows
// from rows_valid on read as zero.
template <typename OutT>
__global__ void __launch_bounds__(256)
transpose_v_kernel(const uint16_t* __restrict__ in, int64_t ld_in, int64_t in_batch,
                   int64_t rows_valid, int64_t rows, OutT* __restrict__ out, int64_t ld_out,
                   int64_t out_batch) {
  __shared__ __attribute__((aligned(16))) uint16_t t[64][72];   // 144-byte rows
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * 64;
  in += blockIdx.z * in_batch + c0;
  out += blockIdx.z * out_batch + r0;
  const int a = threadIdx.x >> 3, b = (threadIdx.x & 7) * 8;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int rr = a + 32 * it;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r0 + rr < rows_valid) v = *reinterpret_cast<const u32x4*>(in + (r0 + rr) * ld_in + b);
    *reinterpret_cast<u32x4*>(&t[rr][b]) = v;
  }
  __syncthreads();
  if (r0 + b >= rows) return;   // whole 8-row pieces (rows % 8 == 0)
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int cc = a + 32 * it;
    u32x4 v;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      v[k] = static_cast<uint32_t>(t[b + 2 * k][cc]) | (static_cast<uint32_t>(t[b + 2 * k + 1][cc]) << 16);
    *reinterpret_cast<u32x4*>(out + (c0 + cc) * ld_out + b) = from_bf16x8<OutT>(v);
  }
}

// Row-wise conversion with 16-byte accesses: grid x over groups of 2048
// columns (256 threads x 8), y over rows with a grid-stride loop. cols,
// leading dimensions and batch strides multiples of 8, 16-byte aligned bases.
template <typename OutT>
__global__ void __launch_bounds__(256)
convert_v_kernel(const uint16_t* __restrict__ in, int64_t ld_in, int64_t in_batch,
                 int64_t rows_valid, int64_t rows, int64_t cols, OutT* __restrict__ out,
                 int64_t ld_out, int64_t out_batch) {
  const int64_t c = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (c >= cols) return;
  in += blockIdx.z * in_batch + c;
  out += blockIdx.z * out_batch + c;
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < rows_valid) v = from_bf16x8<OutT>(*reinterpret_cast<const u32x4*>(in + r * ld_in));
    *reinterpret_cast<u32x4*>(out + r * ld_out) = v;
  }
}

// out[b][r][0..cols) = fp16(in[r][0..cols)) for r < rows_valid, 0 for
// rows_valid <= r < rows; b < batch (out advanced by out_batch). A thread
// converts one 16-byte piece of a row once and writes it to the batch
// entries b = blockIdx.y, blockIdx.y + gridDim.y, ...; cols, ld_in and
// ld_out multiples of 8, rows * cols / 8 below 2^31.
__global__ void __launch_bounds__(256)
broadcast_rows_f16_kernel(const uint16_t* __restrict__ in, int64_t ld_in, int64_t rows_valid,
                          int64_t rows, int cols, _Float16* __restrict__ out, int64_t ld_out,
                          int64_t out_batch, int batch) {
  const int cpr = cols / 8;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= rows * cpr) return;
  const int r = e / cpr, c = e - r * cpr;
  half8 v;
  if (r < rows_valid) {
    v = bf16x8_to_half8(*reinterpret_cast<const u32x4*>(in + r * ld_in + c * 8));
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = static_cast<_Float16>(0.f);
  }
  _Float16* o = out + r * ld_out + c * 8;
  for (int b = blockIdx.y; b < batch; b += gridDim.y)
    *reinterpret_cast<half8*>(o + b * out_batch) = v;
}

}  // namespace

mla_status launch_broadcast_rows_f16(const uint16_t* in, int64_t ld_in, int64_t rows_valid,
                                     int64_t rows, int cols, _Float16* out, int64_t ld_out,
                                     int64_t out_batch, int batch, hipStream_t st,
                                     const char* name) {
  if (cols % 8 || ld_in % 8 || ld_out % 8 || out_batch % 8)
    return fail(MLA_ERR_UNSUPPORTED, "%s: widths must be multiples of 8", name);
  const int64_t pieces = rows * (cols / 8);
  if (pieces >= (int64_t(1) << 31)) return fail(MLA_ERR_UNSUPPORTED, "%s: too many rows", name);
  if (pieces == 0 || batch <= 0) return MLA_OK;
  const unsigned gx = static_cast<unsigned>((pieces + 255) / 256);
  // about 16 batch entries per thread, at least 2048 workgroups when there are that many
  unsigned gy = static_cast<unsigned>((batch + 15) / 16);
  while (gy < static_cast<unsigned>(batch) && static_cast<int64_t>(gx) * gy < 2048) gy *= 2;
  gy = std::min<unsigned>(gy, static_cast<unsigned>(batch));
  KernelTimer kt(name, st);
  hipLaunchKernelGGL(broadcast_rows_f16_kernel, dim3(gx, gy), dim3(256), 0, st, in, ld_in,
                     rows_valid, rows, cols, out, ld_out, out_batch, batch);
  return check_launch(name);
}

static bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

mla_status launch_transpose(const uint16_t* in, int64_t ld_in, int64_t in_batch, int64_t rows_valid,
                            int64_t rows, int64_t cols, void* out, int64_t ld_out,
                            int64_t out_batch, Elem out_t, int batch, hipStream_t st,
                            const char* name) {
  dim3 grid(static_cast<unsigned>((cols + 63) / 64), static_cast<unsigned>((rows + 63) / 64),
            static_cast<unsigned>(batch));
  // every caller passes 64-multiple widths and 16-byte aligned buffers (the
  // fast path's shape checks guarantee them)
  if (cols % 64 != 0 || rows % 8 != 0 || ld_in % 8 != 0 || ld_out % 8 != 0 || in_batch % 8 != 0 ||
      out_batch % 8 != 0 || !al16(in) || !al16(out))
    return fail(MLA_ERR_UNSUPPORTED, "%s: transpose needs 64-column and 8-row multiples, 16-byte alignment", name);
  KernelTimer kt(name, st);
  if (out_t == Elem::F16)
    hipLaunchKernelGGL(transpose_v_kernel<_Float16>, grid, dim3(256), 0, st, in, ld_in, in_batch,
                       rows_valid, rows, static_cast<_Float16*>(out), ld_out, out_batch);
  else
    hipLaunchKernelGGL(transpose_v_kernel<uint16_t>, grid, dim3(256), 0, st, in, ld_in, in_batch,
                       rows_valid, rows, static_cast<uint16_t*>(out), ld_out, out_batch);
  return check_launch(name);
}

mla_status launch_convert(const uint16_t* in, int64_t ld_in, int64_t in_batch, int64_t rows_valid,
                          int64_t rows, int64_t cols, void* out, int64_t ld_out, int64_t out_batch,
                          Elem out_t, int batch, hipStream_t st, const char* name) {
  if (cols % 8 != 0 || ld_in % 8 != 0 || ld_out % 8 != 0 || in_batch % 8 != 0 || out_batch % 8 != 0 ||
      !al16(in) || !al16(out))
    return fail(MLA_ERR_UNSUPPORTED, "%s: conversion needs 8-element multiples, 16-byte alignment", name);
  if (rows <= 0 || cols <= 0) return MLA_OK;
  KernelTimer kt(name, st);
  const dim3 grid(static_cast<unsigned>((cols / 8 + 255) / 256),
                  static_cast<unsigned>(std::min<int64_t>(rows, 65535)), static_cast<unsigned>(batch));
  if (out_t == Elem::F16)
    hipLaunchKernelGGL(convert_v_kernel<_Float16>, grid, dim3(256), 0, st, in, ld_in, in_batch,
                       rows_valid, rows, cols, static_cast<_Float16*>(out), ld_out, out_batch);
  else
    hipLaunchKernelGGL(convert_v_kernel<uint16_t>, grid, dim3(256), 0, st, in, ld_in, in_batch,
                       rows_valid, rows, cols, static_cast<uint16_t*>(out), ld_out, out_batch);
  return check_launch(name);
}

mla_status launch_tile_order(const int32_t* cu, int n_seqs, int64_t S_loc, const RowMap& rm,
                             int64_t key_lo, int64_t Kn, int n_qt, int n_kt, int* qorder,
                             int* korder, hipStream_t st) {
  if (n_qt > kMaxOrderTiles || n_kt > kMaxOrderTiles)
    return fail(MLA_ERR_UNSUPPORTED, "tile order: more than %d tiles", kMaxOrderTiles);
  KernelTimer kt("tile_order", st);
  hipLaunchKernelGGL(tile_order_kernel, dim3(1), dim3(1024), 0, st, cu, n_seqs,
                     static_cast<int>(S_loc), rm, static_cast<int>(key_lo),
                     static_cast<int>(Kn), n_qt, n_kt, qorder, korder);
  return check_launch("tile order");
}

int64_t gemm_splitk_bytes(int64_t R_store, int64_t C_store, int64_t K) {
  const int sp = gemm_splits(R_store, C_store, K);
  if (sp == 1) return 0;
  return static_cast<int64_t>(sp) * ((R_store + GT - 1) / GT) * GT * ((C_store + GT - 1) / GT) * GT * 4;
}

mla_status launch_gemm_nt(const void* X, int64_t ldx, int64_t R, const void* Y, int64_t ldy,
                          int64_t C, int64_t K, void* out, int64_t ldo, int64_t rt_stride,
                          int64_t ct_stride, int64_t R_store, int64_t C_store, Elem in_t,
                          Elem out_t, hipStream_t st, const char* name, float* part,
                          int64_t part_bytes, const float* alpha, bool y_kmajor) {
  if (y_kmajor && (in_t != Elem::F16 || out_t != Elem::F32 || C % 8 != 0))
    return fail(MLA_ERR_UNSUPPORTED, "%s: k-major Y takes fp16 in, fp32 out, C a multiple of 8", name);
  if (K % GK != 0) return fail(MLA_ERR_UNSUPPORTED, "%s: K=%lld not a multiple of 32", name, (long long)K);
  if (C_store % 8 != 0) return fail(MLA_ERR_UNSUPPORTED, "%s: C_store not a multiple of 8", name);
  const int64_t n_tr = (R_store + GT - 1) / GT, n_tc = (C_store + GT - 1) / GT;
  // every tile must hold a valid row of X and of Y (loads clamp to them)
  if (R > 0 && C > 0 && (n_tr != (R + GT - 1) / GT || n_tc != (C + GT - 1) / GT))
    return fail(MLA_ERR_UNSUPPORTED, "%s: stored extent reaches a tile past the operands", name);
  // (lane offsets within a 256-row tile stay below 2^31 bytes)
  if (ldx >= (int64_t(1) << 22) || ldy >= (int64_t(1) << 22) || n_tr * n_tc >= (int64_t(1) << 31))
    return fail(MLA_ERR_UNSUPPORTED, "%s: operand too wide", name);
  int sp = out_t == Elem::F32 ? gemm_splits(R_store, C_store, K) : 1;
  if (sp > 1 && (part == nullptr || part_bytes < gemm_splitk_bytes(R_store, C_store, K))) sp = 1;
  dim3 grid(static_cast<unsigned>(n_tr * n_tc), static_cast<unsigned>(sp));
  float* pp = sp > 1 ? part : nullptr;
  const int64_t kl = K / sp;
  const int ntr = static_cast<int>(n_tr), ntc = static_cast<int>(n_tc);
  KernelTimer kt(name, st);
  // k-major Y first: the other branches read Y k-contiguous
  if (y_kmajor && sp == 1)
    hipLaunchKernelGGL((gemm_nt_kernel<_Float16, float, false, 8, true>), grid, dim3(512), 0, st,
                       static_cast<const _Float16*>(X), ldx, R, static_cast<const _Float16*>(Y),
                       ldy, C, kl, static_cast<float*>(out), ldo, rt_stride, ct_stride, R_store,
                       C_store, nullptr, alpha, ntr, ntc);
  else if (y_kmajor)
    hipLaunchKernelGGL((gemm_nt_kernel<_Float16, float, true, 8, true>), grid, dim3(512), 0, st,
                       static_cast<const _Float16*>(X), ldx, R, static_cast<const _Float16*>(Y),
                       ldy, C, kl, static_cast<float*>(nullptr), ldo, rt_stride, ct_stride,
                       R_store, C_store, pp, nullptr, ntr, ntc);
  else if (in_t == Elem::BF16 && out_t == Elem::F16 && sp == 1)
    hipLaunchKernelGGL((gemm_nt_kernel<__bf16, _Float16, false, 8>), grid, dim3(512), 0, st,
                       static_cast<const __bf16*>(X), ldx, R, static_cast<const __bf16*>(Y), ldy,
                       C, kl, static_cast<_Float16*>(out), ldo, rt_stride, ct_stride, R_store,
                       C_store, nullptr, nullptr, ntr, ntc);
  else if (in_t == Elem::F16 && out_t == Elem::F32 && sp == 1)
    hipLaunchKernelGGL((gemm_nt_kernel<_Float16, float, false, 8>), grid, dim3(512), 0, st,
                       static_cast<const _Float16*>(X), ldx, R, static_cast<const _Float16*>(Y),
                       ldy, C, kl, static_cast<float*>(out), ldo, rt_stride, ct_stride, R_store,
                       C_store, nullptr, alpha, ntr, ntc);
  else if (in_t == Elem::F16 && out_t == Elem::F32)
    hipLaunchKernelGGL((gemm_nt_kernel<_Float16, float, true, 8>), grid, dim3(512), 0, st,
                       static_cast<const _Float16*>(X), ldx, R, static_cast<const _Float16*>(Y),
                       ldy, C, kl, static_cast<float*>(nullptr), ldo, rt_stride, ct_stride,
                       R_store, C_store, pp, nullptr, ntr, ntc);
  else if (in_t == Elem::F16 && out_t == Elem::F16 && sp == 1)
    hipLaunchKernelGGL((gemm_nt_kernel<_Float16, _Float16, false, 8>), grid, dim3(512), 0, st,
                       static_cast<const _Float16*>(X), ldx, R, static_cast<const _Float16*>(Y),
                       ldy, C, kl, static_cast<_Float16*>(out), ldo, rt_stride, ct_stride, R_store,
                       C_store, nullptr, nullptr, ntr, ntc);
  else
    return fail(MLA_ERR_UNSUPPORTED, "%s: GEMM type combination not built", name);
  if (sp > 1) {
    const unsigned gx = static_cast<unsigned>((C_store / 4 + 255) / 256);
    const unsigned gy = static_cast<unsigned>(std::min<int64_t>(R_store, 65535));
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(gx, gy), dim3(256), 0, st, part, sp, n_tr * GT,
                       n_tc * GT, static_cast<float*>(out), ldo, rt_stride, ct_stride, R, C,
                       R_store, C_store, alpha);
  }
  return check_launch(name);
}

}  // namespace mla
