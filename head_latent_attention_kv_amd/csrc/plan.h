// Host-side call plan shared by the C ABI and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "device_common.h"
#include "mla_laga.h"

namespace mla {

constexpr int64_t kAlign = 256;
inline int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Fast-path tile sizes (MFMA kernels).
constexpr int kFastDNope = 128;
constexpr int kFastDV = 128;
constexpr int kFastDRope = 64;
constexpr int kKeyTile = 256;  // key tile of the backward's key-outer kernels; rebuilt-K/V rows are padded to it

struct Plan {
  int n_h, d_c, d_rope, d_nope, d_v, d_qk, n_seqs;
  int64_t S, S_loc, q_offset;
  RowMap rm;      // local row -> global position (the non-empty position blocks)
  bool bf16;
  bool fast;      // forward runs the MFMA path
  bool fast_bwd;  // backward runs the MFMA path
  bool ds_store;  // fast backward: dK/dV stores dS, dQ reads it (no recompute)
  int ds_heads;   // stored dS: heads per group (a buffer holds one group)
  float scale;
  // latent rows the shard needs: [key_lo, key_hi), Kn of them
  int64_t key_lo, key_hi, Kn, Kpad;
  int64_t visible_pairs;
};

// Byte offsets of the workspace regions for one call.
struct FwdLayout {
  // plain fp32 path
  int64_t K, V;
  // fast path: [W_UK | W_UV]^T bf16, keys [n_h][Kpad][192] fp16, V^T [n_h][128][Kpad] fp16
  int64_t WT, Kfull, Vt;
  int64_t order;  // fast path, packed calls: query-tile order (int32 [ceil(S_loc / 256)])
  int64_t total;
};
struct BwdLayout {
  FwdLayout f;  // plain path: K, V; fast path: WT, Kfull (Vt unused)
  // plain path: D [S_loc][n_h], dK/dV fp32 [n_h][Kn][.]
  // fast path:  D [n_h][S_pad], dK = [dK_nope | dV] fp16 [Kpad][2*n_h*128]
  //             (dV unused), dKrope fp32 [n_h][Kpad][64]
  int64_t D, dK, dV, dKrope;
  // fast path only (fp16): V key-major [n_h][Kpad][128], [W_UK | W_UV]
  // [d_c][2*n_h*128], c_kv^T [d_c][Kpad], q and dout per head [n_h][S_pad][.]
  // (the kernels read the transposes of K, q and dout from these row-major
  // tiles with transposed LDS reads)
  int64_t Vkm, W16, ckvT, Qn, dOn;
  int64_t info;  // fast path: per 32-row block {lse*log2e - 15, D, sample start, position} x 32
  int64_t gpart;  // fast path: split-K partial sums of the gradient GEMMs (fp32)
  // fast path, packed calls: query-tile then key-tile order (int32
  // [ceil(S_loc / 256) + Kpad / 128])
  int64_t order;
  // fast path with stored dS: one or (more than one group) two buffers, each
  // fp16 [ds_heads][Kpad / 128][S_pad / 32] blocks of 8 KiB ([4 pairs of 32
  // keys][2 row halves][64 lanes] x 16 bytes, written by dK/dV)
  int64_t dS;
  // fast path: dout scale {2^e, 2^-e} (fp32), then the per-block maxima of
  // |dout| it is chosen from (kScaleBlocks uint32), then per head the
  // largest |2^e dout row| and |D| (2 n_h floats)
  int64_t dscale;
  int64_t total;
};

// Stored dS of the fast backward: all heads in one buffer while that holds at
// most kStoredDsOneBufferBytes; past that, head groups of at most
// kStoredDsGroupBytes each through two buffers (bytes), when a group holds at
// least kStoredDsMinGroupHeads heads (fewer, and the groups' launches cost
// more than recomputing dQ saves).
constexpr int64_t kStoredDsOneBufferBytes = int64_t(16) << 30;
constexpr int64_t kStoredDsGroupBytes = int64_t(1) << 30;
constexpr int kStoredDsMinGroupHeads = 8;
// Workgroups of the fast backward's max|dout| reduction.
constexpr int kScaleBlocks = 1024;

// Decode (absorbed form over the latent cache): one query per sequence.
struct DecodePlan {
  int n_h, batch;
  int64_t S;          // cache rows over all sequences
  float scale;
  int chunk;          // keys per split-KV workgroup (a multiple of 32)
  int nch;            // chunks of the longest sequence
  int64_t total_keys;
};
struct DecodeLayout {
  // W_UV^T fp16 [n_h*128][512]; q_lat, o_lat fp16 [batch][n_h][512];
  // per-chunk partials fp16 [batch][nch][n_h][512] and (max, sum) [batch][nch][n_h]
  int64_t WTv, qlat, olat, opart, ml;
  int64_t total;
};
DecodeLayout decode_layout(const DecodePlan& p);
// Bytes of the library's static decode scratch (one array per GPU).
constexpr int64_t kDecodeScratchBytes = MLA_DECODE_NOALLOC_MAX_BYTES;
// Device address of that scratch on the current device (looked up once per
// device).
mla_status decode_scratch(char** ptr);

FwdLayout fwd_layout(const Plan& p, bool fast);
inline FwdLayout fwd_layout(const Plan& p) { return fwd_layout(p, p.fast); }
BwdLayout bwd_layout(const Plan& p);

// ---- debug mode (debug.hip)
// Bytes after the used workspace that debug mode takes for its canary and
// check slots; the *_workspace_size results include them in that mode.
constexpr int64_t kDebugTailBytes = 256;
struct DebugOutput {
  void* ptr;
  int64_t n;         // fp32 elements
  const char* name;
};
// MLA_LAGA_DEBUG is set (and not "0"); read at every call.
bool debug_mode();
inline int64_t debug_tail() { return debug_mode() ? kDebugTailBytes : 0; }
// Compare cu_dev with cu_host (n_cu values; skipped when either is null),
// fill ws[0, ws_used) and the outputs with all-ones bytes and write the
// canary and check slots at ws + ws_used. Waits for `st`.
mla_status debug_begin(const int32_t* cu_host, const int32_t* cu_dev, int n_cu, char* ws,
                       int64_t ws_used, const DebugOutput* outs, int n_out, hipStream_t st);
// Scan the outputs for NaN, check the canary; waits for `st`.
mla_status debug_end(char* ws, int64_t ws_used, const DebugOutput* outs, int n_out, hipStream_t st);
// Per local row, the inclusive window {lo, hi} of global key positions.
mla_status launch_row_window(const Plan& p, const int32_t* cu_dev, int64_t* window, hipStream_t st);

// Set the thread's last-error message and return `s`.
mla_status fail(mla_status s, const char* fmt, ...);
mla_status check_launch(const char* what);

// Brackets one kernel launch with HIP events on `st` while timing is on.
class KernelTimer {
 public:
  KernelTimer(const char* name, hipStream_t st);
  ~KernelTimer();
  KernelTimer(const KernelTimer&) = delete;
  KernelTimer& operator=(const KernelTimer&) = delete;

 private:
  int slot_ = -1;
  hipStream_t st_;
};

// A second stream on the current device, with a fork and a join event,
// created once per host thread and device (default priority). Work that
// depends only on what the caller's stream has already been given runs there:
// fork() makes it wait for the caller's stream so far, join() makes the
// caller's stream wait for everything given to it so far. From the caller's
// side the call still behaves as if all its work were on the caller's stream.
struct SideStream {
  hipStream_t st = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  hipEvent_t buf_free[2] = {nullptr, nullptr};  // side-stream marks for double-buffered work
};
mla_status side_stream(SideStream* out);
mla_status side_fork(const SideStream& s, hipStream_t main);
mla_status side_join(const SideStream& s, hipStream_t main);
// Joins the side stream back into the caller's on every way out once the
// fork has succeeded, error returns included.
class SideFork {
 public:
  SideFork(const SideStream& s, hipStream_t main) : s_(s), main_(main) {}
  ~SideFork() {
    if (forked_) (void)side_join(s_, main_);
  }
  SideFork(const SideFork&) = delete;
  SideFork& operator=(const SideFork&) = delete;
  mla_status fork() {
    const mla_status r = side_fork(s_, main_);
    forked_ = r == MLA_OK;
    return r;
  }
  mla_status join() {
    forked_ = false;
    return side_join(s_, main_);
  }

 private:
  SideStream s_;
  hipStream_t main_;
  bool forked_ = false;
};

// Segment start of global position p (host version; device twin in kernels).
inline int64_t seg_lo_host(const int32_t* cu, int n_seqs, int64_t p) {
  if (n_seqs == 0 || cu == nullptr) return 0;
  // last k with cu[k] <= p  (upper_bound - 1); skips empty samples
  int lo = 0, hi = n_seqs + 1;  // search in cu[0..n_seqs]
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (cu[mid] <= p) lo = mid; else hi = mid;
  }
  return cu[lo];
}

// ---- plain fp32 path (generic.hip)
mla_status generic_fwd(const Plan& p, const void* q, const void* c_kv, const void* k_rope,
                       const void* W_UK, const void* W_UV, const int32_t* cu_dev, float* out,
                       float* lse, char* ws, hipStream_t st);
mla_status generic_bwd(const Plan& p, const void* dout, const void* q, const void* c_kv,
                       const void* k_rope, const void* W_UK, const void* W_UV,
                       const int32_t* cu_dev, const float* out, const float* lse, float* dq,
                       float* dc_kv, float* dk_rope, float* dW_UK, float* dW_UV, char* ws,
                       hipStream_t st);
mla_status zero_fill(float* p, int64_t n, hipStream_t st);

// ---- fast path (fast_*.hip)
// Bytes of fp32 partial sums launch_gemm_nt uses to split K for an fp32
// output of R_store x C_store (0 when it does not split).
int64_t gemm_splitk_bytes(int64_t R_store, int64_t C_store, int64_t K);
// The fast path's size limits (32-bit element offsets inside the kernels and
// the GEMM operand limits), checked by the workspace queries and again by
// the launchers before anything is enqueued: MLA_ERR_UNSUPPORTED past them.
mla_status fast_fwd_limits(const Plan& p);
mla_status fast_bwd_limits(const Plan& p);
mla_status fast_fwd(const Plan& p, const void* q, const void* c_kv, const void* k_rope,
                    const void* W_UK, const void* W_UV, const int32_t* cu_dev, float* out,
                    float* lse, char* ws, hipStream_t st);
// side: a stream forked from st for the rope-key copy into Kfull, which
// runs beside the GEMMs (st itself when null)
mla_status fast_rebuild_kv(const Plan& p, const void* c_kv, const void* k_rope, const void* W_UK,
                           const void* W_UV, uint16_t* WT, _Float16* Kfull, _Float16* Vt,
                           _Float16* Vkm, hipStream_t st, hipStream_t side,
                           const SideStream* vside = nullptr);
mla_status fast_decode(const DecodePlan& p, const void* q, const void* c_kv, const void* k_rope,
                       const void* W_UK, const void* W_UV, const int32_t* cu_dev, float* out,
                       float* lse, char* ws, hipStream_t st);
mla_status fast_bwd(const Plan& p, const void* dout, const void* q, const void* c_kv,
                    const void* k_rope, const void* W_UK, const void* W_UV,
                    const int32_t* cu_dev, const float* out, const float* lse, float* dq,
                    float* dc_kv, float* dk_rope, float* dW_UK, float* dW_UV, char* ws,
                    hipStream_t st);

}  // namespace mla
