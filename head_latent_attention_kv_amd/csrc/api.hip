// C ABI: argument validation, the call plan, workspace layout and dispatch.
#include <stdlib.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "plan.h"

namespace mla {

namespace {
thread_local char g_last_error[512] = "";
}

mla_status fail(mla_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

mla_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return MLA_OK;
}

// ---------------------------------------------------------------- timing
namespace {
struct TimedLaunch {
  std::string name;
  hipEvent_t start, stop;
};
bool g_timing = false;
std::string g_select;   // ";name;name;" or empty (every kernel)
std::vector<TimedLaunch> g_launches;
std::vector<hipEvent_t> g_event_pool;
std::string g_names;

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void release_records() {
  for (auto& r : g_launches) {
    g_event_pool.push_back(r.start);
    g_event_pool.push_back(r.stop);
  }
  g_launches.clear();
}
}  // namespace

KernelTimer::KernelTimer(const char* name, hipStream_t st) : st_(st) {
  if (!g_timing) return;
  if (!g_select.empty() && g_select.find(";" + std::string(name) + ";") == std::string::npos) return;
  hipEvent_t a = take_event(), b = take_event();
  if (!a || !b) return;
  if (hipEventRecord(a, st) != hipSuccess) {
    g_event_pool.push_back(a);
    g_event_pool.push_back(b);
    return;
  }
  g_launches.push_back({name, a, b});
  slot_ = static_cast<int>(g_launches.size()) - 1;
}

KernelTimer::~KernelTimer() {
  // a start event without its stop makes the record unreadable: drop it
  if (slot_ >= 0 && hipEventRecord(g_launches[slot_].stop, st_) != hipSuccess)
    g_launches[slot_].name = "";
}

mla_status side_stream(SideStream* out) {
  constexpr int kMaxDevices = 64;
  thread_local SideStream per_dev[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(MLA_ERR_HIP, "no current device for the side stream");
  SideStream& s = per_dev[dev];
  if (s.st == nullptr) {
    SideStream n;
    if (hipStreamCreateWithFlags(&n.st, hipStreamNonBlocking) != hipSuccess)
      return fail(MLA_ERR_HIP, "hipStreamCreateWithFlags failed");
    hipEvent_t* evs[4] = {&n.fork, &n.join, &n.buf_free[0], &n.buf_free[1]};
    for (int i = 0; i < 4; ++i)
      if (hipEventCreateWithFlags(evs[i], hipEventDisableTiming) != hipSuccess) {
        for (int j = 0; j < i; ++j) (void)hipEventDestroy(*evs[j]);
        (void)hipStreamDestroy(n.st);
        return fail(MLA_ERR_HIP, "hipEventCreateWithFlags failed");
      }
    s = n;   // kept until the process ends
  }
  *out = s;
  return MLA_OK;
}

mla_status side_fork(const SideStream& s, hipStream_t main) {
  if (hipEventRecord(s.fork, main) != hipSuccess || hipStreamWaitEvent(s.st, s.fork, 0) != hipSuccess)
    return fail(MLA_ERR_HIP, "fork to the side stream failed");
  return MLA_OK;
}

mla_status side_join(const SideStream& s, hipStream_t main) {
  if (hipEventRecord(s.join, s.st) != hipSuccess || hipStreamWaitEvent(main, s.join, 0) != hipSuccess)
    return fail(MLA_ERR_HIP, "join from the side stream failed");
  return MLA_OK;
}

FwdLayout fwd_layout(const Plan& p, bool fast) {
  FwdLayout L{};
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    const int64_t o = off;
    off += align_up(bytes, kAlign);
    return o;
  };
  if (fast) {
    L.K = L.V = -1;
    L.WT = take(static_cast<int64_t>(p.n_h) * (p.d_nope + p.d_v) * p.d_c * 2);  // bf16
    L.Kfull = take(static_cast<int64_t>(p.n_h) * p.Kpad * p.d_qk * 2);         // fp16
    L.Vt = take(static_cast<int64_t>(p.n_h) * p.d_v * p.Kpad * 2);             // fp16
    L.order = take(4 * ((p.S_loc + 255) / 256));
  } else {
    L.WT = L.Kfull = L.Vt = L.order = -1;
    L.K = take(static_cast<int64_t>(p.n_h) * p.Kn * p.d_qk * 4);
    L.V = take(static_cast<int64_t>(p.n_h) * p.Kn * p.d_v * 4);
  }
  L.total = off;
  return L;
}

BwdLayout bwd_layout(const Plan& p) {
  BwdLayout L{};
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    const int64_t o = off;
    off += align_up(bytes, kAlign);
    return o;
  };
  L.Vkm = L.W16 = L.ckvT = L.Qn = L.dOn = L.info = L.gpart = L.order = -1;
  L.dS = L.dscale = -1;
  if (p.fast_bwd) {
    const int64_t nk = static_cast<int64_t>(p.n_h) * 128;
    const int64_t S_pad = align_up(p.S_loc, 64);
    L.f.K = L.f.V = L.f.Vt = L.f.order = -1;
    L.f.WT = take(2 * nk * p.d_c * 2);
    L.f.Kfull = take(p.n_h * p.Kpad * 192 * 2);
    L.Vkm = take(nk * p.Kpad * 2);
    L.W16 = take(static_cast<int64_t>(p.d_c) * 2 * nk * 2);
    L.ckvT = take(static_cast<int64_t>(p.d_c) * p.Kpad * 2);
    L.Qn = take(p.n_h * S_pad * 192 * 2);
    L.dOn = take(p.n_h * S_pad * 128 * 2);
    L.D = take(p.n_h * S_pad * 4);
    L.dK = take(p.Kpad * 2 * nk * 2);
    L.dV = -1;
    L.dKrope = take(p.n_h * p.Kpad * 64 * 4);
    L.info = take(p.n_h * S_pad * 16);
    L.gpart = take(std::max(gemm_splitk_bytes(p.Kn, p.d_c, 2 * nk),
                            gemm_splitk_bytes(p.d_c, nk, p.Kpad)));
    L.order = take(4 * ((p.S_loc + 255) / 256 + p.Kpad / 128));
    L.dscale = take(16 + 4 * kScaleBlocks + 8 * static_cast<int64_t>(p.n_h));
    if (p.ds_store)
      L.dS = take((p.ds_heads < p.n_h ? 2 : 1) * static_cast<int64_t>(p.ds_heads) * p.Kpad * S_pad * 2);
    L.f.total = -1;
  } else {
    L.f = fwd_layout(p, false);
    off = L.f.total;
    L.D = take(p.S_loc * p.n_h * 4);
    L.dK = take(static_cast<int64_t>(p.n_h) * p.Kn * p.d_qk * 4);
    L.dV = take(static_cast<int64_t>(p.n_h) * p.Kn * p.d_v * 4);
    L.dKrope = -1;
  }
  L.total = off;
  return L;
}

static bool fast_shape(const mla_laga_desc* d) {
  return d->in_dtype == MLA_BF16 && !(d->flags & MLA_FLAG_GENERIC) && d->d_nope == kFastDNope &&
         d->d_v == kFastDV && d->d_rope == kFastDRope && d->d_c % 64 == 0 && d->d_c >= 64 &&
         d->d_c <= 4096;
}

// Validate the descriptor (and host cu_seqlens) and fill the plan.
static mla_status make_plan(const mla_laga_desc* d, const int32_t* cu, Plan* p) {
  if (!d) return fail(MLA_ERR_INVALID_ARG, "desc is NULL");
  if (d->n_h < 1 || d->d_c < 1 || d->d_nope < 1 || d->d_v < 1 || d->d_rope < 0)
    return fail(MLA_ERR_INVALID_ARG, "dims must be positive (n_h=%d d_c=%d d_nope=%d d_v=%d d_rope=%d)",
                d->n_h, d->d_c, d->d_nope, d->d_v, d->d_rope);
  if (d->S < 1) return fail(MLA_ERR_INVALID_ARG, "S must be >= 1 (got %lld)", (long long)d->S);
  if (d->S_loc < 0) return fail(MLA_ERR_INVALID_ARG, "S_loc must be >= 0");
  if (d->q_offset < 0 || d->q_offset + d->S_loc > d->S)
    return fail(MLA_ERR_INVALID_ARG, "need 0 <= q_offset and q_offset + S_loc <= S (q_offset=%lld S_loc=%lld S=%lld)",
                (long long)d->q_offset, (long long)d->S_loc, (long long)d->S);
  if (d->S > INT32_MAX) return fail(MLA_ERR_UNSUPPORTED, "S above 2^31-1");
  if (d->in_dtype != MLA_F32 && d->in_dtype != MLA_BF16)
    return fail(MLA_ERR_INVALID_ARG, "in_dtype must be MLA_F32 or MLA_BF16");
  if (d->flags & ~(MLA_FLAG_GENERIC | MLA_FLAG_STORED_DS))
    return fail(MLA_ERR_INVALID_ARG, "unknown flag bits 0x%x",
                static_cast<unsigned>(d->flags & ~(MLA_FLAG_GENERIC | MLA_FLAG_STORED_DS)));
  if (d->n_seqs < 0) return fail(MLA_ERR_INVALID_ARG, "n_seqs must be >= 0");
  if (d->n_seqs > 0) {
    if (!cu) return fail(MLA_ERR_INVALID_ARG, "n_seqs > 0 needs cu_seqlens_host");
    if (cu[0] != 0 || cu[d->n_seqs] != d->S)
      return fail(MLA_ERR_INVALID_ARG, "cu_seqlens must start at 0 and end at S (got %d .. %d)",
                  cu[0], cu[d->n_seqs]);
    for (int k = 0; k < d->n_seqs; ++k)
      if (cu[k + 1] < cu[k])
        return fail(MLA_ERR_INVALID_ARG, "cu_seqlens decreases at index %d", k);
  }
  if (d->n_ranges < 0 || d->n_ranges > MLA_MAX_RANGES)
    return fail(MLA_ERR_INVALID_ARG, "n_ranges must be in [0, %d] (got %d)", MLA_MAX_RANGES,
                d->n_ranges);
  Plan& P = *p;
  P.rm = RowMap{};
  if (d->n_ranges == 0) {
    P.rm.n = 1;
    P.rm.row0[1] = static_cast<int>(d->S_loc);
    P.rm.pos0[0] = static_cast<int>(d->q_offset);
  } else {
    const int64_t* qr = d->q_ranges;
    if (!qr) return fail(MLA_ERR_INVALID_ARG, "n_ranges > 0 needs q_ranges");
    if (d->q_offset != 0) return fail(MLA_ERR_INVALID_ARG, "q_offset must be 0 when n_ranges > 0");
    int64_t rows = 0, prev_end = 0;
    P.rm.n = 0;
    for (int b = 0; b < d->n_ranges; ++b) {
      const int64_t a = qr[2 * b], n = qr[2 * b + 1];
      if (a < 0 || n < 0 || a + n > d->S)
        return fail(MLA_ERR_INVALID_ARG, "q_ranges[%d] = (%lld, %lld) is outside [0, S)", b,
                    (long long)a, (long long)n);
      if (b > 0 && a < prev_end)
        return fail(MLA_ERR_INVALID_ARG, "q_ranges must be ascending and disjoint (block %d starts at %lld, before %lld)",
                    b, (long long)a, (long long)prev_end);
      prev_end = a + n;
      if (n == 0) continue;
      P.rm.row0[P.rm.n] = static_cast<int>(rows);
      P.rm.pos0[P.rm.n] = static_cast<int>(a);
      ++P.rm.n;
      rows += n;
    }
    if (rows != d->S_loc)
      return fail(MLA_ERR_INVALID_ARG, "q_ranges hold %lld rows, S_loc is %lld", (long long)rows,
                  (long long)d->S_loc);
    P.rm.row0[P.rm.n] = static_cast<int>(rows);
    if (P.rm.n == 0) P.rm.n = 1;  // S_loc = 0: one empty block
  }
  P.n_h = d->n_h; P.d_c = d->d_c; P.d_rope = d->d_rope; P.d_nope = d->d_nope; P.d_v = d->d_v;
  P.d_qk = d->d_nope + d->d_rope; P.n_seqs = d->n_seqs;
  P.S = d->S; P.S_loc = d->S_loc; P.q_offset = d->q_offset;
  P.bf16 = d->in_dtype == MLA_BF16;
  P.fast = fast_shape(d);
  P.fast_bwd = P.fast;
  if (!P.fast_bwd && (P.d_qk > 256 || P.d_v > 256))
    return fail(MLA_ERR_UNSUPPORTED, "plain path takes d_nope+d_rope <= 256 and d_v <= 256");
  P.scale = d->softmax_scale > 0.f ? d->softmax_scale : 1.0f / sqrtf(static_cast<float>(P.d_qk));
  if (!(P.scale < INFINITY)) return fail(MLA_ERR_INVALID_ARG, "softmax_scale is not finite");
  if (P.S_loc > 0) {
    // positions increase with the row: the first row has the lowest sample
    // start, the last row the highest position
    P.key_lo = seg_lo_host(cu, P.n_seqs, rm_pos(P.rm, 0));
    P.key_hi = rm_pos(P.rm, static_cast<int>(P.S_loc - 1)) + 1;
  } else {
    P.key_lo = P.key_hi = 0;
  }
  P.Kn = P.key_hi - P.key_lo;
  P.Kpad = align_up(P.Kn, kKeyTile);
  // stored dS: every head in one buffer while it fits kStoredDsOneBufferBytes
  // (dQ then runs once, beside the gradient GEMMs); else head groups of at
  // most kStoredDsGroupBytes, as even as their count allows, if a group holds
  // at least kStoredDsMinGroupHeads heads; else dQ recomputes
  P.ds_store = false;
  P.ds_heads = 0;
  if (P.fast_bwd && (d->flags & MLA_FLAG_STORED_DS)) {
    const int64_t per_head = P.Kpad * align_up(P.S_loc, 64) * 2;
    if (P.n_h * per_head <= kStoredDsOneBufferBytes) {
      P.ds_store = true;
      P.ds_heads = P.n_h;
    } else if (per_head * kStoredDsMinGroupHeads <= kStoredDsGroupBytes) {
      const int64_t most = kStoredDsGroupBytes / per_head;   // heads per group, at most
      const int64_t groups = (P.n_h + most - 1) / most;
      P.ds_store = true;
      P.ds_heads = static_cast<int>((P.n_h + groups - 1) / groups);
    }
  }
  int64_t pairs = 0;
  for (int64_t i = 0; i < P.S_loc; ++i) {
    const int64_t pos = rm_pos(P.rm, static_cast<int>(i));
    pairs += pos - seg_lo_host(cu, P.n_seqs, pos) + 1;
  }
  P.visible_pairs = pairs;
  return MLA_OK;
}

static bool misaligned(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) != 0; }

// Validate a decode call and choose its split: chunks of keys sized so that
// the attention launch has about one workgroup per compute unit (measured
// best against 384 to 2048 workgroups on the 64 x 8192 and long-tailed
// batches).
static mla_status make_decode_plan(const mla_laga_decode_desc* d, const int32_t* cu, DecodePlan* p) {
  if (!d) return fail(MLA_ERR_INVALID_ARG, "desc is NULL");
  if (d->batch < 1) return fail(MLA_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", d->batch);
  if (d->n_h < 1 || d->d_c < 1 || d->d_nope < 1 || d->d_v < 1 || d->d_rope < 0)
    return fail(MLA_ERR_INVALID_ARG, "dims must be positive");
  if (d->S < 1 || d->S > INT32_MAX) return fail(MLA_ERR_INVALID_ARG, "S must be in [1, 2^31)");
  if (d->in_dtype != MLA_F32 && d->in_dtype != MLA_BF16)
    return fail(MLA_ERR_INVALID_ARG, "in_dtype must be MLA_F32 or MLA_BF16");
  if (!cu) return fail(MLA_ERR_INVALID_ARG, "decode needs cu_seqlens_host");
  if (cu[0] != 0 || cu[d->batch] != d->S)
    return fail(MLA_ERR_INVALID_ARG, "cu_seqlens must start at 0 and end at S (got %d .. %d)", cu[0],
                cu[d->batch]);
  int64_t longest = 0;
  for (int b = 0; b < d->batch; ++b) {
    if (cu[b + 1] <= cu[b])
      return fail(MLA_ERR_INVALID_ARG, "sequence %d has no cached row (cu_seqlens must increase)", b);
    longest = std::max<int64_t>(longest, cu[b + 1] - cu[b]);
  }
  if (d->in_dtype != MLA_BF16 || d->d_c != 512 || d->d_rope != 64 || d->d_nope != 128 ||
      d->d_v != 128 || d->n_h % 32 != 0)
    return fail(MLA_ERR_UNSUPPORTED,
                "decode takes bf16 with d_c=512, d_rope=64, d_nope=d_v=128 and n_h a multiple of 32");
  DecodePlan& P = *p;
  P.n_h = d->n_h;
  P.batch = d->batch;
  P.S = d->S;
  P.total_keys = d->S;
  P.scale = d->softmax_scale > 0.f ? d->softmax_scale : 1.0f / sqrtf(static_cast<float>(d->d_nope + d->d_rope));
  if (!(P.scale < INFINITY)) return fail(MLA_ERR_INVALID_ARG, "softmax_scale is not finite");
  const int64_t groups = (d->n_h + 127) / 128;
  const int64_t target = 256;   // workgroups of the attention launch (8 waves, one per CU)
  int64_t chunk = (P.total_keys * groups + target - 1) / target;
  chunk = std::max<int64_t>(256, (chunk + 31) / 32 * 32);
  chunk = std::min<int64_t>(chunk, (longest + 31) / 32 * 32);
  P.chunk = static_cast<int>(chunk);
  P.nch = static_cast<int>((longest + chunk - 1) / chunk);
  return MLA_OK;
}

// Runs `run` (the call's launches), wrapped in the debug-mode checks when
// MLA_LAGA_DEBUG is set. `used`: the workspace bytes the call's layout takes
// (the debug tail follows them).
template <typename F>
static mla_status run_checked(bool debug, const int32_t* cu_host, const int32_t* cu_dev, int n_cu,
                              char* ws, int64_t used, const DebugOutput* outs, int n_out,
                              hipStream_t st, F&& run) {
  if (!debug) return run();
  if (mla_status s = debug_begin(cu_host, cu_dev, n_cu, ws, used, outs, n_out, st); s != MLA_OK)
    return s;
  if (mla_status s = run(); s != MLA_OK) return s;
  return debug_end(ws, used, outs, n_out, st);
}

}  // namespace mla

using namespace mla;

extern "C" {

mla_status mla_laga_fwd_workspace_size(const mla_laga_desc* desc, const int32_t* cu_host,
                                        size_t* bytes) {
  if (!bytes) return fail(MLA_ERR_INVALID_ARG, "bytes is NULL");
  Plan p;
  if (mla_status s = make_plan(desc, cu_host, &p); s != MLA_OK) return s;
  if (p.fast)
    if (mla_status s = fast_fwd_limits(p); s != MLA_OK) return s;
  *bytes = static_cast<size_t>(fwd_layout(p).total + debug_tail());
  return MLA_OK;
}

mla_status mla_laga_bwd_workspace_size(const mla_laga_desc* desc, const int32_t* cu_host,
                                        size_t* bytes) {
  if (!bytes) return fail(MLA_ERR_INVALID_ARG, "bytes is NULL");
  Plan p;
  if (mla_status s = make_plan(desc, cu_host, &p); s != MLA_OK) return s;
  if (p.fast)
    if (mla_status s = fast_bwd_limits(p); s != MLA_OK) return s;
  *bytes = static_cast<size_t>(bwd_layout(p).total + debug_tail());
  return MLA_OK;
}

mla_status mla_laga_count(const mla_laga_desc* desc, const int32_t* cu_host,
                          int64_t* visible_pairs, int64_t* key_lo, int64_t* key_hi) {
  Plan p;
  if (mla_status s = make_plan(desc, cu_host, &p); s != MLA_OK) return s;
  if (visible_pairs) *visible_pairs = p.visible_pairs;
  if (key_lo) *key_lo = p.key_lo;
  if (key_hi) *key_hi = p.key_hi;
  return MLA_OK;
}

int mla_laga_uses_fast_path(const mla_laga_desc* desc) {
  return desc && fast_shape(desc) ? 1 : 0;
}

static mla_status check_common(const Plan& p, const mla_laga_desc* d, const void* q,
                               const void* c_kv, const void* k_rope, const void* W_UK,
                               const void* W_UV, const int32_t* cu_dev, const void* ws,
                               size_t ws_bytes, int64_t need) {
  const void* ptrs[] = {q, c_kv, W_UK, W_UV};
  const char* names[] = {"q", "c_kv", "W_UK", "W_UV"};
  for (int k = 0; k < 4; ++k) {
    if (!ptrs[k]) return fail(MLA_ERR_INVALID_ARG, "%s is NULL", names[k]);
    if (misaligned(ptrs[k])) return fail(MLA_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[k]);
  }
  if (p.d_rope > 0 && (!k_rope || misaligned(k_rope)))
    return fail(MLA_ERR_INVALID_ARG, "k_rope is NULL or not 16-byte aligned");
  if (d->n_seqs > 0 && !cu_dev) return fail(MLA_ERR_INVALID_ARG, "n_seqs > 0 needs cu_seqlens_dev");
  if (need > 0 && (!ws || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1))))
    return fail(MLA_ERR_WORKSPACE, "workspace is NULL or not 256-byte aligned");
  if (static_cast<int64_t>(ws_bytes) < need)
    return fail(MLA_ERR_WORKSPACE, "workspace has %zu bytes, needs %lld", ws_bytes, (long long)need);
  return MLA_OK;
}

mla_status mla_laga_fwd(const mla_laga_desc* desc, const void* q, const void* c_kv,
                        const void* k_rope, const void* W_UK, const void* W_UV,
                        const int32_t* cu_host, const int32_t* cu_dev, float* out, float* lse,
                        void* workspace, size_t workspace_bytes, void* stream) {
  Plan p;
  if (mla_status s = make_plan(desc, cu_host, &p); s != MLA_OK) return s;
  if (p.S_loc == 0) return MLA_OK;
  const FwdLayout L = fwd_layout(p);
  const bool debug = debug_mode();
  if (mla_status s = check_common(p, desc, q, c_kv, k_rope, W_UK, W_UV, cu_dev, workspace,
                                  workspace_bytes, L.total + (debug ? kDebugTailBytes : 0));
      s != MLA_OK)
    return s;
  if (!out || !lse || misaligned(out) || misaligned(lse))
    return fail(MLA_ERR_INVALID_ARG, "out/lse NULL or not 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const DebugOutput outs[] = {{out, p.S_loc * p.n_h * p.d_v, "out"}, {lse, p.S_loc * p.n_h, "lse"}};
  return run_checked(debug, cu_host, cu_dev, p.n_seqs > 0 ? p.n_seqs + 1 : 0, ws, L.total, outs, 2,
                     st, [&] {
                       if (p.fast) return fast_fwd(p, q, c_kv, k_rope, W_UK, W_UV, cu_dev, out, lse, ws, st);
                       return generic_fwd(p, q, c_kv, k_rope, W_UK, W_UV, cu_dev, out, lse, ws, st);
                     });
}

mla_status mla_laga_bwd(const mla_laga_desc* desc, const void* dout, const void* q,
                        const void* c_kv, const void* k_rope, const void* W_UK, const void* W_UV,
                        const int32_t* cu_host, const int32_t* cu_dev, const float* out,
                        const float* lse, float* dq, float* dc_kv, float* dk_rope, float* dW_UK,
                        float* dW_UV, void* workspace, size_t workspace_bytes, void* stream) {
  Plan p;
  if (mla_status s = make_plan(desc, cu_host, &p); s != MLA_OK) return s;
  if (!dc_kv || !dW_UK || !dW_UV || (p.d_rope > 0 && !dk_rope))
    return fail(MLA_ERR_INVALID_ARG, "a gradient output is NULL");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (p.S_loc == 0) {
    // no local query: nothing is visible and every gradient is zero
    mla_status s = zero_fill(dc_kv, p.S * p.d_c, st);
    if (s == MLA_OK) s = zero_fill(dk_rope, p.S * p.d_rope, st);
    if (s == MLA_OK) s = zero_fill(dW_UK, static_cast<int64_t>(p.d_c) * p.n_h * p.d_nope, st);
    if (s == MLA_OK) s = zero_fill(dW_UV, static_cast<int64_t>(p.d_c) * p.n_h * p.d_v, st);
    return s;
  }
  const BwdLayout L = bwd_layout(p);
  const bool debug = debug_mode();
  if (mla_status s = check_common(p, desc, q, c_kv, k_rope, W_UK, W_UV, cu_dev, workspace,
                                  workspace_bytes, L.total + (debug ? kDebugTailBytes : 0));
      s != MLA_OK)
    return s;
  if (!dout || !out || !lse || !dq) return fail(MLA_ERR_INVALID_ARG, "dout/out/lse/dq is NULL");
  const void* al[] = {dout, out, lse, dq, dc_kv, dk_rope, dW_UK, dW_UV};
  for (const void* a : al)
    if (a && misaligned(a)) return fail(MLA_ERR_INVALID_ARG, "a gradient argument is not 16-byte aligned");
  char* ws = static_cast<char*>(workspace);
  const int64_t n_w = static_cast<int64_t>(p.d_c) * p.n_h;
  const DebugOutput outs[] = {{dq, p.S_loc * p.n_h * p.d_qk, "dq"},
                              {dc_kv, p.S * p.d_c, "dc_kv"},
                              {dk_rope, p.S * p.d_rope, "dk_rope"},
                              {dW_UK, n_w * p.d_nope, "dW_UK"},
                              {dW_UV, n_w * p.d_v, "dW_UV"}};
  return run_checked(debug, cu_host, cu_dev, p.n_seqs > 0 ? p.n_seqs + 1 : 0, ws, L.total, outs, 5,
                     st, [&] {
                       if (p.fast_bwd)
                         return fast_bwd(p, dout, q, c_kv, k_rope, W_UK, W_UV, cu_dev, out, lse, dq,
                                         dc_kv, dk_rope, dW_UK, dW_UV, ws, st);
                       return generic_bwd(p, dout, q, c_kv, k_rope, W_UK, W_UV, cu_dev, out, lse, dq,
                                          dc_kv, dk_rope, dW_UK, dW_UV, ws, st);
                     });
}

mla_status mla_laga_decode_workspace_size(const mla_laga_decode_desc* desc, const int32_t* cu_host,
                                           size_t* bytes) {
  if (!bytes) return fail(MLA_ERR_INVALID_ARG, "bytes is NULL");
  DecodePlan p;
  if (mla_status s = make_decode_plan(desc, cu_host, &p); s != MLA_OK) return s;
  *bytes = static_cast<size_t>(decode_layout(p).total + debug_tail());
  return MLA_OK;
}

mla_status mla_laga_decode(const mla_laga_decode_desc* desc, const void* q, const void* c_kv,
                           const void* k_rope, const void* W_UK, const void* W_UV,
                           const int32_t* cu_host, const int32_t* cu_dev, float* out, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream) {
  DecodePlan p;
  if (mla_status s = make_decode_plan(desc, cu_host, &p); s != MLA_OK) return s;
  const void* ptrs[] = {q, c_kv, k_rope, W_UK, W_UV, out, lse};
  const char* names[] = {"q", "c_kv", "k_rope", "W_UK", "W_UV", "out", "lse"};
  for (int k = 0; k < 7; ++k) {
    if (!ptrs[k]) return fail(MLA_ERR_INVALID_ARG, "%s is NULL", names[k]);
    if (misaligned(ptrs[k])) return fail(MLA_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[k]);
  }
  if (!cu_dev) return fail(MLA_ERR_INVALID_ARG, "decode needs cu_seqlens_dev");
  const bool debug = debug_mode();
  const int64_t used = decode_layout(p).total, need = used + (debug ? kDebugTailBytes : 0);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)))
    return fail(MLA_ERR_WORKSPACE, "workspace is NULL or not 256-byte aligned");
  if (static_cast<int64_t>(workspace_bytes) < need)
    return fail(MLA_ERR_WORKSPACE, "workspace has %zu bytes, needs %lld", workspace_bytes,
                (long long)need);
  char* ws = static_cast<char*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const DebugOutput outs[] = {{out, int64_t(p.batch) * p.n_h * kFastDV, "out"},
                              {lse, int64_t(p.batch) * p.n_h, "lse"}};
  return run_checked(debug, cu_host, cu_dev, p.batch + 1, ws, used, outs, 2, st, [&] {
    return fast_decode(p, q, c_kv, k_rope, W_UK, W_UV, cu_dev, out, lse, ws, st);
  });
}

mla_status mla_laga_decode_noalloc(const mla_laga_decode_desc* desc, const void* q,
                                   const void* c_kv, const void* k_rope, const void* W_UK,
                                   const void* W_UV, const int32_t* cu_host,
                                   const int32_t* cu_dev, float* out, float* lse, void* stream) {
  DecodePlan p;
  if (mla_status s = make_decode_plan(desc, cu_host, &p); s != MLA_OK) return s;
  const void* ptrs[] = {q, c_kv, k_rope, W_UK, W_UV, out, lse};
  const char* names[] = {"q", "c_kv", "k_rope", "W_UK", "W_UV", "out", "lse"};
  for (int k = 0; k < 7; ++k) {
    if (!ptrs[k]) return fail(MLA_ERR_INVALID_ARG, "%s is NULL", names[k]);
    if (misaligned(ptrs[k])) return fail(MLA_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[k]);
  }
  if (!cu_dev) return fail(MLA_ERR_INVALID_ARG, "decode needs cu_seqlens_dev");
  const bool debug = debug_mode();
  const int64_t used = decode_layout(p).total, need = used + (debug ? kDebugTailBytes : 0);
  if (need > kDecodeScratchBytes)
    return fail(MLA_ERR_WORKSPACE,
                "decode needs %lld bytes of scratch; the static scratch holds %lld "
                "(use mla_laga_decode with a workspace)",
                (long long)need, (long long)kDecodeScratchBytes);
  char* ws = nullptr;
  if (mla_status s = decode_scratch(&ws); s != MLA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const DebugOutput outs[] = {{out, int64_t(p.batch) * p.n_h * kFastDV, "out"},
                              {lse, int64_t(p.batch) * p.n_h, "lse"}};
  return run_checked(debug, cu_host, cu_dev, p.batch + 1, ws, used, outs, 2, st, [&] {
    return fast_decode(p, q, c_kv, k_rope, W_UK, W_UV, cu_dev, out, lse, ws, st);
  });
}

mla_status mla_laga_row_window(const mla_laga_desc* desc, const int32_t* cu_host,
                               const int32_t* cu_dev, int64_t* window, void* stream) {
  Plan p;
  if (mla_status s = make_plan(desc, cu_host, &p); s != MLA_OK) return s;
  if (p.S_loc == 0) return MLA_OK;
  if (!window || misaligned(window)) return fail(MLA_ERR_INVALID_ARG, "window is NULL or not 16-byte aligned");
  if (p.n_seqs > 0 && !cu_dev) return fail(MLA_ERR_INVALID_ARG, "n_seqs > 0 needs cu_seqlens_dev");
  return launch_row_window(p, cu_dev, window, static_cast<hipStream_t>(stream));
}

const char* mla_laga_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    case MLA_ERR_DEBUG_CHECK: return "MLA_ERR_DEBUG_CHECK";
  }
  return "unknown mla_status";
}

const char* mla_laga_last_error(void) { return g_last_error; }

mla_status mla_laga_timing_enable(int on) {
  for (auto& r : g_launches)
    if (!r.name.empty()) (void)hipEventSynchronize(r.stop);
  release_records();
  g_timing = on != 0;
  return MLA_OK;
}

mla_status mla_laga_timing_select(const char* names) {
  g_select.clear();
  if (names != nullptr && names[0] != '\0') g_select = ";" + std::string(names) + ";";
  return MLA_OK;
}

mla_status mla_laga_timing_read(const char* kernel, double* total_ms, int64_t* launches) {
  if (!kernel || !total_ms || !launches) return fail(MLA_ERR_INVALID_ARG, "NULL argument");
  double tot = 0.0;
  int64_t n = 0;
  for (auto& r : g_launches) {
    if (r.name.empty() || r.name != kernel) continue;
    if (hipEventSynchronize(r.stop) != hipSuccess)
      return fail(MLA_ERR_HIP, "event wait failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
      return fail(MLA_ERR_HIP, "event elapsed time failed");
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return MLA_OK;
}

const char* mla_laga_timing_names(void) {
  g_names.clear();
  for (auto& r : g_launches) {
    const std::string key = r.name + ";";
    if (g_names.find(key) == std::string::npos) g_names += key;
  }
  return g_names.c_str();
}

}  // extern "C"
