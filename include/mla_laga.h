/*
 * mla_laga.h - C ABI of the MI355X (gfx950) latent-attention block library.
 *
 * The operation (LAGA abstract, "A Training-Memory Regression in MLA Sequence
 * Parallelism: Why Megatron-Core Forbids Absorption, and LAGA -- a
 * Communication-Efficient Fix", weekinpapers.com / OpenAlex pages, Abstract):
 * every sequence-parallel rank holds the gathered compressed KV latent of the
 * whole sequence and a contiguous block of query rows. It rebuilds each
 * head's keys and values locally from the latent instead of absorbing the
 * up-projection into the query, then runs causal attention for its rows.
 * The result is the explicit MLA form. One call computes one rank's share:
 *
 *   K_nope[t,h,:] = c_kv[t,:] @ W_UK[:, h*d_nope : (h+1)*d_nope]
 *   V[t,h,:]      = c_kv[t,:] @ W_UV[:, h*d_v    : (h+1)*d_v]
 *   K[t,h,:]      = [ K_nope[t,h,:] | k_rope[t,:] ]          (rope key shared by heads)
 *   s[i,j,h]      = scale * q[i,h,:] . K[j,h,:]              (q row = [nope | rope])
 *   lse[i,h]      = ln sum_{j visible} exp(s[i,j,h])
 *   out[i,h,:]    = sum_{j visible} exp(s[i,j,h] - lse[i,h]) V[j,h,:]
 *
 * Row i sits at global position p = q_offset + i and sees keys j with
 * seg_lo(p) <= j <= p: seg_lo(p) = 0 for one causal sequence, else the start
 * of the packed sample holding p (block-diagonal causal mask of fixed-token
 * packing, Libra review page, "Axiom ledger"). A shard may instead hold
 * several position blocks (zigzag or striped sharding, which evens out
 * causal work across ranks; Libra review page, Related Work beside
 * Fig. 15): its rows are then the blocks laid end to end and p is read off
 * that concatenation (mla_laga_desc.q_ranges). q's rope part and k_rope come
 * already rotated. The backward computes the gradients of sum(out * dout).
 *
 * Conventions for every entry point
 *   - All tensors are dense, row-major, in the shapes given. "Device" means
 *     memory of the current HIP device; "host" means ordinary host memory.
 *   - The caller owns all memory, including the workspace. The library does
 *     not allocate, free, or keep any pointer after a call returns.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     with no host synchronisation. Outputs are valid once the stream has
 *     reached the call. Calls that share a workspace must be ordered.
 *   - The fast forward and backward run some of their kernels on an internal
 *     stream of the current device, forked from `stream` by an event and
 *     joined back into it before the call returns, so ordering on `stream`
 *     is as if all the work were there. That stream and its two events are
 *     created on the first fast forward or backward of each host thread on
 *     each device and kept until the process ends (make that first call
 *     outside graph capture).
 *   - Validation happens on the host before anything is enqueued. On error
 *     nothing is enqueued, the status is returned and a message is kept for
 *     mla_laga_last_error() (per thread). A failed launch returns MLA_ERR_HIP.
 *   - Gradients overwrite their outputs (no accumulation). dc_kv and dk_rope
 *     cover all S latent rows; rows no local query sees are written as 0.
 *   - Precisions: in_dtype MLA_BF16 (the fast path) or MLA_F32 for q, c_kv,
 *     k_rope, W_UK, W_UV and dout; out, lse and all gradients are float32.
 *     The fast path takes d_nope = d_v = 128, d_rope = 64, d_c a multiple of
 *     64 (512 in DeepSeek-V3), any n_h; it keeps the rebuilt K/V and the
 *     softmax weights in fp16 with fp32 accumulation. Every other shape (and
 *     MLA_F32) runs a plain fp32 path of simple kernels.
 *   - Size limits of the fast path (32-bit offsets inside its kernels):
 *     fewer than 2^22 needed keys (the keys the shard's rows see, padded to
 *     256), S below 2^31 - 256, n_h below 32768 for the forward and 16384
 *     for the backward, S_loc below 2^31 / 192 for the backward. Past them
 *     the workspace queries and the calls return MLA_ERR_UNSUPPORTED before
 *     anything is enqueued.
 *   - fp16 ranges of the fast path (normal range 2^-14 .. 65504; below it
 *     values keep an absolute precision of 2^-24, above it they overflow):
 *       forward: q (both parts), k_rope and the rebuilt K_nope = c_kv W_UK
 *       and V = c_kv W_UV are taken in fp16 as they are, so their magnitudes
 *       must stay below 65504, and elements below 2^-14 lose relative
 *       precision (they matter only against larger elements of the same dot
 *       product). Softmax weights are at most 256 by construction. The
 *       scores' absolute rounding grows with the logits: with logits 8 times
 *       those of unit-scale inputs (N(0,1) q and c_kv, weights N(0,1/d_c))
 *       the backward's gradients reach sum|err| / sum|ref| of about 1e-3.
 *       backward: dout is first multiplied by a power of two 2^e that brings
 *       max|dout| into [4, 8) (exact), so the gradients do not depend on the
 *       scale of dout: dout scaled by any power of two gives gradients
 *       scaled by the same power, bit for bit. The dK/dV products take the
 *       softmax weights as P 2^15 and dS = P (dP - D) as dS 2^ex, ex per
 *       key the largest power for which a bound on the key's |dP - D| (from
 *       the largest 2^e dout row norm, the largest |D| and the key's V row
 *       norm) keeps |dS 2^ex| below 2^14; both factors are exact and leave
 *       in fp32, so a key's weights among up to 2^22 keys stay in fp16's
 *       normal range. The per-key rows [dK_nope | dV] are stored in fp16
 *       with the dout factor only: |dV[key]| <= 8 * (the key's total
 *       softmax weight over the shard's rows) must stay below 65504, and
 *       where that total is tiny (a few rows over millions of keys) the rows
 *       fall below 2^-14 and dc_kv loses relative precision (sum|err| /
 *       sum|dc_kv| of 3e-3 at 2^22 keys and 64 rows, 5e-4 at 2^19 keys and
 *       256 rows). The fp32 gradients are multiplied back by 2^-e.
 */
/*
 * Debug mode. With the environment variable MLA_LAGA_DEBUG set to anything
 * but "" or "0" (read at every call), mla_laga_fwd, mla_laga_bwd,
 * mla_laga_decode and mla_laga_decode_noalloc add checks around their work:
 *   - cu_seqlens_dev is copied back and must equal cu_seqlens_host;
 *   - every output and the workspace bytes the call uses are first filled
 *     with all-ones bytes (NaN as fp32, fp16 and bf16), so that an output
 *     element the call does not write, or a result computed from workspace
 *     bytes read before the call wrote them, comes out NaN;
 *   - a canary is written into the 256 bytes after the used workspace (the
 *     *_workspace_size results are 256 bytes larger in this mode, and the
 *     static decode scratch holds 256 bytes less) and must be intact after
 *     the work;
 *   - after the work every output is scanned for NaN.
 * The call then waits for its stream (so it cannot be captured into a
 * graph), and a failed check returns MLA_ERR_DEBUG_CHECK with the first
 * offending value named in mla_laga_last_error(). NaN in the inputs is
 * reported the same way. Results are unchanged when the checks pass.
 */
#ifndef MLA_LAGA_H
#define MLA_LAGA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1, /* bad shape, offset, pointer or cu_seqlens    */
  MLA_ERR_UNSUPPORTED = -2, /* valid, but outside what any path handles     */
  MLA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required   */
  MLA_ERR_HIP = -4,         /* a HIP runtime call or a launch failed        */
  MLA_ERR_DEBUG_CHECK = -5  /* a debug-mode check failed (MLA_LAGA_DEBUG)   */
} mla_status;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;

/* Force the plain fp32 path even where the fast path applies. */
#define MLA_FLAG_GENERIC 1
/* Fast backward, opt-in: the dK/dV kernel keeps dS = P (dP - D) (fp16) in the
 * workspace and dQ is computed from it, instead of recomputing the scores
 * and dP per query tile (the default). Faster, but the workspace then holds
 * dS, one fp16 value per (local row, needed key, head): B = Kpad * S_pad * 2
 * bytes per head (Kpad = needed keys rounded up to 256, S_pad = S_loc
 * rounded up to 64). While n_h * B <= 16 GiB that is n_h * B bytes more
 * (8 GiB at n_h = 128, 16384 keys, 2048 rows). Past that, the heads run in
 * groups of G through two alternating buffers, 2 * G * B bytes more, with
 * G = ceil(n_h / ceil(n_h / floor(2^30 / B))) (groups of at most 1 GiB, as
 * even as their count allows); dQ of one group then shares the GPU with
 * dK/dV of the next, a little slower than the one-buffer form. When 8 heads
 * do not fit one group (8 * B > 1 GiB, with n_h * B past 16 GiB) the flag is
 * ignored and dQ recomputes: so many small groups would cost more than
 * recomputing. Both forms give the same gradients up to fp16 rounding
 * order. */
#define MLA_FLAG_STORED_DS 4
/* The flag value 2 is not used; any flag bit other than these two is
 * rejected with MLA_ERR_INVALID_ARG. */

/* Most position blocks one shard may hold (mla_laga_desc.n_ranges). */
#define MLA_MAX_RANGES 16

typedef struct {
  int32_t n_h;      /* heads                                                  */
  int32_t d_c;      /* latent width                                           */
  int32_t d_rope;   /* shared rope-key width (also the rope part of q)        */
  int32_t d_nope;   /* per-head no-position key width                         */
  int32_t d_v;      /* per-head value width                                   */
  int32_t n_seqs;   /* 0: one causal sequence over [0,S); else packed samples */
  int64_t S;        /* latent (key) length                                    */
  int64_t S_loc;    /* local query rows (0 is a valid empty call)             */
  int64_t q_offset; /* global position of local row 0                         */
  int32_t in_dtype; /* mla_dtype of the inputs                                */
  int32_t flags;    /* MLA_FLAG_* bits                                        */
  float softmax_scale; /* <= 0: 1/sqrt(d_nope + d_rope)                       */
  /* Position blocks of the local rows. n_ranges = 0: one block, rows at
   * q_offset .. q_offset + S_loc - 1. 1 <= n_ranges <= MLA_MAX_RANGES:
   * q_ranges (host memory, read during the call only) holds n_ranges
   * (start, length) int64 pairs; rows are the blocks in that order, so row
   * i of block b (rows counted from the blocks before it) sits at
   * start_b + i. Blocks must be ascending and disjoint (start_b >= start_{b-1}
   * + length_{b-1}), lie in [0, S), and their lengths (0 allowed) must sum
   * to S_loc; q_offset must then be 0. A zigzag rank r of R holds blocks r
   * and 2R-1-r of S/(2R) positions each.                                     */
  int32_t n_ranges;
  const int64_t* q_ranges;
} mla_laga_desc;

/*
 * Workspace bytes mla_laga_fwd / mla_laga_bwd need for `desc` (written to
 * *bytes). cu_seqlens_host: n_seqs+1 int32 sample starts in host memory
 * (cu[0] = 0, cu[n_seqs] = S, non-decreasing), or NULL when n_seqs = 0; it
 * sets how many latent rows the shard needs. Grows linearly in S_loc + q_offset
 * and in n_h.
 */
mla_status mla_laga_fwd_workspace_size(const mla_laga_desc* desc,
                                        const int32_t* cu_seqlens_host,
                                        size_t* bytes);
mla_status mla_laga_bwd_workspace_size(const mla_laga_desc* desc,
                                        const int32_t* cu_seqlens_host,
                                        size_t* bytes);

/*
 * Forward for one query shard (the local computation of LAGA: rebuild K/V
 * from the gathered latent, then attention; LAGA abstract).
 *   q        device [S_loc, n_h, d_nope + d_rope]   in_dtype
 *   c_kv     device [S, d_c]                        in_dtype
 *   k_rope   device [S, d_rope]                     in_dtype
 *   W_UK     device [d_c, n_h * d_nope]             in_dtype (head-major columns)
 *   W_UV     device [d_c, n_h * d_v]                in_dtype (head-major columns)
 *   cu_seqlens_host / cu_seqlens_dev: the same n_seqs+1 int32 values in host
 *            and device memory; both NULL when n_seqs = 0.
 *   out      device [S_loc, n_h, d_v] float32 (written)
 *   lse      device [S_loc, n_h] float32, natural log (written)
 *   workspace device, >= mla_laga_fwd_workspace_size bytes, 256-byte aligned.
 * Device pointers must be 16-byte aligned.
 */
mla_status mla_laga_fwd(const mla_laga_desc* desc, const void* q, const void* c_kv,
                        const void* k_rope, const void* W_UK, const void* W_UV,
                        const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                        float* out, float* lse, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * Backward: gradients of sum(out * dout) (training path; LAGA abstract).
 *   dout     device [S_loc, n_h, d_v] in_dtype
 *   out, lse device, as written by mla_laga_fwd for the same inputs.
 *   dq       device [S_loc, n_h, d_nope + d_rope] float32 (written)
 *   dc_kv    device [S, d_c] float32 (written)
 *   dk_rope  device [S, d_rope] float32 (written)
 *   dW_UK    device [d_c, n_h * d_nope] float32 (written)
 *   dW_UV    device [d_c, n_h * d_v] float32 (written)
 *   workspace device, >= mla_laga_bwd_workspace_size bytes, 256-byte aligned.
 * Other arguments as for mla_laga_fwd.
 */
mla_status mla_laga_bwd(const mla_laga_desc* desc, const void* dout, const void* q,
                        const void* c_kv, const void* k_rope, const void* W_UK,
                        const void* W_UV, const int32_t* cu_seqlens_host,
                        const int32_t* cu_seqlens_dev, const float* out, const float* lse,
                        float* dq, float* dc_kv, float* dk_rope, float* dW_UK, float* dW_UV,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode in the absorbed form (inference only). The LAGA abstract names the
 * absorbed MLA form -- W_UK folded into the query, attention over the
 * compressed latent -- as the one allowed only in inference decode; it needs
 * no per-head K/V. One query per sequence attends to every cached latent row
 * of its sequence (it sits at the sequence's last position, its own latent
 * row already appended):
 *   q_lat = W_UK_h q_nope,  s_j = scale (q_lat . c_kv[j] + q_rope . k_rope[j]),
 *   out   = W_UV_h^T sum_j softmax(s)_j c_kv[j],  lse = ln sum_j exp(s_j)
 * which equals the explicit form (mla_laga_fwd) for that query.
 * Takes bf16 inputs with d_c = 512, d_rope = 64, d_nope = d_v = 128 and n_h a
 * multiple of 32 (MLA_ERR_UNSUPPORTED otherwise).
 */
typedef struct {
  int32_t n_h, d_c, d_rope, d_nope, d_v;
  int32_t batch;       /* sequences, one query each (>= 1)                      */
  int64_t S;           /* cached latent rows over all sequences                 */
  int32_t in_dtype;    /* MLA_BF16                                              */
  float softmax_scale; /* <= 0: 1/sqrt(d_nope + d_rope)                         */
} mla_laga_decode_desc;

/*
 * cu_seqlens_host: batch+1 int32 in host memory; sequence b owns cache rows
 * [cu[b], cu[b+1]), at least one (cu strictly increasing, cu[0] = 0,
 * cu[batch] = S). The workspace grows with batch * n_h * (longest sequence).
 */
mla_status mla_laga_decode_workspace_size(const mla_laga_decode_desc* desc,
                                           const int32_t* cu_seqlens_host, size_t* bytes);

/*
 *   q        device [batch, n_h, d_nope + d_rope] bf16 (rope part rotated)
 *   c_kv     device [S, d_c] bf16, k_rope device [S, d_rope] bf16: the cache
 *   W_UK, W_UV device [d_c, n_h * 128] bf16 (head-major columns)
 *   cu_seqlens_host / cu_seqlens_dev: the same batch+1 values, host and device
 *   out      device [batch, n_h, d_v] float32 (written)
 *   lse      device [batch, n_h] float32, natural log (written)
 *   workspace device, >= mla_laga_decode_workspace_size bytes, 256-byte aligned.
 * Conventions as for mla_laga_fwd.
 */
mla_status mla_laga_decode(const mla_laga_decode_desc* desc, const void* q, const void* c_kv,
                           const void* k_rope, const void* W_UK, const void* W_UV,
                           const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                           float* out, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * Decode that allocates nothing, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation. Same operation, arguments and results as
 * mla_laga_decode, bit for bit, without the workspace: the kernels use a
 * static device buffer of the library's own (MLA_DECODE_NOALLOC_MAX_BYTES,
 * 256 MiB), which each GPU the library runs on holds until the process
 * ends. The call allocates and frees nothing and enqueues no memset; the
 * buffer's address on a device is looked up on the first call with that
 * device current (make that first call outside graph capture).
 *   - A decode whose mla_laga_decode_workspace_size exceeds the buffer is
 *     rejected with MLA_ERR_WORKSPACE before anything is enqueued (64 x 8192
 *     cached rows at n_h = 128 need 64.25 MiB).
 *   - Every call on one GPU shares that GPU's buffer, and nothing in it is
 *     assumed from an earlier call. Calls that overlap on one GPU (other
 *     streams, or other host threads, without ordering between them) race
 *     on it: order them, e.g. on one stream.
 */
#define MLA_DECODE_NOALLOC_MAX_BYTES (256ll << 20)
mla_status mla_laga_decode_noalloc(const mla_laga_decode_desc* desc, const void* q,
                                   const void* c_kv, const void* k_rope, const void* W_UK,
                                   const void* W_UV, const int32_t* cu_seqlens_host,
                                   const int32_t* cu_seqlens_dev, float* out, float* lse,
                                   void* stream);

/*
 * Host-side counts used for FLOP accounting: visible (query, key) pairs per
 * head, and the half-open latent row range [key_lo, key_hi) the shard needs.
 * Attention cost grows with the visible pairs, i.e. with the sum of squared
 * sample lengths for packed data (Libra review page, Eq. 2).
 */
mla_status mla_laga_count(const mla_laga_desc* desc, const int32_t* cu_seqlens_host,
                          int64_t* visible_pairs, int64_t* key_lo, int64_t* key_hi);

/*
 * The key window of every local row, as the kernels compute it: window
 * (device, int64 [S_loc][2], 16-byte aligned) receives for row i the
 * global positions lo = seg_lo(p) and hi = p of the first and last key it
 * sees (p the row's position; see the mask at the top of this file), from
 * the same device code that maps rows to positions and finds sample starts
 * in the attention kernels. For checking the mask against an independent
 * implementation. Arguments and validation as for mla_laga_fwd; enqueued
 * on `stream`.
 */
mla_status mla_laga_row_window(const mla_laga_desc* desc, const int32_t* cu_seqlens_host,
                               const int32_t* cu_seqlens_dev, int64_t* window, void* stream);

/*
 * Kernel timing, for measurement. While enabled, every kernel the library
 * launches is bracketed by two HIP events recorded on the stream it runs
 * on. mla_laga_timing_enable(1) also forgets earlier records.
 * mla_laga_timing_read waits for the recorded events and returns the summed
 * duration (ms) and launch count of the kernels named `kernel` (the names
 * are listed by mla_laga_timing_names, separated by ';'). Not thread-safe:
 * enable, run and read from one host thread.
 * mla_laga_timing_select restricts the bracketing to the kernels whose
 * names appear in `names` (';'-separated, host string, copied); NULL or ""
 * selects every kernel again. Each pair of events adds a few microseconds
 * between launches, so a timed run brackets only the kernels it reports.
 */
mla_status mla_laga_timing_enable(int on);
mla_status mla_laga_timing_select(const char* names);
mla_status mla_laga_timing_read(const char* kernel, double* total_ms, int64_t* launches);
const char* mla_laga_timing_names(void);

/* 1 if `desc` runs the fast (MFMA) path, 0 if the plain fp32 path. */
int mla_laga_uses_fast_path(const mla_laga_desc* desc);

const char* mla_laga_status_string(mla_status status);
const char* mla_laga_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_LAGA_H */
