"""Explicit MLA forward and backward in numpy float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by the tests,
the smoke check and the benchmark's CPU-baseline leg, never by the library.

Sources and readings
--------------------
* LAGA abstract (weekinpapers.com / OpenAlex pages for arXiv 2607.17644,
  Abstract): per-head K/V are rebuilt from the gathered compressed latent;
  the result equals the explicit form; the absorbed form is an algebraic
  reformulation of it (W_UK folded into the query, attention in latent
  space). The page gives no formulas; the plain readings used here are:
    - K_nope[t,h,:] = c_kv[t,:] @ W_UK[:, h*d_nope:(h+1)*d_nope]   (head-major
      weight columns), V[t,h,:] = c_kv[t,:] @ W_UV[:, h*d_v:(h+1)*d_v];
    - a query row is [nope (d_nope) | rope (d_rope)]; the key is
      K[t,h,:] = [K_nope[t,h,:] | k_rope[t,:]], the RoPE key shared by heads;
    - q's rope part and k_rope arrive already rotated (no positions are
      passed, so nothing is rotated here);
    - score s_ij = scale * q_i . K_j with scale = 1/sqrt(d_nope + d_rope)
      unless given; lse is the natural log of the sum of exp of the scaled
      scores.
* Masking. A query's global position is p = q_offset + i when a sequence-
  parallel shard holds one contiguous block of query rows (the full latent
  is gathered). A shard may instead hold several ascending, disjoint blocks
  (zigzag or striped sharding, which evens out causal work across ranks;
  pith.science review of Libra, Related Work beside Fig. 15): its local rows
  are then those blocks concatenated, and row i's position is read off
  that concatenation. Without packing a query sees keys 0..p (causal). With packed
  samples (Libra review page, "Axiom ledger": fixed-token packing, block-
  diagonal causal mask) it sees keys seg_lo(p)..p where seg_lo(p) is the
  start of the sample holding p; empty samples hold no position.
* Backward: the gradients of out = softmax(s) V through s = scale q.K and the
  up-projections, by the chain rule:
    D_i  = dout_i . out_i
    dV_j = sum_i P_ij dout_i          dS_ij = P_ij (dout_i . V_j - D_i)
    dq_i = scale sum_j dS_ij K_j      dK_j  = scale sum_i dS_ij q_i
    dk_rope_j = sum_h dK_j[h, d_nope:]
    dc_kv_j   = sum_h dK_j[h, :d_nope] W_UK_h^T + dV_j[h] W_UV_h^T
    dW_UK_h   = c_kv^T dK[:, h, :d_nope]          dW_UV_h = c_kv^T dV[:, h]

Query rows are processed in chunks only to bound memory: rows are
independent in the definition, so chunking changes no value.
"""

from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

F64 = np.float64


def default_scale(d_nope: int, d_rope: int) -> float:
    """1/sqrt(width of the query-key dot product)."""
    return 1.0 / math.sqrt(d_nope + d_rope)


# ------------------------------------------------------------------- masks
def segment_start(p: np.ndarray, cu_seqlens: Optional[np.ndarray]) -> np.ndarray:
    """Start position of the packed sample that holds global position p.

    cu_seqlens[k] is where sample k starts (cu_seqlens[0] = 0, last = S);
    the holder is the last sample whose start is <= p, which skips empty
    samples (equal neighbouring entries). Without packing it is 0.
    """
    p = np.asarray(p, dtype=np.int64)
    if cu_seqlens is None:
        return np.zeros_like(p)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    k = np.searchsorted(cu, p, side="right") - 1
    return cu[k]


def row_positions(S_loc: int, q_offset: int = 0,
                  q_ranges: Optional[Sequence[Tuple[int, int]]] = None) -> np.ndarray:
    """Global position of every local query row.

    One contiguous block: q_offset + i. With ``q_ranges`` (a list of
    (start, length) blocks), the local rows are the blocks' positions laid
    end to end in the order given; their lengths must add up to S_loc.
    """
    if q_ranges is None:
        return q_offset + np.arange(S_loc, dtype=np.int64)
    parts = [np.arange(int(a), int(a) + int(n), dtype=np.int64) for a, n in q_ranges]
    pos = np.concatenate(parts) if parts else np.zeros(0, np.int64)
    if len(pos) != S_loc:
        raise ValueError(f"q_ranges cover {len(pos)} rows, S_loc is {S_loc}")
    return pos


def visible_range(S_loc: int, q_offset: int,
                  cu_seqlens: Optional[np.ndarray],
                  q_ranges: Optional[Sequence[Tuple[int, int]]] = None
                  ) -> Tuple[np.ndarray, np.ndarray]:
    """Inclusive [lo, hi] key range each local query row sees."""
    p = row_positions(S_loc, q_offset, q_ranges)
    return segment_start(p, cu_seqlens), p


def visible_pairs(S_loc: int, q_offset: int,
                  cu_seqlens: Optional[np.ndarray] = None,
                  q_ranges: Optional[Sequence[Tuple[int, int]]] = None) -> int:
    """Number of (query, key) pairs with nonzero attention weight, per head."""
    lo, hi = visible_range(S_loc, q_offset, cu_seqlens, q_ranges)
    return int(np.sum(hi - lo + 1))


def key_range(S_loc: int, q_offset: int,
              cu_seqlens: Optional[np.ndarray] = None,
              q_ranges: Optional[Sequence[Tuple[int, int]]] = None) -> Tuple[int, int]:
    """Half-open range of keys any local query sees (the latent rows the
    shard rebuilds keys and values for)."""
    lo, hi = visible_range(S_loc, q_offset, cu_seqlens, q_ranges)
    return int(lo.min()), int(hi.max()) + 1


def keys_needed(S_loc: int, q_offset: int,
                cu_seqlens: Optional[np.ndarray] = None,
                q_ranges: Optional[Sequence[Tuple[int, int]]] = None) -> int:
    a, b = key_range(S_loc, q_offset, cu_seqlens, q_ranges)
    return b - a


def attention_flops(n_h: int, d_c: int, d_rope: int, d_nope: int, d_v: int,
                    S_loc: int, q_offset: int,
                    cu_seqlens: Optional[np.ndarray] = None,
                    backward: bool = False,
                    q_ranges: Optional[Sequence[Tuple[int, int]]] = None) -> int:
    """Algorithmic FLOPs of the block: visible pairs plus the up-projection
    of the keys the shard needs (masked work and recomputation earn nothing;
    the backward counts the score recomputation, as flash attention does)."""
    P = visible_pairs(S_loc, q_offset, cu_seqlens, q_ranges)
    Kn = keys_needed(S_loc, q_offset, cu_seqlens, q_ranges)
    d_qk = d_nope + d_rope
    if not backward:
        return 2 * n_h * (d_qk + d_v) * P + 2 * n_h * d_c * (d_nope + d_v) * Kn
    return 2 * n_h * (3 * d_qk + 2 * d_v) * P + 4 * n_h * d_c * (d_nope + d_v) * Kn


# ------------------------------------------------------------- utilities
def _dims(q, k_rope, W_UV):
    S_loc, n_h, d_qk = q.shape
    d_rope = k_rope.shape[1]
    d_nope = d_qk - d_rope
    d_v = W_UV.shape[1] // n_h
    return S_loc, n_h, d_qk, d_rope, d_nope, d_v


def _chunks(idx: np.ndarray, size: int) -> Iterable[np.ndarray]:
    for a in range(0, len(idx), size):
        yield idx[a:a + size]


def _head_kv(c_kv, k_rope, W_UK, W_UV, h, d_nope, d_v, k0, k1):
    """Explicit per-head keys and values for latent rows k0..k1-1."""
    c = c_kv[k0:k1]
    k_nope = c @ W_UK[:, h * d_nope:(h + 1) * d_nope]
    K = np.concatenate([k_nope, k_rope[k0:k1]], axis=1)
    V = c @ W_UV[:, h * d_v:(h + 1) * d_v]
    return K, V


def _softmax_rows(s: np.ndarray, vis: np.ndarray):
    """Masked row softmax: returns P and lse (natural log). Rows with no
    visible key (impossible under the call's preconditions) give P = 0 and
    lse = -inf."""
    sm = np.where(vis, s, -np.inf)
    m = sm.max(axis=1, keepdims=True)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.where(vis, np.exp(sm - m_safe), 0.0)
    tot = e.sum(axis=1, keepdims=True)
    with np.errstate(divide="ignore"):
        lse = m_safe + np.log(tot)
    P = np.where(tot > 0, e / np.where(tot > 0, tot, 1.0), 0.0)
    return P, lse[:, 0]


# --------------------------------------------------------------- forward
def mla_forward(q, c_kv, k_rope, W_UK, W_UV, q_offset: int = 0,
                cu_seqlens: Optional[np.ndarray] = None,
                scale: Optional[float] = None,
                heads: Optional[Sequence[int]] = None,
                rows: Optional[Sequence[int]] = None,
                chunk: int = 512,
                q_ranges: Optional[Sequence[Tuple[int, int]]] = None):
    """Explicit MLA forward for one query shard.

    q [S_loc, n_h, d_nope+d_rope], c_kv [S, d_c], k_rope [S, d_rope],
    W_UK [d_c, n_h*d_nope], W_UV [d_c, n_h*d_v]. Returns out
    [len(rows), len(heads), d_v] and lse [len(rows), len(heads)] in float64
    (all rows/heads by default). ``q_ranges`` replaces q_offset when the
    shard's rows are several position blocks (see ``row_positions``).
    """
    q = np.asarray(q, F64); c_kv = np.asarray(c_kv, F64)
    k_rope = np.asarray(k_rope, F64)
    W_UK = np.asarray(W_UK, F64); W_UV = np.asarray(W_UV, F64)
    S_loc, n_h, d_qk, d_rope, d_nope, d_v = _dims(q, k_rope, W_UV)
    if scale is None:
        scale = default_scale(d_nope, d_rope)
    heads = list(range(n_h)) if heads is None else list(heads)
    rows = np.arange(S_loc) if rows is None else np.asarray(rows, dtype=np.int64)
    lo, hi = visible_range(S_loc, q_offset, cu_seqlens, q_ranges)
    k0 = int(lo[rows].min()); k1 = int(hi[rows].max()) + 1
    keys = np.arange(k0, k1)
    out = np.zeros((len(rows), len(heads), d_v), F64)
    lse = np.zeros((len(rows), len(heads)), F64)
    for hi_, h in enumerate(heads):
        K, V = _head_kv(c_kv, k_rope, W_UK, W_UV, h, d_nope, d_v, k0, k1)
        for ci in _chunks(np.arange(len(rows)), chunk):
            r = rows[ci]
            s = scale * (q[r, h, :] @ K.T)
            vis = (keys[None, :] >= lo[r][:, None]) & (keys[None, :] <= hi[r][:, None])
            P, l = _softmax_rows(s, vis)
            out[ci, hi_, :] = P @ V
            lse[ci, hi_] = l
    return out, lse


def mla_forward_absorbed(q, c_kv, k_rope, W_UK, W_UV, q_offset: int = 0,
                         cu_seqlens: Optional[np.ndarray] = None,
                         scale: Optional[float] = None,
                         q_ranges: Optional[Sequence[Tuple[int, int]]] = None):
    """The absorbed reformulation (LAGA abstract: the form that folds W_UK
    into the query and attends in latent space). Per head h:
        s_ij  = scale * ((W_UK_h q_nope_i) . c_kv_j + q_rope_i . k_rope_j)
        out_i = (sum_j P_ij c_kv_j) W_UV_h
    It is a different association of the same products, so it must equal
    the explicit form up to rounding; used only to pin ``mla_forward``.
    """
    q = np.asarray(q, F64); c_kv = np.asarray(c_kv, F64)
    k_rope = np.asarray(k_rope, F64)
    W_UK = np.asarray(W_UK, F64); W_UV = np.asarray(W_UV, F64)
    S_loc, n_h, d_qk, d_rope, d_nope, d_v = _dims(q, k_rope, W_UV)
    if scale is None:
        scale = default_scale(d_nope, d_rope)
    lo, hi = visible_range(S_loc, q_offset, cu_seqlens, q_ranges)
    keys = np.arange(c_kv.shape[0])
    vis = (keys[None, :] >= lo[:, None]) & (keys[None, :] <= hi[:, None])
    out = np.zeros((S_loc, n_h, d_v), F64)
    lse = np.zeros((S_loc, n_h), F64)
    for h in range(n_h):
        Wk = W_UK[:, h * d_nope:(h + 1) * d_nope]        # [d_c, d_nope]
        q_lat = q[:, h, :d_nope] @ Wk.T                   # [S_loc, d_c]
        s = scale * (q_lat @ c_kv.T + q[:, h, d_nope:] @ k_rope.T)
        P, l = _softmax_rows(s, vis)
        ctx = P @ c_kv                                    # [S_loc, d_c]
        out[:, h, :] = ctx @ W_UV[:, h * d_v:(h + 1) * d_v]
        lse[:, h] = l
    return out, lse


# -------------------------------------------------------------- backward
def mla_backward(dout, q, c_kv, k_rope, W_UK, W_UV, q_offset: int = 0,
                 cu_seqlens: Optional[np.ndarray] = None,
                 scale: Optional[float] = None,
                 heads: Optional[Sequence[int]] = None,
                 chunk: int = 512,
                 q_ranges: Optional[Sequence[Tuple[int, int]]] = None):
    """Gradients of sum(out * dout) with respect to every input.

    Returns dq [S_loc,n_h,d_qk], dc_kv [S,d_c], dk_rope [S,d_rope],
    dW_UK [d_c,n_h*d_nope], dW_UV [d_c,n_h*d_v], all float64. With ``heads``
    given, only those heads contribute (the others' dq/dW blocks stay zero);
    this equals the full result when dout is zero on the other heads.
    """
    dout = np.asarray(dout, F64)
    q = np.asarray(q, F64); c_kv = np.asarray(c_kv, F64)
    k_rope = np.asarray(k_rope, F64)
    W_UK = np.asarray(W_UK, F64); W_UV = np.asarray(W_UV, F64)
    S_loc, n_h, d_qk, d_rope, d_nope, d_v = _dims(q, k_rope, W_UV)
    S, d_c = c_kv.shape
    if scale is None:
        scale = default_scale(d_nope, d_rope)
    heads = list(range(n_h)) if heads is None else list(heads)
    lo, hi = visible_range(S_loc, q_offset, cu_seqlens, q_ranges)
    k0 = int(lo.min()); k1 = int(hi.max()) + 1
    keys = np.arange(k0, k1)

    dq = np.zeros((S_loc, n_h, d_qk), F64)
    dc_kv = np.zeros((S, d_c), F64)
    dk_rope = np.zeros((S, d_rope), F64)
    dW_UK = np.zeros((d_c, n_h * d_nope), F64)
    dW_UV = np.zeros((d_c, n_h * d_v), F64)
    for h in heads:
        K, V = _head_kv(c_kv, k_rope, W_UK, W_UV, h, d_nope, d_v, k0, k1)
        dK = np.zeros_like(K)
        dV = np.zeros_like(V)
        for r in _chunks(np.arange(S_loc), chunk):
            s = scale * (q[r, h, :] @ K.T)
            vis = (keys[None, :] >= lo[r][:, None]) & (keys[None, :] <= hi[r][:, None])
            P, _ = _softmax_rows(s, vis)
            o = P @ V
            dO = dout[r, h, :]
            D = np.sum(dO * o, axis=1, keepdims=True)
            dV += P.T @ dO
            dS = P * (dO @ V.T - D)
            dq[r, h, :] = scale * (dS @ K)
            dK += scale * (dS.T @ q[r, h, :])
        Wk = W_UK[:, h * d_nope:(h + 1) * d_nope]
        Wv = W_UV[:, h * d_v:(h + 1) * d_v]
        dK_nope = dK[:, :d_nope]
        dk_rope[k0:k1] += dK[:, d_nope:]
        dc_kv[k0:k1] += dK_nope @ Wk.T + dV @ Wv.T
        dW_UK[:, h * d_nope:(h + 1) * d_nope] = c_kv[k0:k1].T @ dK_nope
        dW_UV[:, h * d_v:(h + 1) * d_v] = c_kv[k0:k1].T @ dV
    return dq, dc_kv, dk_rope, dW_UK, dW_UV
