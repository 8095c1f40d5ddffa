"""Seeded synthetic workloads for the latent-attention block.

This module only draws random numbers and packs them into arrays. It holds
none of the attention arithmetic: both the fp64 oracle (under ``oracle/``) and
the GPU library's tests and benchmark take their inputs from here, and nothing
here depends on either of them.

Workload shapes follow the five configurations the library is checked on:
DeepSeek-V3-sized MLA heads (latent width 512, shared RoPE key 64, per-head
no-position key 128 and value 128, so a query row is 192 wide), one sequence-
parallel query shard per call, and a packed variable-length case whose sample
lengths are long-tailed (lognormal) as in the packed-training workloads the
Libra review describes (pith.science review of Libra, "Axiom ledger", fixed-
token packing with a block-diagonal causal mask; Fig. 1, long-tailed length
distributions).

Conventions (each is a reading, recorded with the design notes):
  * every tensor is drawn as float32 from ``numpy.random.default_rng(seed)``
    (PCG64) with ``standard_normal`` and scaled by its standard deviation;
  * N(0, 1/d_c) names the variance, so the weights' std is 1/sqrt(d_c);
  * one generator draws, in this order: q, c_kv, k_rope, W_UK, W_UV, dout;
  * bf16 configurations round each float32 value to bf16 with
    round-to-nearest-even; the oracle then reads those exact bf16 values.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np

__all__ = [
    "MLAConfig",
    "CONFIGS",
    "config",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "lognormal_lengths",
    "cu_seqlens_from_lengths",
    "make_inputs",
    "zigzag_blocks",
    "decode_config",
    "lognormal_count",
    "DECODE_CONFIGS",
]


@dataclasses.dataclass(frozen=True)
class MLAConfig:
    """Shape of one call: one query shard of a (possibly packed) sequence."""

    name: str
    n_h: int
    d_c: int
    d_rope: int
    d_nope: int
    d_v: int
    S: int            # latent (key) length
    S_loc: int        # number of local query rows
    q_offset: int     # global position of local row 0
    dtype: str        # "bf16" or "f32" (input precision)
    backward: bool = False
    # packed variable-length samples (None: one causal sequence over [0, S))
    varlen_median: Optional[int] = None
    varlen_sigma: Optional[float] = None
    varlen_cap: Optional[int] = None
    seed: int = 0
    # several position blocks instead of [q_offset, q_offset + S_loc): a
    # tuple of (start, length); q_offset is then 0
    q_ranges: Optional[Tuple[Tuple[int, int], ...]] = None
    # explicit sample lengths (packed samples; overrides the lognormal draw)
    seq_lens: Optional[Tuple[int, ...]] = None

    @property
    def d_qk(self) -> int:
        return self.d_nope + self.d_rope

    def with_(self, **kw) -> "MLAConfig":
        return dataclasses.replace(self, **kw)

    def cu_seqlens(self) -> Optional[np.ndarray]:
        if self.seq_lens is not None:
            return cu_seqlens_from_lengths(self.seq_lens)
        if self.varlen_median is None:
            return None
        lens = lognormal_lengths(self.S, self.varlen_median, self.varlen_sigma,
                                 self.varlen_cap, self.seed)
        return cu_seqlens_from_lengths(lens)


_DSV3 = dict(d_c=512, d_rope=64, d_nope=128, d_v=128)


def zigzag_blocks(S: int, rank: int, world: int) -> Tuple[Tuple[int, int], ...]:
    """Zigzag sequence-parallel shard: of 2*world equal position blocks, rank
    r holds blocks r and 2*world-1-r, which evens out causal work (Libra
    review page, Related Work beside Fig. 15: ring schemes arrange shards
    against causal imbalance)."""
    C = S // (2 * world)
    return ((rank * C, C), ((2 * world - 1 - rank) * C, C))


CONFIGS: Dict[str, MLAConfig] = {
    # tiny fp32 case, all queries local
    "tiny_f32": MLAConfig("tiny_f32", n_h=4, d_c=32, d_rope=8, d_nope=16, d_v=16,
                          S=128, S_loc=128, q_offset=0, dtype="f32"),
    # DeepSeek-V3 per-head dims, 16 heads, full causal sequence of 4096
    "h16_s4k": MLAConfig("h16_s4k", n_h=16, S=4096, S_loc=4096, q_offset=0,
                         dtype="bf16", **_DSV3),
    # full head count, last of 8 contiguous shards of a 16384-long sequence
    "h128_s16k_shard": MLAConfig("h128_s16k_shard", n_h=128, S=16384, S_loc=2048,
                                 q_offset=14336, dtype="bf16", **_DSV3),
    # full head count, forward + backward, 8192 causal
    "h128_s8k_bwd": MLAConfig("h128_s8k_bwd", n_h=128, S=8192, S_loc=8192,
                              q_offset=0, dtype="bf16", backward=True, **_DSV3),
    # packed varlen, 65536 tokens of lognormal samples, last 8192-query shard
    "h128_varlen64k": MLAConfig("h128_varlen64k", n_h=128, S=65536, S_loc=8192,
                                q_offset=57344, dtype="bf16", backward=True,
                                varlen_median=2048, varlen_sigma=1.0,
                                varlen_cap=32768, **_DSV3),
}

# further parity and measurement cases beyond the five configurations:
# zigzag ranks of the 16384-long sequence over 8 ranks. Rank 0 holds blocks
# 0 and 15 (it rebuilds K/V for every latent row); every rank sees the same
# number of pairs.
for _r in (0, 7):
    CONFIGS[f"h128_s16k_zigzag_r{_r}"] = MLAConfig(
        f"h128_s16k_zigzag_r{_r}", n_h=128, S=16384, S_loc=2048, q_offset=0, dtype="bf16",
        backward=True, q_ranges=zigzag_blocks(16384, _r, 8), **_DSV3)



# the five configurations, in the order they are listed with the method's targets
CONFIG_ORDER: List[str] = ["tiny_f32", "h16_s4k", "h128_s16k_shard",
                           "h128_s8k_bwd", "h128_varlen64k"]


def config(name: str) -> MLAConfig:
    return CONFIGS[name]


# ---------------------------------------------------------------- bf16 bytes
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even.

    NaN inputs become a quiet NaN; this is a storage conversion, not part of
    the method.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded = rounded.copy()
        rounded[nan] = 0x7FC0
    return rounded


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------- packed lengths
def lognormal_lengths(total: int, median: int, sigma: float, cap: int,
                      seed: int = 0) -> List[int]:
    """Sample lengths L_k = clip(round(exp(ln(median) + sigma*z_k)), 1, cap).

    z_k is drawn one at a time from a fresh ``default_rng(seed)``; sampling
    stops once the lengths reach ``total`` and the last one is cut so that
    they sum to exactly ``total``.
    """
    rng = np.random.default_rng(seed)
    lens: List[int] = []
    acc = 0
    mu = math.log(median)
    while acc < total:
        z = float(rng.standard_normal())
        L = int(round(math.exp(mu + sigma * z)))
        L = max(1, min(cap, L))
        L = min(L, total - acc)
        lens.append(L)
        acc += L
    return lens


def cu_seqlens_from_lengths(lens) -> np.ndarray:
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lens, dtype=np.int64))
    return cu


# ------------------------------------------------------------------ inputs
def make_inputs(cfg: MLAConfig, seed: Optional[int] = None,
                with_dout: Optional[bool] = None) -> Dict[str, np.ndarray]:
    """Draw one call's inputs.

    Returns float32 arrays holding exactly the values the library receives:
    for bf16 configurations they are already rounded to bf16, and the raw
    bit patterns are returned too under ``<name>_bits``. Keys: q [S_loc,n_h,
    d_qk], c_kv [S,d_c], k_rope [S,d_rope], W_UK [d_c,n_h*d_nope],
    W_UV [d_c,n_h*d_v], and dout [S_loc,n_h,d_v] when requested.
    """
    seed = cfg.seed if seed is None else seed
    with_dout = cfg.backward if with_dout is None else with_dout
    rng = np.random.default_rng(seed)
    w_std = 1.0 / math.sqrt(cfg.d_c)
    shapes = [
        ("q", (cfg.S_loc, cfg.n_h, cfg.d_qk), 1.0),
        ("c_kv", (cfg.S, cfg.d_c), 1.0),
        ("k_rope", (cfg.S, cfg.d_rope), 1.0),
        ("W_UK", (cfg.d_c, cfg.n_h * cfg.d_nope), w_std),
        ("W_UV", (cfg.d_c, cfg.n_h * cfg.d_v), w_std),
    ]
    if with_dout:
        shapes.append(("dout", (cfg.S_loc, cfg.n_h, cfg.d_v), 1.0))
    out: Dict[str, np.ndarray] = {}
    for name, shape, std in shapes:
        x = rng.standard_normal(size=shape, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        if cfg.dtype == "bf16":
            bits = f32_to_bf16_bits(x)
            out[name + "_bits"] = bits
            out[name] = bf16_bits_to_f32(bits)
        else:
            out[name] = x
    cu = cfg.cu_seqlens()
    if cu is not None:
        out["cu_seqlens"] = cu
    return out

def decode_config(name: str, n_h: int, lens, seed: int = 0) -> MLAConfig:
    """Decode batch: one query per sequence, at the last position of its
    cached latent rows (the packed cache holds the sequences end to end).
    The query rows are those last positions, so the oracle reads them as
    one-row position blocks."""
    lens = tuple(int(x) for x in lens)
    cu = cu_seqlens_from_lengths(lens)
    last = tuple((int(cu[b + 1]) - 1, 1) for b in range(len(lens)))
    return MLAConfig(name, n_h=n_h, S=int(cu[-1]), S_loc=len(lens), q_offset=0, dtype="bf16",
                     seq_lens=lens, q_ranges=last, seed=seed, **_DSV3)


def lognormal_count(count: int, median: int, sigma: float, cap: int, seed: int = 0) -> List[int]:
    """`count` lengths clip(round(exp(ln(median) + sigma z)), 1, cap), z drawn
    one at a time from a fresh default_rng(seed)."""
    rng = np.random.default_rng(seed)
    mu = math.log(median)
    return [max(1, min(cap, int(round(math.exp(mu + sigma * float(rng.standard_normal()))))))
            for _ in range(count)]


# decode batches (absorbed form over the latent cache): 64 sequences of 8192
# cached rows, and 32 sequences of long-tailed lengths (median 4096)
DECODE_CONFIGS: Dict[str, MLAConfig] = {
    "decode_h128_b64_l8k": decode_config("decode_h128_b64_l8k", 128, [8192] * 64),
    "decode_h128_b32_mixed": decode_config("decode_h128_b32_mixed", 128,
                                           lognormal_count(32, 4096, 1.0, 32768, seed=0)),
}
CONFIGS.update(DECODE_CONFIGS)
