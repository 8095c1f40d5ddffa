"""GPU parity of the training path (the backward), beyond the per-shape
elementwise cases of test_gpu_parity.py.

- Every head active at the full head count: dc_kv sums over 2 * 128 per-head
  products of 128-wide rows (a 32768-deep reduction) and dk_rope over 128
  heads, so both are compared with the oracle when all heads contribute.
- The scale of dout: the fast backward holds dout, dP, dS and the per-key
  gradient rows in fp16 after an exact power-of-two prescale. Gradients of
  realistic size (dout far below 2^-14) must meet the same bar, and scaling
  dout by 2^-k must scale every gradient by 2^-k bit for bit.
- The benchmark's own workload (n_h = 128, 16384 keys, 2048 rows at 14336):
  its latent and rope-key gradients on sampled heads (dout zero on the other
  heads) and its weight-gradient blocks, in the benchmark's launch
  configuration.
"""

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import announce, check
from tests.test_gpu_parity import DSV3, GRADS, oracle_args, positions, run

pytestmark = pytest.mark.gpu

ALL = ("out", "lse") + GRADS

FULL_HEADS = [
    workloads.MLAConfig("h128_causal_1536", n_h=128, S=1536, S_loc=1536, q_offset=0,
                        dtype="bf16", backward=True, seed=11, **DSV3),
    # a packed shard: samples of 300, 1 and 800 tokens before it, the shard
    # starting inside the fourth sample
    workloads.MLAConfig("h128_packed_shard", n_h=128, S=2048, S_loc=1024, q_offset=1024,
                        dtype="bf16", backward=True, seed=12, seq_lens=(300, 1, 800, 947),
                        **DSV3),
]


def scaled(x, k):
    """x with dout multiplied by 2^-k (exact in bf16 for these magnitudes)."""
    d = x["dout"] * np.float32(2.0 ** -k)
    bits = workloads.f32_to_bf16_bits(d)
    assert np.array_equal(workloads.bf16_bits_to_f32(bits), d)
    return dict(x, dout=d, dout_bits=bits)


@pytest.mark.parametrize("stored_ds", [False, True], ids=["default", "stored_ds"])
@pytest.mark.parametrize("cfg", FULL_HEADS, ids=[c.name for c in FULL_HEADS])
def test_all_heads_active_every_output(cfg, stored_ds):
    cu = cfg.cu_seqlens()
    announce(f"{cfg.name} all 128 heads, every output, stored_ds={stored_ds}")
    x = workloads.make_inputs(cfg, with_dout=True)
    g = run(cfg, x, cu, backward=True, stored_ds=stored_ds)
    assert g["fast"]
    ro, rl = oracle.mla_forward(*oracle_args(x), cu_seqlens=cu, **positions(cfg))
    rg = oracle.mla_backward(x["dout"], *oracle_args(x), cu_seqlens=cu, **positions(cfg))
    for name, ref in zip(ALL, (ro, rl) + tuple(rg)):
        check(name, g[name], ref)


@pytest.mark.parametrize("k", [12, 20])
def test_small_dout_scale(k):
    """dout scaled by 2^-k: gradients equal 2^-k times those of dout, bit for
    bit, and meet the bar against the oracle run on the scaled dout."""
    cfg = FULL_HEADS[1]
    cu = cfg.cu_seqlens()
    announce(f"{cfg.name} dout x 2^-{k}")
    x = workloads.make_inputs(cfg, with_dout=True)
    base = run(cfg, x, cu, backward=True)
    xs = scaled(x, k)
    g = run(cfg, xs, cu, backward=True)
    for name in GRADS:
        assert np.array_equal(g[name], base[name] * np.float32(2.0 ** -k)), name
    rg = oracle.mla_backward(xs["dout"], *oracle_args(x), cu_seqlens=cu, **positions(cfg))
    for name, ref in zip(GRADS, rg):
        check(name, g[name], ref)


def test_large_dout_scale():
    """dout scaled up by 2^10: the prescale brings it back down (bit-exact
    scaling again)."""
    cfg = FULL_HEADS[0].with_(n_h=16, S=700, S_loc=700)
    announce(f"{cfg.name} dout x 2^10")
    x = workloads.make_inputs(cfg, with_dout=True)
    base = run(cfg, x, backward=True)
    g = run(cfg, scaled(x, -10), backward=True)
    for name in GRADS:
        assert np.array_equal(g[name], base[name] * np.float32(1024.0)), name


@pytest.mark.parametrize("k", [12])
def test_varlen64k_backward_scaled_dout_sampled_heads(k):
    """The packed 65536-token workload's backward with dout on two heads only
    (zero elsewhere), so that the latent and rope-key gradients are the
    sampled heads' own; dout scaled by 2^-k."""
    cfg = workloads.config("h128_varlen64k")
    cu = cfg.cu_seqlens()
    heads = [17, 100]
    announce(f"{cfg.name} fwd+bwd, dout x 2^-{k} on heads {heads}")
    x = workloads.make_inputs(cfg, with_dout=True)
    dz = np.zeros_like(x["dout"])
    dz[:, heads] = x["dout"][:, heads] * np.float32(2.0 ** -k)
    x0 = dict(x, dout=dz, dout_bits=workloads.f32_to_bf16_bits(dz))
    g = run(cfg, x0, cu, backward=True)
    assert g["fast"]
    rg = oracle.mla_backward(dz, *oracle_args(x), cu_seqlens=cu, heads=heads, **positions(cfg))
    for nm, ref in zip(GRADS, rg):
        if nm == "dq":
            check(nm, g[nm][:, heads], ref[:, heads])
        else:
            check(nm, g[nm], ref)


def test_benchmark_shard_backward_sampled_heads():
    """The benchmark workload's backward in its launch configuration: dc_kv,
    dk_rope and the weight gradients with dout on two heads (zero elsewhere:
    the sums over heads are then the sampled heads' own), and dq on those
    heads."""
    cfg = workloads.config("h128_s16k_shard")
    heads = [3, 90]
    announce(f"{cfg.name} fwd+bwd, dout only on heads {heads}")
    x = workloads.make_inputs(cfg, with_dout=True)
    dz = np.zeros_like(x["dout"])
    dz[:, heads] = x["dout"][:, heads]
    x0 = dict(x, dout=dz, dout_bits=workloads.f32_to_bf16_bits(dz))
    g = run(cfg, x0, backward=True)
    assert g["fast"]
    rg = oracle.mla_backward(dz, *oracle_args(x), heads=heads, **positions(cfg))
    for nm, ref in zip(GRADS, rg):
        if nm == "dq":
            check(nm, g[nm][:, heads], ref[:, heads])
        else:
            check(nm, g[nm], ref)
