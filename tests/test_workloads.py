"""The seeded input generator and the stored fixtures."""

import math
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_golden_ints(name):
    with open(os.path.join(GOLDEN, name)) as f:
        lines = [ln for ln in f if not ln.startswith("#")]
    return lines


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 65504.0, 1e-40,
                  np.inf, -np.inf, 3.0 + 2 ** -7], np.float32)
    bits = workloads.f32_to_bf16_bits(x)
    back = workloads.bf16_bits_to_f32(bits)
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.0 + 2 ** -6
    assert back[3] == -2.5 and np.isinf(back[6]) and np.isinf(back[7])
    assert back[8] == 3.0  # 3 + 2^-7 is a tie at bf16 spacing 2^-6 -> even
    assert np.isnan(workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(np.array([np.nan], np.float32))))[0]
    # matches torch's conversion on random values
    import torch
    r = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 100
    tb = torch.from_numpy(r).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(tb, workloads.f32_to_bf16_bits(r))


def test_inputs_deterministic_and_distributed():
    cfg = workloads.config("h16_s4k").with_(S=512, S_loc=512)
    a = workloads.make_inputs(cfg)
    b = workloads.make_inputs(cfg)
    for k in ("q", "c_kv", "k_rope", "W_UK", "W_UV"):
        assert np.array_equal(a[k], b[k])
    assert abs(a["q"].std() - 1.0) < 0.01
    assert abs(a["W_UK"].std() * math.sqrt(512) - 1.0) < 0.01
    assert a["q"].shape == (512, 16, 192) and a["W_UV"].shape == (512, 16 * 128)
    # values are exactly bf16
    assert np.array_equal(workloads.bf16_bits_to_f32(a["q_bits"]), a["q"])


def test_varlen_boundaries_fixture():
    line = read_golden_ints("varlen64k_cu_seqlens.txt")[0]
    cu = np.array([int(v) for v in line.split()])
    got = workloads.config("h128_varlen64k").cu_seqlens()
    assert np.array_equal(cu, got)
    lens = np.diff(cu)
    assert cu[0] == 0 and cu[-1] == 65536 and len(lens) == 25 and lens.max() == 8031


def test_config_counts_fixture():
    rows = {ln.split()[0]: [int(v) for v in ln.split()[1:]]
            for ln in read_golden_ints("config_counts.txt")}
    # independent figures for these shapes: n(n+1)/2 for full causal
    # sequences, S_loc*q_off + S_loc(S_loc+1)/2 for a shard, and for the
    # packed shard the pairs counted sample by sample
    assert rows["h16_s4k"][0] == 4096 * 4097 // 2
    assert rows["h128_s8k_bwd"][0] == 8192 * 8193 // 2
    assert rows["h128_s16k_shard"][0] == 2048 * 14336 + 2048 * 2049 // 2
    cu = workloads.config("h128_varlen64k").cu_seqlens()
    pairs = 0
    for a, b in zip(cu[:-1], cu[1:]):
        lo, hi = max(a, 57344), min(b, 65536)
        if hi > lo:   # rows lo..hi-1 of sample [a,b) see keys a..p
            pairs += sum(p - a + 1 for p in range(lo, hi))
    assert rows["h128_varlen64k"][0] == pairs == 15_619_141
    assert rows["h128_varlen64k"][1] == 65536 - 56898 == 8638
    for name in workloads.CONFIG_ORDER:
        c = workloads.config(name)
        cu = c.cu_seqlens()
        assert rows[name][0] == oracle.visible_pairs(c.S_loc, c.q_offset, cu)
        assert rows[name][3] == oracle.attention_flops(c.n_h, c.d_c, c.d_rope, c.d_nope, c.d_v,
                                                       c.S_loc, c.q_offset, cu)


def test_tiny_oracle_samples_fixture():
    cfg = workloads.config("tiny_f32")
    x = workloads.make_inputs(cfg, with_dout=True)
    args = [x[k] for k in ("q", "c_kv", "k_rope", "W_UK", "W_UV")]
    out, lse = oracle.mla_forward(*args)
    g = oracle.mla_backward(x["dout"], *args)
    t = dict(out=out, lse=lse, dq=g[0], dc_kv=g[1], dk_rope=g[2], dW_UK=g[3], dW_UV=g[4])
    for ln in read_golden_ints("tiny_f32_samples.txt"):
        name, k, v = ln.split()
        assert abs(t[name].reshape(-1)[int(k)] - float(v)) <= 1e-12 * max(1.0, abs(float(v)))
