"""Write the text fixtures under tests/golden/.

Calls only the seeded input generator (workloads) and the fp64 oracle;
nothing here touches the GPU library. Run from the repository root:

    python tests/golden/make_golden.py
"""

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads  # noqa: E402


def write_cu_seqlens():
    cfg = workloads.config("h128_varlen64k")
    cu = cfg.cu_seqlens()
    path = os.path.join(HERE, "varlen64k_cu_seqlens.txt")
    with open(path, "w") as f:
        f.write("# Packed-sample boundaries of the 65536-token varlen workload.\n")
        f.write("# Lengths ~ clip(round(exp(ln 2048 + 1.0 z)), 1, 32768), z drawn one at a\n")
        f.write("# time from numpy default_rng(0); the last sample is cut so the total is\n")
        f.write("# 65536. Stand-in for the long-tailed packed training data of the Libra\n")
        f.write("# review page (Fig. 1; 'Axiom ledger', fixed-token packing).\n")
        f.write(" ".join(str(int(v)) for v in cu) + "\n")


def write_counts():
    path = os.path.join(HERE, "config_counts.txt")
    with open(path, "w") as f:
        f.write("# name visible_pairs_per_head keys_needed key_lo flops_fwd flops_bwd\n")
        f.write("# Counts from the fp64 oracle's mask (one sample's block-diagonal causal\n")
        f.write("# mask; LAGA abstract for the shard setting).\n")
        for name in workloads.CONFIG_ORDER:
            c = workloads.config(name)
            cu = c.cu_seqlens()
            P = oracle.visible_pairs(c.S_loc, c.q_offset, cu)
            lo, hi = oracle.key_range(c.S_loc, c.q_offset, cu)
            Ff = oracle.attention_flops(c.n_h, c.d_c, c.d_rope, c.d_nope, c.d_v,
                                        c.S_loc, c.q_offset, cu)
            Fb = oracle.attention_flops(c.n_h, c.d_c, c.d_rope, c.d_nope, c.d_v,
                                        c.S_loc, c.q_offset, cu, backward=True)
            f.write(f"{name} {P} {hi - lo} {lo} {Ff} {Fb}\n")


def write_tiny_samples():
    """A few oracle outputs of the tiny fp32 workload, as a regression pin."""
    cfg = workloads.config("tiny_f32")
    x = workloads.make_inputs(cfg, with_dout=True)
    args = [x[k] for k in ("q", "c_kv", "k_rope", "W_UK", "W_UV")]
    out, lse = oracle.mla_forward(*args)
    dq, dc, dkr, dwk, dwv = oracle.mla_backward(x["dout"], *args)
    rng = np.random.default_rng(123)
    path = os.path.join(HERE, "tiny_f32_samples.txt")
    with open(path, "w") as f:
        f.write("# tensor flat_index value (fp64 oracle on the tiny fp32 workload, seed 0)\n")
        for name, t in [("out", out), ("lse", lse), ("dq", dq), ("dc_kv", dc),
                        ("dk_rope", dkr), ("dW_UK", dwk), ("dW_UV", dwv)]:
            for k in sorted(rng.choice(t.size, size=6, replace=False)):
                f.write(f"{name} {int(k)} {float(t.reshape(-1)[k])!r}\n")


if __name__ == "__main__":
    write_cu_seqlens()
    write_counts()
    write_tiny_samples()
