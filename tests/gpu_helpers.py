"""Shared helpers for the GPU parity tests (inputs to device, error metrics)."""

import sys

import numpy as np
import torch

import workloads

# Bar for every checked tensor (bf16 inputs): max |x - ref| and the ratio of
# means sum|x - ref| / sum|ref|.
MAX_ABS = 2e-2
MEAN_REL = 1e-3


def announce(msg: str):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_device(x: dict, cfg: workloads.MLAConfig, names=("q", "c_kv", "k_rope", "W_UK", "W_UV", "dout")):
    out = {}
    for n in names:
        if n not in x:
            continue
        if cfg.dtype == "bf16":
            t = torch.from_numpy(x[n + "_bits"].view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(x[n]))
        out[n] = t.to("cuda").contiguous()
    return out


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite values in GPU output"
    d = np.abs(got - ref)
    denom = np.sum(np.abs(ref))
    return float(d.max()) if d.size else 0.0, float(d.sum() / denom) if denom > 0 else float(d.sum())


def check(name, got, ref, max_abs=MAX_ABS, mean_rel=MEAN_REL):
    ma, mr = errors(got, ref)
    print(f"    {name:8s} max_abs={ma:.3e} mean_rel={mr:.3e}", flush=True)
    assert ma <= max_abs, f"{name}: max_abs {ma:.3e} > {max_abs}"
    assert mr <= mean_rel, f"{name}: mean_rel {mr:.3e} > {mean_rel}"
    return ma, mr
