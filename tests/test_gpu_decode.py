"""GPU parity of the decode path (absorbed form over the latent cache).

Each decode query sits at the last position of its sequence's cached latent
rows, so the fp64 oracle's explicit form with one-row position blocks at
those positions is the reference (the absorbed and explicit forms are the
same function; the oracle pins that). Small batches are compared element by
element, the full-size batches on sampled heads; the mask is checked
exactly with q = 0.
"""

import numpy as np
import pytest
import torch

import head_latent_attention_kv_amd as hla
import oracle
import workloads
from tests.gpu_helpers import announce, check, to_device

pytestmark = pytest.mark.gpu


def run_decode(cfg, x, q_override=None):
    dev = to_device(x, cfg, names=("q", "c_kv", "k_rope", "W_UK", "W_UV"))
    q = dev["q"] if q_override is None else q_override
    out, lse = hla.mla_laga_decode(q, dev["c_kv"], dev["k_rope"], dev["W_UK"], dev["W_UV"],
                                   cfg.cu_seqlens())
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def reference(cfg, x, heads=None):
    return oracle.mla_forward(*[x[k] for k in ("q", "c_kv", "k_rope", "W_UK", "W_UV")],
                              cu_seqlens=cfg.cu_seqlens(), q_ranges=cfg.q_ranges, heads=heads)


SMALL = [
    # one block, ragged blocks, one-key sequences
    ("ragged", 32, [1, 2, 31, 32, 33, 95, 300]),
    # several key chunks per sequence (chunks are at least 256 keys)
    ("chunks", 64, [5000, 1, 700, 257]),
    # two head groups, the second one partly filled (160 heads)
    ("two_head_groups", 160, [129, 1030, 64]),
]


@pytest.mark.parametrize("name,n_h,lens", SMALL, ids=[s[0] for s in SMALL])
def test_decode_small_elementwise(name, n_h, lens):
    cfg = workloads.decode_config(f"dec_{name}", n_h, lens, seed=5)
    announce(f"decode {name} n_h={n_h} lens={lens}")
    x = workloads.make_inputs(cfg, with_dout=False)
    out, lse = run_decode(cfg, x)
    ro, rl = reference(cfg, x)
    check("out", out, ro)
    check("lse", lse, rl)


@pytest.mark.parametrize("name", list(workloads.DECODE_CONFIGS))
def test_decode_full_size_sampled_heads(name):
    cfg = workloads.config(name)
    heads = [0, 77]
    announce(f"{name} decode, heads {heads}")
    x = workloads.make_inputs(cfg, with_dout=False)
    out, lse = run_decode(cfg, x)
    ro, rl = reference(cfg, x, heads=heads)
    check("out", out[:, heads], ro)
    check("lse", lse[:, heads], rl)


@pytest.mark.parametrize("name", list(workloads.DECODE_CONFIGS) + ["ragged"])
def test_decode_mask_probe_exact_counts(name):
    """q = 0: every score is exactly 0, so exp(lse) is the sequence length."""
    if name == "ragged":
        cfg = workloads.decode_config("dec_probe", 32, [1, 2, 31, 32, 33, 95, 300, 4097])
    else:
        cfg = workloads.config(name)
    announce(f"decode mask probe {name}")
    x = workloads.make_inputs(cfg, with_dout=False)
    dev = to_device(x, cfg, names=("q",))
    _, lse = run_decode(cfg, x, q_override=torch.zeros_like(dev["q"]))
    counts = np.rint(np.exp(lse.astype(np.float64))).astype(np.int64)
    expect = np.asarray(cfg.seq_lens, np.int64)[:, None]
    bad = np.argwhere(counts != expect)
    assert bad.size == 0, f"{len(bad)} (sequence, head) with a wrong key count, first {bad[:3]}"


def test_decode_matches_explicit_library_path():
    """Up to 16 sequences fit the explicit path's position blocks: both library
    paths must agree with the oracle and with each other."""
    cfg = workloads.decode_config("dec_vs_explicit", 128, [300, 1, 1030, 64, 700], seed=9)
    announce("decode vs explicit path")
    x = workloads.make_inputs(cfg, with_dout=False)
    out, lse = run_decode(cfg, x)
    dev = to_device(x, cfg, names=("q", "c_kv", "k_rope", "W_UK", "W_UV"))
    eo, el = hla.mla_laga_fwd(dev["q"], dev["c_kv"], dev["k_rope"], dev["W_UK"], dev["W_UV"],
                              cu_seqlens=cfg.cu_seqlens(), q_ranges=cfg.q_ranges)
    torch.cuda.synchronize()
    check("out", out, eo.cpu().numpy())
    check("lse", lse, el.cpu().numpy())


def test_decode_graph_replays_match_eager():
    """Decode captured into a HIP graph (through torch) and replayed three
    times, with eager fills and host synchronisations between replays: every
    replay gives the eager call's bits."""
    cfg = workloads.decode_config("dec_graph", 64, [5000, 1, 700, 257], seed=6)
    announce("decode graph capture and replay")
    x = workloads.make_inputs(cfg, with_dout=False)
    dev = to_device(x, cfg, names=("q", "c_kv", "k_rope", "W_UK", "W_UV"))
    args = [dev[k] for k in ("q", "c_kv", "k_rope", "W_UK", "W_UV")]
    call = hla.MLADecodeCall(*args, cfg.cu_seqlens())
    out, lse = call(*args)
    torch.cuda.synchronize()
    ref_out, ref_lse = out.cpu().numpy(), lse.cpu().numpy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                  # warm-up off the default stream
        call(*args, out=out, lse=lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(*args, out=out, lse=lse)
    torch.cuda.synchronize()
    for _ in range(3):
        out.fill_(7.0)
        lse.fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref_out)
        assert np.array_equal(lse.cpu().numpy(), ref_lse)
