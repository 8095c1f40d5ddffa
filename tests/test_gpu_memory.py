"""Device memory of the block (the LAGA abstract's claim is about training
memory: rebuilding K/V from the latent keeps the explicit form's activation
memory, while the absorbed form inflates it).

The library allocates nothing itself: every byte is the caller's, through
torch's caching allocator here. So the peaks of the bytes requested from
the allocator (torch's requested_bytes statistics, which count what was
asked for rather than the cached blocks that serve it) must equal the sizes
the library reports and the output tensors, exactly:
  forward:  workspace + out + lse (+ the device copy of cu_seqlens);
  held from forward to backward: out + lse only (the rebuilt K/V are not kept);
  backward: workspace + the five gradients, for the default backward
            (dQ recomputes the scores: no rows x keys term) and for the
            stored-dS form (its workspace holds one fp16 dS value per
            local row, needed key and head more, or, past 16 GiB of that,
            two buffers of one head group each).
"""

import pytest
import torch

import head_latent_attention_kv_amd as hla
import workloads
from tests.gpu_helpers import announce, to_device
from tests.test_abi import stored_ds_bytes

pytestmark = pytest.mark.gpu


def rounded(nbytes):
    """Bytes torch requests for a tensor of `nbytes` (no rounding)."""
    return int(nbytes)


def requested():
    return torch.cuda.memory_stats()["requested_bytes.all.current"]


def peak_of(fn):
    torch.cuda.synchronize()
    before = requested()
    torch.cuda.reset_peak_memory_stats()
    res = fn()
    torch.cuda.synchronize()
    peak = torch.cuda.memory_stats()["requested_bytes.all.peak"]
    return res, peak - before, requested() - before


CASES = [
    workloads.MLAConfig("mem_shard", n_h=16, S=4096, S_loc=1024, q_offset=3072, dtype="bf16",
                        backward=True, d_c=512, d_rope=64, d_nope=128, d_v=128),
    workloads.MLAConfig("mem_packed", n_h=8, S=3000, S_loc=1000, q_offset=2000, dtype="bf16",
                        backward=True, seq_lens=(700, 1, 1299, 1000), d_c=512, d_rope=64,
                        d_nope=128, d_v=128),
    # 16.25 GiB of dS: the stored form runs 17 head groups through two buffers
    workloads.MLAConfig("mem_ds_groups", n_h=130, S=16384, S_loc=4096, q_offset=12288,
                        dtype="bf16", backward=True, d_c=64, d_rope=64, d_nope=128, d_v=128),
]


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_allocator_peaks_equal_the_reported_sizes(cfg):
    announce(f"memory {cfg.name}")
    cu = cfg.cu_seqlens()
    x = workloads.make_inputs(cfg, with_dout=True)
    dev = to_device(x, cfg)
    a = [dev[k] for k in ("q", "c_kv", "k_rope", "W_UK", "W_UV")]
    torch.cuda.empty_cache()
    f32 = 4
    out_b = rounded(cfg.S_loc * cfg.n_h * cfg.d_v * f32)
    lse_b = rounded(cfg.S_loc * cfg.n_h * f32)
    cu_b = 0 if cu is None else rounded(len(cu) * 4)   # the device copy of cu_seqlens
    grads_b = sum(rounded(n * f32) for n in (
        cfg.S_loc * cfg.n_h * (cfg.d_nope + cfg.d_rope), cfg.S * cfg.d_c, cfg.S * cfg.d_rope,
        cfg.d_c * cfg.n_h * cfg.d_nope, cfg.d_c * cfg.n_h * cfg.d_v))

    def fwd():
        call = hla.MLACall(*a, q_offset=cfg.q_offset, cu_seqlens=cu)
        out, lse = call.fwd(*a)
        return call, out, lse

    (call, out, lse), fpeak, _ = peak_of(fwd)
    ws_f = hla.mla_laga_fwd_workspace_size(call.desc, call.cu)
    assert fpeak == rounded(ws_f) + cu_b + out_b + lse_b
    del call
    torch.cuda.synchronize()
    # what stays from forward to backward: out and lse
    held = out.numel() * 4 + lse.numel() * 4
    assert rounded(out.numel() * 4) + rounded(lse.numel() * 4) == out_b + lse_b
    assert held == cfg.S_loc * cfg.n_h * (cfg.d_v + 1) * 4

    sizes = {}
    for stored in (False, True):
        def bwd():
            c = hla.MLACall(*a, q_offset=cfg.q_offset, cu_seqlens=cu, backward=True,
                            stored_ds=stored)
            g = c.bwd(dev["dout"], *a, out, lse)
            return c, g
        (c, g), bpeak, _ = peak_of(bwd)
        ws_b = hla.mla_laga_bwd_workspace_size(c.desc, c.cu)
        assert c.ws_bwd.numel() == max(ws_b, 1)
        # the forward workspace MLACall also allocates up front
        assert bpeak == rounded(ws_b) + rounded(hla.mla_laga_fwd_workspace_size(c.desc, c.cu)) + \
            cu_b + grads_b
        sizes[stored] = ws_b
        del c, g
        torch.cuda.empty_cache()
    # the stored-dS workspace is the default one plus dS: one fp16 value per
    # (row padded to 64, needed key padded to 256, head) of all heads or of
    # two head groups
    pairs, k_lo, k_hi = hla.mla_laga_count(hla.MLACall(*a, q_offset=cfg.q_offset,
                                                       cu_seqlens=cu).desc, cu)
    ds = stored_ds_bytes(cfg.n_h, k_hi - k_lo, cfg.S_loc)
    assert ds > 0
    assert sizes[True] - sizes[False] == (ds + 255) // 256 * 256
