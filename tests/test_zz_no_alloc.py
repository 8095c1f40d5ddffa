"""mla_laga_decode_noalloc: the decode with the library's static scratch
instead of a caller's workspace, for callers that cannot allocate device
memory. Called through the C ABI (ctypes) with buffers allocated up front;
its results must equal mla_laga_decode's bit for bit (same kernels, same
plan), on two calls in a row, the second with a smaller batch, so that the
second call runs over what the first left in the shared scratch.
"""

import ctypes

import numpy as np
import pytest
import torch

import head_latent_attention_kv_amd as hla
import workloads
from tests.gpu_helpers import announce, to_device


def _desc(cfg):
    d = hla.MLADecodeDesc()
    d.n_h, d.d_c, d.d_rope, d.d_nope, d.d_v = cfg.n_h, cfg.d_c, cfg.d_rope, cfg.d_nope, cfg.d_v
    d.batch, d.S = cfg.S_loc, cfg.S
    d.in_dtype = hla.MLA_BF16
    d.softmax_scale = 0.0
    return d


def test_noalloc_rejects_a_decode_larger_than_its_scratch():
    """Host-side check before anything is enqueued: 1024 sequences of 4096
    rows at 128 heads need more than the static scratch holds. The pointers
    are never dereferenced (the call fails on the size first)."""
    lib = hla.load_library()
    cfg = workloads.decode_config("too_big", 128, [4096] * 1024)
    cu = cfg.cu_seqlens()
    d = _desc(cfg)
    need = hla.mla_laga_decode_workspace_size(d, cu)
    assert need > hla.MLA_DECODE_NOALLOC_MAX_BYTES
    fake = ctypes.c_void_p(1 << 20)   # 16-byte aligned, never read
    st = lib.mla_laga_decode_noalloc(ctypes.byref(d), fake, fake, fake, fake, fake,
                                     cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), fake,
                                     fake, fake, None)
    assert st == hla.MLA_ERR_WORKSPACE
    assert "static scratch" in lib.mla_laga_last_error().decode()


@pytest.mark.gpu
def test_noalloc_decode_equals_workspace_decode_twice():
    lib = hla.load_library()
    for lens in ([700, 1, 2500, 64, 300, 4097], [33, 5, 200]):
        cfg = workloads.decode_config("noalloc", 64, lens, seed=9 + len(lens))
        announce(f"decode_noalloc n_h=64 lens={lens}")
        x = workloads.make_inputs(cfg, with_dout=False)
        dev = to_device(x, cfg, names=("q", "c_kv", "k_rope", "W_UK", "W_UV"))
        args = [dev[k] for k in ("q", "c_kv", "k_rope", "W_UK", "W_UV")]
        cu = cfg.cu_seqlens()
        ref_out, ref_lse = hla.mla_laga_decode(*args, cu)
        cu_dev = torch.from_numpy(cu).cuda()
        out = torch.full((cfg.S_loc, 64, 128), 7.0, dtype=torch.float32, device="cuda")
        lse = torch.full((cfg.S_loc, 64), 7.0, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        d = _desc(cfg)
        stream = torch.cuda.current_stream().cuda_stream
        st = lib.mla_laga_decode_noalloc(
            ctypes.byref(d), *[ctypes.c_void_p(t.data_ptr()) for t in args],
            cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), ctypes.c_void_p(cu_dev.data_ptr()),
            ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(lse.data_ptr()),
            ctypes.c_void_p(stream))
        assert st == hla.MLA_OK, lib.mla_laga_last_error().decode()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref_out.cpu().numpy())
        assert np.array_equal(lse.cpu().numpy(), ref_lse.cpu().numpy())
