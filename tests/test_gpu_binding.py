"""The binding refuses tensors the library would read or write past: every
per-call tensor of a forward or backward (inputs, dout, out, lse, caller
gradients) is checked for shape, dtype, contiguity and device before the
library is called. Each case raises ValueError, and the output buffers the
call would have written keep their contents (nothing was launched)."""

import pytest
import torch

import head_latent_attention_kv_amd as hla
import workloads
from tests.gpu_helpers import announce, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def prepared():
    cfg = workloads.MLAConfig("binding", n_h=2, S=300, S_loc=200, q_offset=100, dtype="bf16",
                              backward=True, d_c=512, d_rope=64, d_nope=128, d_v=128)
    x = workloads.make_inputs(cfg, with_dout=True)
    dev = to_device(x, cfg)
    a = [dev[k] for k in ("q", "c_kv", "k_rope", "W_UK", "W_UV")]
    call = hla.MLACall(*a, q_offset=cfg.q_offset, backward=True)
    out, lse = call.fwd(*a)
    torch.cuda.synchronize()
    return cfg, dev, a, call, out, lse


def _raises(fn, *args, **kw):
    with pytest.raises(ValueError) as e:
        fn(*args, **kw)
    return str(e.value)


def test_forward_rejects_bad_tensors(prepared):
    cfg, dev, a, call, out, lse = prepared
    announce("binding forward checks")
    q, c_kv, k_rope, W_UK, W_UV = a
    # inputs: dtype, shape, contiguity, device
    assert "q" in _raises(call.fwd, q.float(), c_kv, k_rope, W_UK, W_UV)
    assert "c_kv" in _raises(call.fwd, q, c_kv[:-1], k_rope, W_UK, W_UV)
    assert "contiguous" in _raises(call.fwd, q, c_kv, k_rope, W_UK.t().contiguous().t(), W_UV)
    assert "device" in _raises(call.fwd, q, c_kv.cpu(), k_rope, W_UK, W_UV)
    # outputs: dtype and shape
    sentinel = torch.full_like(out, 7.0)
    lse_s = torch.full_like(lse, 7.0)
    assert "out" in _raises(call.fwd, *a, out=sentinel.to(torch.bfloat16), lse=lse_s)
    assert "lse" in _raises(call.fwd, *a, out=sentinel, lse=lse_s[:-1])
    assert "out" in _raises(call.fwd, *a, out=sentinel[:, :, :64], lse=lse_s)
    torch.cuda.synchronize()
    assert bool((sentinel == 7.0).all()) and bool((lse_s == 7.0).all())


def test_backward_rejects_bad_tensors(prepared):
    cfg, dev, a, call, out, lse = prepared
    announce("binding backward checks")
    dout = dev["dout"]
    # dout: the input dtype (an fp32 dout would be read as bf16) and shape
    assert "dout" in _raises(call.bwd, dout.float(), *a, out, lse)
    assert "dout" in _raises(call.bwd, dout[:-1], *a, out, lse)
    assert "dout" in _raises(call.bwd, dout.transpose(0, 1).contiguous().transpose(0, 1), *a, out, lse)
    # out and lse as the forward wrote them: fp32 and their shapes
    assert "out" in _raises(call.bwd, dout, *a, out.to(torch.bfloat16), lse)
    assert "lse" in _raises(call.bwd, dout, *a, out, lse[:, :1].contiguous())
    # caller gradients: fp32, shapes, contiguity
    f32 = dict(dtype=torch.float32, device="cuda")
    good = [torch.full((cfg.S_loc, cfg.n_h, 192), 7.0, **f32), torch.full((cfg.S, 512), 7.0, **f32),
            torch.full((cfg.S, 64), 7.0, **f32), torch.full((512, cfg.n_h * 128), 7.0, **f32),
            torch.full((512, cfg.n_h * 128), 7.0, **f32)]
    names = ("dq", "dc_kv", "dk_rope", "dW_UK", "dW_UV")
    for k, name in enumerate(names):
        bad = list(good)
        bad[k] = good[k].to(torch.bfloat16)
        assert name in _raises(call.bwd, dout, *a, out, lse, grads=tuple(bad))
        bad[k] = good[k].reshape(-1)[1:]
        assert name in _raises(call.bwd, dout, *a, out, lse, grads=tuple(bad))
    assert "grads" in _raises(call.bwd, dout, *a, out, lse, grads=tuple(good[:4]))
    torch.cuda.synchronize()
    assert all(bool((g == 7.0).all()) for g in good)
    # and the good buffers still work
    call.bwd(dout, *a, out, lse, grads=tuple(good))
    torch.cuda.synchronize()
    assert all(bool(torch.isfinite(g).all()) and not bool((g == 7.0).all()) for g in good[:2])
