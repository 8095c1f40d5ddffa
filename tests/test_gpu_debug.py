"""The kernels' key windows, and debug mode.

Key windows: the first and last key each local row sees, as the library's
device code computes them (the row-to-position map and the sample-start
search every attention kernel uses), must equal the oracle's integers
exactly. Shapes: every workload, zigzag ranks, and packed shards whose rows
straddle sample starts, skip empty samples or lie in several blocks. This
complements the q = 0 count probe, which a window shifted by one key leaves
unchanged.

Debug mode (MLA_LAGA_DEBUG=1): outputs and the used workspace are filled
with NaN before the work, a canary follows the workspace, and the outputs
are scanned afterwards. Every path must pass those checks (no output left
unwritten, no workspace byte read before it is written, nothing written
past the workspace) and give the same bits as a normal call. NaN in an
input and a device copy of cu_seqlens that differs from the host copy are
reported with MLA_ERR_DEBUG_CHECK.
"""

import numpy as np
import pytest
import torch

import head_latent_attention_kv_amd as hla
import oracle
import workloads
from tests.gpu_helpers import announce, to_device

pytestmark = pytest.mark.gpu

DSV3 = dict(d_c=512, d_rope=64, d_nope=128, d_v=128)
GRADS = ("dq", "dc_kv", "dk_rope", "dW_UK", "dW_UV")


def meta_desc(cfg, cu):
    """Descriptor of a workload from shape-only tensors (nothing allocated)."""
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    m = lambda *s: torch.empty(s, dtype=dt, device="meta")  # noqa: E731
    return hla.make_desc(m(cfg.S_loc, cfg.n_h, cfg.d_nope + cfg.d_rope), m(cfg.S, cfg.d_c),
                         m(cfg.S, cfg.d_rope), m(cfg.d_c, cfg.n_h * cfg.d_v), cfg.q_offset, cu,
                         q_ranges=cfg.q_ranges)


def small(name, S, S_loc, q_offset, cu=None, q_ranges=None, n_h=2):
    if q_ranges is not None:
        S_loc, q_offset = sum(n for _, n in q_ranges), 0
    cfg = workloads.MLAConfig(name, n_h=n_h, S=S, S_loc=S_loc, q_offset=q_offset, dtype="bf16",
                              backward=True, seed=5, q_ranges=q_ranges, **DSV3)
    return cfg, (None if cu is None else np.array(cu, np.int32))


WINDOW_SHAPES = [(workloads.config(n), workloads.config(n).cu_seqlens())
                 for n in workloads.CONFIG_ORDER + ["h128_s16k_zigzag_r0", "h128_s16k_zigzag_r7"]]
WINDOW_SHAPES += [
    small("varlen_empty_samples", 600, 450, 150, cu=[0, 1, 1, 130, 131, 400, 600]),
    small("blocks_varlen", 600, 0, 0, cu=[0, 1, 1, 130, 131, 400, 600],
          q_ranges=((5, 120), (300, 200))),
    small("sixteen_blocks", 2000, 0, 0, cu=[0, 3, 400, 401, 1250, 2000],
          q_ranges=tuple((125 * k + 11 * (k % 3), 1 + 6 * k) for k in range(16))),
    small("single_row_samples", 64, 64, 0, cu=list(range(65))),
    small("last_row_only", 257, 1, 256),
]


@pytest.mark.parametrize("cfg,cu", WINDOW_SHAPES, ids=[c.name for c, _ in WINDOW_SHAPES])
def test_row_windows_equal_the_oracle(cfg, cu):
    announce(f"row window {cfg.name} S={cfg.S} S_loc={cfg.S_loc}")
    d, cu_h, _keep = meta_desc(cfg, cu)
    cu_dev = None if cu_h is None else torch.from_numpy(cu_h).cuda()
    w = hla.mla_laga_row_window(d, cu_h, cu_dev).cpu().numpy()
    lo, hi = oracle.visible_range(cfg.S_loc, cfg.q_offset, cu, cfg.q_ranges)
    assert w.shape == (cfg.S_loc, 2)
    bad = np.flatnonzero((w[:, 0] != lo) | (w[:, 1] != hi))
    assert bad.size == 0, f"{bad.size} rows differ, first row {bad[0]}: {w[bad[0]]} vs " \
                          f"({lo[bad[0]]}, {hi[bad[0]]})"


# ---------------------------------------------------------------- debug mode
DEBUG_SHAPES = [
    small("causal_ragged", 300, 300, 0),
    small("shard_ragged", 700, 333, 367, n_h=3),
    small("varlen_empty_samples", 600, 450, 150, cu=[0, 1, 1, 130, 131, 400, 600]),
    small("blocks_unseen_sample", 700, 0, 0, cu=[0, 200, 450, 700],
          q_ranges=((10, 150), (470, 200))),
    small("one_token", 1, 1, 0, n_h=1),
]


def run_all(cfg, cu, dev, generic, stored_ds):
    a = [dev[k] for k in ("q", "c_kv", "k_rope", "W_UK", "W_UV")]
    call = hla.MLACall(*a, q_offset=cfg.q_offset, cu_seqlens=cu, generic=generic, backward=True,
                       q_ranges=cfg.q_ranges, stored_ds=stored_ds)
    out, lse = call.fwd(*a)
    g = call.bwd(dev["dout"], *a, out, lse)
    torch.cuda.synchronize()
    return call, dict(zip(("out", "lse") + GRADS, [t.cpu().numpy() for t in (out, lse, *g)]))


@pytest.mark.parametrize("path", ["default", "stored_ds", "plain"])
@pytest.mark.parametrize("cfg,cu", DEBUG_SHAPES, ids=[c.name for c, _ in DEBUG_SHAPES])
def test_debug_mode_checks_pass_and_change_nothing(cfg, cu, path, monkeypatch):
    announce(f"debug mode {cfg.name} path={path}")
    x = workloads.make_inputs(cfg, with_dout=True)
    dev = to_device(x, cfg)
    kw = dict(generic=path == "plain", stored_ds=path == "stored_ds")
    monkeypatch.delenv("MLA_LAGA_DEBUG", raising=False)
    plain_call, ref = run_all(cfg, cu, dev, **kw)
    monkeypatch.setenv("MLA_LAGA_DEBUG", "1")
    dbg_call, got = run_all(cfg, cu, dev, **kw)
    # the debug tail: 256 bytes more workspace per call
    assert dbg_call.ws_fwd.numel() == plain_call.ws_fwd.numel() + 256
    assert dbg_call.ws_bwd.numel() == plain_call.ws_bwd.numel() + 256
    for k in ref:
        assert np.array_equal(got[k], ref[k]), k


@pytest.mark.parametrize("packed", [False, True], ids=["causal", "packed"])
def test_debug_mode_stored_ds_head_groups(packed, monkeypatch):
    """The head-grouped stored-dS backward (130 heads, 17 groups through two
    dS buffers) in debug mode. The workspace starts as NaN: with packed
    samples the dS blocks of the second sample's rows against earlier keys
    are written by no group, so a dQ that let them through would leave NaN
    in dq; the canary past the buffers checks the group offsets. Every
    output equals the plain call's bits."""
    from tests.test_gpu_parity import GROUPED
    cfg = GROUPED.with_(seq_lens=(16000, 384)) if packed else GROUPED
    cu = cfg.cu_seqlens()
    announce(f"debug mode, stored dS in head groups, packed={packed}")
    x = workloads.make_inputs(cfg, with_dout=True)
    dev = to_device(x, cfg)
    monkeypatch.delenv("MLA_LAGA_DEBUG", raising=False)
    plain_call, ref = run_all(cfg, cu, dev, generic=False, stored_ds=True)
    monkeypatch.setenv("MLA_LAGA_DEBUG", "1")
    dbg_call, got = run_all(cfg, cu, dev, generic=False, stored_ds=True)
    assert dbg_call.ws_bwd.numel() == plain_call.ws_bwd.numel() + 256
    for k in ref:
        assert np.array_equal(got[k], ref[k]), k


def test_debug_mode_reports_nan_inputs(monkeypatch):
    cfg, cu = small("nan_input", 300, 200, 100, cu=[0, 50, 180, 300])
    announce("debug mode NaN input")
    x = workloads.make_inputs(cfg, with_dout=True)
    dev = to_device(x, cfg)
    a = [dev[k] for k in ("q", "c_kv", "k_rope", "W_UK", "W_UV")]
    monkeypatch.setenv("MLA_LAGA_DEBUG", "1")
    call = hla.MLACall(*a, q_offset=cfg.q_offset, cu_seqlens=cu, backward=True)
    out, lse = call.fwd(*a)                     # clean inputs pass
    q_bad = a[0].clone()
    q_bad[5, 1, 0] = float("nan")               # row 5, head 1
    with pytest.raises(hla.MLAError) as e:
        call.fwd(q_bad, *a[1:])
    assert e.value.status == hla.MLA_ERR_DEBUG_CHECK
    assert f"out[{(5 * cfg.n_h + 1) * cfg.d_v}]" in str(e.value)
    dout_bad = dev["dout"].clone()
    dout_bad[7, 0, 3] = float("nan")            # row 7, head 0
    with pytest.raises(hla.MLAError) as e:
        call.bwd(dout_bad, *a, out, lse)
    assert e.value.status == hla.MLA_ERR_DEBUG_CHECK
    assert f"dq[{7 * cfg.n_h * (cfg.d_nope + cfg.d_rope)}]" in str(e.value)
    call.bwd(dev["dout"], *a, out, lse)         # and clean ones again
    torch.cuda.synchronize()


def test_debug_mode_compares_device_cu_seqlens(monkeypatch):
    cfg, cu = small("cu_mismatch", 300, 200, 100, cu=[0, 50, 180, 300])
    announce("debug mode cu_seqlens mismatch")
    x = workloads.make_inputs(cfg)
    dev = to_device(x, cfg)
    a = [dev[k] for k in ("q", "c_kv", "k_rope", "W_UK", "W_UV")]
    monkeypatch.setenv("MLA_LAGA_DEBUG", "1")
    call = hla.MLACall(*a, q_offset=cfg.q_offset, cu_seqlens=cu)
    # another valid partition on the device: the check fails before any launch
    call.cu_dev = torch.tensor([0, 60, 180, 300], dtype=torch.int32, device="cuda")
    with pytest.raises(hla.MLAError) as e:
        call.fwd(*a)
    assert e.value.status == hla.MLA_ERR_DEBUG_CHECK
    assert "cu_seqlens_dev[1] = 60" in str(e.value)


def test_debug_mode_decode(monkeypatch):
    cfg = workloads.decode_config("dbg_decode", 64, [700, 1, 2500, 64, 300], seed=21)
    announce("debug mode decode")
    x = workloads.make_inputs(cfg, with_dout=False)
    dev = to_device(x, cfg, names=("q", "c_kv", "k_rope", "W_UK", "W_UV"))
    a = [dev[k] for k in ("q", "c_kv", "k_rope", "W_UK", "W_UV")]
    cu = cfg.cu_seqlens()
    monkeypatch.delenv("MLA_LAGA_DEBUG", raising=False)
    ref = [t.cpu().numpy() for t in hla.mla_laga_decode(*a, cu)]
    monkeypatch.setenv("MLA_LAGA_DEBUG", "1")
    got = [t.cpu().numpy() for t in hla.mla_laga_decode(*a, cu)]
    out = torch.empty((cfg.S_loc, 64, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((cfg.S_loc, 64), dtype=torch.float32, device="cuda")
    hla.mla_laga_decode_noalloc(*a, cu, torch.from_numpy(cu).cuda(), out, lse)
    torch.cuda.synchronize()
    for r, g, n in zip(ref, got, ("out", "lse")):
        assert np.array_equal(g, r), n
    assert np.array_equal(out.cpu().numpy(), ref[0]) and np.array_equal(lse.cpu().numpy(), ref[1])
