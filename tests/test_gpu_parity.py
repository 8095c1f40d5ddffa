"""GPU parity: the HIP path against the fp64 oracle on the same seeded inputs.

Small shapes (several tiles and a ragged tail) are compared element by
element. The full-size workloads run in the same launch configuration the
benchmark uses and are compared on sampled heads: every output of a head
depends only on that head's inputs, except the latent and rope-key gradients,
which sum over heads and are checked with dout zero outside the sampled heads.
The mask is checked exactly with q = 0, where every visible score is 0, so
exp(lse) is the number of visible keys of the row.
"""

import numpy as np
import pytest
import torch

import head_latent_attention_kv_amd as hla
import oracle
import workloads
from tests.gpu_helpers import MAX_ABS, MEAN_REL, announce, check, to_device

pytestmark = pytest.mark.gpu

DSV3 = dict(d_c=512, d_rope=64, d_nope=128, d_v=128)
GRADS = ("dq", "dc_kv", "dk_rope", "dW_UK", "dW_UV")


def small(name, n_h, S, S_loc, q_offset, cu=None, backward=True, seed=3, q_ranges=None):
    if q_ranges is not None:
        S_loc, q_offset = sum(n for _, n in q_ranges), 0
    cfg = workloads.MLAConfig(name, n_h=n_h, S=S, S_loc=S_loc, q_offset=q_offset, dtype="bf16",
                              backward=backward, seed=seed, q_ranges=q_ranges, **DSV3)
    return cfg, (None if cu is None else np.array(cu, np.int32))


def small_dc(name, d_c, n_h, S, S_loc, q_offset, cu=None):
    """Fast path at another latent width (d_c a multiple of 64)."""
    cfg = workloads.MLAConfig(name, n_h=n_h, d_c=d_c, d_rope=64, d_nope=128, d_v=128, S=S,
                              S_loc=S_loc, q_offset=q_offset, dtype="bf16", backward=True, seed=4)
    return cfg, (None if cu is None else np.array(cu, np.int32))


def positions(cfg):
    """Oracle keyword arguments that place the rows (one block or several)."""
    return dict(q_offset=cfg.q_offset, q_ranges=cfg.q_ranges)


# With one visible key a row's softmax weight is exactly 1, so dS = P (dP - D)
# is zero and dq, dK (hence dk_rope and dW_UK) vanish analytically: the
# oracle's values are rounding noise, and a ratio of sums against them means
# nothing. Such tensors get an absolute bound instead.
VANISHING = {"one_token": {"dq", "dk_rope", "dW_UK"}}

SMALL = [
    small("causal_ragged", 2, 300, 300, 0),
    small("shard_ragged", 3, 700, 333, 367),
    small("varlen_shard", 2, 600, 450, 150, cu=[0, 1, 1, 130, 131, 400, 600]),
    small("one_token", 1, 1, 1, 0),
    small("last_row_only", 2, 257, 1, 256),
    small("varlen_len1_and_empty", 2, 520, 520, 0, cu=[0, 1, 1, 2, 258, 258, 259, 520]),
    # several position blocks; tiles straddle block ends
    small("blocks_ragged", 2, 1000, 0, 0, q_ranges=((37, 150), (400, 230), (900, 100))),
    small("blocks_varlen", 2, 600, 0, 0, cu=[0, 1, 1, 130, 131, 400, 600],
          q_ranges=((5, 120), (300, 200))),
    # the middle sample lies between the blocks: its keys get zero gradients
    small("blocks_unseen_sample", 2, 700, 0, 0, cu=[0, 200, 450, 700],
          q_ranges=((10, 150), (470, 200))),
    small("zigzag_r1_of_4", 2, 1024, 0, 0, q_ranges=workloads.zigzag_blocks(1024, 1, 4)),
    # the most position blocks a call takes, over packed samples
    small("sixteen_blocks", 2, 2000, 0, 0, cu=[0, 3, 400, 401, 1250, 2000],
          q_ranges=tuple((125 * k + 11 * (k % 3), 1 + 6 * k) for k in range(16))),
    # other latent widths on the fast path
    small_dc("d_c_256", 256, 3, 700, 333, 367),
    small_dc("d_c_1024", 1024, 2, 600, 450, 150, cu=[0, 1, 1, 130, 131, 400, 600]),
    # the narrowest latent the fast path takes, and one that is not a power of
    # two: the gradient GEMMs' latent-side tiles end mid-tile
    small_dc("d_c_64", 64, 2, 500, 300, 200),
    small_dc("d_c_320", 320, 3, 700, 333, 367, cu=[0, 90, 91, 400, 700]),
]


def run(cfg, x, cu=None, generic=False, backward=False, dout_override=None, stored_ds=False):
    dev = to_device(x, cfg)
    if dout_override is not None:
        dev["dout"] = dout_override
    call = hla.MLACall(dev["q"], dev["c_kv"], dev["k_rope"], dev["W_UK"], dev["W_UV"],
                       q_offset=cfg.q_offset, cu_seqlens=cu, generic=generic, backward=backward,
                       q_ranges=cfg.q_ranges, stored_ds=stored_ds)
    out, lse = call.fwd(dev["q"], dev["c_kv"], dev["k_rope"], dev["W_UK"], dev["W_UV"])
    res = {"out": out, "lse": lse, "fast": call.fast}
    if backward:
        g = call.bwd(dev["dout"], dev["q"], dev["c_kv"], dev["k_rope"], dev["W_UK"], dev["W_UV"],
                     out, lse)
        res.update(dict(zip(GRADS, g)))
    torch.cuda.synchronize()
    return {k: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for k, v in res.items()}


def oracle_args(x):
    return [x[k] for k in ("q", "c_kv", "k_rope", "W_UK", "W_UV")]


# default: the fast path with dQ recomputing S and dP; stored_ds: the fast
# path with dQ read from the stored dS; plain: the fp32 path
@pytest.mark.parametrize("path", ["default", "stored_ds", "plain"])
@pytest.mark.parametrize("cfg,cu", SMALL, ids=[c.name for c, _ in SMALL])
def test_small_fwd_bwd_elementwise(cfg, cu, path):
    announce(f"small {cfg.name} path={path} n_h={cfg.n_h} S={cfg.S} S_loc={cfg.S_loc} q_off={cfg.q_offset}")
    x = workloads.make_inputs(cfg, with_dout=True)
    g = run(cfg, x, cu, generic=path == "plain", backward=True, stored_ds=path == "stored_ds")
    assert g["fast"] == (path != "plain")
    ro, rl = oracle.mla_forward(*oracle_args(x), cu_seqlens=cu, **positions(cfg))
    check("out", g["out"], ro)
    check("lse", g["lse"], rl)
    rg = oracle.mla_backward(x["dout"], *oracle_args(x), cu_seqlens=cu, **positions(cfg))
    for name, ref in zip(GRADS, rg):
        if name in VANISHING.get(cfg.name, ()):
            assert np.abs(ref).max() < 1e-12
            check(name, g[name], ref, max_abs=2e-3, mean_rel=np.inf)
        else:
            check(name, g[name], ref)


def test_tiny_f32_config():
    cfg = workloads.config("tiny_f32")
    announce("tiny_f32 fwd+bwd")
    x = workloads.make_inputs(cfg, with_dout=True)
    g = run(cfg, x, backward=True)
    ro, rl = oracle.mla_forward(*oracle_args(x))
    rg = oracle.mla_backward(x["dout"], *oracle_args(x))
    # fp32 inputs on the plain fp32 path: far inside the bf16 bar
    for name, got, ref in [("out", g["out"], ro), ("lse", g["lse"], rl)] + \
            [(n, g[n], r) for n, r in zip(GRADS, rg)]:
        ma, mr = check(name, got, ref)
        assert ma < 1e-4 and mr < 1e-5, name


def test_h16_s4k_full_forward():
    cfg = workloads.config("h16_s4k")
    announce("h16_s4k fwd full")
    x = workloads.make_inputs(cfg)
    g = run(cfg, x)
    ro, rl = oracle.mla_forward(*oracle_args(x))
    check("out", g["out"], ro)
    check("lse", g["lse"], rl)


def _set(x, name, values):
    """x with input `name` replaced by `values` (exact in bf16)."""
    bits = workloads.f32_to_bf16_bits(np.asarray(values, np.float32))
    return dict(x, **{name: workloads.bf16_bits_to_f32(bits), name + "_bits": bits})


@pytest.mark.parametrize("v_exp", [-10, 8])
@pytest.mark.parametrize("path", ["default", "stored_ds"])
def test_value_scale_and_zero_rows_bwd(v_exp, path):
    """The backward's per-key dS factor comes from a bound on |dP - D| built
    from the key's V row norm and the per-head maxima of |dout row| and |D|.
    V scaled by 2^v_exp (W_UV times a power of two, exact in bf16) moves the
    factor's exponent far from its usual range, and a run of latent rows set
    to zero (V = K_nope = 0 there) leaves the largest |D| as the whole bound
    of those keys. Every output against the oracle: the sum ratio at the
    full bar (it does not depend on the scale of the values); the max-abs bar,
    set for unit-scale inputs, scaled by the same 2^v_exp when v_exp > 0,
    since out, dq and the key-side gradients grow with V."""
    cfg, cu = small("v_scale", 2, 700, 333, 367, cu=[0, 90, 91, 400, 700], seed=9)
    announce(f"value scale 2^{v_exp}, zero latent rows, path={path}")
    x = workloads.make_inputs(cfg, with_dout=True)
    x = _set(x, "W_UV", x["W_UV"] * np.float32(2.0 ** v_exp))
    ckv = x["c_kv"].copy()
    ckv[380:450] = 0.0
    x = _set(x, "c_kv", ckv)
    g = run(cfg, x, cu, backward=True, stored_ds=path == "stored_ds")
    assert g["fast"]
    ro, rl = oracle.mla_forward(*oracle_args(x), cu_seqlens=cu, **positions(cfg))
    bar = MAX_ABS * 2.0 ** max(v_exp, 0)
    check("out", g["out"], ro, max_abs=bar)
    check("lse", g["lse"], rl)
    rg = oracle.mla_backward(x["dout"], *oracle_args(x), cu_seqlens=cu, **positions(cfg))
    for name, ref in zip(GRADS, rg):
        check(name, g[name], ref, max_abs=bar)


@pytest.mark.parametrize("k_mul", [4])
def test_sharp_softmax_bwd(k_mul):
    """Scores k_mul times larger (W_UK times a power of two, exact in bf16):
    the softmax puts most weight on a few keys per row, so P 2^15 comes close
    to its ceiling of 2^15 for them while most keys' weights fall far below
    fp16's range. Every output against the oracle; the max-abs bar scaled by
    k_mul, since dq and dK grow with K. (At 8 times the gradients reach the
    1e-3 sum-ratio bar, as they did before the dS factors: the scores come
    from fp16 q and K, and sharper logits magnify their rounding.)"""
    cfg, cu = small("sharp", 2, 600, 450, 150, cu=[0, 1, 1, 130, 131, 400, 600], seed=11)
    announce(f"sharp softmax (W_UK x {k_mul})")
    x = workloads.make_inputs(cfg, with_dout=True)
    x = _set(x, "W_UK", x["W_UK"] * np.float32(k_mul))
    g = run(cfg, x, cu, backward=True)
    assert g["fast"]
    ro, rl = oracle.mla_forward(*oracle_args(x), cu_seqlens=cu, **positions(cfg))
    check("out", g["out"], ro)
    check("lse", g["lse"], rl)
    rg = oracle.mla_backward(x["dout"], *oracle_args(x), cu_seqlens=cu, **positions(cfg))
    for name, ref in zip(GRADS, rg):
        check(name, g[name], ref, max_abs=k_mul * MAX_ABS)


@pytest.mark.parametrize("S,S_loc,stored_ds", [(1 << 17, 1024, False), (1 << 17, 1024, True),
                                               (1 << 19, 256, False)])
def test_long_context_bwd(S, S_loc, stored_ds):
    """Long latents with a short shard of rows at the end: the softmax weights
    of a key are about 1 / S (2^-17 and 2^-19), below fp16's normal range
    (2^-14). The dK/dV products take them with power-of-two factors (P 2^15,
    dS 2^ex per key) that keep them normal; every output at the full bar, also
    with dQ taken from the stored dS (written without the factor)."""
    cfg = workloads.MLAConfig(f"long_{S}", n_h=1, d_c=64, d_rope=64, d_nope=128, d_v=128, S=S,
                              S_loc=S_loc, q_offset=S - S_loc, dtype="bf16", backward=True, seed=7)
    announce(f"long context fwd+bwd: S={S}, last {S_loc} rows, stored_ds={stored_ds}")
    x = workloads.make_inputs(cfg, with_dout=True)
    g = run(cfg, x, backward=True, stored_ds=stored_ds)
    assert g["fast"]
    ro, rl = oracle.mla_forward(*oracle_args(x), q_offset=cfg.q_offset)
    check("out", g["out"], ro)
    check("lse", g["lse"], rl)
    rg = oracle.mla_backward(x["dout"], *oracle_args(x), q_offset=cfg.q_offset)
    for name, ref in zip(GRADS, rg):
        check(name, g[name], ref)


def test_max_keys_fwd_bwd():
    """The fast path at its key limit: one head and the last 64 rows of a
    latent of 2^22 - 256 rows (the most needed keys the fast path takes), so
    every offset into the rebuilt K, V^T and key-major V tiles, the gradient
    rows and every 32-bit DMA offset is at its largest. Every key is visible
    to these rows. All seven outputs element by element against the oracle
    (the narrowest latent, d_c = 64, keeps the oracle's fp64 copies small).

    dc_kv alone has a wider mean bound. Each key's [dK_nope | dV] row is
    stored in fp16 (times the dout factor 2^e, max|2^e dout| in [4, 8)):
    dV[key] sums 64 rows' weights of about 2^-22 each, so its elements are
    near 2^-19, inside fp16's subnormal range, where the spacing is a fixed
    2^-24. Rounding to that spacing costs up to 2^-25 / 2^-19 = 2^-6 of each
    element, about 2^-8 on average over the row's sizes, i.e. 4e-3. The
    measured sum|err| / sum|ref| is 3.0e-3; the bound is 5e-3. Its max-abs
    stays at the full bar, and the other outputs meet the full bar."""
    S = (1 << 22) - 256
    cfg = workloads.MLAConfig("max_keys", n_h=1, d_c=64, d_rope=64, d_nope=128, d_v=128, S=S,
                              S_loc=64, q_offset=S - 64, dtype="bf16", backward=True, seed=5)
    announce(f"max keys fwd+bwd: S={S}, last {cfg.S_loc} rows")
    x = workloads.make_inputs(cfg, with_dout=True)
    g = run(cfg, x, backward=True)
    assert g["fast"]
    ro, rl = oracle.mla_forward(*oracle_args(x), q_offset=cfg.q_offset)
    check("out", g["out"], ro)
    check("lse", g["lse"], rl)
    del ro, rl
    rg = oracle.mla_backward(x["dout"], *oracle_args(x), q_offset=cfg.q_offset)
    for name, ref in zip(GRADS, rg):
        check(name, g[name], ref, mean_rel=5e-3 if name == "dc_kv" else MEAN_REL)


@pytest.mark.parametrize("heads", [[0, 37, 64, 127]])
def test_h128_s16k_shard_forward_sampled_heads(heads):
    cfg = workloads.config("h128_s16k_shard")
    announce(f"h128_s16k_shard fwd, heads {heads}")
    x = workloads.make_inputs(cfg)
    g = run(cfg, x)
    ro, rl = oracle.mla_forward(*oracle_args(x), q_offset=cfg.q_offset, heads=heads)
    check("out", g["out"][:, heads], ro)
    check("lse", g["lse"][:, heads], rl)


@pytest.mark.parametrize("name", ["h128_s8k_bwd", "h128_varlen64k", "h128_s16k_zigzag_r0"])
def test_full_size_backward_sampled_heads(name):
    """Default fast path (dQ from the stored dS)."""
    cfg = workloads.config(name)
    cu = cfg.cu_seqlens()
    heads = [5, 122]
    announce(f"{name} fwd+bwd, dout only on heads {heads}")
    x = workloads.make_inputs(cfg, with_dout=True)
    dz = np.zeros_like(x["dout"])
    dz[:, heads] = x["dout"][:, heads]
    x0 = dict(x, dout=dz, dout_bits=workloads.f32_to_bf16_bits(dz))
    g = run(cfg, x0, cu, backward=True)
    ro, rl = oracle.mla_forward(*oracle_args(x), cu_seqlens=cu, heads=heads, **positions(cfg))
    check("out", g["out"][:, heads], ro)
    check("lse", g["lse"][:, heads], rl)
    rg = oracle.mla_backward(dz, *oracle_args(x), cu_seqlens=cu, heads=heads, **positions(cfg))
    for nm, ref in zip(GRADS, rg):
        check(nm, g[nm], ref)

    announce(f"{name} fwd+bwd, full dout; dq and weight blocks of heads {heads}")
    g = run(cfg, x, cu, backward=True)
    rg = oracle.mla_backward(x["dout"], *oracle_args(x), cu_seqlens=cu, heads=heads,
                             **positions(cfg))
    check("dq", g["dq"][:, heads], rg[0][:, heads])
    cols_k = np.concatenate([np.arange(h * 128, (h + 1) * 128) for h in heads])
    check("dW_UK", g["dW_UK"][:, cols_k], rg[3][:, cols_k])
    check("dW_UV", g["dW_UV"][:, cols_k], rg[4][:, cols_k])


@pytest.mark.parametrize("name", workloads.CONFIG_ORDER + ["h128_s16k_zigzag_r0",
                                                           "h128_s16k_zigzag_r7"])
def test_mask_probe_exact_counts(name):
    """q = 0: every visible score is exactly 0, so exp(lse) counts the visible
    keys of each row; it must equal the oracle's integer count exactly."""
    cfg = workloads.config(name)
    cu = cfg.cu_seqlens()
    announce(f"mask probe {name}")
    x = workloads.make_inputs(cfg)
    dev = to_device(x, cfg)
    q0 = torch.zeros_like(dev["q"])
    call = hla.MLACall(q0, dev["c_kv"], dev["k_rope"], dev["W_UK"], dev["W_UV"],
                       q_offset=cfg.q_offset, cu_seqlens=cu, q_ranges=cfg.q_ranges)
    _, lse = call.fwd(q0, dev["c_kv"], dev["k_rope"], dev["W_UK"], dev["W_UV"])
    counts = np.rint(np.exp(lse.double().cpu().numpy())).astype(np.int64)
    lo, hi = oracle.visible_range(cfg.S_loc, cfg.q_offset, cu, cfg.q_ranges)
    expect = (hi - lo + 1)[:, None]
    bad = np.argwhere(counts != expect)
    assert bad.size == 0, f"{len(bad)} rows with wrong visible-key count, first {bad[:3]}"


@pytest.mark.parametrize("generic", [False, True], ids=["default", "plain"])
def test_shard_concatenation_identity(generic):
    """Eight contiguous query shards reproduce the single-rank call (LAGA
    abstract: equivalence across sequence-parallel degrees)."""
    cfg = workloads.MLAConfig("sp", n_h=4, S=2048, S_loc=2048, q_offset=0, dtype="bf16", **DSV3)
    announce(f"shard identity generic={generic}")
    x = workloads.make_inputs(cfg)
    full = run(cfg, x, generic=generic)
    n = 256
    outs, lses = [], []
    for r in range(8):
        c = cfg.with_(S_loc=n, q_offset=r * n)
        xr = dict(x, q=x["q"][r * n:(r + 1) * n], q_bits=x["q_bits"][r * n:(r + 1) * n])
        g = run(c, xr, generic=generic)
        outs.append(g["out"]); lses.append(g["lse"])
    o, l = np.concatenate(outs), np.concatenate(lses)
    assert np.array_equal(o, full["out"]) and np.array_equal(l, full["lse"])


@pytest.mark.parametrize("generic", [False, True], ids=["default", "plain"])
def test_zigzag_concatenation_identity(generic):
    """Four zigzag ranks (blocks r and 7-r of eight) reproduce the single-rank
    call row for row, bit for bit, and their latent and weight gradients sum
    to the single-rank gradients (LAGA abstract: equivalence across
    sequence-parallel degrees)."""
    cfg = workloads.MLAConfig("zz", n_h=4, S=2048, S_loc=2048, q_offset=0, dtype="bf16",
                              backward=True, **DSV3)
    announce(f"zigzag identity generic={generic}")
    x = workloads.make_inputs(cfg, with_dout=True)
    full = run(cfg, x, generic=generic, backward=True)
    out = np.full_like(full["out"], np.nan)
    lse = np.full_like(full["lse"], np.nan)
    dq = np.full_like(full["dq"], np.nan)
    sums = {k: np.zeros_like(full[k], dtype=np.float64) for k in GRADS[1:]}
    for r in range(4):
        blocks = workloads.zigzag_blocks(2048, r, 4)
        rows = np.concatenate([np.arange(a, a + n) for a, n in blocks])
        c = cfg.with_(S_loc=len(rows), q_ranges=blocks)
        xr = dict(x)
        for k in ("q", "dout"):
            xr[k] = x[k][rows]
            xr[k + "_bits"] = x[k + "_bits"][rows]
        g = run(c, xr, generic=generic, backward=True)
        out[rows], lse[rows], dq[rows] = g["out"], g["lse"], g["dq"]
        for k in sums:
            sums[k] += g[k]
    assert np.array_equal(out, full["out"]) and np.array_equal(lse, full["lse"])
    check("dq", dq, full["dq"], max_abs=1e-5, mean_rel=1e-6)
    rg = oracle.mla_backward(x["dout"], *oracle_args(x))
    for k, ref in zip(GRADS[1:], rg[1:]):
        check(k, sums[k], ref)


@pytest.mark.parametrize("name", ["h128_s16k_shard", "h128_varlen64k"])
def test_full_size_dq_paths_agree(name):
    """dQ read from the stored dS and dQ recomputed per query tile, both on
    the full-size shard, checked against the oracle on sampled heads."""
    cfg = workloads.config(name)
    cu = cfg.cu_seqlens()
    heads = [3, 90]
    x = workloads.make_inputs(cfg, with_dout=True)
    rg = oracle.mla_backward(x["dout"], *oracle_args(x), cu_seqlens=cu, heads=heads,
                             **positions(cfg))
    for stored in (False, True):
        announce(f"{name} dq, stored_ds={stored}, heads {heads}")
        g = run(cfg, x, cu, backward=True, stored_ds=stored)
        check("dq", g["dq"][:, heads], rg[0][:, heads])


# 130 heads x 128 MiB of dS: the stored-dS backward in 17 head groups
GROUPED = workloads.MLAConfig("ds_groups", n_h=130, d_c=64, d_rope=64, d_nope=128, d_v=128,
                              S=16384, S_loc=4096, q_offset=12288, dtype="bf16", backward=True,
                              seed=11)


@pytest.mark.parametrize("packed", [False, True], ids=["causal", "packed"])
def test_stored_ds_head_groups(packed):
    """Stored dS past its one-buffer limit (16 GiB): 130 heads of 4096 rows
    over 16384 keys hold 128 MiB of dS each, 16.25 GiB in all, so the
    backward runs them in 16 groups of 8 heads and one of 2 through two
    alternating 1 GiB buffers: group g + 2 writes the buffer of group g once
    dQ of group g has read it. Heads 0 and 16 use the first slot of buffer 0
    in groups 0 and 2; head 129 is in the last group, which also uses buffer
    0. dout is zero outside those three heads, so every output is checked in
    full against the oracle over them (the idle heads give exactly zero dq
    and weight gradients). Packed: a second sample starts at 16000, so the
    dS blocks of its rows against earlier keys are never written and still
    hold an earlier group's values, which dQ must mask."""
    cfg = GROUPED.with_(seq_lens=(16000, 384)) if packed else GROUPED
    cu = cfg.cu_seqlens()
    heads = [0, 16, 129]
    idle = [h for h in range(cfg.n_h) if h not in heads]
    announce(f"stored dS in 17 head groups, dout on heads {heads}")
    x = workloads.make_inputs(cfg, with_dout=True)
    dz = np.zeros_like(x["dout"])
    dz[:, heads] = x["dout"][:, heads]
    x = _set(x, "dout", dz)
    g = run(cfg, x, cu, backward=True, stored_ds=True)
    assert g["fast"]
    rg = oracle.mla_backward(x["dout"], *oracle_args(x), cu_seqlens=cu, q_offset=cfg.q_offset,
                             heads=heads)
    check("dq", g["dq"][:, heads], rg[0][:, heads])
    check("dc_kv", g["dc_kv"], rg[1])
    check("dk_rope", g["dk_rope"], rg[2])
    cols = np.concatenate([np.arange(h * 128, (h + 1) * 128) for h in heads])
    cols_idle = np.concatenate([np.arange(h * 128, (h + 1) * 128) for h in idle])
    check("dW_UK", g["dW_UK"][:, cols], rg[3][:, cols])
    check("dW_UV", g["dW_UV"][:, cols], rg[4][:, cols])
    assert not g["dq"][:, idle].any()
    assert not g["dW_UK"][:, cols_idle].any() and not g["dW_UV"][:, cols_idle].any()


def test_forward_backward_deterministic():
    cfg = workloads.MLAConfig("det", n_h=8, S=1500, S_loc=1000, q_offset=500, dtype="bf16",
                              backward=True, **DSV3)
    announce("determinism")
    x = workloads.make_inputs(cfg, with_dout=True)
    a = run(cfg, x, backward=True)
    b = run(cfg, x, backward=True)
    for k in ("out", "lse") + GRADS:
        assert np.array_equal(a[k], b[k]), k


def test_backward_ordered_on_caller_streams():
    """The fast backward runs part of its kernels on an internal stream, forked
    from the caller's stream and joined back into it. Work enqueued on the
    caller's stream right after the call (no host sync in between) must see
    the final gradients, and calls on two other caller streams must give the
    same bits as a call on the default stream."""
    cfg = workloads.MLAConfig("streams", n_h=8, S=1500, S_loc=1000, q_offset=500, dtype="bf16",
                              backward=True, **DSV3)
    announce("backward on caller streams")
    x = workloads.make_inputs(cfg, with_dout=True)
    ref = run(cfg, x, backward=True)
    dev = to_device(x, cfg)
    args = [dev[k] for k in ("q", "c_kv", "k_rope", "W_UK", "W_UV")]
    torch.cuda.synchronize()
    copies = []
    for s in (torch.cuda.Stream(), torch.cuda.Stream()):
        with torch.cuda.stream(s):
            call = hla.MLACall(*args, q_offset=cfg.q_offset, backward=True)
            out, lse = call.fwd(*args)
            g = call.bwd(dev["dout"], *args, out, lse)
            copies.append([t.clone() for t in g])   # same stream, right after the call
    torch.cuda.synchronize()
    for got in copies:
        for k, t in zip(GRADS, got):
            assert np.array_equal(t.cpu().numpy(), ref[k]), k


GRAPH_CASES = {
    "default": (workloads.MLAConfig("graph", n_h=8, S=1500, S_loc=1000, q_offset=500,
                                    dtype="bf16", backward=True, **DSV3), False),
    "stored_ds": (workloads.MLAConfig("graph", n_h=8, S=1500, S_loc=1000, q_offset=500,
                                      dtype="bf16", backward=True, **DSV3), True),
    # 17 head groups through two dS buffers (16.25 GiB of dS in one buffer)
    "stored_ds_groups": (workloads.MLAConfig("graph_groups", n_h=130, d_c=64, d_rope=64,
                                             d_nope=128, d_v=128, S=16384, S_loc=4096,
                                             q_offset=12288, dtype="bf16", backward=True,
                                             seed=12), True),
}


@pytest.mark.parametrize("form", list(GRAPH_CASES))
def test_graph_replays_match_eager(form):
    """Forward and backward captured into one HIP graph (through torch) and
    replayed: every replay, with eager work and a host synchronisation
    between replays, gives the eager call's bits. The library enqueues no
    memset or allocation, and the backward's side stream joins the capture
    through its fork event and leaves it through its join event; in the
    head-grouped stored-dS form the waits for a free dS buffer are captured
    as well."""
    cfg, stored = GRAPH_CASES[form]
    announce(f"graph capture and replay, {form}")
    x = workloads.make_inputs(cfg, with_dout=True)
    ref = run(cfg, x, backward=True, stored_ds=stored)
    dev = to_device(x, cfg)
    args = [dev[k] for k in ("q", "c_kv", "k_rope", "W_UK", "W_UV")]
    call = hla.MLACall(*args, q_offset=cfg.q_offset, backward=True, stored_ds=stored)
    out, lse = call.fwd(*args)
    grads = call.bwd(dev["dout"], *args, out, lse)   # eager: also creates the side stream
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                     # warm-up off the default stream
        call.fwd(*args, out=out, lse=lse)
        call.bwd(dev["dout"], *args, out, lse, grads=grads)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call.fwd(*args, out=out, lse=lse)
        call.bwd(dev["dout"], *args, out, lse, grads=grads)
    torch.cuda.synchronize()
    for _ in range(3):
        for t in (out, lse, *grads):
            t.fill_(7.0)                               # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref["out"])
        assert np.array_equal(lse.cpu().numpy(), ref["lse"])
        for k, t in zip(GRADS, grads):
            assert np.array_equal(t.cpu().numpy(), ref[k]), k


def test_empty_shard():
    cfg = workloads.MLAConfig("empty", n_h=2, S=64, S_loc=0, q_offset=64, dtype="bf16",
                              backward=True, **DSV3)
    announce("empty shard")
    x = workloads.make_inputs(cfg, with_dout=True)
    dev = to_device(x, cfg)
    call = hla.MLACall(dev["q"], dev["c_kv"], dev["k_rope"], dev["W_UK"], dev["W_UV"],
                       q_offset=64, backward=True)
    out, lse = call.fwd(dev["q"], dev["c_kv"], dev["k_rope"], dev["W_UK"], dev["W_UV"])
    assert out.numel() == 0 and lse.numel() == 0
    grads = [torch.full_like(t, 7.0) for t in call.bwd(dev["dout"], dev["q"], dev["c_kv"],
                                                      dev["k_rope"], dev["W_UK"], dev["W_UV"],
                                                      out, lse)]
    grads = call.bwd(dev["dout"], dev["q"], dev["c_kv"], dev["k_rope"], dev["W_UK"], dev["W_UV"],
                     out, lse, grads=grads)
    torch.cuda.synchronize()
    for t in grads[1:]:
        assert torch.count_nonzero(t).item() == 0
