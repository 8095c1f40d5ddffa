"""Pins for the fp64 oracle, none of which re-types its formulas.

* brute-force per-element loops (tests/oracle_brute.py) on tiny inputs,
  causal, sharded and packed (with an empty and a length-1 sample);
* the absorbed reformulation (LAGA abstract: W_UK folded into the query,
  attention over the latent) equals the explicit form;
* the special case n_h=1, identity weights, zero rope part is textbook causal
  scaled-dot-product attention, checked with torch's library routine in fp64;
* closed forms: one visible key gives out = V_j and lse = s_jj; q = 0 gives
  uniform weights (lse = ln|vis|, out = mean of visible V); constant values
  give out = that constant (softmax weights sum to one);
* a packed call equals independent calls on each sample (block-diagonal
  causal mask, Libra review page, "Axiom ledger");
* sequence-parallel shards concatenate to the single-rank result and their
  latent / weight gradients sum to it (LAGA abstract: equivalence across SP
  degrees), for contiguous shards and for zigzag shards of two position
  blocks each (Libra review page, Related Work beside Fig. 15);
* gradients against central finite differences of the forward.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import mla_oracle as M
from tests.oracle_brute import MacCounter, brute_backward, brute_forward, brute_visible_pairs


def rand_inputs(n_h=2, d_c=6, d_rope=2, d_nope=3, d_v=4, S=9, S_loc=None, seed=1,
                w_std=None):
    rng = np.random.default_rng(seed)
    S_loc = S if S_loc is None else S_loc
    w_std = 1.0 / math.sqrt(d_c) if w_std is None else w_std
    return dict(
        q=rng.standard_normal((S_loc, n_h, d_nope + d_rope)),
        c_kv=rng.standard_normal((S, d_c)),
        k_rope=rng.standard_normal((S, d_rope)),
        W_UK=rng.standard_normal((d_c, n_h * d_nope)) * w_std,
        W_UV=rng.standard_normal((d_c, n_h * d_v)) * w_std,
    )


CASES = [
    # (S, S_loc, q_offset, cu_seqlens)
    (9, 9, 0, None),
    (9, 5, 4, None),
    (12, 12, 0, [0, 3, 3, 4, 9, 12]),      # empty sample and a length-1 sample
    (12, 7, 5, [0, 3, 3, 4, 9, 12]),       # shard starting inside a sample
    (10, 3, 7, [0, 10]),                   # one packed sample == causal
]


@pytest.mark.parametrize("S,S_loc,q_offset,cu", CASES)
def test_forward_matches_brute_force(S, S_loc, q_offset, cu):
    x = rand_inputs(S=S, S_loc=S_loc, seed=S + S_loc + q_offset)
    cu_a = None if cu is None else np.array(cu, dtype=np.int32)
    out, lse = oracle.mla_forward(**x, q_offset=q_offset, cu_seqlens=cu_a)
    bo, bl = brute_forward(x["q"].tolist(), x["c_kv"].tolist(), x["k_rope"].tolist(),
                           x["W_UK"].tolist(), x["W_UV"].tolist(), q_offset, cu)
    np.testing.assert_allclose(out, np.array(bo), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(bl), rtol=0, atol=1e-12)


def test_forward_rows_heads_subset_matches_full():
    x = rand_inputs(n_h=3, S=11, S_loc=8)
    out, lse = oracle.mla_forward(**x, q_offset=3)
    rows, heads = [0, 5, 7], [2, 0]
    o2, l2 = oracle.mla_forward(**x, q_offset=3, rows=rows, heads=heads)
    np.testing.assert_allclose(o2, out[np.ix_(rows, heads)], rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, lse[np.ix_(rows, heads)], rtol=0, atol=1e-13)


@pytest.mark.parametrize("S,S_loc,q_offset,cu", CASES)
def test_absorbed_equals_explicit(S, S_loc, q_offset, cu):
    x = rand_inputs(n_h=3, d_c=7, d_rope=3, d_nope=5, d_v=4, S=S, S_loc=S_loc, seed=7)
    cu_a = None if cu is None else np.array(cu, dtype=np.int32)
    o1, l1 = oracle.mla_forward(**x, q_offset=q_offset, cu_seqlens=cu_a)
    o2, l2 = oracle.mla_forward_absorbed(**x, q_offset=q_offset, cu_seqlens=cu_a)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-12, atol=1e-13)


def test_reduces_to_textbook_causal_sdpa():
    torch.manual_seed(0)
    D, d_rope, S = 8, 4, 33
    rng = np.random.default_rng(3)
    q = rng.standard_normal((S, 1, D + d_rope))
    q[:, :, D:] = 0.0                      # rope part off
    c_kv = rng.standard_normal((S, D))
    k_rope = rng.standard_normal((S, d_rope))
    eye = np.eye(D)
    out, lse = oracle.mla_forward(q, c_kv, k_rope, eye, eye)
    scale = 1.0 / math.sqrt(D + d_rope)
    qt = torch.from_numpy(q[:, 0, :D]).double()[None, None]
    kv = torch.from_numpy(c_kv).double()[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kv, kv, is_causal=True,
                                                           scale=scale)[0, 0].numpy()
    np.testing.assert_allclose(out[:, 0, :], ref, rtol=0, atol=1e-12)
    # lse from the same library: logsumexp of the masked scaled scores
    s = torch.from_numpy(q[:, 0, :D] @ c_kv.T * scale)
    s = s.masked_fill(torch.triu(torch.ones(S, S, dtype=torch.bool), 1), float("-inf"))
    np.testing.assert_allclose(lse[:, 0], torch.logsumexp(s, dim=1).numpy(), rtol=0, atol=1e-12)


def test_shard_reduces_to_sdpa_with_offset_mask():
    D, S, q_off = 6, 20, 13
    rng = np.random.default_rng(4)
    q = np.concatenate([rng.standard_normal((S - q_off, 1, D)), np.zeros((S - q_off, 1, 2))], 2)
    c_kv = rng.standard_normal((S, D))
    eye = np.eye(D)
    out, _ = oracle.mla_forward(q, c_kv, rng.standard_normal((S, 2)), eye, eye, q_offset=q_off)
    allowed = np.arange(S)[None, :] <= (q_off + np.arange(S - q_off))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q[:, 0, :D])[None], torch.from_numpy(c_kv)[None],
        torch.from_numpy(c_kv)[None], attn_mask=torch.from_numpy(allowed)[None],
        scale=1.0 / math.sqrt(D + 2))[0].numpy()
    np.testing.assert_allclose(out[:, 0, :], ref, rtol=0, atol=1e-12)


def test_single_visible_key_closed_form():
    # rows at position 0 and at each sample start see exactly one key
    cu = np.array([0, 4, 5, 9], dtype=np.int32)
    x = rand_inputs(S=9, seed=11)
    out, lse = oracle.mla_forward(**x, cu_seqlens=cu)
    sc = oracle.default_scale(3, 2)
    for p in [0, 4, 5]:
        for h in range(2):
            kn = x["c_kv"][p] @ x["W_UK"][:, h * 3:(h + 1) * 3]
            v = x["c_kv"][p] @ x["W_UV"][:, h * 4:(h + 1) * 4]
            s = sc * (x["q"][p, h, :3] @ kn + x["q"][p, h, 3:] @ x["k_rope"][p])
            np.testing.assert_allclose(out[p, h], v, rtol=0, atol=1e-13)
            assert abs(lse[p, h] - s) <= 1e-13


@pytest.mark.parametrize("S,S_loc,q_offset,cu", CASES)
def test_zero_query_gives_uniform_weights(S, S_loc, q_offset, cu):
    x = rand_inputs(S=S, S_loc=S_loc, seed=5)
    x["q"][:] = 0.0
    cu_a = None if cu is None else np.array(cu, dtype=np.int32)
    out, lse = oracle.mla_forward(**x, q_offset=q_offset, cu_seqlens=cu_a)
    for i in range(S_loc):
        p = q_offset + i
        lo = 0 if cu is None else max(c for c in cu if c <= p)
        n = p - lo + 1
        assert abs(lse[i, 0] - math.log(n)) < 1e-13
        V = x["c_kv"][lo:p + 1] @ x["W_UV"][:, 4:8]
        np.testing.assert_allclose(out[i, 1], V.mean(axis=0), rtol=0, atol=1e-13)


def test_weights_sum_to_one_constant_values():
    # append a constant-one latent column; W_UV reads only that column, so
    # every value row is the same vector u and out must equal u
    x = rand_inputs(n_h=2, d_c=5, S=10, S_loc=6)
    x["c_kv"][:, -1] = 1.0
    u = np.array([[0.5, -2.0, 3.0, 1.25], [-1.0, 0.0, 2.5, 7.0]])
    x["W_UV"][:] = 0.0
    x["W_UV"][-1, :] = u.reshape(-1)
    out, _ = oracle.mla_forward(**x, q_offset=4, cu_seqlens=np.array([0, 3, 10], np.int32))
    for h in range(2):
        np.testing.assert_allclose(out[:, h, :], np.broadcast_to(u[h], (6, 4)), rtol=0, atol=1e-13)


def test_packed_equals_independent_samples():
    cu = np.array([0, 5, 5, 6, 13, 20], dtype=np.int32)
    x = rand_inputs(n_h=2, S=20, seed=9)
    out, lse = oracle.mla_forward(**x, cu_seqlens=cu)
    for a, b in zip(cu[:-1], cu[1:]):
        if a == b:
            continue
        o, l = oracle.mla_forward(x["q"][a:b], x["c_kv"][a:b], x["k_rope"][a:b], x["W_UK"], x["W_UV"])
        np.testing.assert_allclose(out[a:b], o, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[a:b], l, rtol=0, atol=1e-13)


@pytest.mark.parametrize("cu", [None, [0, 7, 7, 8, 21, 32]])
@pytest.mark.parametrize("SP", [2, 4, 8])
def test_sequence_parallel_shard_identity(SP, cu):
    S = 32
    cu_a = None if cu is None else np.array(cu, dtype=np.int32)
    x = rand_inputs(n_h=2, S=S, seed=21)
    dout = np.random.default_rng(22).standard_normal((S, 2, 4))
    o1, l1 = oracle.mla_forward(**x, cu_seqlens=cu_a)
    g1 = oracle.mla_backward(dout, **x, cu_seqlens=cu_a)
    n = S // SP
    outs, lses, dqs = [], [], []
    sums = [np.zeros_like(g) for g in g1[1:]]
    for r in range(SP):
        xs = dict(x, q=x["q"][r * n:(r + 1) * n])
        o, l = oracle.mla_forward(**xs, q_offset=r * n, cu_seqlens=cu_a)
        g = oracle.mla_backward(dout[r * n:(r + 1) * n], **xs, q_offset=r * n, cu_seqlens=cu_a)
        outs.append(o); lses.append(l); dqs.append(g[0])
        for acc, gi in zip(sums, g[1:]):
            acc += gi
    np.testing.assert_allclose(np.concatenate(outs), o1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(np.concatenate(lses), l1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(np.concatenate(dqs), g1[0], rtol=1e-12, atol=1e-14)
    for acc, ref in zip(sums, g1[1:]):
        np.testing.assert_allclose(acc, ref, rtol=1e-12, atol=1e-13)


RANGE_CASES = [
    # (S, q_ranges, cu_seqlens): rows are the blocks laid end to end
    (24, [(2, 3), (9, 4), (20, 2)], None),
    (24, [(0, 1), (23, 1)], None),
    (24, [(3, 5), (8, 2), (17, 7)], [0, 4, 4, 5, 11, 18, 24]),   # touching blocks
    (24, [(4, 1), (10, 6)], [0, 4, 4, 5, 11, 18, 24]),           # a length-1 sample
]


@pytest.mark.parametrize("S,ranges,cu", RANGE_CASES)
def test_forward_ranges_match_brute_force(S, ranges, cu):
    S_loc = sum(n for _, n in ranges)
    x = rand_inputs(S=S, S_loc=S_loc, seed=S + 3 * S_loc)
    cu_a = None if cu is None else np.array(cu, dtype=np.int32)
    out, lse = oracle.mla_forward(**x, cu_seqlens=cu_a, q_ranges=ranges)
    pos = [a + k for a, n in ranges for k in range(n)]
    bo, bl = brute_forward(x["q"].tolist(), x["c_kv"].tolist(), x["k_rope"].tolist(),
                           x["W_UK"].tolist(), x["W_UV"].tolist(), cu=cu, positions=pos)
    np.testing.assert_allclose(out, np.array(bo), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(bl), rtol=0, atol=1e-12)
    assert oracle.visible_pairs(S_loc, 0, cu_a, ranges) == sum(
        brute_visible_pairs(1, p, cu) for p in pos)


@pytest.mark.parametrize("cu", [None, [0, 7, 7, 8, 21, 32]])
@pytest.mark.parametrize("SP", [2, 4])
def test_zigzag_shard_identity(SP, cu):
    """Rank r of SP holds blocks r and 2SP-1-r of 2SP equal blocks."""
    S = 32
    C = S // (2 * SP)
    cu_a = None if cu is None else np.array(cu, dtype=np.int32)
    x = rand_inputs(n_h=2, S=S, seed=23)
    dout = np.random.default_rng(24).standard_normal((S, 2, 4))
    o1, l1 = oracle.mla_forward(**x, cu_seqlens=cu_a)
    g1 = oracle.mla_backward(dout, **x, cu_seqlens=cu_a)
    out = np.full_like(o1, np.nan); lse = np.full_like(l1, np.nan); dq = np.full_like(g1[0], np.nan)
    sums = [np.zeros_like(g) for g in g1[1:]]
    for r in range(SP):
        ranges = [(r * C, C), ((2 * SP - 1 - r) * C, C)]
        rows = np.concatenate([np.arange(a, a + n) for a, n in ranges])
        xs = dict(x, q=x["q"][rows])
        o, l = oracle.mla_forward(**xs, cu_seqlens=cu_a, q_ranges=ranges)
        g = oracle.mla_backward(dout[rows], **xs, cu_seqlens=cu_a, q_ranges=ranges)
        out[rows] = o; lse[rows] = l; dq[rows] = g[0]
        for acc, gi in zip(sums, g[1:]):
            acc += gi
    np.testing.assert_allclose(out, o1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, l1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dq, g1[0], rtol=1e-12, atol=1e-14)
    for acc, ref in zip(sums, g1[1:]):
        np.testing.assert_allclose(acc, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("SP", [1, 2, 4, 8])
def test_zigzag_ranks_have_equal_pairs(SP):
    """Block k of C rows holds k*C^2 + C(C+1)/2 causal pairs, so blocks r and
    2SP-1-r together hold (2SP-1)C^2 + C(C+1) on every rank."""
    C = 16
    for r in range(SP):
        ranges = [(r * C, C), ((2 * SP - 1 - r) * C, C)]
        assert oracle.visible_pairs(2 * C, 0, None, ranges) == (2 * SP - 1) * C * C + C * (C + 1)


def test_zero_gradient_for_keys_between_blocks():
    # the middle sample [6, 12) lies between the two blocks: nobody sees it
    cu = np.array([0, 6, 12, 18], np.int32)
    ranges = [(2, 3), (14, 3)]
    x = rand_inputs(S=18, S_loc=6, seed=63)
    dout = np.random.default_rng(64).standard_normal((6, 2, 4))
    _, dc, dkr, _, _ = oracle.mla_backward(dout, **x, cu_seqlens=cu, q_ranges=ranges)
    assert np.all(dc[6:12] == 0) and np.all(dkr[6:12] == 0)
    assert np.all(dc[5:6] == 0) and np.all(dc[17:] == 0)
    assert np.any(dc[:5] != 0) and np.any(dc[12:17] != 0)


def test_row_positions_rejects_wrong_total():
    with pytest.raises(ValueError):
        oracle.row_positions(5, 0, [(0, 2), (4, 2)])


# ----------------------------------------------------------- gradients
def _loss(x, dout, q_offset, cu, q_ranges=None):
    out, _ = oracle.mla_forward(**x, q_offset=q_offset, cu_seqlens=cu, q_ranges=q_ranges)
    return float(np.sum(out * dout))


def test_backward_ranges_directional_finite_differences():
    ranges = [(1, 4), (9, 5)]
    cu_a = np.array([0, 3, 3, 4, 10, 16], np.int32)
    x = rand_inputs(n_h=2, d_c=8, d_rope=4, d_nope=4, d_v=6, S=16, S_loc=9, seed=33)
    rng = np.random.default_rng(34)
    dout = rng.standard_normal((9, 2, 6))
    grads = oracle.mla_backward(dout, **x, cu_seqlens=cu_a, q_ranges=ranges)
    eps = 1e-5
    for name, g in zip(["q", "c_kv", "k_rope", "W_UK", "W_UV"], grads):
        for _ in range(3):
            v = rng.standard_normal(x[name].shape)
            xp = dict(x); xp[name] = x[name] + eps * v
            xm = dict(x); xm[name] = x[name] - eps * v
            fd = (_loss(xp, dout, 0, cu_a, ranges) - _loss(xm, dout, 0, cu_a, ranges)) / (2 * eps)
            an = float(np.sum(g * v))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


GRAD_CASES = [(16, 16, 0, None), (16, 11, 5, [0, 3, 3, 4, 10, 16])]


@pytest.mark.parametrize("S,S_loc,q_offset,cu", GRAD_CASES)
def test_backward_directional_finite_differences(S, S_loc, q_offset, cu):
    x = rand_inputs(n_h=2, d_c=8, d_rope=4, d_nope=4, d_v=6, S=S, S_loc=S_loc, seed=31)
    cu_a = None if cu is None else np.array(cu, dtype=np.int32)
    rng = np.random.default_rng(32)
    dout = rng.standard_normal((S_loc, 2, 6))
    grads = oracle.mla_backward(dout, **x, q_offset=q_offset, cu_seqlens=cu_a)
    names = ["q", "c_kv", "k_rope", "W_UK", "W_UV"]
    eps = 1e-5
    for name, g in zip(names, grads):
        for _ in range(3):
            v = rng.standard_normal(x[name].shape)
            xp = dict(x); xp[name] = x[name] + eps * v
            xm = dict(x); xm[name] = x[name] - eps * v
            fd = (_loss(xp, dout, q_offset, cu_a) - _loss(xm, dout, q_offset, cu_a)) / (2 * eps)
            an = float(np.sum(g * v))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


def test_backward_single_elements_finite_differences():
    x = rand_inputs(n_h=2, d_c=5, d_rope=2, d_nope=3, d_v=3, S=7, S_loc=4, seed=41)
    dout = np.random.default_rng(42).standard_normal((4, 2, 3))
    grads = oracle.mla_backward(dout, **x, q_offset=3)
    names = ["q", "c_kv", "k_rope", "W_UK", "W_UV"]
    eps = 1e-6
    for name, g in zip(names, grads):
        flat = x[name].reshape(-1)
        for k in range(0, flat.size, max(1, flat.size // 9)):
            xp = dict(x); xp[name] = x[name].copy(); xp[name].reshape(-1)[k] += eps
            xm = dict(x); xm[name] = x[name].copy(); xm[name].reshape(-1)[k] -= eps
            fd = (_loss(xp, dout, 3, None) - _loss(xm, dout, 3, None)) / (2 * eps)
            assert abs(fd - g.reshape(-1)[k]) <= 1e-7, (name, k)


def test_backward_head_subset_with_zero_dout():
    x = rand_inputs(n_h=4, S=12, S_loc=9, seed=51)
    dout = np.random.default_rng(52).standard_normal((9, 4, 4))
    keep = [1, 3]
    dz = np.zeros_like(dout); dz[:, keep] = dout[:, keep]
    full = oracle.mla_backward(dz, **x, q_offset=3)
    part = oracle.mla_backward(dz, **x, q_offset=3, heads=keep)
    for a, b in zip(full, part):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)


def test_zero_gradient_for_keys_nobody_sees():
    cu = np.array([0, 6, 12], np.int32)
    x = rand_inputs(S=12, S_loc=4, seed=61)
    dout = np.random.default_rng(62).standard_normal((4, 2, 4))
    _, dc, dkr, _, _ = oracle.mla_backward(dout, **x, q_offset=8, cu_seqlens=cu)
    assert np.all(dc[:6] == 0) and np.all(dkr[:6] == 0)   # earlier sample
    assert np.all(dc[12:] == 0)
    assert np.any(dc[6:12] != 0)


# -------------------------------------------------------------- counting
@pytest.mark.parametrize("S", [1, 2, 7, 100])
def test_visible_pairs_causal_closed_form(S):
    assert oracle.visible_pairs(S, 0) == S * (S + 1) // 2


@pytest.mark.parametrize("S_loc,q_off", [(1, 0), (5, 3), (2048, 14336)])
def test_visible_pairs_shard_closed_form(S_loc, q_off):
    assert oracle.visible_pairs(S_loc, q_off) == S_loc * q_off + S_loc * (S_loc + 1) // 2


@pytest.mark.parametrize("S_loc,q_off,cu", [(12, 0, [0, 3, 3, 4, 9, 12]),
                                            (7, 5, [0, 3, 3, 4, 9, 12]),
                                            (20, 10, [0, 1, 2, 15, 15, 30])])
def test_visible_pairs_varlen_brute(S_loc, q_off, cu):
    assert oracle.visible_pairs(S_loc, q_off, np.array(cu)) == brute_visible_pairs(S_loc, q_off, cu)


# The FLOP count of the block (what the throughput figures divide by) is the
# multiply-adds of the method's products, two FLOPs each, counted on visible
# (row, key) pairs only, plus the up-projection of the keys the shard needs.
# Forward: rebuild K_nope and V, scores, weights times V. Backward: the
# scores again (counted, as flash attention counts its recomputation), dP,
# dV, dq, dK, then dc_kv and dW, each over the needed keys; rebuilding K and
# V for the backward and the row sums D are not counted. The per-product
# multiply-adds come from running the element-by-element loops of
# tests/oracle_brute.py, whose values are pinned to the oracle first.
FLOP_CASES = [
    (6, 6, 0, None), (9, 5, 4, None), (12, 7, 5, [0, 3, 3, 4, 9, 12]),
    (10, 4, 6, [0, 1, 7, 10]), (7, 1, 6, None),
]
FWD_PRODUCTS = ("rebuild_K", "rebuild_V", "score", "PV")
BWD_PRODUCTS = ("score", "dP", "dV", "dq", "dK", "dc_kv", "dW")


@pytest.mark.parametrize("S,S_loc,q_offset,cu", FLOP_CASES)
def test_flops_count_the_products_of_brute_force_loops(S, S_loc, q_offset, cu):
    n_h, d_c, d_rope, d_nope, d_v = 2, 5, 2, 3, 4
    x = rand_inputs(n_h=n_h, d_c=d_c, d_rope=d_rope, d_nope=d_nope, d_v=d_v, S=S,
                    S_loc=S_loc, seed=S + S_loc)
    cu_a = None if cu is None else np.array(cu, np.int32)
    rng = np.random.default_rng(5)
    dout = rng.standard_normal((S_loc, n_h, d_v))
    L = {k: v.tolist() for k, v in x.items()}
    fc = MacCounter()
    bo, bl = brute_forward(L["q"], L["c_kv"], L["k_rope"], L["W_UK"], L["W_UV"],
                           q_offset=q_offset, cu=cu, counter=fc)
    bc = MacCounter()
    bg = brute_backward(dout.tolist(), L["q"], L["c_kv"], L["k_rope"], L["W_UK"], L["W_UV"], bo,
                        q_offset=q_offset, cu=cu, counter=bc)
    # the loops compute the oracle's values ...
    o, lse = oracle.mla_forward(**x, q_offset=q_offset, cu_seqlens=cu_a)
    np.testing.assert_allclose(np.array(bo), o, rtol=1e-11, atol=1e-12)
    g = oracle.mla_backward(dout, **x, q_offset=q_offset, cu_seqlens=cu_a)
    for got, ref in zip(bg, g):
        np.testing.assert_allclose(np.array(got), ref, rtol=1e-10, atol=1e-11)
    # ... and the FLOP counts are twice their multiply-adds
    args = (n_h, d_c, d_rope, d_nope, d_v, S_loc, q_offset, cu_a)
    assert oracle.attention_flops(*args) == 2 * sum(fc[k] for k in FWD_PRODUCTS)
    assert oracle.attention_flops(*args, backward=True) == 2 * sum(bc[k] for k in BWD_PRODUCTS)
    assert set(fc) == set(FWD_PRODUCTS)
    assert set(bc) == set(BWD_PRODUCTS) | {"rebuild_K", "rebuild_V", "D"}


def test_flops_headline_shard():
    # n_h=128, S=16384, last of 8 shards: 31,458,304 pairs/head, 16384 keys
    f = oracle.attention_flops(128, 512, 64, 128, 128, 2048, 14336)
    pairs = 2048 * 14336 + 2048 * 2049 // 2
    assert oracle.visible_pairs(2048, 14336) == pairs == 31_458_304
    assert f == 2 * 128 * 320 * pairs + 2 * 128 * 512 * 256 * 16384
    assert abs(f / 1e12 - 3.127) < 1e-3


def test_decode_batch_absorbed_equals_explicit():
    """A decode batch (one query per packed sequence, at its last position)
    computed in the absorbed form equals the explicit form (LAGA abstract:
    the absorbed form is a reformulation, used for decode)."""
    lens = [1, 4, 9, 2]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    last = [(int(cu[b + 1]) - 1, 1) for b in range(len(lens))]
    x = rand_inputs(n_h=3, S=int(cu[-1]), S_loc=len(lens), seed=71)
    o1, l1 = oracle.mla_forward(**x, cu_seqlens=cu, q_ranges=last)
    o2, l2 = oracle.mla_forward_absorbed(**x, cu_seqlens=cu, q_ranges=last)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=1e-12, atol=1e-13)
    # the one-key sequence attends to its own row only: out = V of that row
    c = x["c_kv"][0]
    for h in range(3):
        np.testing.assert_allclose(o1[0, h], c @ x["W_UV"][:, 4 * h:4 * (h + 1)], rtol=1e-12)
