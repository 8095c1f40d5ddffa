"""The pins have teeth: plant plausible mistakes in a copy of the oracle's
source (on the CPU, never in the library) and check that a pin rejects each.
"""

import math
import types

import numpy as np
import pytest

from oracle import mla_oracle as M
from tests.oracle_brute import brute_forward
from tests.test_oracle_pins import rand_inputs


def mutant(old: str, new: str) -> types.ModuleType:
    src = open(M.__file__).read()
    assert src.count(old) >= 1, old
    mod = types.ModuleType("oracle_mutant")
    mod.__dict__["__name__"] = "oracle_mutant"
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def brute_error(mod, S=12, S_loc=7, q_offset=5, cu=(0, 3, 3, 4, 9, 12)):
    x = rand_inputs(S=S, S_loc=S_loc, seed=77)
    cu_a = None if cu is None else np.array(cu, dtype=np.int32)
    out, lse = mod.mla_forward(**x, q_offset=q_offset, cu_seqlens=cu_a)
    bo, bl = brute_forward(x["q"].tolist(), x["c_kv"].tolist(), x["k_rope"].tolist(),
                           x["W_UK"].tolist(), x["W_UV"].tolist(), q_offset,
                           None if cu is None else list(cu))
    return max(np.abs(out - np.array(bo)).max(), np.abs(lse - np.array(bl)).max())


def fd_error(mod):
    x = rand_inputs(n_h=2, d_c=8, d_rope=4, d_nope=4, d_v=6, S=16, S_loc=11, seed=31)
    cu = np.array([0, 3, 3, 4, 10, 16], np.int32)
    rng = np.random.default_rng(5)
    dout = rng.standard_normal((11, 2, 6))
    grads = mod.mla_backward(dout, **x, q_offset=5, cu_seqlens=cu)
    worst = 0.0
    for name, g in zip(["q", "c_kv", "k_rope", "W_UK", "W_UV"], grads):
        v = rng.standard_normal(x[name].shape)
        def loss(z):
            xx = dict(x); xx[name] = z
            return float(np.sum(M.mla_forward(**xx, q_offset=5, cu_seqlens=cu)[0] * dout))
        eps = 1e-5
        fd = (loss(x[name] + eps * v) - loss(x[name] - eps * v)) / (2 * eps)
        worst = max(worst, abs(fd - float(np.sum(g * v))))
    return worst


def test_unmutated_passes():
    assert brute_error(M) < 1e-12
    assert fd_error(M) < 1e-6


FWD_MUTANTS = [
    # rope part of the key dropped
    ("K = np.concatenate([k_nope, k_rope[k0:k1]], axis=1)",
     "K = np.concatenate([k_nope, 0 * k_rope[k0:k1]], axis=1)"),
    # heads taken as interleaved weight columns instead of head-major blocks
    ("k_nope = c @ W_UK[:, h * d_nope:(h + 1) * d_nope]",
     "k_nope = c @ W_UK[:, h::W_UK.shape[1] // d_nope]"),
    # diagonal excluded from the causal mask
    ("(keys[None, :] <= hi[r][:, None])\n            P, l",
     "(keys[None, :] < hi[r][:, None]) | (keys[None, :] == lo[r][:, None])\n            P, l"),
    # sample start taken from the wrong side (first start > p)
    ('k = np.searchsorted(cu, p, side="right") - 1', 'k = np.searchsorted(cu, p, side="left") - 1'),
    # scale forgotten
    ("s = scale * (q[r, h, :] @ K.T)\n            vis", "s = (q[r, h, :] @ K.T)\n            vis"),
    # lse in log2 instead of natural log
    ("lse = m_safe + np.log(tot)", "lse = m_safe + np.log2(tot)"),
]


@pytest.mark.parametrize("old,new", FWD_MUTANTS)
def test_forward_mutant_caught_by_brute_force(old, new):
    assert brute_error(mutant(old, new)) > 1e-6


BWD_MUTANTS = [
    ("dS = P * (dO @ V.T - D)", "dS = P * (D - dO @ V.T)"),            # sign
    ("dS = P * (dO @ V.T - D)", "dS = P * (dO @ V.T)"),                # dropped D term
    ("dq[r, h, :] = scale * (dS @ K)", "dq[r, h, :] = (dS @ K)"),      # missing scale
    ("dc_kv[k0:k1] += dK_nope @ Wk.T + dV @ Wv.T", "dc_kv[k0:k1] += dV @ Wv.T"),
    ("dW_UK[:, h * d_nope:(h + 1) * d_nope] = c_kv[k0:k1].T @ dK_nope",
     "dW_UK[:, h * d_nope:(h + 1) * d_nope] = c_kv[k0:k1].T @ dK[:, d_rope:]"),
    ("dK += scale * (dS.T @ q[r, h, :])", "dK += scale * (dS @ K).T[:, :0].sum() + scale * (P.T @ q[r, h, :])"),
]


@pytest.mark.parametrize("old,new", BWD_MUTANTS)
def test_backward_mutant_caught_by_finite_differences(old, new):
    assert fd_error(mutant(old, new)) > 1e-4


def ranges_error(mod):
    ranges = [(3, 5), (8, 2), (16, 7)]
    cu = [0, 4, 4, 5, 11, 18, 24]
    x = rand_inputs(S=24, S_loc=14, seed=78)
    out, lse = mod.mla_forward(**x, cu_seqlens=np.array(cu, np.int32), q_ranges=ranges)
    pos = [a + k for a, n in ranges for k in range(n)]
    bo, bl = brute_forward(x["q"].tolist(), x["c_kv"].tolist(), x["k_rope"].tolist(),
                           x["W_UK"].tolist(), x["W_UV"].tolist(), cu=cu, positions=pos)
    err = np.concatenate([np.abs(out - np.array(bo)).ravel(), np.abs(lse - np.array(bl)).ravel()])
    return float(err.max()) if np.all(np.isfinite(err)) else math.inf


RANGE_MUTANTS = [
    # each block's rows counted from position 0 of the block list
    ("parts = [np.arange(int(a), int(a) + int(n), dtype=np.int64) for a, n in q_ranges]",
     "parts = [np.arange(0, int(n), dtype=np.int64) + int(q_ranges[0][0]) for a, n in q_ranges]"),
    # blocks laid end to end in reverse
    ("pos = np.concatenate(parts) if parts else",
     "pos = np.concatenate(parts[::-1]) if parts else"),
    # block end treated as inclusive, start shifted to compensate
    ("parts = [np.arange(int(a), int(a) + int(n), dtype=np.int64) for a, n in q_ranges]",
     "parts = [np.arange(int(a) + 1, int(a) + int(n) + 1, dtype=np.int64) for a, n in q_ranges]"),
]


def test_ranges_unmutated_passes():
    assert ranges_error(M) < 1e-12


@pytest.mark.parametrize("old,new", RANGE_MUTANTS)
def test_ranges_mutant_caught_by_brute_force(old, new):
    assert ranges_error(mutant(old, new)) > 1e-6


def flop_error(mod):
    """Largest difference between the module's FLOP counts and twice the
    multiply-adds that the brute-force loops perform (forward products; the
    backward's products less the K/V rebuild and the row sums D)."""
    from tests.oracle_brute import MacCounter, brute_backward
    from tests.test_oracle_pins import BWD_PRODUCTS, FWD_PRODUCTS
    worst = 0
    for S, S_loc, q_offset, cu in ((9, 5, 4, None), (12, 7, 5, [0, 3, 3, 4, 9, 12])):
        x = rand_inputs(n_h=2, d_c=5, d_rope=2, d_nope=3, d_v=4, S=S, S_loc=S_loc, seed=9)
        L = {k: v.tolist() for k, v in x.items()}
        dout = np.ones((S_loc, 2, 4)).tolist()
        fc, bc = MacCounter(), MacCounter()
        bo, _ = brute_forward(L["q"], L["c_kv"], L["k_rope"], L["W_UK"], L["W_UV"], q_offset, cu,
                              counter=fc)
        brute_backward(dout, L["q"], L["c_kv"], L["k_rope"], L["W_UK"], L["W_UV"], bo, q_offset,
                       cu, counter=bc)
        cu_a = None if cu is None else np.array(cu, np.int32)
        args = (2, 5, 2, 3, 4, S_loc, q_offset, cu_a)
        worst = max(worst, abs(mod.attention_flops(*args) - 2 * sum(fc[k] for k in FWD_PRODUCTS)),
                    abs(mod.attention_flops(*args, backward=True) - 2 * sum(bc[k] for k in BWD_PRODUCTS)))
    return worst


FLOP_MUTANTS = [
    # the backward's score recomputation not counted
    ("return 2 * n_h * (3 * d_qk + 2 * d_v) * P", "return 2 * n_h * (2 * d_qk + 2 * d_v) * P"),
    # dP or dV dropped
    ("return 2 * n_h * (3 * d_qk + 2 * d_v) * P", "return 2 * n_h * (3 * d_qk + d_v) * P"),
    # the backward's up-projection gradients counted once
    ("+ 4 * n_h * d_c * (d_nope + d_v) * Kn", "+ 2 * n_h * d_c * (d_nope + d_v) * Kn"),
    # the forward without the up-projection
    ("return 2 * n_h * (d_qk + d_v) * P + 2 * n_h * d_c * (d_nope + d_v) * Kn",
     "return 2 * n_h * (d_qk + d_v) * P"),
    # the forward's value width taken as d_qk
    ("return 2 * n_h * (d_qk + d_v) * P + 2", "return 2 * n_h * (2 * d_qk) * P + 2"),
]


def test_flops_unmutated_passes():
    assert flop_error(M) == 0


@pytest.mark.parametrize("old,new", FLOP_MUTANTS)
def test_flop_mutant_caught_by_counted_loops(old, new):
    assert flop_error(mutant(old, new)) > 0
