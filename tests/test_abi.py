"""C ABI checks that need no GPU: the library loads, exports every entry
point the header declares, validates arguments on the host before touching
the device, and its host-side counts agree with the oracle's mask."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import workloads

hla = pytest.importorskip("head_latent_attention_kv_amd")


@pytest.fixture(scope="module")
def lib():
    return hla.load_library()


def header_symbols(root):
    src = open(os.path.join(root, "include", "mla_laga.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_laga_\w+)\s*\(", src)))


def test_exports_every_declared_symbol(lib, root_dir):
    names = header_symbols(root_dir)
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
        assert n in hla.EXPORTED, f"binding does not wrap {n}"


def desc_for(cfg, **kw):
    d = hla.MLADesc()
    d.n_h, d.d_c, d.d_rope, d.d_nope, d.d_v = cfg.n_h, cfg.d_c, cfg.d_rope, cfg.d_nope, cfg.d_v
    cu = cfg.cu_seqlens()
    d.n_seqs = 0 if cu is None else len(cu) - 1
    d.S, d.S_loc, d.q_offset = cfg.S, cfg.S_loc, cfg.q_offset
    d.in_dtype = hla.MLA_BF16 if cfg.dtype == "bf16" else hla.MLA_F32
    d.flags, d.softmax_scale = 0, 0.0
    for k, v in kw.items():
        setattr(d, k, v)
    return d, cu


@pytest.mark.parametrize("name", workloads.CONFIG_ORDER)
def test_counts_match_oracle(name):
    cfg = workloads.config(name)
    d, cu = desc_for(cfg)
    pairs, lo, hi = hla.mla_laga_count(d, cu)
    assert pairs == oracle.visible_pairs(cfg.S_loc, cfg.q_offset, cu)
    assert (lo, hi) == oracle.key_range(cfg.S_loc, cfg.q_offset, cu)


@pytest.mark.parametrize("S,S_loc,q_off,cu", [
    (12, 12, 0, [0, 3, 3, 4, 9, 12]), (12, 7, 5, [0, 3, 3, 4, 9, 12]),
    (40, 9, 31, [0, 31, 31, 31, 40]), (5, 1, 4, None), (33, 0, 33, None)])
def test_counts_edge_cases(S, S_loc, q_off, cu):
    cfg = workloads.config("tiny_f32").with_(S=S, S_loc=S_loc, q_offset=q_off)
    d, _ = desc_for(cfg)
    cu_a = None if cu is None else np.array(cu, np.int32)
    d.n_seqs = 0 if cu is None else len(cu) - 1
    pairs, lo, hi = hla.mla_laga_count(d, cu_a)
    assert pairs == oracle.visible_pairs(S_loc, q_off, cu_a)
    if S_loc:
        assert (lo, hi) == oracle.key_range(S_loc, q_off, cu_a)


def with_ranges(d, ranges):
    """Point the descriptor at (start, length) blocks; returns the array that
    must stay alive while it is used."""
    arr = np.ascontiguousarray(np.asarray(ranges, np.int64).reshape(-1, 2))
    d.n_ranges = len(arr)
    d.q_ranges = arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    d.S_loc = int(arr[:, 1].sum())
    d.q_offset = 0
    return arr


RANGE_COUNT_CASES = [
    (16384, workloads.zigzag_blocks(16384, 0, 8), None),
    (16384, workloads.zigzag_blocks(16384, 7, 8), None),
    (600, [(5, 120), (300, 200)], [0, 1, 1, 130, 131, 400, 600]),
    (700, [(10, 150), (470, 200)], [0, 200, 450, 700]),    # a sample nobody sees
    (50, [(0, 0), (3, 1), (4, 0), (49, 1)], None),          # empty and one-row blocks
]


@pytest.mark.parametrize("S,ranges,cu", RANGE_COUNT_CASES)
def test_counts_with_ranges_match_oracle(S, ranges, cu):
    cfg = workloads.config("tiny_f32").with_(S=S)
    d, _ = desc_for(cfg)
    keep = with_ranges(d, ranges)
    cu_a = None if cu is None else np.array(cu, np.int32)
    d.n_seqs = 0 if cu is None else len(cu) - 1
    pairs, lo, hi = hla.mla_laga_count(d, cu_a)
    S_loc = int(keep[:, 1].sum())
    rl = [tuple(r) for r in keep.tolist()]
    assert pairs == oracle.visible_pairs(S_loc, 0, cu_a, rl)
    assert (lo, hi) == oracle.key_range(S_loc, 0, cu_a, rl)


def test_zigzag_ranks_balance_pairs():
    per_rank = []
    for r in range(8):
        d, _ = desc_for(workloads.config("tiny_f32").with_(S=16384))
        keep = with_ranges(d, workloads.zigzag_blocks(16384, r, 8))
        per_rank.append(hla.mla_laga_count(d, None)[0])
    assert len(set(per_rank)) == 1
    d, _ = desc_for(workloads.config("h128_s16k_shard"))
    contiguous_last = hla.mla_laga_count(d, None)[0]
    assert contiguous_last > 1.8 * per_rank[0]


def test_invalid_ranges_rejected_on_host():
    E = hla.MLA_ERR_INVALID_ARG
    cfg = workloads.config("tiny_f32").with_(S=100)
    cases = [
        [(50, 10), (20, 10)],          # descending
        [(10, 20), (25, 10)],          # overlapping
        [(-1, 5)],                     # before 0
        [(95, 10)],                    # past S
        [(10, -2), (20, 4)],           # negative length
    ]
    for ranges in cases:
        d, _ = desc_for(cfg)
        keep = with_ranges(d, ranges)
        bad(E, hla.mla_laga_fwd_workspace_size, d, None)
    d, _ = desc_for(cfg)
    keep = with_ranges(d, [(0, 10), (40, 10)])
    d.S_loc = 21                                            # rows do not add up
    assert "S_loc" in bad(E, hla.mla_laga_count, d, None)
    d.S_loc = 20
    d.q_offset = 3                                          # q_offset with ranges
    assert "q_offset" in bad(E, hla.mla_laga_count, d, None)
    d.q_offset = 0
    d.q_ranges = None                                       # NULL blocks
    bad(E, hla.mla_laga_count, d, None)
    d, _ = desc_for(cfg)
    keep = with_ranges(d, [(2 * k, 1) for k in range(hla.MLA_MAX_RANGES + 1)])
    bad(E, hla.mla_laga_count, d, None)
    keep = with_ranges(d, [(2 * k, 1) for k in range(hla.MLA_MAX_RANGES)])
    assert hla.mla_laga_count(d, None)[0] == sum(2 * k + 1 for k in range(hla.MLA_MAX_RANGES))


def test_workspace_linear_in_rows_and_heads():
    # the rebuilt K/V dominate the workspace: affine in the key count and in n_h
    base = workloads.config("h128_s16k_shard")
    def ws(**kw):
        d, cu = desc_for(base.with_(**kw))
        return hla.mla_laga_fwd_workspace_size(d, cu)
    a, b, c = ws(S=4096, S_loc=1024, q_offset=3072), ws(S=8192, S_loc=1024, q_offset=7168), \
        ws(S=12288, S_loc=1024, q_offset=11264)
    assert b - a == c - b and b > a
    h1, h2, h3 = ws(n_h=8), ws(n_h=16), ws(n_h=24)
    assert h2 - h1 == h3 - h2 and h2 > h1


def stored_ds_bytes(n_h, keys, rows):
    """Workspace the stored-dS backward adds: fp16 dS per (row padded to 64,
    needed key padded to 256, head). All heads in one buffer while that is
    at most 16 GiB; else head groups of at most 1 GiB each, as even as their
    count allows, through two group buffers, if 8 heads fit a group; else 0
    (dQ recomputes)."""
    per_head = (keys + 255) // 256 * 256 * ((rows + 63) // 64 * 64) * 2
    if n_h * per_head <= 16 << 30:
        return n_h * per_head
    if 8 * per_head > 1 << 30:   # a group would hold fewer than 8 heads
        return 0
    groups = -(-n_h // ((1 << 30) // per_head))
    return 2 * -(-n_h // groups) * per_head


def test_stored_ds_workspace():
    """The default backward recomputes the scores for dQ, so its workspace is
    a sum of per-row and per-key terms: the mixed second difference over
    (rows, keys) vanishes. With MLA_FLAG_STORED_DS it holds dS (fp16) as
    well: n_h x Kpad x S_pad while that fits 16 GiB, else two buffers of one
    head group (at most 1 GiB, at least 8 heads) each."""
    base = workloads.config("h128_s16k_shard")

    def ws(S_loc, S, flags=0, n_h=128):
        d, cu = desc_for(base.with_(S=S, S_loc=S_loc, q_offset=S - S_loc, n_h=n_h))
        d.flags = flags
        return hla.mla_laga_bwd_workspace_size(d, cu)

    for flags, term in ((0, 0), (hla.MLA_FLAG_STORED_DS, 128 * 8192 * 1024 * 2)):
        mixed = ws(2048, 16384, flags) - ws(1024, 16384, flags) - ws(2048, 8192, flags) \
            + ws(1024, 8192, flags)
        assert mixed == term, (flags, mixed)
    S = hla.MLA_FLAG_STORED_DS
    cases = [
        (128, 16384, 2048, 8 << 30),             # one buffer
        (128, 32768, 2048, 16 << 30),            # one buffer, at its limit
        (129, 32768, 2048, 2 * 8 * (128 << 20)),  # past it: 17 groups of 8 (the last of 1)
        (130, 16384, 4096, 2 * 8 * (128 << 20)),  # 16 groups of 8 and one of 2
        (256, 32768, 4096, 0),                   # four heads of 256 MiB per group: recomputes
        (128, 32769, 2048, 0),                   # 7 heads of 129 MiB per group: recomputes
        (47, 24576, 8192, 0),                    # 384 MiB heads, 17.6 GiB: recomputes
        (8, 131072, 8192, 16 << 30),             # 2 GiB heads, but one buffer holds them
        (128, 131072, 8192, 0),                  # neither: dQ recomputes
    ]
    for n_h, keys, rows, want in cases:
        assert stored_ds_bytes(n_h, keys, rows) == want, (n_h, keys, rows)
        assert ws(rows, keys, S, n_h) - ws(rows, keys, 0, n_h) == want, (n_h, keys, rows)


def test_unknown_flags_rejected():
    d, cu = desc_for(workloads.config("h16_s4k"))
    for f in (2, 8, 1 << 30):
        d.flags = f
        with pytest.raises(hla.MLAError) as e:
            hla.mla_laga_fwd_workspace_size(d, cu)
        assert e.value.status == hla.MLA_ERR_INVALID_ARG
        assert "flag" in str(e.value)


def bad(status, fn, *args):
    with pytest.raises(hla.MLAError) as e:
        fn(*args)
    assert e.value.status == status
    return str(e.value)


def test_invalid_arguments_rejected_on_host():
    cfg = workloads.config("h16_s4k")
    E = hla.MLA_ERR_INVALID_ARG
    d, _ = desc_for(cfg, q_offset=1)                       # q_offset + S_loc > S
    assert "q_offset" in bad(E, hla.mla_laga_fwd_workspace_size, d, None)
    d, _ = desc_for(cfg, n_h=0)
    bad(E, hla.mla_laga_fwd_workspace_size, d, None)
    d, _ = desc_for(cfg, in_dtype=7)
    bad(E, hla.mla_laga_fwd_workspace_size, d, None)
    d, _ = desc_for(cfg, n_seqs=2)                         # cu missing
    bad(E, hla.mla_laga_fwd_workspace_size, d, None)
    d, _ = desc_for(cfg, n_seqs=2)
    bad(E, hla.mla_laga_fwd_workspace_size, d, np.array([0, 5, 4000], np.int32))  # end != S
    bad(E, hla.mla_laga_fwd_workspace_size, d, np.array([0, 5000, 4096], np.int32))  # decreasing
    d, _ = desc_for(cfg, d_nope=300, in_dtype=hla.MLA_F32)
    bad(hla.MLA_ERR_UNSUPPORTED, hla.mla_laga_fwd_workspace_size, d, None)


def test_fast_path_size_limits_rejected_on_host(lib):
    """Shapes past the fast kernels' 32-bit offsets and GEMM operand limits
    are refused by the workspace queries and by the calls, before any
    launch (no GPU is touched here)."""
    cfg = workloads.config("h128_s16k_shard")
    U = hla.MLA_ERR_UNSUPPORTED
    S = 1 << 22                         # one query at the end: 2^22 needed keys
    d, _ = desc_for(cfg, S=S, S_loc=1, q_offset=S - 1, n_h=1)
    assert lib.mla_laga_uses_fast_path(ctypes.byref(d)) == 1
    assert "2^22" in bad(U, hla.mla_laga_fwd_workspace_size, d, None)
    assert "2^22" in bad(U, hla.mla_laga_bwd_workspace_size, d, None)
    good = ctypes.c_void_p(1 << 20)    # never dereferenced: the limits come first
    huge = ctypes.c_size_t(1 << 44)
    assert lib.mla_laga_fwd(ctypes.byref(d), good, good, good, good, good, None, None,
                            good, good, good, huge, None) == U
    assert lib.mla_laga_bwd(ctypes.byref(d), good, good, good, good, good, good, None, None,
                            good, good, good, good, good, good, good, good, huge, None) == U
    # one key fewer fits
    d, _ = desc_for(cfg, S=S - 256, S_loc=1, q_offset=S - 257, n_h=1)
    assert hla.mla_laga_fwd_workspace_size(d, None) > 0
    assert hla.mla_laga_bwd_workspace_size(d, None) > 0
    # n_h: the backward's GEMMs take fewer heads than the forward's
    d, _ = desc_for(cfg, S=256, S_loc=256, q_offset=0, n_h=16384)
    assert hla.mla_laga_fwd_workspace_size(d, None) > 0
    assert "n_h" in bad(U, hla.mla_laga_bwd_workspace_size, d, None)
    d, _ = desc_for(cfg, S=256, S_loc=256, q_offset=0, n_h=32768)
    assert "n_h" in bad(U, hla.mla_laga_fwd_workspace_size, d, None)


def test_null_and_misaligned_pointers_rejected_before_launch(lib):
    cfg = workloads.config("h16_s4k")
    d, _ = desc_for(cfg)
    ws = hla.mla_laga_fwd_workspace_size(d, None)
    good = ctypes.c_void_p(1 << 20)        # never dereferenced: validation fails first
    odd = ctypes.c_void_p((1 << 20) + 8)
    args = [good] * 5
    st = lib.mla_laga_fwd(ctypes.byref(d), None, *args[1:], None, None, good, good, good, ws, None)
    assert st == hla.MLA_ERR_INVALID_ARG and b"q" in lib.mla_laga_last_error()
    st = lib.mla_laga_fwd(ctypes.byref(d), odd, *args[1:], None, None, good, good, good, ws, None)
    assert st == hla.MLA_ERR_INVALID_ARG and b"aligned" in lib.mla_laga_last_error()
    st = lib.mla_laga_fwd(ctypes.byref(d), *args, None, None, good, good, good, ws - 1, None)
    assert st == hla.MLA_ERR_WORKSPACE
    st = lib.mla_laga_fwd(ctypes.byref(d), *args, None, None, good, good, None, ws, None)
    assert st == hla.MLA_ERR_WORKSPACE
    st = lib.mla_laga_fwd(ctypes.byref(d), *args, None, None, None, good, good, ws, None)
    assert st == hla.MLA_ERR_INVALID_ARG


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4, -5):
        assert lib.mla_laga_status_string(s).startswith(b"MLA_")
    assert lib.mla_laga_status_string(hla.MLA_ERR_DEBUG_CHECK) == b"MLA_ERR_DEBUG_CHECK"


def test_debug_mode_adds_a_256_byte_tail_to_every_workspace(monkeypatch):
    """MLA_LAGA_DEBUG is read at every call: the workspace sizes grow by the
    canary tail while it is set (and not "0"), and only then."""
    cfg = workloads.config("h128_varlen64k")
    d, cu = desc_for(cfg)
    dd = decode_desc()
    dcu = np.array([0, 10, 11, 60, 100], np.int32)

    def sizes():
        return (hla.mla_laga_fwd_workspace_size(d, cu), hla.mla_laga_bwd_workspace_size(d, cu),
                hla.mla_laga_decode_workspace_size(dd, dcu))

    monkeypatch.delenv("MLA_LAGA_DEBUG", raising=False)
    base = sizes()
    for v, extra in (("1", 256), ("0", 0), ("", 0), ("yes", 256)):
        monkeypatch.setenv("MLA_LAGA_DEBUG", v)
        assert sizes() == tuple(b + extra for b in base), v


def test_row_window_validated_on_host(lib):
    cfg = workloads.config("h128_varlen64k")
    d, cu = desc_for(cfg)
    fake = ctypes.c_void_p(1 << 20)   # never dereferenced: validation fails first
    cup = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    assert lib.mla_laga_row_window(ctypes.byref(d), cup, fake, None, None) == hla.MLA_ERR_INVALID_ARG
    assert b"window" in lib.mla_laga_last_error()
    assert lib.mla_laga_row_window(ctypes.byref(d), cup, None, fake, None) == hla.MLA_ERR_INVALID_ARG
    assert b"cu_seqlens_dev" in lib.mla_laga_last_error()
    odd = ctypes.c_void_p((1 << 20) + 8)
    assert lib.mla_laga_row_window(ctypes.byref(d), cup, fake, odd, None) == hla.MLA_ERR_INVALID_ARG
    d.S_loc = 0
    d.q_offset = 0
    assert lib.mla_laga_row_window(ctypes.byref(d), cup, None, None, None) == hla.MLA_OK


def decode_desc(n_h=128, batch=4, S=100, d_c=512, d_rope=64, d_nope=128, d_v=128, dtype=None):
    d = hla.MLADecodeDesc()
    d.n_h, d.d_c, d.d_rope, d.d_nope, d.d_v = n_h, d_c, d_rope, d_nope, d_v
    d.batch, d.S = batch, S
    d.in_dtype = hla.MLA_BF16 if dtype is None else dtype
    d.softmax_scale = 0.0
    return d


def test_decode_validation_and_workspace():
    cu = np.array([0, 10, 11, 60, 100], np.int32)
    ws = hla.mla_laga_decode_workspace_size(decode_desc(), cu)
    assert ws > 128 * 128 * 512 * 2            # at least W_UV^T in fp16
    longer = np.array([0, 10, 11, 60, 100000], np.int32)
    assert hla.mla_laga_decode_workspace_size(decode_desc(S=100000), longer) > ws
    E, U = hla.MLA_ERR_INVALID_ARG, hla.MLA_ERR_UNSUPPORTED
    bad(E, hla.mla_laga_decode_workspace_size, decode_desc(batch=0), np.array([0], np.int32))
    bad(E, hla.mla_laga_decode_workspace_size, decode_desc(), np.array([0, 10, 10, 60, 100], np.int32))
    bad(E, hla.mla_laga_decode_workspace_size, decode_desc(), np.array([0, 10, 11, 60, 99], np.int32))
    bad(E, hla.mla_laga_decode_workspace_size, decode_desc(), None)
    bad(U, hla.mla_laga_decode_workspace_size, decode_desc(d_c=256), cu)
    bad(U, hla.mla_laga_decode_workspace_size, decode_desc(n_h=48), cu)
    bad(U, hla.mla_laga_decode_workspace_size, decode_desc(dtype=hla.MLA_F32), cu)
