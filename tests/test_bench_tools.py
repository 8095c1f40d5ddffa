"""Host-side tools of bench.py that turn rocprofv3 counter csv files into the
traffic record and the utilisation table (no GPU): the second step of a
counter run is selected, counters are scaled by the plain copy's reading, and
the utilisation ratios follow the profiler's own formulas."""

import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
          "Counter_Value", "Start_Timestamp", "End_Timestamp"]
FWD = "_ZN3mla12_GLOBAL__N_115attn_fwd_kernelILi1ELi8EEEvPKt"
DKDV = "_ZN3mla12_GLOBAL__N_120attn_bwd_dkdv_kernelEPKDF16_"
COPY = "__amd_rocclr_copyBuffer"


def write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for disp, name, counter, value, t0, t1 in rows:
            w.writerow({k: 0 for k in FIELDS} | {
                "Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": counter,
                "Counter_Value": value, "Start_Timestamp": t0, "End_Timestamp": t1})


def test_traffic_counts_second_step_scaled_by_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(tmp_path / "traffic.json"))
    copy_units = 262144.0   # what FETCH_SIZE reads for the 512 MiB copy: 2048 B per unit
    fetch = [(1, FWD, "FETCH_SIZE", 999999.0, 0, 1), (2, DKDV, "FETCH_SIZE", 888888.0, 0, 1),
             (5, FWD, "FETCH_SIZE", 1000.0, 0, 1), (6, DKDV, "FETCH_SIZE", 3000.0, 0, 1),
             (9, COPY, "FETCH_SIZE", copy_units, 0, 1)]
    write = [(1, FWD, "WRITE_SIZE", 777777.0, 0, 1), (2, DKDV, "WRITE_SIZE", 666666.0, 0, 1),
             (5, FWD, "WRITE_SIZE", 10.0, 0, 1), (6, DKDV, "WRITE_SIZE", 20.0, 0, 1),
             (9, COPY, "WRITE_SIZE", 524288.0, 0, 1)]
    write_csv(tmp_path / "f.csv", fetch)
    write_csv(tmp_path / "w.csv", write)
    table = bench.traffic_from_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "wl")
    fwd, dkdv = table["attn_fwd@wl"], table["attn_bwd_dkdv@wl"]
    # first-step dispatches (1, 2) are ignored; FETCH_SIZE scales by 2048 B, WRITE_SIZE by 1 KiB
    assert fwd["fetch_bytes"] == 1000 * 2048 and fwd["write_bytes"] == 10 * 1024
    assert dkdv["bytes_per_launch"] == 3000 * 2048 + 20 * 1024
    assert dkdv["sha"] == bench.sources_sha(dkdv["sources"])
    assert json.load(open(tmp_path / "traffic.json")) == table


def test_utilisation_formulas(tmp_path):
    # one second-step dispatch of 1 ms on 8 XCDs at 2.0 GHz: 2e6 active cycles per XCD
    t0, t1 = 0, 1_000_000
    grbm = 8 * 2.0e6
    a = [(3, FWD, "GRBM_GUI_ACTIVE", grbm, t0, t1),
         (3, FWD, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * 2.0e6 * 1024, t0, t1),
         (3, FWD, "SQ_INSTS_VALU_MFMA_MOPS_F16", 1.0e12 / 512, t0, t1),
         (3, FWD, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0, t0, t1),
         (3, FWD, "SQ_LDS_IDX_ACTIVE", 0.25 * 2.0e6 * 256, t0, t1),
         (3, FWD, "SQ_LDS_BANK_CONFLICT", 0.1 * 0.25 * 2.0e6 * 256, t0, t1),
         (3, FWD, "SQ_BUSY_CU_CYCLES", 0.0, t0, t1),
         (3, FWD, "SQ_ACTIVE_INST_VALU", 200.0, t0, t1),
         (3, FWD, "SQ_INSTS_VALU_TRANS_F32", 0.0, t0, t1),
         (1, FWD, "GRBM_GUI_ACTIVE", 1e12, t0, t1)]          # first step: ignored
    b = [(3, FWD, "SQ_WAVE_CYCLES", 1000.0, t0, t1), (3, FWD, "SQ_ACTIVE_INST_LDS", 50.0, t0, t1),
         (3, FWD, "SQ_WAIT_INST_ANY", 400.0, t0, t1), (3, FWD, "GRBM_GUI_ACTIVE", grbm, t0, t1)]
    write_csv(tmp_path / "a.csv", a)
    write_csv(tmp_path / "b.csv", b)
    rows = bench.utilisation_from_counters(str(tmp_path / "a.csv"), str(tmp_path / "b.csv"))
    line = [ln for ln in rows.splitlines() if ln.startswith("| attn_fwd_kernel")][0]
    cells = [c.strip() for c in line.strip("|").split("|")]
    name, launches, ms, clk, busy, tf, frac, lds, conflict, valu, ldsi, wait = cells
    assert launches == "1" and ms == "1.000" and clk == "2.00"
    assert busy == "50.0%" and tf == "1000.0" and lds == "25.0%" and conflict == "10.0%"
    # 1000 TFLOP/s against the dense peak scaled to 2.0 GHz
    assert frac == f"{100 * 1000.0 / (bench.PEAK_TFLOPS * 2.0 / 2.4):.1f}%"
    assert (valu, ldsi, wait) == ("20.0%", "5.0%", "40.0%")


# ---------------------------------------------------------------- FLOP counts
def _golden_counts():
    rows = {}
    for line in open(os.path.join(ROOT, "tests", "golden", "config_counts.txt")):
        if line.startswith("#") or not line.strip():
            continue
        name, P, kn, lo, ff, fb = line.split()
        rows[name] = tuple(int(v) for v in (P, kn, lo, ff, fb))
    return rows


def test_bench_flops_match_the_oracle_count_on_every_configuration():
    """bench.flops (the numerator of the headline value) equals the oracle's
    count, forward and backward, on all five configurations, and both equal
    the stored counts."""
    import oracle
    import workloads
    golden = _golden_counts()
    for name in workloads.CONFIG_ORDER:
        c = workloads.config(name)
        cu = c.cu_seqlens()
        P = oracle.visible_pairs(c.S_loc, c.q_offset, cu)
        kn = oracle.keys_needed(c.S_loc, c.q_offset, cu)
        args = (c.n_h, c.d_c, c.d_rope, c.d_nope, c.d_v, c.S_loc, c.q_offset, cu)
        for bwd, col in ((False, 3), (True, 4)):
            f = bench.flops(c, P, kn, bwd)
            assert f == oracle.attention_flops(*args, backward=bwd) == golden[name][col], (name, bwd)
        assert golden[name][:2] == (P, kn)


def test_flops_of_the_full_head_configurations_by_hand():
    """Hand counts at DeepSeek-V3 head dims (d_qk = 192, d_v = 128, d_c =
    512, 128 heads). Per visible pair and head: forward 192 + 128
    multiply-adds (scores, weights x V), backward 3 x 192 + 2 x 128 (scores
    again, dq, dK; dP, dV). Per needed key and head: forward 512 x 256
    (rebuilding K_nope and V), backward twice that (dc_kv, dW).
    Full causal 8192: 8192 x 8193 / 2 = 33,558,528 pairs, 8192 keys.
    The 2048-row shard at 14336 of 16384: 2048 x 14336 + 2048 x 2049 / 2 =
    31,458,304 pairs, 16384 keys."""
    import workloads
    pair_f, pair_b = 2 * 128 * 320, 2 * 128 * 832
    key_f, key_b = 2 * 128 * 512 * 256, 4 * 128 * 512 * 256
    for name, P, kn in (("h128_s8k_bwd", 33_558_528, 8192),
                        ("h128_s16k_shard", 31_458_304, 16384)):
        c = workloads.config(name)
        assert bench.flops(c, P, kn, False) == pair_f * P + key_f * kn
        assert bench.flops(c, P, kn, True) == pair_b * P + key_b * kn
    c = workloads.config("h128_s8k_bwd")
    assert round(bench.flops(c, 33_558_528, 8192, True) / 1e12, 3) == 7.697
    assert round(bench.flops(c, 33_558_528, 8192, False) / 1e12, 3) == 3.024
    c = workloads.config("h128_varlen64k")
    assert round(bench.flops(c, 15_619_141, 8638, True) / 1e12, 3) == 3.906


def test_kernel_flops_split_the_step_count():
    """The per-kernel algorithmic counts of bench.kernel_flops add up to the
    step's count: forward = 2 up-projection launches + attention; backward =
    dK/dV (S, dP, dV, dK) + dQ (dq) + the latent-gradient GEMM + 2 weight
    GEMMs; the backward's K/V rebuild launches are not credited."""
    import workloads
    c = workloads.config("h128_s16k_shard")
    P, kn = 31_458_304, 16384
    kf = lambda n: bench.kernel_flops(n, c, P, kn)[0]  # noqa: E731
    assert 2 * kf("upproj") + kf("attn_fwd") == bench.flops(c, P, kn, False)
    for dq in ("attn_bwd_dq", "attn_bwd_dq_ds"):
        assert kf("attn_bwd_dkdv") + kf(dq) + kf("grad_latent") + 2 * kf("grad_w") == \
            bench.flops(c, P, kn, True)
