"""Benchmark: one step = forward + backward of the latent-attention block on
one query shard (synthetic seeded inputs, resident in HBM before timing).

    python bench.py [--steps K] [--warmup W] [--workload NAME]
    python bench.py --sp-sweep 8 [--steps K]   (per-rank times of an 8-way split)
    python bench.py --memory [--workload NAME]   (activation and workspace bytes)
    python bench.py --decode decode_h128_b64_l8k   (absorbed decode over the latent cache)

Prints one JSON line. `value` is the step's algorithmic TFLOP/s: visible
(query, key) pairs times 2*n_h*(d_qk+d_v) forward and 2*n_h*(3*d_qk+2*d_v)
backward, plus the latent up-projection of the keys the shard needs (once
forward, twice backward); masked work and the backward's K/V recomputation
earn nothing. `roofline` is for the kernel with the largest share of the
step's time, timed live with HIP events on the stream it runs on.
`cpu_baseline` times the fp64 oracle on a few heads of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA attn-block fwd/bwd TFLOP/s + % bf16 MFMA peak, n_h=128 S=16384 shard"
PEAK_TFLOPS = 2516.6   # MI355X dense fp16/bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0


def flops(cfg, pairs, kn, backward):
    d_qk = cfg.d_nope + cfg.d_rope
    up = 2 * cfg.n_h * cfg.d_c * (cfg.d_nope + cfg.d_v) * kn
    if not backward:
        return 2 * cfg.n_h * (d_qk + cfg.d_v) * pairs + up
    return 2 * cfg.n_h * (3 * d_qk + 2 * cfg.d_v) * pairs + 2 * up


def kernel_flops(name, cfg, pairs, kn):
    """(algorithmic, executed) FLOPs of one launch of `name`; None if it is
    not a contraction. The algorithmic figures split the step's FLOP count
    (640 per visible pair and head forward, 1664 backward, plus the
    up-projection of the needed keys) over the kernels, each product once:
    the backward's S = Q K^T and dP = dO V^T go to the dK/dV kernel; the dQ
    kernel either reads the dS the dK/dV kernel stored or recomputes them,
    and the backward's K/V rebuild launches recompute the up-projection."""
    d_qk = cfg.d_nope + cfg.d_rope
    up = 2 * cfg.n_h * cfg.d_c * (cfg.d_nope + cfg.d_v) * kn
    per_pair = lambda d: 2 * cfg.n_h * d * pairs  # noqa: E731
    table = {
        # forward launches rebuild K_nope and V separately (half each)
        "upproj": (up // 2, up // 2), "plain_upproj": (up, up),
        "attn_fwd": (per_pair(d_qk + cfg.d_v),) * 2,
        "plain_attn_fwd": (per_pair(d_qk + cfg.d_v),) * 2,
        # paired dK/dV: S, dP, dV += P^T dO, dK += dS^T Q (each once)
        "attn_bwd_dkdv": (per_pair(2 * d_qk + 2 * cfg.d_v),) * 2,
        # dQ: dQ = dS K (S and dP recomputed)
        "attn_bwd_dq": (per_pair(d_qk), per_pair(2 * d_qk + cfg.d_v)),
        # dQ = dS K from the dS the dK/dV kernel stored
        "attn_bwd_dq_ds": (per_pair(d_qk),) * 2,
        "plain_attn_bwd_dkdv": (per_pair(2 * d_qk + 2 * cfg.d_v),) * 2,
        "plain_attn_bwd_dq": (per_pair(d_qk), per_pair(2 * d_qk + cfg.d_v)),
        # dc_kv = [dK_nope | dV] W^T and dW = c_kv^T [dK_nope | dV]: one up-projection each
        "grad_latent": (up, up), "plain_grad_latent": (up, up),
        # dW_UK and dW_UV are separate launches on the fast path
        "grad_w": (up // 2, up // 2), "plain_grad_w": (up, up),
    }
    return table.get(name)


# Kernels the fast backward runs on its side stream, next to the main
# stream's kernels: their event times are wall times while sharing the CUs,
# not the time they take alone.
SIDE_STREAM_KERNELS = ("prep_rope", "zero_rows", "prep_w16", "prep_ckvT", "dout_scale", "bwd_prep", "attn_bwd_dq",
                       "attn_bwd_dq_ds")

TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "head_latent_attention_kv_amd", "csrc")
# kernel symbol fragment -> (timer name, sources whose text decides its code)
COUNTED_KERNELS = {
    "attn_fwd_kernel": ("attn_fwd", ["fast_fwd.hip", "fast_common.h", "device_common.h"]),
    "attn_bwd_dkdv_kernel": ("attn_bwd_dkdv", ["fast_bwd.hip", "fast_common.h", "device_common.h"]),
    "attn_bwd_dq_kernel": ("attn_bwd_dq", ["fast_bwd.hip", "fast_common.h", "device_common.h"]),
    "attn_bwd_dq_ds_kernel": ("attn_bwd_dq_ds", ["fast_bwd.hip", "fast_common.h", "device_common.h"]),
}
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 512 * 2**20


def sources_sha(sources):
    h = hashlib.sha256()
    for name in sources:
        h.update(open(os.path.join(CSRC, name), "rb").read())
    h.update(open(os.path.join(ROOT, "head_latent_attention_kv_amd", "build.py"), "rb").read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the kernel source (and build flags) as they are now."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    rec = json.load(open(TRAFFIC_JSON)).get(f"{kernel}@{workload}")
    if not rec:
        return None
    if any(not os.path.exists(os.path.join(CSRC, s)) for s in rec["sources"]):
        return None
    if sources_sha(rec["sources"]) != rec["sha"]:
        return None
    return rec["bytes_per_launch"]


def traffic_from_counters(fetch_csv, write_csv, workload):
    """Turn two rocprofv3 --pmc csv files (FETCH_SIZE, WRITE_SIZE; KiB per
    dispatch) of a --counter-step run into HBM bytes per launch of its second
    step. Each counter is scaled by bytes / counter of the plain device copy
    in the same run."""
    import csv
    from collections import defaultdict

    def per_kernel(path, counter):
        # the run's second step only (dispatches from the last forward-attention
        # launch on): the first step's launches also touch fresh pages and
        # load code objects
        rows = list(csv.DictReader(open(path)))
        first = max([int(r["Dispatch_Id"]) for r in rows if "attn_fwd" in r["Kernel_Name"]] or [0])
        vals = defaultdict(list)
        for r in rows:
            if r["Counter_Name"] == counter and int(r["Dispatch_Id"]) >= first:
                vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return vals

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    fcopy = [v for k, v in fetch.items() if COPY_KERNEL in k][0]
    wcopy = [v for k, v in write.items() if COPY_KERNEL in k][0]
    fscale = COPY_BYTES / (sum(fcopy) / len(fcopy))
    wscale = COPY_BYTES / (sum(wcopy) / len(wcopy))
    table = json.load(open(TRAFFIC_JSON)) if os.path.exists(TRAFFIC_JSON) else {}
    # drop records taken on sources that have changed since
    table = {k: v for k, v in table.items() if v.get("sha") == sources_sha(v.get("sources", []))}
    for frag, (timer, sources) in COUNTED_KERNELS.items():
        fk = [v for k, v in fetch.items() if frag in k]
        wk = [v for k, v in write.items() if frag in k]
        if not fk or not wk:
            continue
        fb = sum(fk[0]) / len(fk[0]) * fscale
        wb = sum(wk[0]) / len(wk[0]) * wscale
        table[f"{timer}@{workload}"] = {
            "bytes_per_launch": int(round(fb + wb)), "fetch_bytes": int(round(fb)),
            "write_bytes": int(round(wb)), "fetch_scale": round(fscale, 4),
            "write_scale": round(wscale, 4), "sources": sources, "sha": sources_sha(sources)}
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")
    return table


# Counters of one --counter-step run, collected in two rocprofv3 --pmc passes
# (each pass within the per-block limits of one run).
UTIL_PASS_A = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_F16",
               "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT",
               "SQ_BUSY_CU_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_VALU_TRANS_F32",
               "GRBM_GUI_ACTIVE")
UTIL_PASS_B = ("SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_LDS", "SQ_INSTS_LDS",
               "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_ANY",
               "GRBM_GUI_ACTIVE")


def kernel_key(name):
    """Short name of a kernel from a profiler's (demangled or mangled) name:
    the function's identifier plus its template arguments."""
    import re
    m = re.search(r"::(\w+)(<[^(]*>)?\(", name)
    z = re.search(r"_GLOBAL__N_1(\d+)(\w+)", name)
    if m:
        return m.group(1) + (m.group(2) or "")
    if z:   # a mangled name: the length-prefixed identifier, then its template args
        ln, rest = int(z.group(1)), z.group(2)
        # template arguments run to the "EE" that closes them
        return rest[:ln] + (f"<{rest[ln + 1:rest.find('EE', ln)]}>" if rest[ln:ln + 1] == "I" else "")
    return name.split("(")[0]


def utilisation_from_counters(csv_a, csv_b, n_xcd=8, n_cu=256, n_simd=1024):
    """Markdown table of per-kernel unit utilisation from the two passes.

    Per kernel (summed over its dispatches): the shader clock, GRBM_GUI_ACTIVE
    per XCD over the dispatch time; MFMA busy, SQ_VALU_MFMA_BUSY_CYCLES over
    (active cycles x SIMDs), the counter tool's own MfmaUtil formula; the MFMA
    rate the executed MOPS give (512 FLOP each) and its fraction of the
    dense peak at the measured clock; LDS busy, SQ_LDS_IDX_ACTIVE over (active
    cycles x CUs); bank-conflict cycles as a share of LDS-active cycles; and
    the shares of wave time spent issuing VALU and LDS instructions and
    waiting. Only the run's second step counts (dispatches from the last
    forward-attention launch on): the first launch of each kernel also
    loads its code object."""
    import csv
    from collections import defaultdict

    def load(path):
        cnt = defaultdict(lambda: defaultdict(float))
        dur = defaultdict(dict)
        rows = list(csv.DictReader(open(path)))
        first = max([int(r["Dispatch_Id"]) for r in rows if "attn_fwd" in r["Kernel_Name"]] or [0])
        for r in rows:
            if int(r["Dispatch_Id"]) < first:
                continue
            k = kernel_key(r["Kernel_Name"])
            cnt[k][r["Counter_Name"]] += float(r["Counter_Value"])
            dur[k][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
        return cnt, {k: (sum(v.values()), len(v)) for k, v in dur.items()}

    A, tA = load(csv_a)
    B, _ = load(csv_b)
    rows = ["| kernel | launches | ms per launch | clock GHz | MFMA busy | MFMA TFLOP/s executed "
            "| of dense peak at that clock | LDS busy | bank-conflict share | VALU issue / wave time "
            "| LDS issue / wave time | waiting / wave time |",
            "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for k in sorted(A, key=lambda k: -tA[k][0]):
        a, b = A[k], B.get(k, {})
        t, n = tA[k]
        if a["SQ_INSTS_VALU_MFMA_MOPS_F16"] + a["SQ_INSTS_VALU_MFMA_MOPS_BF16"] == 0 and t / n < 1e-4:
            continue
        g = a["GRBM_GUI_ACTIVE"] / n_xcd
        clk = g / t / 1e9
        tf = (a["SQ_INSTS_VALU_MFMA_MOPS_F16"] + a["SQ_INSTS_VALU_MFMA_MOPS_BF16"]) * 512 / t / 1e12
        wc = max(b.get("SQ_WAVE_CYCLES", 0.0), 1.0)
        pct = lambda x: f"{100 * x:.1f}%"  # noqa: E731
        rows.append(
            f"| {k} | {n} | {t / n * 1e3:.3f} | {clk:.2f} | {pct(a['SQ_VALU_MFMA_BUSY_CYCLES'] / (g * n_simd))} "
            f"| {tf:.1f} | {pct(tf / (PEAK_TFLOPS * clk / 2.4))} | {pct(a['SQ_LDS_IDX_ACTIVE'] / (g * n_cu))} "
            f"| {pct(a['SQ_LDS_BANK_CONFLICT'] / max(a['SQ_LDS_IDX_ACTIVE'], 1.0))} "
            f"| {pct(a['SQ_ACTIVE_INST_VALU'] / wc)} | {pct(b.get('SQ_ACTIVE_INST_LDS', 0.0) / wc)} "
            f"| {pct(b.get('SQ_WAIT_INST_ANY', 0.0) / wc)} |")
    return "\n".join(rows)


def host_cpu():
    """Model name of the host CPU (lscpu), and the BLAS library numpy uses
    with its thread count (threadpoolctl)."""
    import subprocess
    info = {"model": None, "logical_cpus": os.cpu_count(), "blas": None, "blas_threads": None}
    try:
        txt = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in txt.splitlines():
            if line.startswith("Model name:"):
                info["model"] = line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if blas:
            info["blas"] = f"{blas[0].get('internal_api')} {blas[0].get('version')}"
            info["blas_threads"] = max(p.get("num_threads", 1) for p in blas)
    except Exception:  # noqa: BLE001
        pass
    return info


def cpu_one_core_forward(budget_heads=2):
    """The oracle's forward on one core for the two small configurations:
    the tiny fp32 one whole, and `budget_heads` of the 16 heads of the
    16-head 4096-token one (its rate on those heads)."""
    import oracle
    import workloads
    from threadpoolctl import threadpool_limits
    res = {}
    with threadpool_limits(limits=1):
        for name, heads in (("tiny_f32", None), ("h16_s4k", list(range(budget_heads)))):
            cfg = workloads.config(name)
            xx = workloads.make_inputs(cfg)
            args = [xx[k] for k in ("q", "c_kv", "k_rope", "W_UK", "W_UV")]
            oracle.mla_forward(*args, heads=[0])   # import and first-call costs
            t0 = time.perf_counter()
            oracle.mla_forward(*args, heads=heads)
            dt = time.perf_counter() - t0
            nh = cfg.n_h if heads is None else len(heads)
            pairs = oracle.visible_pairs(cfg.S_loc, cfg.q_offset)
            F = oracle.attention_flops(cfg.n_h, cfg.d_c, cfg.d_rope, cfg.d_nope, cfg.d_v,
                                       cfg.S_loc, cfg.q_offset) * nh / cfg.n_h
            res[name] = {"forward_s": round(dt, 4), "heads": nh, "of_heads": cfg.n_h,
                         "gflops": round(F / dt / 1e9, 3), "visible_pairs_per_head": pairs}
    return res


def kernel_stats_from_trace(trace_csv, skip_first=True):
    """Markdown table of per-kernel durations from a rocprofv3 --kernel-trace
    csv. With skip_first, each kernel's first dispatch (which also loads its
    code object) is left out: the table holds warm launches only."""
    import csv
    from collections import defaultdict
    rows = list(csv.DictReader(open(trace_csv)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    per = defaultdict(list)
    seen = set()
    for r in rows:
        key = kernel_key(r["Kernel_Name"])
        if skip_first and key not in seen:
            seen.add(key)
            continue
        per[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
    total = sum(sum(v) for v in per.values())
    out = ["| kernel | warm launches | total ms | average us | min us | max us | % |",
           "|---|---|---|---|---|---|---|"]
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"| {k} | {len(v)} | {sum(v) / 1e3:.3f} | {sum(v) / len(v):.1f} | {min(v):.1f} "
                   f"| {max(v):.1f} | {100 * sum(v) / total:.2f} |")
    return "\n".join(out)


def cpu_baseline(cfg, x, cu, pairs, kn, budget_s=15.0, max_heads=16):
    """The fp64 oracle, as it stands, on whole heads of the workload (all rows,
    forward and backward) until about `budget_s` seconds have been spent; the
    host's CPU model and BLAS; and one-core forward runs of the two small
    configurations."""
    import oracle
    host = host_cpu()
    threads = host["blas_threads"] or os.cpu_count() or 1
    args = [x[k] for k in ("q", "c_kv", "k_rope", "W_UK", "W_UV")]
    heads = 0
    t0 = time.perf_counter()
    while heads < min(max_heads, cfg.n_h) and time.perf_counter() - t0 < budget_s:
        h = [heads]
        oracle.mla_forward(*args, q_offset=cfg.q_offset, cu_seqlens=cu, heads=h,
                           q_ranges=cfg.q_ranges)
        oracle.mla_backward(x["dout"], *args, q_offset=cfg.q_offset, cu_seqlens=cu, heads=h,
                            q_ranges=cfg.q_ranges)
        heads += 1
    dt = time.perf_counter() - t0
    F = (flops(cfg, pairs, kn, False) + flops(cfg, pairs, kn, True)) * heads / cfg.n_h
    res = {"value": round(F / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
           "kind": "oracle",
           "sample": f"fp64 numpy oracle, forward+backward of heads 0..{heads - 1} of {cfg.n_h} "
                     f"(all {cfg.S_loc} rows), {dt:.1f} s",
           "host": host}
    try:
        res["one_core_forward"] = cpu_one_core_forward()
    except Exception as e:  # noqa: BLE001
        res["one_core_forward"] = {"error": str(e)}
    return res


def memory_report(name):
    """Device bytes of one attention block on a query shard (prints one JSON
    line). The LAGA figures are the caching allocator's peaks around this
    library's calls, above the resident inputs: forward (workspace and
    outputs), backward with the stored dS and with dQ recomputed (workspace
    and gradients), and what stays allocated from forward to backward (out,
    lse: the K/V rebuilt from the latent are not kept). For comparison, the
    tensors that the other two forms of the block keep for their backward are
    allocated (not computed) and measured the same way, in bf16:
      explicit: per-head K = [K_nope | k_rope] and V for the keys the shard
                attends to, and, as the smaller reading, for its own rows only;
      absorbed: per query row and head the latent-space query (W_UK_h q_nope
                with q_rope, 576 wide) and output (512 wide)."""
    import numpy as np
    import torch

    import head_latent_attention_kv_amd as hla
    import workloads

    cfg = workloads.config(name)
    x = workloads.make_inputs(cfg, with_dout=True)
    dev = {k: torch.from_numpy(x[k + "_bits"].view(np.int16)).view(torch.bfloat16).cuda()
           for k in ("q", "c_kv", "k_rope", "W_UK", "W_UV", "dout")}
    a = [dev[k] for k in ("q", "c_kv", "k_rope", "W_UK", "W_UV")]
    cu = cfg.cu_seqlens()

    def requested():
        return torch.cuda.memory_stats()["requested_bytes.all.current"]

    torch.cuda.synchronize()
    inputs = requested()

    def peak_of(fn):
        # bytes requested from the caching allocator (not the cached blocks
        # that serve them)
        torch.cuda.synchronize()
        before = requested()
        torch.cuda.reset_peak_memory_stats()
        res = fn()
        torch.cuda.synchronize()
        return res, torch.cuda.memory_stats()["requested_bytes.all.peak"] - before

    def fwd_call():
        call = hla.MLACall(*a, q_offset=cfg.q_offset, cu_seqlens=cu, q_ranges=cfg.q_ranges)
        out, lse = call.fwd(*a)
        return call, out, lse

    (call, out, lse), fwd_peak = peak_of(fwd_call)
    del call
    torch.cuda.synchronize()
    held = requested() - inputs
    res = {"metric": "attention-block device bytes per query shard", "workload": cfg.name,
           "config": {"n_h": cfg.n_h, "S": cfg.S, "S_loc": cfg.S_loc, "q_offset": cfg.q_offset},
           "laga": {"forward_peak": fwd_peak, "held_forward_to_backward": held}}
    for recompute in (False, True):
        def bwd_call():
            c = hla.MLACall(*a, q_offset=cfg.q_offset, cu_seqlens=cu, q_ranges=cfg.q_ranges,
                            backward=True, stored_ds=not recompute)
            g = c.bwd(dev["dout"], *a, out, lse)
            return c, g
        (c, g), peak = peak_of(bwd_call)
        key = "backward_peak_recompute_dq" if recompute else "backward_peak_stored_ds"
        res["laga"][key] = peak
        res["laga"][key.replace("peak", "workspace")] = c.ws_bwd.numel()
        del c, g
    pairs, k_lo, k_hi = hla.mla_laga_count(hla.MLACall(*a, q_offset=cfg.q_offset, cu_seqlens=cu,
                                                        q_ranges=cfg.q_ranges).desc, cu)
    kn = k_hi - k_lo
    d_qk = cfg.d_nope + cfg.d_rope

    def held_bytes(shapes):
        torch.cuda.synchronize()
        before = requested()
        ts = [torch.empty(sh, dtype=torch.bfloat16, device="cuda") for sh in shapes]
        torch.cuda.synchronize()
        b = requested() - before
        del ts
        return b

    res["explicit_saved_kv_all_keys"] = held_bytes([(kn, cfg.n_h, d_qk), (kn, cfg.n_h, cfg.d_v)])
    res["explicit_saved_kv_own_rows"] = held_bytes([(cfg.S_loc, cfg.n_h, d_qk), (cfg.S_loc, cfg.n_h, cfg.d_v)])
    res["absorbed_saved_latent_q_and_out"] = held_bytes([(cfg.S_loc, cfg.n_h, cfg.d_c + cfg.d_rope),
                                                         (cfg.S_loc, cfg.n_h, cfg.d_c)])
    res["keys_needed"] = kn
    print(json.dumps(res), flush=True)


def sp_sweep(base_name, world, steps, warmup):
    """Time every rank's forward+backward of a `world`-way sequence-parallel
    split of the workload's sequence, contiguous and zigzag, one rank after
    another on this GPU. With all ranks running at once, a step lasts as
    long as the slowest rank, so `max` is the split's step time."""
    import numpy as np
    import torch

    import head_latent_attention_kv_amd as hla
    import workloads

    base = workloads.config(base_name)
    S, n = base.S, base.S // world
    out = {"sp_sweep": {"workload": base.name, "world": world, "S": S, "steps": steps}}
    for sharding in ("contiguous", "zigzag"):
        ms, pairs = [], []
        for r in range(world):
            if sharding == "contiguous":
                cfg = base.with_(S_loc=n, q_offset=r * n, q_ranges=None)
            else:
                cfg = base.with_(S_loc=n, q_offset=0, q_ranges=workloads.zigzag_blocks(S, r, world))
            x = workloads.make_inputs(cfg, with_dout=True)
            a = [torch.from_numpy(x[k + "_bits"].view(np.int16)).view(torch.bfloat16).cuda()
                 for k in ("q", "c_kv", "k_rope", "W_UK", "W_UV", "dout")]
            dout = a.pop()
            call = hla.MLACall(*a, q_offset=cfg.q_offset, cu_seqlens=cfg.cu_seqlens(),
                               backward=True, q_ranges=cfg.q_ranges)
            pairs.append(hla.mla_laga_count(call.desc, call.cu)[0])
            o, l = call.fwd(*a)
            g = call.bwd(dout, *a, o, l)
            for _ in range(warmup):
                call.fwd(*a, out=o, lse=l)
                call.bwd(dout, *a, o, l, grads=g)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                call.fwd(*a, out=o, lse=l)
                call.bwd(dout, *a, o, l, grads=g)
            torch.cuda.synchronize()
            ms.append((time.perf_counter() - t0) * 1e3 / steps)
            print(f"  {sharding} rank {r}: {ms[-1]:.3f} ms per step", file=sys.stderr, flush=True)
            del call, a, dout, o, l, g
            torch.cuda.empty_cache()
        out["sp_sweep"][sharding] = {"ms_per_step": [round(v, 4) for v in ms],
                                     "max_ms": round(max(ms), 4),
                                     "mean_ms": round(sum(ms) / len(ms), 4),
                                     "visible_pairs_per_head": pairs}
    print(json.dumps(out), flush=True)


def decode_bench(name, steps, warmup):
    """Time the decode path (absorbed form over the latent cache) on a decode
    batch; prints its own JSON line. Algorithmic work per cached row and
    head: 2 (576 + 512) FLOP for the scores and the latent-weighted sum; the
    dominant kernel streams each cached row (1152 bytes in bf16) once."""
    import numpy as np
    import torch

    import head_latent_attention_kv_amd as hla
    import workloads

    cfg = workloads.config(name)
    cu = cfg.cu_seqlens()
    x = workloads.make_inputs(cfg, with_dout=False)
    a = [torch.from_numpy(x[k + "_bits"].view(np.int16)).view(torch.bfloat16).cuda()
         for k in ("q", "c_kv", "k_rope", "W_UK", "W_UV")]
    call = hla.MLADecodeCall(*a, cu)
    out, lse = call(*a)
    for _ in range(warmup):
        call(*a, out=out, lse=lse)
    torch.cuda.synchronize()
    # per-kernel breakdown in a short pass of its own (every kernel bracketed
    # by events); the timed region brackets only the attention kernel
    n_brk = max(1, min(5, steps))
    hla.timing_select(None)
    hla.timing_enable(True)
    for _ in range(n_brk):
        call(*a, out=out, lse=lse)
    torch.cuda.synchronize()
    kern = {}
    for kname in hla.timing_names():
        tot, n = hla.timing_read(kname)
        kern[kname] = {"ms_per_launch": round(tot / max(n, 1), 4),
                       "launches_per_step": n / n_brk}
    hla.timing_enable(False)
    hla.timing_select(["decode_attn"])
    hla.timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call(*a, out=out, lse=lse)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    tot, n = hla.timing_read("decode_attn")
    if n:
        kern["decode_attn"] = {"ms_per_launch": round(tot / n, 4), "launches_per_step": n / steps}
    hla.timing_enable(False)
    hla.timing_select(None)
    keys = int(cu[-1])
    n_h, B = cfg.n_h, cfg.S_loc
    f_attn = 2 * n_h * (576 + 512) * keys
    f_proj = 2 * B * n_h * 128 * 512 * 2
    cache_bytes = keys * 1152
    t_attn = kern.get("decode_attn", {}).get("ms_per_launch")
    roofline = None
    if t_attn:
        gbs = cache_bytes / (t_attn / 1e3) / 1e9
        roofline = {"kernel": "decode_attn", "bound": "hbm", "achieved": round(gbs, 1),
                    "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                    "traffic": None, "ms_per_launch": t_attn,
                    "tflops": round(f_attn / (t_attn / 1e3) / 1e12, 2),
                    # each score and output product runs once (the waves of a
                    # pair split the score contraction); only the padding of a
                    # sequence's last 32-key block is executed beyond this
                    "mfma_tflops_executed": round(f_attn / (t_attn / 1e3) / 1e12, 2)}
    res = {"metric": "MLA absorbed decode step (latent cache), TFLOP/s",
           "value": round((f_attn + f_proj) / (ms / 1e3) / 1e12, 2), "unit": "TFLOP/s",
           "ms_per_step": round(ms, 4), "steps": steps, "warmup": warmup,
           "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": cfg.name, "n_h": n_h, "batch": B, "cached_rows": keys,
                      "longest": int(max(cfg.seq_lens)), "flop": f_attn + f_proj,
                      "cache_bytes": cache_bytes},
           "cache_gbs": round(cache_bytes / (ms / 1e3) / 1e9, 1),
           "roofline": roofline, "kernels": kern}
    print(json.dumps(res), flush=True)


def device_info(torch):
    """Compute units and the maximum shader clock of GPU 0, and the dense
    fp16/bf16 MFMA peak they imply (4096 FLOP per clock per CU). The clock
    comes from rocminfo; null when it cannot be read."""
    import subprocess
    props = torch.cuda.get_device_properties(0)
    info = {"name": props.name, "arch": getattr(props, "gcnArchName", None),
            "cus": props.multi_processor_count, "max_sclk_mhz": None, "peak_tflops_derived": None}
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=30).stdout
        gpu = False
        for line in txt.splitlines():
            if "Name:" in line and "gfx" in line:
                gpu = True
            if gpu and "Max Clock Freq. (MHz):" in line:
                info["max_sclk_mhz"] = int(line.split(":")[1].split()[0])
                break
    except (OSError, subprocess.SubprocessError, ValueError):
        pass
    if info["max_sclk_mhz"]:
        info["peak_tflops_derived"] = round(info["cus"] * info["max_sclk_mhz"] * 1e6 * 4096 / 1e12, 1)
    return info


def spread(v):
    """Median, min and 90th percentile of a list of times (ms)."""
    import numpy as np
    return {"ms_median": round(float(np.median(v)), 4), "ms_min": round(float(min(v)), 4),
            "ms_p90": round(float(np.percentile(v, 90)), 4)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="h128_s16k_shard")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-bwd-forms", action="store_true",
                    help="skip timing the stored-dS backward and the allocator peaks of both "
                         "forms (so that a profiled run holds the default form only)")
    ap.add_argument("--cold-steps", type=int, default=5,
                    help="extra steps timed after a 512 MiB write that evicts the caches")
    ap.add_argument("--counter-step", action="store_true",
                    help="run one warm-up and one step, then a plain 512 MiB device copy "
                         "(the scale reference for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--utilisation-from", nargs=2, metavar=("PASS_A_CSV", "PASS_B_CSV"),
                    help="print per-kernel MFMA/LDS/VALU utilisation from two --counter-step "
                         "rocprofv3 --pmc runs (counters: UTIL_PASS_A, then UTIL_PASS_B)")
    ap.add_argument("--kernel-stats-from", metavar="TRACE_CSV",
                    help="print warm-launch kernel durations from a rocprofv3 --kernel-trace csv "
                         "(each kernel's first dispatch left out)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two --counter-step counter csv files")
    ap.add_argument("--decode", metavar="NAME",
                    help="time the absorbed decode path on a decode batch "
                         "(decode_h128_b64_l8k, decode_h128_b32_mixed); prints its own JSON line")
    ap.add_argument("--memory", action="store_true",
                    help="device bytes of the block on the workload (prints its own JSON line)")
    ap.add_argument("--sp-sweep", type=int, metavar="WORLD",
                    help="time each rank of a WORLD-way contiguous and zigzag split of the "
                         "workload's sequence, one after another (prints its own JSON line)")
    args = ap.parse_args()
    if args.utilisation_from:
        print(utilisation_from_counters(*args.utilisation_from))
        return
    if args.kernel_stats_from:
        print(kernel_stats_from_trace(args.kernel_stats_from))
        return
    if args.traffic_from:
        print(json.dumps(traffic_from_counters(*args.traffic_from, args.workload), indent=1))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's query shard: the library has no multi-GPU path "
              "(the latent all-gather is not part of it); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.decode:
        decode_bench(args.decode, args.steps, args.warmup)
        return
    if args.memory:
        memory_report(args.workload)
        return
    if args.sp_sweep:
        sp_sweep(args.workload, args.sp_sweep, args.steps, args.warmup)
        return

    import numpy as np
    import torch

    import head_latent_attention_kv_amd as hla
    import workloads

    cfg = workloads.config(args.workload)
    x = workloads.make_inputs(cfg, with_dout=True)
    cu = cfg.cu_seqlens()
    dev = {}
    for k in ("q", "c_kv", "k_rope", "W_UK", "W_UV", "dout"):
        if cfg.dtype == "bf16":
            dev[k] = torch.from_numpy(x[k + "_bits"].view(np.int16)).view(torch.bfloat16).cuda()
        else:
            dev[k] = torch.from_numpy(x[k]).cuda()
    a = [dev[k] for k in ("q", "c_kv", "k_rope", "W_UK", "W_UV")]
    call = hla.MLACall(*a, q_offset=cfg.q_offset, cu_seqlens=cu, backward=True,
                       q_ranges=cfg.q_ranges)   # the default backward (dQ recomputes)
    pairs, k_lo, k_hi = hla.mla_laga_count(call.desc, call.cu)
    kn = k_hi - k_lo
    F_fwd, F_bwd = flops(cfg, pairs, kn, False), flops(cfg, pairs, kn, True)
    out, lse = call.fwd(*a)
    grads = call.bwd(dev["dout"], *a, out, lse)

    def step():
        call.fwd(*a, out=out, lse=lse)
        call.bwd(dev["dout"], *a, out, lse, grads=grads)

    if args.counter_step:
        step()
        src = torch.full((COPY_BYTES // 4,), 1.0, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"counter step done: {cfg.name}, copy of {COPY_BYTES} bytes", flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    # Per-kernel breakdown: a short pass with every kernel bracketed by HIP
    # events (each pair adds a few microseconds between launches, so this
    # pass is not the timed one). It also names the dominant kernel.
    n_brk = max(1, min(5, args.steps))
    hla.timing_select(None)
    hla.timing_enable(True)
    for _ in range(n_brk):
        step()
    torch.cuda.synchronize()
    kern = {}
    for name in hla.timing_names():
        tot, n = hla.timing_read(name)
        kern[name] = {"ms_per_launch": tot / max(n, 1), "launches_per_step": n / n_brk,
                      "ms_per_step": tot / n_brk}
    hla.timing_enable(False)
    dom = max(kern, key=lambda k: kern[k]["ms_per_step"]) if kern else None

    # Timed region: only the dominant kernel is bracketed (for the roofline).
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    hla.timing_select([dom] if dom else None)
    hla.timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1, e2 in ev:
        e0.record(stream)
        call.fwd(*a, out=out, lse=lse)
        e1.record(stream)
        call.bwd(dev["dout"], *a, out, lse, grads=grads)
        e2.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = [e0.elapsed_time(e1) for e0, e1, _ in ev]
    bwd_ms = [e1.elapsed_time(e2) for _, e1, e2 in ev]
    step_ms = wall * 1e3 / args.steps
    if dom:
        tot, n = hla.timing_read(dom)
        kern[dom].update({"ms_per_launch": tot / max(n, 1), "ms_per_step": tot / args.steps,
                          "launches_per_step": n / args.steps})
    hla.timing_enable(False)
    hla.timing_select(None)
    roofline = None
    if dom:
        kf = kernel_flops(dom, cfg, pairs, kn)
        per_launch_s = kern[dom]["ms_per_launch"] / 1e3
        traffic = recorded_traffic(dom, cfg.name)
        if kf is not None:
            ach = kf[0] / per_launch_s / 1e12
            roofline = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2),
                        "peak": PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_TFLOPS, 4),
                        "traffic": traffic, "ms_per_launch": round(kern[dom]["ms_per_launch"], 4),
                        "mfma_tflops_executed": round(kf[1] / per_launch_s / 1e12, 2)}
    for name, k in kern.items():
        kf = kernel_flops(name, cfg, pairs, kn)
        if kf is not None:
            k["tflops"] = round(kf[0] / (k["ms_per_launch"] / 1e3) / 1e12, 2)
            k["mfma_tflops_executed"] = round(kf[1] / (k["ms_per_launch"] / 1e3) / 1e12, 2)
        for f in ("ms_per_launch", "ms_per_step"):
            k[f] = round(k[f], 4)

    # cold caches: a 512 MiB write (twice the last-level cache) before each
    # step, outside the timed events
    cold = None
    if args.cold_steps > 0:
        flush = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        cev = []
        for i in range(args.cold_steps):
            flush.fill_(float(i))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            cev.append((e0, e1))
        torch.cuda.synchronize()
        cold = spread([e0.elapsed_time(e1) for e0, e1 in cev])
        del flush

    med = lambda v: float(np.median(v))  # noqa: E731
    for name, k in kern.items():
        if name in SIDE_STREAM_KERNELS:
            k["stream"] = "side (wall time while sharing the CUs)"

    # The two backward forms. The default recomputes the scores and dP for
    # dQ; the stored-dS form (opt-in) keeps dS in the workspace, which grows
    # with rows x keys up to 16 GiB (past that it runs head groups of at least
    # 8 heads through two buffers of at most 1 GiB). Each form's backward is timed on its own call, and its
    # allocator peak (workspace and gradients of a fresh call) is measured.
    def bwd_peak(stored):
        # bytes requested from the caching allocator by a fresh call's
        # workspaces and the gradients
        torch.cuda.synchronize()
        before = torch.cuda.memory_stats()["requested_bytes.all.current"]
        torch.cuda.reset_peak_memory_stats()
        c = hla.MLACall(*a, q_offset=cfg.q_offset, cu_seqlens=cu, backward=True,
                        q_ranges=cfg.q_ranges, stored_ds=stored)
        g = c.bwd(dev["dout"], *a, out, lse)
        torch.cuda.synchronize()
        peak = torch.cuda.memory_stats()["requested_bytes.all.peak"] - before
        ws = c.ws_bwd.numel()
        del c, g
        torch.cuda.empty_cache()
        return peak, ws

    forms = {}
    for stored in (() if args.no_bwd_forms else (False, True)):
        peak, ws = bwd_peak(stored)
        entry = {"workspace_bytes": ws, "backward_peak_bytes": peak}
        if not stored:
            entry.update({"default": True, "bwd_ms_median": round(med(bwd_ms), 4),
                          "step_ms": round(step_ms, 4)})
        else:
            cs = hla.MLACall(*a, q_offset=cfg.q_offset, cu_seqlens=cu, backward=True,
                             q_ranges=cfg.q_ranges, stored_ds=True)
            gs = cs.bwd(dev["dout"], *a, out, lse)
            for _ in range(2):
                cs.bwd(dev["dout"], *a, out, lse, grads=gs)
            n_s = max(3, min(10, args.steps))
            sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
                    torch.cuda.Event(enable_timing=True)) for _ in range(n_s)]
            torch.cuda.synchronize()
            for e0, e1, e2 in sev:
                e0.record(stream)
                cs.fwd(*a, out=out, lse=lse)
                e1.record(stream)
                cs.bwd(dev["dout"], *a, out, lse, grads=gs)
                e2.record(stream)
            torch.cuda.synchronize()
            sb = [e1.elapsed_time(e2) for _, e1, e2 in sev]
            ss = [e0.elapsed_time(e2) for e0, _, e2 in sev]
            entry.update({"default": False, "bwd_ms_median": round(med(sb), 4),
                          "step_ms": round(med(ss), 4), "steps": n_s,
                          "step_tflops": round((F_fwd + F_bwd) / (med(ss) / 1e3) / 1e12, 2)})
            del cs, gs
            torch.cuda.empty_cache()
        forms["stored_ds" if stored else "recompute_dq"] = entry

    value = (F_fwd + F_bwd) / (step_ms / 1e3) / 1e12
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "n_h": cfg.n_h, "d_c": cfg.d_c, "d_rope": cfg.d_rope,
                   "d_nope": cfg.d_nope, "d_v": cfg.d_v, "S": cfg.S, "S_loc": cfg.S_loc,
                   "q_offset": cfg.q_offset, "packed_samples": None if cu is None else len(cu) - 1,
                   "q_ranges": None if cfg.q_ranges is None else [list(r) for r in cfg.q_ranges],
                   "step": "forward+backward", "fast_path": call.fast,
                   "visible_pairs_per_head": pairs, "keys_needed": kn,
                   "flop_fwd": F_fwd, "flop_bwd": F_bwd},
        "frac_peak": round(value / PEAK_TFLOPS, 4),
        "fwd": {**spread(fwd_ms), "tflops": round(F_fwd / (med(fwd_ms) / 1e3) / 1e12, 2),
                "frac_peak": round(F_fwd / (med(fwd_ms) / 1e3) / 1e12 / PEAK_TFLOPS, 4)},
        "bwd": {**spread(bwd_ms), "tflops": round(F_bwd / (med(bwd_ms) / 1e3) / 1e12, 2),
                "frac_peak": round(F_bwd / (med(bwd_ms) / 1e3) / 1e12 / PEAK_TFLOPS, 4)},
        "step_events": spread([f + b for f, b in zip(fwd_ms, bwd_ms)]),
        "bwd_forms": forms,
        "step_cold_caches": cold,
        "device": device_info(torch),
        "roofline": roofline,
        "kernels": kern,
        "kernels_breakdown_steps": n_brk,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, x, cu, pairs, kn, budget_s=args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
