#!/usr/bin/env python3
"""Benchmark of the fused causal grouped-query attention hot path on one MI355X.

The default line ("headline") measures the path at the model card's attention
shapes, with seeded synthetic inputs already resident in HBM:
  * the forward at the card's head layout (128 query heads over 16 kv heads, d=64)
    with a 16,384-key sliding window and 2,048 sinks at S=65,536, B=1: the largest
    single-GPU workload, whose throughput is the line's ``value``;
  * the plain causal forward at the same head layout, S=16,384;
  * the backward (delta, dK/dV, dQ; each kernel timed on its own) at B=4, H=32,
    G=8, S=4096, from the forward's O and lse.
Each kernel carries its own roofline record; the dominant one (the windowed
forward) is the line's ``roofline``.  Other workloads: ``--workload``; ``step``
is one forward + backward pass at B=4 H=32 G=8 S=2048.

Work is counted only on visible (query, key) pairs: forward 4*d*pairs*B*H flop
(Q K^T and P V), backward 10*d*pairs*B*H flop (S, dP, dV, dK, dQ), where the
pair count comes from the library's host-side rule.  The printed JSON line
carries the step throughput, a roofline record for the dominant kernel (timed
with HIP events on the stream the kernels run on) and the CPU fp64 oracle
timed on a bounded sample of the same work on the host's cores.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--rope | --fp8]
                       [--workload headline|step|c2|c3|c4|c5|long|decode|decode16|rope_k]
                       [--no-cpu-baseline]
Every workload also warms up for at least WARMUP_FLOOR_S seconds of GPU work,
whatever --warmup says: the device settles at its sustained clocks only after
that.  Counter summaries: --reduce-counters (HBM bytes), --reduce-sq-counters
(matrix-core busy and issue statistics), --reduce-kernel-trace (per-kernel
durations, split by launch shape).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6  # 256 CUs x 2.4 GHz x 4096 flop/clk/CU (published 2.5 PFLOP/s dense)
MFMA_FP8_PEAK_TFLOPS = 5033.2   # twice the bf16 rate (published 5.0 PFLOP/s dense)
HBM_PEAK_GBS = 8000.0
METRIC = "causal GQA attention TFLOP/s (fwd, bwd) at d=64 + % of MI355X bf16 MFMA peak"
WARMUP_FLOOR_S = 1.0  # seconds of GPU work before any timed step
N_SIMDS = 256 * 4     # MI355X: 256 compute units of 4 SIMDs
N_XCDS = 8
KERNEL_SOURCES = ["gqa_fwd.hip", "gqa_bwd.hip", "gqa_decode.hip", "gqa_rope.hip", "gqa_fwd_fp8.hip",
                  "gqa_device.h", "gqa_internal.h"]


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU takes tens of milliseconds of sustained work to reach its steady clocks, so the
    # defaults warm up for 50 steps before timing 100 (3 and 1 at the long-context workload,
    # whose step takes seconds)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="headline",
                    choices=["headline", "step", "c2", "c3", "c4", "c5", "long", "decode", "decode16", "rope_k"])
    ap.add_argument("--rope", action="store_true",
                    help="YaRN RoPE (factor 32) on q and k in front of attention: rotation of K, the "
                         "forward with Q rotated in registers, and dQ / dK rotated back after the backward")
    ap.add_argument("--fp8", action="store_true",
                    help="forward only, with FP8 (e4m3) Q, K, V and per-tensor scales, on the FP8 matrix cores")
    ap.add_argument("--split-grads", action="store_true",
                    help="backward workloads: dK/dV and dQ as two launches (the library's path for grids "
                         "beyond two rounds of workgroup slots), each timed on its own")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter calibration runs)")
    ap.add_argument("--reduce-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc counter_collection.csv "
                         "files (FETCH_SIZE, WRITE_SIZE) of a --copy-calibration run of --workload, then exit")
    ap.add_argument("--reduce-sq-counters", metavar="SQ_CSV",
                    help="write profiles/counters.json (and print a summary) from a rocprofv3 --pmc "
                         "counter_collection.csv with the SQ counters of SQ_COUNTERS for --workload, then exit")
    ap.add_argument("--reduce-kernel-trace", metavar="TRACE_CSV",
                    help="print per-kernel duration statistics, split by launch shape, from a rocprofv3 "
                         "--kernel-trace kernel_trace.csv, then exit")
    return ap.parse_args()


def workload(name):
    from synth import WORKLOADS

    if name == "step":
        w = WORKLOADS["c2"].with_(name="step", direction="fwd+bwd")
    elif name == "c5":
        w = WORKLOADS["c5"].with_(direction="fwd+bwd")
    else:
        w = WORKLOADS[name]
    return w


def source_digest():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "transformer_attention_07_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, wname, path=None):
    """HBM bytes per launch of `kernel` from the committed counter summary (or `path`), if
    it was taken on the current kernel sources; None otherwise."""
    path = path or os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get("kernels", {}).get(f"{kernel}@{wname}")
    if not ent or rec.get("source_digest") != source_digest():
        return None
    return ent.get("bytes_per_launch")


KERNEL_KEYS = {"rope_kernel": "rope", "fwd_fp8_kernel": "fwd_fp8", "vt_permute_kernel": "vt_permute",
               "fwd_mfma_kernel": "fwd", "bwd_preprocess_kernel": "bwd_preprocess",
               "bwd_fused_kernel": "bwd_grads", "bwd_dkdv_kernel": "bwd_dkdv", "bwd_dq_kernel": "bwd_dq",
               "decode_split_kernel": "decode", "decode_shared_kernel": "decode", "decode_merge_kernel": "decode_merge", "copyBuffer": "copy"}
COPY_BYTES = 1 << 30


def reduce_counters(fetch_csv, write_csv, wname, path=None):
    """HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each
    scaled so that the 1 GiB calibration copy reads as exactly 1 GiB in and 1 GiB out;
    recorded under ``wname`` in ``path`` (default profiles/traffic.json)."""
    import csv

    def per_kernel(path, counter):
        # a kernel's launches are alike: their mean.  The calibration copy is the largest
        # copy dispatch: the runtime's copy kernel also serves small copies (reading a
        # result back to the host), which must not dilute it.
        acc = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                key = next((v for k, v in KERNEL_KEYS.items() if k in r["Kernel_Name"]), None)
                if key:
                    acc.setdefault(key, []).append(float(r["Counter_Value"]) * 1024.0)
        return {k: max(v) if k == "copy" else sum(v) / len(v) for k, v in acc.items()}

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    f_scale, w_scale = COPY_BYTES / fetch["copy"], COPY_BYTES / write["copy"]
    path = path or os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    if rec.get("source_digest") != source_digest():
        rec = {"kernels": {}}
    rec.update(source_digest=source_digest(),
               note="HBM bytes per launch = FETCH_SIZE*fetch_scale + WRITE_SIZE*write_scale (counters in KiB); "
                    "scales make a plain 1 GiB device copy read 1 GiB in and 1 GiB out")
    rec.setdefault("calibration", {})[wname] = {"fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5)}
    for k in fetch:
        if k == "copy" or k not in write:
            continue
        rec["kernels"][f"{k}@{wname}"] = {
            "fetch_bytes": round(fetch[k] * f_scale), "write_bytes": round(write[k] * w_scale),
            "bytes_per_launch": round(fetch[k] * f_scale + write[k] * w_scale)}
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(rec["kernels"], indent=1))


SQ_COUNTERS = ["SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES",
               "SQ_WAVE_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_ANY",
               "SQ_LDS_BANK_CONFLICT", "GRBM_GUI_ACTIVE"]


def _kernel_key(name):
    return next((v for k, v in KERNEL_KEYS.items() if k in name), None)


def _dispatch_table(path):
    """rocprofv3 counter_collection.csv as {dispatch id: (kernel key, {counter: value}, duration ns)}."""
    import csv

    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            key = _kernel_key(r["Kernel_Name"])
            if key is None:
                continue
            d = out.setdefault(r["Dispatch_Id"], [key, {}, None])
            d[1][r["Counter_Name"]] = d[1].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            if r.get("Start_Timestamp") and r.get("End_Timestamp"):
                d[2] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    return out


def sq_derived(c, duration_ns=None):
    """Matrix-core and issue statistics of one dispatch from its SQ counters.  The GRBM
    counter arrives summed over the XCDs, so the GPU's own cycle count is a 1/N_XCDS of it;
    the matrix cores were busy SQ_VALU_MFMA_BUSY_CYCLES out of that times N_SIMDS
    SIMD-cycles.  Each executed bf16 MFMA operation counts 512 flop."""
    gpu_cycles = c["GRBM_GUI_ACTIVE"] / N_XCDS
    wave = c["SQ_WAVE_CYCLES"]
    busy = c["SQ_VALU_MFMA_BUSY_CYCLES"]
    d = {"mfma_busy": busy / (gpu_cycles * N_SIMDS),
         "mfma_flop_executed": c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0,
         "mfma_coexec_valu": c["SQ_VALU_MFMA_COEXEC_CYCLES"] / busy if busy else 0.0,
         "valu_active_per_wave_cycle": c["SQ_ACTIVE_INST_VALU"] / wave,
         "lds_active_per_wave_cycle": c["SQ_ACTIVE_INST_LDS"] / wave,
         "wait_issue_per_wave_cycle": c["SQ_WAIT_INST_ANY"] / wave,
         "lds_bank_conflicts": c["SQ_LDS_BANK_CONFLICT"],
         "gpu_cycles": gpu_cycles}
    if duration_ns:
        d["clock_mhz"] = gpu_cycles / (duration_ns * 1e-3)
        d["duration_us"] = duration_ns * 1e-3
    return d


def reduce_sq_counters(sq_csv, wname, path=None):
    """profiles/counters.json entries kernel@wname: the mean over a kernel's dispatches of
    each statistic of ``sq_derived``, recorded with the kernel sources' digest (a bench line
    reads them only while the sources are unchanged).  Returns a printable summary."""
    table = _dispatch_table(sq_csv)
    per = {}
    for key, cnt, dur in table.values():
        if key == "copy" or not all(n in cnt for n in SQ_COUNTERS):
            continue
        per.setdefault(key, []).append(sq_derived(cnt, dur))
    path = path or os.path.join(ROOT, "profiles", "counters.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    if rec.get("source_digest") != source_digest():
        rec = {"kernels": {}}
    rec.update(source_digest=source_digest(), counters=SQ_COUNTERS,
               note="mean over a kernel's dispatches; mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / "
                    "(GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs); per-wave-cycle ratios over SQ_WAVE_CYCLES")
    lines = []
    for key, ds in sorted(per.items()):
        mean = {k: sum(d[k] for d in ds) / len(ds) for k in ds[0] if all(k in d for d in ds)}
        ent = {k: round(v, 6) if abs(v) < 1e6 else float(f"{v:.6e}") for k, v in mean.items()}
        ent["dispatches"] = len(ds)
        rec["kernels"][f"{key}@{wname}"] = ent
        lines.append(f"{key}@{wname}: {len(ds)} dispatches; MFMA busy {100 * mean['mfma_busy']:.1f} %, "
                     f"executed bf16 MFMA flop {mean['mfma_flop_executed']:.4e}, MFMA cycles co-executing "
                     f"with VALU {mean['mfma_coexec_valu']:.2f}; per wave cycle: VALU active "
                     f"{mean['valu_active_per_wave_cycle']:.2f}, LDS active {mean['lds_active_per_wave_cycle']:.2f}, "
                     f"waiting on issue {mean['wait_issue_per_wave_cycle']:.2f}; LDS bank conflicts "
                     f"{mean['lds_bank_conflicts']:.0f}"
                     + (f"; {mean['clock_mhz']:.0f} MHz over {mean['duration_us']:.1f} us" if "clock_mhz" in mean else ""))
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    return "\n".join(lines)


def load_counters(kernel, wname, path=None):
    """The counters.json entry of kernel@wname if it was taken on the current kernel
    sources, else None."""
    path = path or os.path.join(ROOT, "profiles", "counters.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != source_digest():
        return None
    return rec.get("kernels", {}).get(f"{kernel}@{wname}")


def reduce_kernel_trace(trace_csv):
    """Per-kernel duration statistics from a rocprofv3 kernel_trace.csv, one row per kernel
    and launch shape (workgroups), so that one kernel run at several shapes in one process
    is reported per shape.  Returns the table as text."""
    import csv

    groups = {}
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            grid = int(float(r.get("Grid_Size_X") or r.get("Grid_Size") or 0))
            wg = int(float(r.get("Workgroup_Size_X") or r.get("Workgroup_Size") or 1)) or 1
            dur = (float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) * 1e-3
            name = _kernel_key(r["Kernel_Name"]) or r["Kernel_Name"][:60]
            groups.setdefault((name, grid // wg), []).append(dur)
    rows = [f"{'kernel':<22}{'workgroups':>11}{'calls':>7}{'avg us':>11}{'median us':>11}{'min us':>10}{'max us':>10}"]
    for (name, nwg), ds in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        ds_sorted = sorted(ds)
        rows.append(f"{name:<22}{nwg:>11}{len(ds):>7}{sum(ds) / len(ds):>11.1f}{ds_sorted[len(ds) // 2]:>11.1f}"
                    f"{ds_sorted[0]:>10.1f}{ds_sorted[-1]:>10.1f}")
    return "\n".join(rows)


def row_decomposition(w):
    """Workgroups of the forward and dQ launches (heads per workgroup as the library picks
    them: 4, 2 or 1 dividing H/G; one 64-row tile per wave) and of the dK/dV launch
    (128 keys per workgroup); used to label launches in kernel traces."""
    hpg = w.H // w.G
    hpw = 4 if hpg % 4 == 0 else 2 if hpg % 2 == 0 else 1
    n_qblk = -(-w.S // (64 * (4 // hpw)))
    return {"fwd": n_qblk * w.B * (w.H // hpw), "bwd_dq": n_qblk * w.B * (w.H // hpw),
            "bwd_dkdv": -(-w.S // 128) * w.B * w.G}


def host_cpu():
    """The host CPU's model name (for the CPU baseline's record)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown CPU"


def cpu_baseline(w, inputs, budget_s, rope=False, rows_sample=None):
    """The oracle, as it stands, on whole kv groups of the same workload until the
    time budget is used: forward rows of every head of the group plus its backward.
    At the long-context workload one group alone would take hours, so there it times
    forward rows (chunks of 256 consecutive rows at seeded positions) instead."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle.attention as ref
    from transformer_attention_07_amd import gqa_visible_pairs

    if rope:
        import oracle.rope as ref  # the same entry points, with the rotation in front

    q, k, v, do = inputs
    if rows_sample is None:
        rows_sample = w.per_slab
    if rows_sample:
        kw = dict(scale=w.scale, causal=w.causal, window=w.window, num_sinks=w.num_sinks)
        rng = np.random.default_rng(w.seed)
        t0 = time.perf_counter()
        flop, nrows = 0.0, 0
        while time.perf_counter() - t0 < budget_s:
            b, h, i0 = int(rng.integers(w.B)), int(rng.integers(w.H)), int(rng.integers(w.S - 256))
            rows = np.arange(i0, i0 + 256)
            ref.forward_rows(q, k, v, b, h, rows, **kw)
            vis = np.minimum(rows + 1, w.window) + np.minimum(w.num_sinks, np.maximum(0, rows - w.window + 1))
            flop += 4.0 * w.D * float(vis.sum())
            nrows += rows.size
        dt = time.perf_counter() - t0
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
                "sample": f"{nrows} forward rows (chunks of 256 at seeded positions), {dt:.1f} s, fp64 numpy on {host_cpu()}"}
    hpg = w.H // w.G
    pairs = gqa_visible_pairs(w.S, w.causal, w.window, w.num_sinks)
    kw = dict(scale=w.scale, causal=w.causal, window=w.window, num_sinks=w.num_sinks)
    rows = np.arange(w.S)
    t0 = time.perf_counter()
    groups = 0
    flop = 0.0
    for b in range(w.B):
        for g in range(w.G):
            for h in range(g * hpg, (g + 1) * hpg):
                ref.forward_rows(q, k, v, b, h, rows, **kw)
            flop += 4.0 * w.D * pairs * hpg
            if "bwd" in w.direction:
                ref.backward_group(q, k, v, do, b, g, **kw)
                flop += 10.0 * w.D * pairs * hpg
            groups += 1
            if time.perf_counter() - t0 > budget_s:
                break
        else:
            continue
        break
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{groups} of {w.B * w.G} kv groups (all {hpg} heads each, "
                      f"{'fwd+bwd' if 'bwd' in w.direction else 'fwd'}), {dt:.1f} s, fp64 numpy on {host_cpu()}"}


def warm_up(call, steps, floor_s=WARMUP_FLOOR_S):
    """At least ``steps`` calls and at least ``floor_s`` seconds of wall time with the
    device synchronised (so the seconds are GPU work, not queued launches).  Returns the
    number of calls and the seconds spent."""
    import torch

    t0 = time.perf_counter()
    n = 0
    while n < steps or time.perf_counter() - t0 < floor_s:
        call()
        n += 1
        torch.cuda.synchronize()
    return n, time.perf_counter() - t0


def time_units(units, steps, stream):
    """Time ``steps`` passes over ``units`` (a list of callables run in order on
    ``stream``): per-unit mean milliseconds from HIP events recorded on that stream, and
    the wall-clock milliseconds per pass between device synchronisations."""
    import torch

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(units) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        ev[s][0].record(stream)
        for i, u in enumerate(units):
            u()
            ev[s][i + 1].record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    per = [sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)) / steps for i in range(len(units))]
    return per, wall_ms


def clock_under_load(kernel, wname, probe_mhz, value, peak):
    """The shader clock to scale the peak by: the one the counters measured during the
    kernel's own dispatches (GRBM_GUI_ACTIVE over the dispatch time) when profiles/
    counters.json holds them for the current sources, else the clock probe's (MFMA chains
    right after the timed steps, not under the kernel's own power draw)."""
    ctr = load_counters(kernel, wname)
    if ctr and ctr.get("clock_mhz"):
        mhz, src = ctr["clock_mhz"], f"rocprofv3 counters of {kernel}@{wname} (GRBM_GUI_ACTIVE over its dispatches)"
    else:
        mhz, src = probe_mhz, "gqa_clock_probe after the timed steps"
    return {"clock_mhz_for_peak": round(mhz, 1), "clock_source": src,
            "pct_of_peak_at_measured_clock": round(100 * value / (peak * mhz / 2400.0), 2)}


def kernel_record(kernel, wname, ms, flop=None, nbytes=None):
    """One kernel's entry of a bench line: its event-timed milliseconds, its rate against
    its roofline (bf16 MFMA for the attention products, HBM for the delta pass), and what
    the committed counter summaries say about it (null once the sources have changed)."""
    traffic = load_traffic(kernel, wname)
    ctr = load_counters(kernel, wname)
    d = {"ms": round(ms, 5)}
    if flop:
        ach = flop / (ms * 1e-3) / 1e12
        d.update(tflops=round(ach, 1), pct_peak=round(100 * ach / MFMA_BF16_PEAK_TFLOPS, 2))
        rf = {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
              "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4)}
    else:
        ach = nbytes / (ms * 1e-3) / 1e9
        d.update(gbs=round(ach, 1), pct_peak=round(100 * ach / HBM_PEAK_GBS, 2))
        rf = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
              "frac": round(ach / HBM_PEAK_GBS, 4)}
    rf["traffic"] = traffic
    rf["hbm_gbs"] = round(traffic / (ms * 1e-3) / 1e9, 1) if traffic else None
    rf["mfma_busy"] = round(ctr["mfma_busy"], 4) if ctr else None
    d["roofline"] = rf
    return d


def run_headline(args):
    """The default line: the windowed forward at S=65,536 (value), the causal forward at
    S=16,384 and the backward at B=4 H=32 S=4096, each kernel with its own roofline."""
    import torch

    import transformer_attention_07_amd as gqa
    from synth import WORKLOADS, make_inputs

    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    kernels, notes = {}, {}

    def fwd_unit(w):
        print(f"[bench] {w}", file=sys.stderr, flush=True)
        q, k, v, _ = make_inputs(w, with_do=False)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        o = torch.empty_like(qd)
        lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)
        kw = dict(causal=w.causal, window=w.window, num_sinks=w.num_sinks, scale=w.scale)
        call = lambda: gqa.gqa_attn_fwd(qd, kd, vd, out=o, lse=lse, stream=stream, **kw)  # noqa: E731
        n, secs = warm_up(call, args.warmup)
        (ms,), wall = time_units([call], args.steps, stream)
        pairs = gqa.gqa_visible_pairs(w.S, w.causal, w.window, w.num_sinks)
        flop = 4.0 * w.D * pairs * w.B * w.H
        notes[w.name] = {"warmup_calls": n, "warmup_s": round(secs, 2)}
        kernels[f"fwd@{w.name}"] = kernel_record("fwd", w.name, ms, flop=flop)
        kernels[f"fwd@{w.name}"]["workgroups"] = row_decomposition(w)["fwd"]
        return (q, k, v), flop, wall

    c4 = WORKLOADS["c4"]
    c4_inputs, c4_flop, c4_wall = fwd_unit(c4)
    fwd_unit(WORKLOADS["c3"])

    w5 = WORKLOADS["c5"]
    print(f"[bench] {w5}", file=sys.stderr, flush=True)
    q, k, v, do = make_inputs(w5, with_do=True)
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    kw = dict(causal=w5.causal, window=w5.window, num_sinks=w5.num_sinks, scale=w5.scale)
    o, lse, o_lo = gqa.gqa_attn_fwd(qd, kd, vd, keep_residual=True, stream=stream, **kw)  # as in training
    delta = torch.empty_like(lse)
    dq = torch.empty(qd.shape, dtype=torch.float32, device=dev)
    dk = torch.empty(kd.shape, dtype=torch.float32, device=dev)
    dv = torch.empty(kd.shape, dtype=torch.float32, device=dev)
    units = [lambda: gqa.gqa_attn_bwd_preprocess(o, dod, delta=delta, o_lo=o_lo, stream=stream),
             lambda: gqa.gqa_attn_bwd_dkdv(qd, kd, vd, lse, dod, delta, dk=dk, dv=dv, stream=stream, **kw),
             lambda: gqa.gqa_attn_bwd_dq(qd, kd, vd, lse, dod, delta, dq=dq, stream=stream, **kw),
             # dK/dV and dQ as the library runs them inside gqa_attn_bwd (one launch or two)
             lambda: gqa.gqa_attn_bwd_grads(qd, kd, vd, lse, dod, delta, dq=dq, dk=dk, dv=dv, stream=stream, **kw)]
    n, secs = warm_up(lambda: [u() for u in units], args.warmup)
    notes["c5"] = {"warmup_calls": n, "warmup_s": round(secs, 2)}
    (ms_pre, ms_dkdv, ms_dq, ms_grads), _ = time_units(units, args.steps, stream)
    clock_mhz = gqa.gqa_clock_probe()  # right after the timed steps, the device still warm

    pairs5 = gqa.gqa_visible_pairs(w5.S, True, 0, 0)
    bh5 = w5.B * w5.H
    shapes5 = row_decomposition(w5)
    kernels["bwd_preprocess@c5"] = kernel_record("bwd_preprocess", "c5", ms_pre,
                                                 nbytes=3.0 * bh5 * w5.S * w5.D * 2 + bh5 * w5.S * 4)
    kernels["bwd_dkdv@c5"] = kernel_record("bwd_dkdv", "c5", ms_dkdv, flop=8.0 * w5.D * pairs5 * bh5)
    kernels["bwd_dkdv@c5"]["workgroups"] = shapes5["bwd_dkdv"]
    kernels["bwd_dq@c5"] = kernel_record("bwd_dq", "c5", ms_dq, flop=2.0 * w5.D * pairs5 * bh5)
    kernels["bwd_dq@c5"]["workgroups"] = shapes5["bwd_dq"]
    kernels["bwd_grads@c5"] = kernel_record("bwd_grads", "c5", ms_grads, flop=10.0 * w5.D * pairs5 * bh5)
    kernels["bwd_grads@c5"]["note"] = "dK/dV and dQ in the launch(es) gqa_attn_bwd uses"
    bwd_ms = ms_pre + ms_grads
    bwd_t = 10.0 * w5.D * pairs5 * bh5 / (bwd_ms * 1e-3) / 1e12
    kernels["bwd@c5"] = {"ms": round(bwd_ms, 5), "tflops": round(bwd_t, 1),
                         "pct_peak": round(100 * bwd_t / MFMA_BF16_PEAK_TFLOPS, 2),
                         "note": "delta + grads (the whole gqa_attn_bwd); 10*d*pairs*B*H flop (S, dP, dV, dK, dQ)"}

    value = c4_flop / (c4_wall * 1e-3) / 1e12
    dom = kernels["fwd@c4"]
    roofline = dict(dom["roofline"], kernel="fwd@c4 (fwd_mfma_kernel)")

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(c4, (*c4_inputs, None), args.cpu_seconds, rows_sample=True)

    pairs4 = gqa.gqa_visible_pairs(c4.S, True, c4.window, c4.num_sinks)
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(c4_wall, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic N(0,1), seeded",
        "config": {"workload": f"causal GQA fwd with sliding window + sinks, B={c4.B} H={c4.H} G={c4.G} "
                               f"S={c4.S} d={c4.D} window={c4.window} sinks={c4.num_sinks}, bf16 "
                               "(the model card's head layout; the largest single-GPU workload)",
                   "B": c4.B, "H": c4.H, "G": c4.G, "S": c4.S, "D": c4.D, "causal": True, "window": c4.window,
                   "num_sinks": c4.num_sinks, "visible_pairs_per_head": pairs4, "flop_per_step": c4_flop,
                   "parallelism": "none (1 GPU)",
                   "also_timed": "fwd at B=1 H=128 G=16 S=16384 (causal); bwd at B=4 H=32 G=8 S=4096 (causal)"},
        "pct_of_peak": round(100 * value / MFMA_BF16_PEAK_TFLOPS, 2),
        "mfma_clock_mhz": round(clock_mhz, 1),
        **clock_under_load("fwd", c4.name, clock_mhz, value, MFMA_BF16_PEAK_TFLOPS),
        "mfma_busy": roofline["mfma_busy"], "hbm_gbs": roofline["hbm_gbs"],
        "kernels": kernels, "warmup_detail": notes,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def decode_bytes(w):
    """Algorithmic HBM bytes of one decode call: every cache row visible to at least one of
    the Sq rows, K and V, read once per kv head; Q read and O written once; lse written."""
    W, NS, Skv, Sq = w.window, w.num_sinks, w.Skv, w.Sq
    if W >= Skv:
        W = 0
    if W == 0 or NS >= Skv:
        W, NS = 0, 0
    lo = max(0, Skv - Sq - W + 1) if W else 0  # first window key of the oldest row
    keys = (Skv - lo) + min(NS, lo)
    elem = 2
    return (w.B * w.G * keys * w.D * 2 * elem + 2 * w.B * w.H * w.Sq * w.D * elem
            + w.B * w.H * w.Sq * 4)


def run_decode(args, w):
    import numpy as np
    import torch

    import transformer_attention_07_amd as gqa
    from synth import make_decode_inputs

    print(f"[bench] decode workload {w}", file=sys.stderr, flush=True)
    q, k, v = make_decode_inputs(w)
    dev = torch.device("cuda", 0)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)
    ws = torch.empty(max(16, gqa.gqa_attn_decode_workspace_bytes(qd, kd, w.window, w.num_sinks)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def call():
        gqa.gqa_attn_decode(qd, kd, vd, window=w.window, num_sinks=w.num_sinks, scale=w.scale, out=o, lse=lse,
                            workspace=ws, stream=stream)

    warm_up(call, args.warmup)
    if args.copy_calibration:  # a plain copy of known size, for counter calibration
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_call = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    ms_step = wall * 1e3 / args.steps
    nbytes = decode_bytes(w)
    value = nbytes / (ms_step * 1e-3) / 1e9
    ach = nbytes / (ms_call * 1e-3) / 1e9
    roofline = {"bound": "hbm", "kernel": "decode (split-KV pass + merge, one call)", "achieved": round(ach, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                "traffic": load_traffic("decode", w.name)}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle.attention as ref
        from threadpoolctl import threadpool_info

        print("[bench] timing the CPU oracle on one sequence", file=sys.stderr, flush=True)
        t1 = time.perf_counter()
        ref.decode(q[:1], k[:1], v[:1], scale=w.scale, window=w.window, num_sinks=w.num_sinks)
        dt = time.perf_counter() - t1
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        cpu = {"value": nbytes / w.B / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
               "sample": f"batch element 0 of {w.B} (all {w.H} heads, {w.Sq} rows each), {dt:.1f} s, fp64 numpy on {host_cpu()}"}
    wl = (f"decode, B={w.B} H={w.H} G={w.G} Sq={w.Sq} Skv={w.Skv} d={w.D}"
          + (f" window={w.window} sinks={w.num_sinks}" if w.window else "") + f", {w.dtype}")
    line = {
        "metric": "decode attention HBM throughput (algorithmic bytes / time)", "value": round(value, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic N(0,1), seeded",
        "config": {"workload": wl, "B": w.B, "H": w.H, "G": w.G, "Sq": w.Sq, "Skv": w.Skv, "D": w.D,
                   "window": w.window, "num_sinks": w.num_sinks, "bytes_per_step": nbytes,
                   "parallelism": "none (1 GPU)"},
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "kernels": {"decode": {"ms": round(ms_call, 5), "gbs": round(ach, 1)}},
        "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def run_rope_k(args):
    """The rotation kernel alone, on the model card's long-context K shape
    [2][16][204800][64] bf16 at positions 0 .. 204,799: each call reads and writes every
    element once (HBM-bound)."""
    import torch

    import transformer_attention_07_amd as gqa

    B, G, S, D = 2, 16, 204800, 64
    print(f"[bench] rotation of K [{B}][{G}][{S}][{D}] bf16", file=sys.stderr, flush=True)
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev).manual_seed(1250)
    x = torch.randn(B, G, S, D, generator=g, device=dev).to(torch.bfloat16)
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream(dev)
    warm_up(lambda: gqa.gqa_rope_apply(x, out=y, stream=stream), args.warmup)
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        gqa.gqa_rope_apply(x, out=y, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_call = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    ms_step = wall * 1e3 / args.steps
    nbytes = 2.0 * x.numel() * x.element_size()
    value = nbytes / (ms_step * 1e-3) / 1e9
    ach = nbytes / (ms_call * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle.rope as ref
        from threadpoolctl import threadpool_info

        print("[bench] timing the CPU oracle on one slab", file=sys.stderr, flush=True)
        xs = x[0, 0].cpu()
        t1 = time.perf_counter()
        ref.rope(xs, list(range(S)))
        dt = time.perf_counter() - t1
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        cpu = {"value": 2.0 * xs.numel() * 2 / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
               "sample": f"one [{S}][{D}] slab of {B * G}, {dt:.1f} s, fp64 numpy on {host_cpu()}"}
    line = {
        "metric": "YaRN rotary embedding HBM throughput (algorithmic bytes / time)", "value": round(value, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic N(0,1), seeded",
        "config": {"workload": f"YaRN RoPE (factor 32) of K [{B}][{G}][{S}][{D}] bf16, positions 0..{S - 1}",
                   "bytes_per_step": nbytes, "rope": dict(gqa.YARN_ROPE), "parallelism": "none (1 GPU)"},
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "kernels": {"rope": {"ms": round(ms_call, 5), "gbs": round(ach, 1)}},
        "roofline": {"bound": "hbm", "kernel": "rope", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": load_traffic("rope", "rope_k")},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def run_fp8(args, w):
    """The FP8 forward on a forward workload: e4m3 Q, K, V with per-tensor scales; one call
    = the V^T permute pre-pass + the forward kernel."""
    import torch

    import transformer_attention_07_amd as gqa
    from synth import make_fp8_inputs

    print(f"[bench] fp8 workload {w}", file=sys.stderr, flush=True)
    q8, k8, v8, sc = make_fp8_inputs(w)
    dev = torch.device("cuda", 0)
    q8d, k8d, v8d = q8.to(dev), k8.to(dev), v8.to(dev)
    kw = dict(causal=w.causal, window=w.window, num_sinks=w.num_sinks, scale=w.scale)
    o = torch.empty(q8.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(q8.shape[:3], dtype=torch.float32, device=dev)
    ws = torch.empty(max(16, gqa.gqa_attn_fwd_fp8_workspace_bytes(q8d, k8d, w.causal, w.window, w.num_sinks)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def call():
        gqa.gqa_attn_fwd_fp8(q8d, k8d, v8d, *sc, out=o, lse=lse, workspace=ws, stream=stream, **kw)

    warm_up(call, args.warmup)
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clock_mhz = gqa.gqa_clock_probe()
    ms_call = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    ms_step = wall * 1e3 / args.steps
    pairs = gqa.gqa_visible_pairs(w.S, w.causal, w.window, w.num_sinks)
    flop = 4.0 * w.D * pairs * w.B * w.H
    value = flop / (ms_step * 1e-3) / 1e12
    ach = flop / (ms_call * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        deq = tuple(x.to(torch.float32) * s for x, s in zip((q8, k8, v8), sc)) + (None,)
        cpu = cpu_baseline(w, deq, args.cpu_seconds)
    wl = (f"causal GQA fwd, FP8 e4m3 Q/K/V (per-tensor scales) and P, B={w.B} H={w.H} G={w.G} S={w.S} d={w.D}"
          + (f" window={w.window} sinks={w.num_sinks}" if w.window else "") + ", O bf16")
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8 e4m3", "data": "synthetic N(0,1) quantised per tensor, seeded",
        "config": {"workload": wl, "B": w.B, "H": w.H, "G": w.G, "S": w.S, "D": w.D, "causal": w.causal,
                   "window": w.window, "num_sinks": w.num_sinks, "visible_pairs_per_head": pairs,
                   "flop_per_step": flop, "parallelism": "none (1 GPU)"},
        "pct_of_peak": round(100 * value / MFMA_FP8_PEAK_TFLOPS, 2),
        "pct_of_bf16_peak": round(100 * value / MFMA_BF16_PEAK_TFLOPS, 2),
        "mfma_clock_mhz": round(clock_mhz, 1),
        "pct_of_peak_at_measured_clock": round(100 * value / (MFMA_FP8_PEAK_TFLOPS * clock_mhz / 2400.0), 2),
        "kernels": {"fwd_fp8": {"ms": round(ms_call, 5), "tflops": round(ach, 1)}},
        "roofline": {"bound": "mfma", "kernel": "fwd_fp8 (V^T permute + forward, one call)", "achieved": round(ach, 2),
                     "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / MFMA_FP8_PEAK_TFLOPS, 4),
                     "traffic": load_traffic("fwd_fp8", w.name)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: the attention path is built and measured on a "
              "single MI355X (no collectives, no sharding); use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.reduce_kernel_trace:
        print(reduce_kernel_trace(args.reduce_kernel_trace))
        return
    if args.reduce_sq_counters:
        print(reduce_sq_counters(args.reduce_sq_counters, args.workload))
        return
    if args.reduce_counters:
        special = args.workload.startswith("decode") or args.workload == "rope_k"
        name = args.workload if special else (workload(args.workload).name + ("_rope" if args.rope else "")
                                              + ("_fp8" if args.fp8 else ""))
        reduce_counters(*args.reduce_counters, name)
        return
    long_step = args.workload == "long"
    if args.steps is None:
        args.steps = 3 if long_step else 20
    if args.warmup is None:
        args.warmup = 1 if long_step else 5
    if args.workload == "headline":
        if args.rope or args.fp8:
            print("--rope and --fp8 apply to a single workload (--workload c3, c4, c5, step)", file=sys.stderr)
            sys.exit(2)
        import torch

        import transformer_attention_07_amd as gqa

        if not torch.cuda.is_available():
            print("bench.py needs a GPU", file=sys.stderr)
            sys.exit(1)
        gqa.library()  # fail loudly if the HIP library is not built
        run_headline(args)
        return
    if args.workload == "rope_k":
        import torch

        import transformer_attention_07_amd as gqa

        if not torch.cuda.is_available():
            print("bench.py needs a GPU", file=sys.stderr)
            sys.exit(1)
        gqa.library()
        run_rope_k(args)
        return
    if args.workload.startswith("decode"):
        import torch

        import transformer_attention_07_amd as gqa
        from synth import DECODE_WORKLOADS

        if not torch.cuda.is_available():
            print("bench.py needs a GPU", file=sys.stderr)
            sys.exit(1)
        gqa.library()
        run_decode(args, DECODE_WORKLOADS[args.workload])
        return

    import torch

    import transformer_attention_07_amd as gqa
    from synth import make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    gqa.library()  # fail loudly if the HIP library is not built
    w = workload(args.workload)
    if args.fp8:
        if args.rope or "bwd" in w.direction:
            print("--fp8 is a forward-only mode without --rope (workloads c2, c3, c4)", file=sys.stderr)
            sys.exit(2)
        run_fp8(args, w.with_(name=w.name + "_fp8"))
        return
    if args.rope:
        w = w.with_(name=w.name + "_rope")
    do_bwd = "bwd" in w.direction
    print(f"[bench] workload {w}", file=sys.stderr, flush=True)
    q, k, v, do = make_inputs(w, with_do=do_bwd)
    dev = torch.device("cuda", 0)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    dod = do.to(dev) if do_bwd else None
    kw = dict(causal=w.causal, window=w.window, num_sinks=w.num_sinks, scale=w.scale)
    o = torch.empty_like(qd)
    o_lo = torch.empty_like(qd) if do_bwd else None  # O's rounding residual, kept for the backward
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)
    delta = torch.empty_like(lse)
    dq = torch.empty(qd.shape, dtype=torch.float32, device=dev)
    dk = torch.empty(kd.shape, dtype=torch.float32, device=dev)
    dv = torch.empty(kd.shape, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    if args.split_grads and (args.rope or not do_bwd):
        print("--split-grads applies to backward workloads without --rope", file=sys.stderr)
        sys.exit(2)
    grads = ["bwd_dkdv", "bwd_dq"] if args.split_grads else ["bwd_grads"]
    kernels = ["fwd"] + (["bwd_preprocess"] + grads if do_bwd else [])
    q_rot = k_rot = None
    if args.rope:
        # the rotated Q (kept for the backward) and K; the backward rotates dQ and dK back as
        # its kernels store them
        q_rot = torch.empty_like(qd) if do_bwd else None
        k_rot = torch.empty_like(kd)
        ws = torch.empty(max(gqa.gqa_attn_bwd_workspace_bytes(qd, kd, **kw), 16), dtype=torch.uint8, device=dev)
        kernels = ["fwd_rope"] + (["bwd_rope"] if do_bwd else [])

    def step(events=None):
        def mark(i):
            if events is not None:
                events[i].record(stream)
        mark(0)
        if args.rope:  # rotation of K, then the forward with Q rotated in registers
            gqa.gqa_attn_fwd_rope(qd, kd, vd, out=o, lse=lse, o_lo=o_lo, q_rot=q_rot, k_rot=k_rot,
                                  keep_q_rot=do_bwd, stream=stream, **kw)
        else:
            gqa.gqa_attn_fwd(qd, kd, vd, out=o, lse=lse, o_lo=o_lo, stream=stream, **kw)
        mark(1)
        if do_bwd and args.rope:  # delta, then dK/dV and dQ with the back-rotation at the store
            gqa.gqa_attn_bwd_rope(q_rot, k_rot, vd, o, lse, dod, dq=dq, dk=dk, dv=dv, workspace=ws, o_lo=o_lo,
                                  stream=stream, **kw)
            mark(2)
        elif do_bwd:
            gqa.gqa_attn_bwd_preprocess(o, dod, delta=delta, o_lo=o_lo, stream=stream)
            mark(2)
            if args.split_grads:
                gqa.gqa_attn_bwd_dkdv(qd, kd, vd, lse, dod, delta, dk=dk, dv=dv, stream=stream, **kw)
                mark(3)
                gqa.gqa_attn_bwd_dq(qd, kd, vd, lse, dod, delta, dq=dq, stream=stream, **kw)
                mark(4)
            else:
                # dK, dV and dQ: one fused launch when the dK/dV grid fills at most two rounds
                # of workgroup slots, else the two passes back to back
                gqa.gqa_attn_bwd_grads(qd, kd, vd, lse, dod, delta, dq=dq, dk=dk, dv=dv, stream=stream, **kw)
                mark(3)

    warm_up(step, args.warmup, floor_s=0.0 if long_step else WARMUP_FLOOR_S)

    if args.copy_calibration:  # a plain copy of known size, for counter calibration
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(kernels) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(ev[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    clock_mhz = gqa.gqa_clock_probe()  # right after the timed steps, the device still warm

    per_kernel_ms = {}
    for i, name in enumerate(kernels):
        per_kernel_ms[name] = sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)) / args.steps
    ms_per_step = wall * 1e3 / args.steps

    pairs = gqa.gqa_visible_pairs(w.S, w.causal, w.window, w.num_sinks)
    bh = w.B * w.H
    # with --rope, fwd_rope is the rotation of K plus the forward, bwd_rope delta plus dK/dV and dQ
    flop = {"fwd": 4.0 * w.D * pairs * bh, "fwd_rope": 4.0 * w.D * pairs * bh, "bwd_preprocess": 0.0,
            "bwd_grads": 10.0 * w.D * pairs * bh, "bwd_rope": 10.0 * w.D * pairs * bh,
            "bwd_dkdv": 8.0 * w.D * pairs * bh, "bwd_dq": 2.0 * w.D * pairs * bh}
    elem = 2 if w.dtype in ("bf16", "f16") else 4
    hbm_bytes = {"bwd_preprocess": 3.0 * bh * w.S * w.D * elem + bh * w.S * 4}  # O, o_lo, dO in; delta out
    step_flop = flop["fwd"] + (10.0 * w.D * pairs * bh if do_bwd else 0.0)
    value = step_flop / (ms_per_step * 1e-3) / 1e12

    detail = {}
    for name in kernels:
        ms = per_kernel_ms[name]
        d = {"ms": round(ms, 5)}
        if flop[name] > 0:
            t = flop[name] / (ms * 1e-3) / 1e12
            d.update(tflops=round(t, 1), pct_peak=round(100 * t / MFMA_BF16_PEAK_TFLOPS, 1))
        else:
            d.update(gbs=round(hbm_bytes[name] / (ms * 1e-3) / 1e9, 1))
        detail[name] = d
    fwd_tflops = flop[kernels[0]] / (per_kernel_ms[kernels[0]] * 1e-3) / 1e12
    if do_bwd:
        bwd_ms = sum(per_kernel_ms[n] for n in kernels[1:])
        detail["bwd_total"] = {"ms": round(bwd_ms, 5),
                               "tflops": round(10.0 * w.D * pairs * bh / (bwd_ms * 1e-3) / 1e12, 1)}
    detail["fwd_tflops"] = round(fwd_tflops, 1)

    # (with --rope the timed units are the two calls, each two launches; per-kernel times of
    # that run come from the kernel trace)
    dominant = max((n for n in kernels if flop[n] > 0), key=lambda n: per_kernel_ms[n])
    ach = flop[dominant] / (per_kernel_ms[dominant] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dominant, "achieved": round(ach, 2),
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": load_traffic(dominant, w.name)}

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, (q, k, v, do), args.cpu_seconds, rope=args.rope)

    wl = (f"causal GQA {'fwd+bwd' if do_bwd else 'fwd'}, B={w.B} H={w.H} G={w.G} S={w.S} d={w.D}"
          + (f" window={w.window} sinks={w.num_sinks}" if w.window else "")
          + (", YaRN RoPE x32 on q and k" if args.rope else "") + f", {w.dtype}")
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic N(0,1), seeded",
        "config": {"workload": wl, "B": w.B, "H": w.H, "G": w.G, "S": w.S, "D": w.D, "causal": w.causal,
                   "window": w.window, "num_sinks": w.num_sinks, "visible_pairs_per_head": pairs,
                   "flop_per_step": step_flop, "parallelism": "none (1 GPU)",
                   "rope": dict(gqa.YARN_ROPE) if args.rope else None,
                   "grads_launches": ("two (--split-grads)" if args.split_grads else "as gqa_attn_bwd chooses")
                   if do_bwd else None},
        "pct_of_peak": round(100 * value / MFMA_BF16_PEAK_TFLOPS, 2),
        "mfma_clock_mhz": round(clock_mhz, 1),
        "pct_of_peak_at_measured_clock": round(100 * value / (MFMA_BF16_PEAK_TFLOPS * clock_mhz / 2400.0), 2),
        "kernels": detail,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
