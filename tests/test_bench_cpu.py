"""Host-side pieces of bench.py that need no GPU: the reduction of rocprofv3 counter files
to HBM bytes per launch."""

from __future__ import annotations

import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

FIELDS = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]


def _write(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, kib) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Grid_Size": 64, "Counter_Name": counter,
                        "Counter_Value": kib})


def test_counter_reduction_calibrates_on_the_large_copy(tmp_path):
    # The 1 GiB calibration copy reads as 512 MiB fetched and 1 GiB written.  A small copy
    # that reads a result back uses the same runtime kernel; it must not dilute the
    # calibration.  A forward kernel launched twice fetches 100 MiB and writes 40 MiB per
    # launch on the calibrated scale.
    copy, small = "__amd_rocclr_copyBuffer", "__amd_rocclr_copyBuffer"
    fwd = "void gqa::(anonymous namespace)::fwd_mfma_kernel<1, false>(gqa::FwdParams)"
    mib = 1024.0  # KiB per MiB
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _write(fetch, "FETCH_SIZE", [(copy, 512 * mib), (fwd, 50 * mib), (fwd, 50 * mib), (small, 3.4)])
    _write(write, "WRITE_SIZE", [(copy, 1024 * mib), (fwd, 40 * mib), (fwd, 40 * mib), (small, 4.0)])
    out = tmp_path / "traffic.json"
    bench.reduce_counters(str(fetch), str(write), "wl", path=str(out))
    rec = json.loads(out.read_text())
    assert rec["calibration"]["wl"] == {"fetch_scale": 2.0, "write_scale": 1.0}
    ent = rec["kernels"]["fwd@wl"]
    assert ent["fetch_bytes"] == 100 << 20 and ent["write_bytes"] == 40 << 20
    assert ent["bytes_per_launch"] == 140 << 20
    assert rec["source_digest"] == bench.source_digest()
    # what the bench line's roofline reads back
    assert bench.load_traffic("fwd", "wl", path=str(out)) == 140 << 20
    assert bench.load_traffic("fwd", "other", path=str(out)) is None


def test_committed_counters_read_back():
    # every bench line reads the committed summaries: they must parse and hold the default
    # line's kernels.  After a kernel change their digest is stale until counters are taken
    # again on a GPU, and the bench then reports traffic, hbm_gbs and mfma_busy as null.
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        rec = json.load(f)
    with open(os.path.join(ROOT, "profiles", "counters.json")) as f:
        ctr = json.load(f)
    # the default line's kernels: the windowed forward (its roofline), the causal forward and
    # the backward's kernels
    for key in ("fwd@c4", "fwd@c3", "bwd_dkdv@c5", "bwd_dq@c5", "bwd_preprocess@c5"):
        assert key in rec["kernels"] and key in ctr["kernels"], key
    assert rec["calibration"]
    if rec["source_digest"] != bench.source_digest() or ctr["source_digest"] != bench.source_digest():
        pytest.skip("counters predate the current kernel sources")
    assert bench.load_traffic("fwd", "c4") == rec["kernels"]["fwd@c4"]["bytes_per_launch"]
    assert 0 < bench.load_counters("fwd", "c4")["mfma_busy"] < 1


SQ_FIELDS = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value", "Start_Timestamp",
             "End_Timestamp"]


def test_sq_counter_reduction(tmp_path):
    # Two dispatches of the forward.  The GRBM counter is summed over the 8 XCDs: 8e6 means
    # 1e6 GPU cycles; over 500 us that is 2000 MHz.  The matrix cores were busy 512e6
    # SIMD-cycles out of 1e6 x 1024: 50 %.  1e9 executed MFMA operations of 512 flop.
    fwd = "void gqa::(anonymous namespace)::fwd_mfma_kernel<1, false>(gqa::FwdParams)"
    vals = {"SQ_INSTS_VALU_MFMA_MOPS_BF16": 1e9, "SQ_VALU_MFMA_BUSY_CYCLES": 512e6,
            "SQ_VALU_MFMA_COEXEC_CYCLES": 128e6, "SQ_WAVE_CYCLES": 4e8, "SQ_ACTIVE_INST_VALU": 1e8,
            "SQ_ACTIVE_INST_LDS": 2e7, "SQ_WAIT_INST_ANY": 2e8, "SQ_LDS_BANK_CONFLICT": 0.0, "GRBM_GUI_ACTIVE": 8e6}
    path = tmp_path / "sq.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=SQ_FIELDS)
        w.writeheader()
        for d in (1, 2):
            for name, v in vals.items():
                w.writerow({"Dispatch_Id": d, "Kernel_Name": fwd, "Grid_Size": 64, "Counter_Name": name,
                            "Counter_Value": v, "Start_Timestamp": 1000, "End_Timestamp": 1000 + 500_000})
        # a copy dispatch and a kernel of no interest are ignored
        w.writerow({"Dispatch_Id": 3, "Kernel_Name": "__amd_rocclr_copyBuffer", "Grid_Size": 64,
                    "Counter_Name": "GRBM_GUI_ACTIVE", "Counter_Value": 1, "Start_Timestamp": 0, "End_Timestamp": 1})
    out = tmp_path / "counters.json"
    text = bench.reduce_sq_counters(str(path), "wl", path=str(out))
    rec = json.loads(out.read_text())
    ent = rec["kernels"]["fwd@wl"]
    assert ent["dispatches"] == 2
    assert ent["mfma_busy"] == pytest.approx(0.5)
    assert ent["mfma_flop_executed"] == pytest.approx(512e9)
    assert ent["mfma_coexec_valu"] == pytest.approx(0.25)
    assert ent["valu_active_per_wave_cycle"] == pytest.approx(0.25)
    assert ent["wait_issue_per_wave_cycle"] == pytest.approx(0.5)
    assert ent["clock_mhz"] == pytest.approx(2000.0)
    assert "MFMA busy 50.0 %" in text
    assert bench.load_counters("fwd", "wl", path=str(out))["mfma_busy"] == pytest.approx(0.5)
    assert bench.load_counters("fwd", "other", path=str(out)) is None
    # a stale digest hides the entry from bench lines
    rec["source_digest"] = "0" * 16
    out.write_text(json.dumps(rec))
    assert bench.load_counters("fwd", "wl", path=str(out)) is None


def test_kernel_trace_reduction_splits_launch_shapes(tmp_path):
    # one kernel at two launch shapes (2048 and 32768 workgroups of 256 lanes): one row each
    fwd = "void gqa::(anonymous namespace)::fwd_mfma_kernel<1, false>(gqa::FwdParams)"
    path = tmp_path / "kernel_trace.csv"
    fields = ["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Start_Timestamp", "End_Timestamp"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for dur_us, wgs in [(100, 2048), (110, 2048), (30000, 32768), (32000, 32768), (31000, 32768)]:
            w.writerow({"Kernel_Name": fwd, "Grid_Size_X": wgs * 256, "Workgroup_Size_X": 256,
                        "Start_Timestamp": 0, "End_Timestamp": dur_us * 1000})
    rows = bench.reduce_kernel_trace(str(path)).splitlines()
    assert len(rows) == 3
    big = rows[1].split()
    assert big[0] == "fwd" and big[1] == "32768" and big[2] == "3" and float(big[3]) == pytest.approx(31000.0)
    small = rows[2].split()
    assert small[1] == "2048" and float(small[3]) == pytest.approx(105.0)


def test_row_decomposition_labels():
    # the launch shapes the library picks (4 heads per workgroup when H/G allows, 64 rows
    # per wave; 128 keys per dK/dV workgroup)
    from synth import WORKLOADS

    assert bench.row_decomposition(WORKLOADS["c4"])["fwd"] == 1024 * 32
    assert bench.row_decomposition(WORKLOADS["c3"])["fwd"] == 256 * 32
    c5 = bench.row_decomposition(WORKLOADS["c5"])
    assert c5["fwd"] == 64 * 4 * 8 and c5["bwd_dkdv"] == 32 * 4 * 8


@pytest.mark.parametrize("flag", ["--rope", "--fp8"])
def test_default_line_rejects_single_workload_flags(flag):
    # --rope / --fp8 change one workload's kernels; the default line times several, so the
    # combination is refused before anything touches a GPU
    import subprocess

    r = subprocess.run([sys.executable, os.path.join(os.path.dirname(bench.__file__), "bench.py"), flag],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "--workload" in r.stderr


def test_clock_under_load_prefers_the_kernels_own_counters(tmp_path, monkeypatch):
    # the peak is scaled by the clock the counters saw during the kernel's dispatches when
    # they match the sources, else by the probe's
    rec = {"source_digest": bench.source_digest(), "kernels": {"fwd@c4": {"clock_mhz": 1950.0}}}
    path = tmp_path / "counters.json"
    path.write_text(json.dumps(rec))
    real = bench.load_counters
    monkeypatch.setattr(bench, "load_counters", lambda k, w, path_=str(path): real(k, w, path=path_))
    got = bench.clock_under_load("fwd", "c4", 2100.0, 1000.0, 2516.6)
    assert got["clock_mhz_for_peak"] == 1950.0 and "counters" in got["clock_source"]
    assert abs(got["pct_of_peak_at_measured_clock"] - 100 * 1000.0 / (2516.6 * 1950.0 / 2400.0)) < 0.01
    got = bench.clock_under_load("fwd", "c3", 2100.0, 1000.0, 2516.6)
    assert got["clock_mhz_for_peak"] == 2100.0 and "probe" in got["clock_source"]
