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


def test_committed_traffic_reads_back():
    # every bench line reads the committed summary: it must parse and hold the default
    # step's dominant kernel.  After a kernel change its digest is stale until counters are
    # taken again on a GPU, and the bench then reports traffic as null.
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        rec = json.load(f)
    assert "bwd_grads@step" in rec["kernels"] and rec["calibration"]
    if rec["source_digest"] != bench.source_digest():
        pytest.skip("counters predate the current kernel sources")
    assert bench.load_traffic("bwd_grads", "step") == rec["kernels"]["bwd_grads@step"]["bytes_per_launch"]
