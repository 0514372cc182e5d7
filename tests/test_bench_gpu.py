"""bench.py on every workload it offers (short runs): it exits 0 and prints one JSON line
with the contract's fields, a roofline record and the CPU baseline where asked for.  The
benchmark runs as a child process, one workload after another."""

from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FIELDS = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
          "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline")

CASES = [
    ([], True),                       # the default line, with the CPU baseline
    (["--workload", "step"], False),
    (["--workload", "c5"], False),
    (["--workload", "c5", "--split-grads"], False),
    (["--workload", "c3"], False),
    (["--workload", "decode16"], False),
    (["--workload", "rope_k"], False),
    (["--rope", "--workload", "step"], False),
    (["--fp8", "--workload", "c2"], False),
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("args,cpu", CASES, ids=lambda a: " ".join(a) if isinstance(a, list) else str(a))
def test_bench_line(args, cpu):
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1", *args]
    if cpu:
        cmd += ["--cpu-seconds", "2"]
    else:
        cmd += ["--no-cpu-baseline"]
    print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=280)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for f in FIELDS:
        assert f in d, f
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["value"] > 0
    assert "workload" in d["config"]
    rf = d["roofline"]
    assert rf["bound"] in ("mfma", "hbm") and rf["achieved"] > 0 and 0 < rf["frac"] < 1
    if not args:  # the default line: the windowed forward at S=65536, with the other headline kernels
        assert d["config"]["S"] == 65536 and d["config"]["window"] == 16384 and d["config"]["num_sinks"] == 2048
        for k in ("fwd@c4", "fwd@c3", "bwd_preprocess@c5", "bwd_dkdv@c5", "bwd_dq@c5", "bwd_grads@c5", "bwd@c5"):
            assert d["kernels"][k]["ms"] > 0, k
        kc5 = d["kernels"]
        assert abs(kc5["bwd@c5"]["ms"] - kc5["bwd_preprocess@c5"]["ms"] - kc5["bwd_grads@c5"]["ms"]) < 1e-3
        for k in ("fwd@c4", "fwd@c3", "bwd_dkdv@c5", "bwd_dq@c5", "bwd_grads@c5"):
            r = d["kernels"][k]["roofline"]
            assert r["bound"] == "mfma" and 0 < r["frac"] < 1, k
        assert d["roofline"]["achieved"] == d["kernels"]["fwd@c4"]["roofline"]["achieved"]
        assert "mfma_busy" in d and "hbm_gbs" in d
        assert d["clock_mhz_for_peak"] > 0 and d["clock_source"] and d["pct_of_peak_at_measured_clock"] > 0
        assert d["warmup_detail"]["c4"]["warmup_s"] >= 1.0
    if "--split-grads" in args:
        assert d["kernels"]["bwd_dkdv"]["ms"] > 0 and d["kernels"]["bwd_dq"]["ms"] > 0
        assert "bwd_grads" not in d["kernels"] and "two" in d["config"]["grads_launches"]
    if cpu:
        c = d["cpu_baseline"]
        assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["sample"]
    else:
        assert d["cpu_baseline"] is None
