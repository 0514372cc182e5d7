"""Build libgqa.so for gfx950 with hipcc, in-tree (next to this file).

``python -m transformer_attention_07_amd.build`` or ``build_library()``.  Every
source is compiled each time (each translation unit in parallel), then linked.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgqa.so")

SOURCES = ["gqa_api.cpp", "gqa_fwd.hip", "gqa_bwd.hip", "gqa_f32.hip", "gqa_decode.hip", "gqa_rope.hip", "gqa_fwd_fp8.hip", "gqa_clock.hip",
           "gqa_noalloc.hip"]
ARCH = os.environ.get("GQA_OFFLOAD_ARCH", "gfx950")

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU instructions.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
                "-Wall", "-Wno-unused-function"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libgqa)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)
    return out


def build_library(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([hipcc, *COMMON_FLAGS, *DEVICE_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(len(cmds), 4)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


def resource_usage(src: str) -> dict:
    """Per-kernel register and scratch usage of one HIP source, compiled for the device
    only, from the compiler's kernel-resource-usage remarks: {kernel symbol: {"vgprs",
    "agprs", "sgprs", "scratch_bytes_per_lane", "occupancy"}}."""
    import re

    cmd = [_hipcc(), *COMMON_FLAGS, *DEVICE_FLAGS, "-x", "hip", "--offload-device-only", "-c",
           os.path.join(CSRC, src), "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
    out = _run(cmd, False)
    fields = {"VGPRs": "vgprs", "AGPRs": "agprs", "TotalSGPRs": "sgprs",
              "ScratchSize [bytes/lane]": "scratch_bytes_per_lane", "Occupancy [waves/SIMD]": "occupancy"}
    res, cur = {}, None
    for line in out.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            cur = res.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z][^:]*): (\d+)", line)
        if m and cur is not None and m.group(1).strip() in fields:
            cur[fields[m.group(1).strip()]] = int(m.group(2))
    return res


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
