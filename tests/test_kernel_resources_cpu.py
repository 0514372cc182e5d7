"""Register and scratch usage of every gfx950 kernel, from the compiler's
kernel-resource-usage remarks (device-only compiles, no GPU needed).

No kernel may use scratch memory: a per-lane stack (a spilled register, a copied
argument block or the callee-saved registers of an out-of-line call) turns into
HBM traffic that scales with the grid.  The matrix-core kernels must keep two
waves per SIMD, which their launch bounds ask for.
"""

from __future__ import annotations

import pytest

from transformer_attention_07_amd.build import SOURCES, resource_usage

HIP_SOURCES = [s for s in SOURCES if s.endswith(".hip")]
TWO_WAVES = ("fwd_mfma_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel", "bwd_fused_kernel", "fwd_fp8_kernel")


@pytest.mark.slow
@pytest.mark.parametrize("src", HIP_SOURCES)
def test_no_scratch_and_occupancy(src):
    import os

    from transformer_attention_07_amd.build import CSRC

    usage = resource_usage(src)
    with open(os.path.join(CSRC, src)) as f:
        has_kernels = "__global__" in f.read()
    assert bool(usage) == has_kernels, f"{src}: kernel-resource-usage remarks {sorted(usage)}"
    for name, u in usage.items():
        assert "scratch_bytes_per_lane" in u and "occupancy" in u, (name, u)
        assert u["scratch_bytes_per_lane"] == 0, f"{src}: {name} uses {u['scratch_bytes_per_lane']} B/lane of scratch"
        if any(k in name for k in TWO_WAVES):
            assert u["occupancy"] >= 2, f"{src}: {name} at {u['occupancy']} wave(s) per SIMD"


def test_backward_kernels_take_one_argument_block():
    # the backward kernels read their parameters and rotation table from one by-value block,
    # so nothing depends on a hand-computed argument offset
    import os
    import re

    from transformer_attention_07_amd.build import CSRC

    with open(os.path.join(CSRC, "gqa_bwd.hip")) as f:
        src = f.read()
    for k in ("bwd_dkdv_kernel", "bwd_dq_kernel", "bwd_fused_kernel"):
        m = re.search(k + r"\(([^)]*)\)\s*\{", src)
        assert m and m.group(1).strip() == "BwdArgs a", (k, m and m.group(1))
    assert "kernarg_segment_ptr" not in src
