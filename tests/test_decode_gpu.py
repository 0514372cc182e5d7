"""Decode attention (gqa_attn_decode, through the C-ABI) against the CPU fp64 oracle.

Tolerances as for the forward: O max abs 2e-2 and mean abs 2e-3, lse max abs 1e-3.
Every output row is compared, at small shapes that span several key tiles, splits,
row blocks and row chunks with ragged tails, and at the two full-size decode workloads.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle.attention as ref
import transformer_attention_07_amd as gqa
from synth import DECODE_WORKLOADS, DecodeWorkload, make_decode_inputs

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-3


def _check(w: DecodeWorkload):
    print(f"[decode] {w}", flush=True)
    q, k, v = make_decode_inputs(w)
    o, lse = gqa.gqa_attn_decode(q.cuda(), k.cuda(), v.cuda(), window=w.window, num_sinks=w.num_sinks,
                                 scale=w.scale)
    torch.cuda.synchronize()
    O, L = ref.decode(q, k, v, scale=w.scale, window=w.window, num_sinks=w.num_sinks)
    eo = np.abs(o.float().cpu().numpy().astype(np.float64) - O)
    el = np.abs(lse.cpu().numpy().astype(np.float64) - L)
    print(f"  O: max {eo.max():.3e} mean {eo.mean():.3e}; lse: max {el.max():.3e}", flush=True)
    assert np.isfinite(eo).all() and np.isfinite(el).all()
    assert eo.max() <= O_MAX and eo.mean() <= O_MEAN
    assert el.max() <= LSE_MAX
    return q, k, v, o, lse


# (B, H, G, Sq, Skv, window, sinks, dtype): one key, ragged tails, 1..4 row blocks (rows =
# H/G * Sq up to 128 per chunk: the shared-tile kernel with 2, 3 and 4 waves at 48, 72/84
# and 112/128 rows), two row chunks, MHA, f16, Sq == Skv, a window that starts inside the
# sinks' reach, many splits
SMALL = [
    (1, 4, 2, 1, 1, 0, 0, "bf16"),
    (2, 8, 2, 3, 100, 0, 0, "bf16"),
    (1, 16, 2, 16, 777, 0, 0, "bf16"),
    (1, 8, 8, 5, 300, 64, 4, "bf16"),
    (1, 32, 2, 7, 1000, 200, 10, "bf16"),
    (1, 40, 2, 8, 500, 0, 0, "bf16"),
    (3, 8, 4, 2, 4100, 1000, 64, "f16"),
    (2, 16, 2, 9, 9, 0, 0, "bf16"),
    (1, 8, 2, 4, 70000, 16384, 2048, "bf16"),
    (1, 12, 4, 3, 5000, 0, 0, "bf16"),
    (1, 4, 1, 2, 200, 130, 70, "bf16"),
    (1, 16, 2, 6, 3000, 500, 16, "bf16"),
    (1, 24, 2, 7, 2000, 0, 0, "f16"),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}H{}G{}Sq{}Skv{}W{}N{}{}".format(*c))
def test_decode_small(case):
    B, H, G, Sq, Skv, W, NS, dt = case
    _check(DecodeWorkload("small", B=B, H=H, G=G, Sq=Sq, Skv=Skv, window=W, num_sinks=NS, dtype=dt,
                          seed=1300 + Skv + Sq))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", sorted(DECODE_WORKLOADS))
def test_decode_full_size(name):
    _check(DECODE_WORKLOADS[name])


def test_decode_is_deterministic_and_reuses_workspace():
    w = DecodeWorkload("det", B=2, H=16, G=4, Sq=3, Skv=3000, window=512, num_sinks=32, seed=1299)
    q, k, v = (t.cuda() for t in make_decode_inputs(w))
    ws = torch.full((gqa.gqa_attn_decode_workspace_bytes(q, k, w.window, w.num_sinks),), 255,
                    dtype=torch.uint8, device="cuda")
    o1, l1 = gqa.gqa_attn_decode(q, k, v, window=w.window, num_sinks=w.num_sinks, workspace=ws)
    o2, l2 = gqa.gqa_attn_decode(q, k, v, window=w.window, num_sinks=w.num_sinks, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("sq", [1, 16])
def test_decode_maximum_jumps_inside_tiles(sq):
    # cache keys whose scores jump by 2^46, then 2^92 (log2 units) between the halves of a
    # 64-key tile: every partial's running maximum is raised in the middle of a tile
    B, H, G, Skv = 1, 8, 1, 320
    q = torch.full((B, H, sq, 64), 2.0)
    k = torch.zeros((B, G, Skv, 64))
    k[:, :, 32:64] = 2.0
    k[:, :, 64:96] = 2.0
    k[:, :, 96:128] = 4.0
    v = torch.randn((B, G, Skv, 64), generator=torch.Generator().manual_seed(7320))
    q, k, v = (x.to(torch.bfloat16) for x in (q, k, v))
    o, lse = gqa.gqa_attn_decode(q.cuda(), k.cuda(), v.cuda())
    torch.cuda.synchronize()
    O, L = ref.decode(q, k, v)
    eo = np.abs(o.float().cpu().numpy().astype(np.float64) - O)
    el = np.abs(lse.cpu().numpy().astype(np.float64) - L)
    print(f"  O: max {eo.max():.3e} mean {eo.mean():.3e}; lse: max {el.max():.3e}", flush=True)
    assert np.isfinite(eo).all() and np.isfinite(el).all()
    assert eo.max() <= O_MAX and eo.mean() <= O_MEAN and el.max() <= LSE_MAX


@pytest.mark.parametrize("sq", [1, 16])
def test_decode_first_keys_far_below_the_rest(sq):
    # the first 64 cache keys score about -1000 (log2 units), keys 160..223 about +23: the
    # partials that hold only low keys keep a maximum near -1000 and get merge weight 0, the
    # others raise theirs by ~1000 and scale what came before by exactly 0
    B, H, G, Skv = 1, 8, 1, 320
    c = 1000.0 / (2.0 * 64 * (64 ** -0.5) * math.log2(math.e))
    q = torch.full((B, H, sq, 64), 2.0)
    k = torch.zeros((B, G, Skv, 64))
    k[:, :, :64] = -c
    k[:, :, 160:224] = 1.0
    v = torch.randn((B, G, Skv, 64), generator=torch.Generator().manual_seed(7333))
    q, k, v = (x.to(torch.bfloat16) for x in (q, k, v))
    o, lse = gqa.gqa_attn_decode(q.cuda(), k.cuda(), v.cuda())
    torch.cuda.synchronize()
    O, L = ref.decode(q, k, v)
    eo = np.abs(o.float().cpu().numpy().astype(np.float64) - O)
    el = np.abs(lse.cpu().numpy().astype(np.float64) - L)
    print(f"  O: max {eo.max():.3e} mean {eo.mean():.3e}; lse: max {el.max():.3e}", flush=True)
    assert np.isfinite(eo).all() and np.isfinite(el).all()
    assert eo.max() <= O_MAX and eo.mean() <= O_MEAN and el.max() <= LSE_MAX
