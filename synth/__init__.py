"""Seeded synthetic inputs for the attention workloads.

This module holds no attention arithmetic: it only names the workload shapes
and draws i.i.d. N(0, 1) tensors from a seeded CPU generator, so that the
oracle, the tests and the benchmark all see bit-identical inputs.

Recipe: ``torch.Generator('cpu').manual_seed(seed)`` with ``seed = 1234 + k``
for workload k (1..5); ``torch.randn`` in fp32 in the fixed order Q, K, V, dO;
each tensor then cast (round to nearest even) to the workload dtype on the CPU.
Shapes follow the model card's attention layout (128 query heads over 16 KV
heads, head dimension 64) and the tiny gate program's grouping (H=4, G=2).
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "sample_rows", "sample_rows_c4"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    G: int
    S: int
    D: int = 64
    dtype: str = "bf16"          # "f32", "bf16" or "f16"
    causal: bool = True
    window: int = 0
    num_sinks: int = 0
    direction: str = "fwd"       # "fwd", "bwd" or "fwd+bwd"
    seed: int = 0
    desc: str = ""

    @property
    def torch_dtype(self):
        return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[self.dtype]

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "c1": Workload("c1", B=1, H=4, G=2, S=128, dtype="f32", direction="fwd+bwd", seed=1235,
                   desc="tiny causal GQA fwd+bwd, fp32"),
    "c2": Workload("c2", B=4, H=32, G=8, S=2048, dtype="bf16", direction="fwd", seed=1236,
                   desc="causal GQA fwd, bf16 in / fp32 accumulate"),
    "c3": Workload("c3", B=1, H=128, G=16, S=16384, dtype="bf16", direction="fwd", seed=1237,
                   desc="causal GQA fwd at the model card's head layout"),
    "c4": Workload("c4", B=1, H=128, G=16, S=65536, dtype="bf16", window=16384, num_sinks=2048,
                   direction="fwd", seed=1238, desc="sliding-window + sink causal GQA fwd"),
    "c5": Workload("c5", B=4, H=32, G=8, S=4096, dtype="bf16", direction="bwd", seed=1239,
                   desc="causal GQA bwd from saved logsumexp, fp32 gradients"),
}


def make_inputs(w: Workload, with_do: bool | None = None, seed: int | None = None):
    """Return CPU tensors (q, k, v, do) in the workload dtype; do is None when
    the direction has no backward and ``with_do`` is not forced."""
    if with_do is None:
        with_do = "bwd" in w.direction
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed if seed is None else seed)
    shapes = [(w.B, w.H, w.S, w.D), (w.B, w.G, w.S, w.D), (w.B, w.G, w.S, w.D), (w.B, w.H, w.S, w.D)]
    out = []
    for n, shp in enumerate(shapes):
        if n == 3 and not with_do:
            out.append(None)
            break
        t = torch.randn(shp, generator=gen, dtype=torch.float32)
        out.append(t.to(w.torch_dtype).contiguous())
    return tuple(out)


def sample_rows(B: int, H: int, S: int, n: int, seed: int, forced_rows=()):
    """Distinct (b, h, i) triples: ``n`` drawn uniformly without replacement
    from numpy's seeded default_rng, plus every forced position ``i`` for the
    first, middle and last head of batch 0 and of the last batch."""
    rng = np.random.default_rng(seed)
    total = B * H * S
    flat = rng.choice(total, size=min(n, total), replace=False)
    trip = set(zip(*np.unravel_index(flat, (B, H, S))))
    for b in sorted({0, B - 1}):
        for h in sorted({0, H // 2, H - 1}):
            for i in forced_rows:
                if 0 <= i < S:
                    trip.add((b, h, i))
    trip = sorted((int(b), int(h), int(i)) for b, h, i in trip)
    return np.array(trip, dtype=np.int64).reshape(-1, 3)


def sample_rows_c4(w: Workload, n: int = 4096):
    """Rows checked at the sliding-window + sink workload: ``n`` seeded random
    (h, i) pairs of batch 0 plus rows at the sink, window and tile edges for
    heads 0, 7, 8 and 127 (first/last head of two neighbouring kv groups)."""
    rng = np.random.default_rng(w.seed)
    flat = rng.choice(w.H * w.S, size=n, replace=False)
    trip = {(0, int(f // w.S), int(f % w.S)) for f in flat}
    W, NS = w.window, w.num_sinks
    forced = [0, 1, 63, 64, NS - 1, NS, W - 1, W, W + NS - 1, W + NS, w.S - 1]
    for h in (0, 7, 8, w.H - 1):
        for i in forced:
            if 0 <= i < w.S:
                trip.add((0, h, i))
    trip = sorted(trip)
    return np.array(trip, dtype=np.int64).reshape(-1, 3)
