"""Seeded synthetic inputs for the attention workloads.

This module holds no attention arithmetic: it only names the workload shapes
and draws i.i.d. N(0, 1) tensors from a seeded CPU generator, so that the
oracle, the tests and the benchmark all see bit-identical inputs.

Recipe: ``torch.Generator('cpu').manual_seed(seed)`` with ``seed = 1234 + k``
for workload k (1..5); ``torch.randn`` in fp32 in the fixed order Q, K, V, dO;
each tensor then cast (round to nearest even) to the workload dtype on the CPU.
Shapes follow the model card's attention layout (128 query heads over 16 KV
heads, head dimension 64) and the tiny gate program's grouping (H=4, G=2).

The long-context workload (k = 6: the model card's window 65,536 and 2,048
sinks at S = 204,800, B = 2) holds 3.4e9 elements per query-sized tensor, so it
is drawn per slab instead: slab (tensor n, batch b, head h) -- n = 0..3 in the
order Q, K, V, dO -- gets its own generator seeded with
``seed * 1_000_003 + (n * 4096 + b) * 4096 + h`` and ``torch.randn`` of one
[S, D] fp32 slab, cast to the dtype; slabs are independent, so they are drawn
on a thread pool.
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "make_fp8_inputs", "sample_rows", "sample_rows_c4",
           "sample_rows_long", "DecodeWorkload", "DECODE_WORKLOADS", "make_decode_inputs"]


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
    per_slab: bool = False       # draw each [S, D] slab from its own generator (see above)

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
    "long": Workload("long", B=2, H=128, G=16, S=204800, dtype="bf16", window=65536, num_sinks=2048,
                     direction="fwd+bwd", seed=1240, per_slab=True,
                     desc="the model card's long-context setting: window 65,536, 2,048 sinks, S=204,800"),
}


def make_inputs(w: Workload, with_do: bool | None = None, seed: int | None = None):
    """Return CPU tensors (q, k, v, do) in the workload dtype; do is None when
    the direction has no backward and ``with_do`` is not forced."""
    if with_do is None:
        with_do = "bwd" in w.direction
    base = w.seed if seed is None else seed
    if w.per_slab:
        return _make_inputs_per_slab(w, with_do, base)
    gen = torch.Generator(device="cpu")
    gen.manual_seed(base)
    shapes = [(w.B, w.H, w.S, w.D), (w.B, w.G, w.S, w.D), (w.B, w.G, w.S, w.D), (w.B, w.H, w.S, w.D)]
    out = []
    for n, shp in enumerate(shapes):
        if n == 3 and not with_do:
            out.append(None)
            break
        t = torch.randn(shp, generator=gen, dtype=torch.float32)
        out.append(t.to(w.torch_dtype).contiguous())
    return tuple(out)


def make_fp8_inputs(w: Workload, seed: int | None = None):
    """FP8 inputs of a workload: the same fp32 N(0, 1) draws as ``make_inputs`` (Q, K, V),
    each divided by its own scale max|x| / 448 and rounded to OCP e4m3 (nearest even) by
    PyTorch's conversion.  Returns CPU tensors (q8, k8, v8) of torch.float8_e4m3fn and the
    scales (sq, sk, sv): element value = scale * code value."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed if seed is None else seed)
    shapes = [(w.B, w.H, w.S, w.D), (w.B, w.G, w.S, w.D), (w.B, w.G, w.S, w.D)]
    out, scales = [], []
    for shp in shapes:
        t = torch.randn(shp, generator=gen, dtype=torch.float32)
        sc = float(t.abs().max()) / 448.0 if t.numel() else 1.0
        out.append((t / sc).to(torch.float8_e4m3fn).contiguous())
        scales.append(sc)
    return out[0], out[1], out[2], tuple(scales)


def _make_inputs_per_slab(w: Workload, with_do: bool, base: int):
    from concurrent.futures import ThreadPoolExecutor
    heads = [w.H, w.G, w.G, w.H]
    out = [torch.empty((w.B, heads[n], w.S, w.D), dtype=w.torch_dtype) for n in range(4 if with_do else 3)]

    def slab(job):
        n, b, h = job
        gen = torch.Generator(device="cpu")
        gen.manual_seed(base * 1_000_003 + (n * 4096 + b) * 4096 + h)
        out[n][b, h] = torch.randn((w.S, w.D), generator=gen, dtype=torch.float32).to(w.torch_dtype)

    jobs = [(n, b, h) for n in range(len(out)) for b in range(w.B) for h in range(heads[n])]
    with ThreadPoolExecutor(max_workers=16) as ex:
        list(ex.map(slab, jobs))
    if not with_do:
        out.append(None)
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


def sample_rows_long(w: Workload, n: int = 512):
    """Rows checked at the long-context workload: ``n`` seeded random (b, h, i)
    triples plus rows at the sink, window and tile edges and at 2^17 (first and
    last head of two neighbouring kv groups in both batches)."""
    rng = np.random.default_rng(w.seed)
    flat = rng.choice(w.B * w.H * w.S, size=n, replace=False)
    trip = set(zip(*[a.tolist() for a in np.unravel_index(flat, (w.B, w.H, w.S))]))
    W, NS = w.window, w.num_sinks
    forced = [0, 1, 63, 64, NS - 1, NS, W - 1, W, W + NS - 1, W + NS, 131071, 131072, w.S - 64, w.S - 1]
    for b in (0, w.B - 1):
        for h in (0, 7, 8, w.H - 1):
            for i in forced:
                if 0 <= i < w.S:
                    trip.add((b, h, i))
    trip = sorted((int(b), int(h), int(i)) for b, h, i in trip)
    return np.array(trip, dtype=np.int64).reshape(-1, 3)


@dataclass(frozen=True)
class DecodeWorkload:
    """Decode against a key/value cache: Sq query rows per head at the newest positions of
    Skv keys.  Inputs: the same recipe as above (one seeded generator, fp32 normals in the
    order Q [B,H,Sq,D], K [B,G,Skv,D], V [B,G,Skv,D], each cast to the dtype)."""
    name: str
    B: int
    H: int
    G: int
    Sq: int
    Skv: int
    D: int = 64
    dtype: str = "bf16"
    window: int = 0
    num_sinks: int = 0
    seed: int = 0
    desc: str = ""

    @property
    def torch_dtype(self):
        return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[self.dtype]

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))


DECODE_WORKLOADS = {
    # one new token per sequence, four sequences, the card's head layout, window and sinks
    "decode": DecodeWorkload("decode", B=4, H=128, G=16, Sq=1, Skv=131072, window=65536, num_sinks=2048,
                             seed=1241, desc="decode of one token against a 131,072-key cache"),
    # sixteen new tokens (speculative / chunked decode) at the card's longest sequence
    "decode16": DecodeWorkload("decode16", B=1, H=128, G=16, Sq=16, Skv=204800, window=65536,
                               num_sinks=2048, seed=1242, desc="16 query rows against a 204,800-key cache"),
}


def make_decode_inputs(w: DecodeWorkload, seed: int | None = None):
    """CPU tensors (q, k, v) in the workload dtype."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed if seed is None else seed)
    shapes = [(w.B, w.H, w.Sq, w.D), (w.B, w.G, w.Skv, w.D), (w.B, w.G, w.Skv, w.D)]
    return tuple(torch.randn(shp, generator=gen, dtype=torch.float32).to(w.torch_dtype).contiguous()
                 for shp in shapes)
