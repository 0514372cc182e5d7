"""CPU fp64 oracle for YaRN-scaled rotary position embedding (RoPE) on the queries and
keys of causal grouped-query attention, and for that attention's forward and backward
with the rotation in front of it.

TEST INFRASTRUCTURE ONLY, like ``oracle.attention``: only the test suite, the package's
smoke check and the benchmark's CPU-baseline leg may import it; the product path never
does, and nothing here shares code with the HIP kernels.

What the pages state: the "SnapKitty Transformer 8B" model card lists YaRN RoPE with a
32x factor (Model Specifications table), ``rope_yarn: true`` and
``rope_yarn_factor: 32.0`` with ``head_dim: 64`` and ``max_seq_len: 204800`` (Training
Configuration), and, in its Protected Inventions list, YaRN-scaled RoPE for
204800-length sequences inside the attention kernels and the FlashAttention-3 forward.
The card gives no formula.  This module follows the published methods it names, with
these readings (each is a choice where the card is silent):

* Rotary embedding (Su et al., "RoFormer"): the pair of dimensions (2i, 2i+1),
  i = 0 .. D/2 - 1, of the vector at position p is rotated by the angle p * theta_i,
  theta_i = base^(-2i/D), base = 10000 (that paper's value).  Written as complex
  numbers z_i = x_{2i} + 1j x_{2i+1}, the rotation is z_i * exp(1j p theta_i).
* YaRN (Peng et al., "YaRN: Efficient Context Window Extension of Large Language
  Models"), "NTK-by-parts" frequencies: scale s = 32, original context
  L = 204800 / 32 = 6400, r_i = L theta_i / (2 pi) rotations of dimension pair i over
  L, ramp gamma_i = clip((r_i - alpha) / (beta - alpha), 0, 1) with alpha = 1,
  beta = 32 (that paper's values), theta'_i = (1 - gamma_i) theta_i / s + gamma_i theta_i:
  fast pairs keep their frequency, slow ones are interpolated by 1/s.  The paper's
  attention temperature sqrt(1/t) = 0.1 ln(s) + 1 multiplies each rotated q and k.
* Positions: in the forward and backward, query and key i sit at position i (the
  same sequence); in decode, query row t sits at Skv - Sq + t.
* The backward of y = m R(p) x is dx = m R(p)^T dy, so dQ and dK are the attention
  gradients with respect to the rotated Q and K, rotated back.
* ``operand_dtype``: the library's interface stores the rotated q and k in the input
  element type (its rotated-key output is what a key/value cache holds), so for 16-bit
  inputs the attention runs over those roundings.  With ``operand_dtype`` set (a torch
  dtype) the oracle rounds its fp64 rotation the same way -- to fp32, then to that type,
  each to nearest even, by PyTorch's conversions -- before the attention; with None it
  uses the exact rotation.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from oracle import attention as attn


@dataclass(frozen=True)
class YarnConfig:
    base: float = 10000.0
    factor: float = 32.0
    orig_ctx: float = 6400.0
    alpha: float = 1.0
    beta: float = 32.0
    mscale: float | None = None   # None: YaRN's 0.1 ln(s) + 1 (1 for s == 1)


YARN = YarnConfig()
PLAIN = YarnConfig(factor=1.0)


def rope_frequencies(D: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/D), i = 0 .. D/2 - 1 (radians per position)."""
    return base ** (-2.0 * np.arange(D // 2, dtype=np.float64) / D)


def yarn_frequencies(D: int, cfg: YarnConfig = YARN) -> np.ndarray:
    """YaRN's per-pair frequencies theta'_i (radians per position), fp64."""
    theta = rope_frequencies(D, cfg.base)
    if cfg.factor == 1.0:
        return theta
    r = cfg.orig_ctx * theta / (2.0 * np.pi)
    gamma = np.clip((r - cfg.alpha) / (cfg.beta - cfg.alpha), 0.0, 1.0)
    return (1.0 - gamma) * theta / cfg.factor + gamma * theta


def yarn_mscale(cfg: YarnConfig = YARN) -> float:
    """Factor applied to each rotated vector (YaRN's attention temperature)."""
    if cfg.mscale is not None:
        return float(cfg.mscale)
    return 1.0 if cfg.factor <= 1.0 else 0.1 * float(np.log(cfg.factor)) + 1.0


def _rotate_pairs(x, ang):
    """Rotate each pair (x[..., 2i], x[..., 2i+1]) by ang[..., i] (counter-clockwise)."""
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = x0 * c - x1 * s
    y[..., 1::2] = x0 * s + x1 * c
    return y


def rope(x, positions, inverse: bool = False, cfg: YarnConfig = YARN) -> np.ndarray:
    """m R(p) x (or m R(p)^T x with ``inverse``) on the last axis of x [..., S, D];
    ``positions`` holds the S positions, fp64."""
    x = attn._f64(x)
    D = x.shape[-1]
    ang = np.asarray(positions, dtype=np.float64)[:, None] * yarn_frequencies(D, cfg)[None, :]
    return yarn_mscale(cfg) * _rotate_pairs(x, -ang if inverse else ang)


def _stored(x, operand_dtype):
    """x as the library stores a rotated operand: unchanged for None, else rounded to fp32
    and then to ``operand_dtype`` (nearest even, PyTorch's conversions), back in fp64."""
    if operand_dtype is None:
        return x
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32).to(operand_dtype)
    return t.to(torch.float64).numpy()


def _rot(x, positions, cfg, operand_dtype):
    return _stored(rope(x, positions, cfg=cfg), operand_dtype)


def _rot_qk(q, k, cfg, operand_dtype=None):
    S = q.shape[2]
    pos = np.arange(S)
    return _rot(q, pos, cfg, operand_dtype), _rot(k, pos, cfg, operand_dtype)


def forward(q, k, v, scale=None, causal=True, window=0, num_sinks=0, cfg: YarnConfig = YARN,
            operand_dtype=None):
    """O [B,H,S,D] and lse [B,H,S] of attention over the rotated q and k, fp64."""
    qr, kr = _rot_qk(q, k, cfg, operand_dtype)
    return attn.forward(qr, kr, v, scale, causal, window, num_sinks)


def forward_rows(q, k, v, b: int, h: int, rows, scale=None, causal=True, window=0, num_sinks=0,
                 cfg: YarnConfig = YARN, operand_dtype=None):
    """O[b, h, rows, :] and lse[b, h, rows] with the rotation: the rows of q are rotated
    at their positions and the whole key slab of their kv head at 0 .. S-1."""
    B, H, S, D = q.shape
    g = int(attn.kv_head(h, H, k.shape[1]))
    rows = np.asarray(rows, dtype=np.int64)
    qr = np.zeros((1, 1, S, D))
    qr[0, 0, rows] = _rot(attn._f64(q[b, h, rows]), rows, cfg, operand_dtype)
    kr = _rot(attn._f64(k[b, g]), np.arange(S), cfg, operand_dtype)[None, None]
    return attn.forward_rows(qr, kr, attn._f64(v[b, g])[None, None], 0, 0, rows, scale, causal, window,
                             num_sinks)


def backward(q, k, v, do, scale=None, causal=True, window=0, num_sinks=0, cfg: YarnConfig = YARN,
             operand_dtype=None):
    """dQ, dK, dV of L = <O, dO> through the rotation, fp64: the attention gradients with
    respect to the rotated q and k, rotated back with m R^T."""
    S = q.shape[2]
    qr, kr = _rot_qk(q, k, cfg, operand_dtype)
    dqr, dkr, dv = attn.backward(qr, kr, v, do, scale, causal, window, num_sinks)
    pos = np.arange(S)
    return rope(dqr, pos, inverse=True, cfg=cfg), rope(dkr, pos, inverse=True, cfg=cfg), dv


def _group_rotated(q, k, b, g, cfg, operand_dtype=None):
    """Rotated q slabs of the heads of kv group g and the rotated k slab, as [1,hpg,S,D]
    and [1,1,S,D] arrays (kv head 0 of a one-group problem)."""
    B, H, S, D = q.shape
    hpg = H // k.shape[1]
    pos = np.arange(S)
    qr = _rot(attn._f64(q[b, g * hpg:(g + 1) * hpg]), pos, cfg, operand_dtype)[None]
    kr = _rot(attn._f64(k[b, g]), pos, cfg, operand_dtype)[None, None]
    return qr, kr


def backward_group(q, k, v, do, b: int, g: int, scale=None, causal=True, window=0, num_sinks=0,
                   cfg: YarnConfig = YARN, operand_dtype=None):
    """dQ [H/G, S, D] of the heads of kv group g (in head order) and dK, dV [S, D] of that
    kv head, through the rotation, fp64."""
    B, H, S, D = q.shape
    hpg = H // k.shape[1]
    qr, kr = _group_rotated(q, k, b, g, cfg, operand_dtype)
    dqr, dkr, dv = attn.backward_group(qr, kr, attn._f64(v[b, g])[None, None],
                                       attn._f64(do[b, g * hpg:(g + 1) * hpg])[None], 0, 0, scale, causal,
                                       window, num_sinks)
    pos = np.arange(S)
    return rope(dqr, pos, inverse=True, cfg=cfg), rope(dkr, pos, inverse=True, cfg=cfg), dv


def backward_rows(q, k, v, do, b: int, h: int, rows, scale=None, causal=True, window=0, num_sinks=0,
                  cfg: YarnConfig = YARN, operand_dtype=None):
    """dQ[b, h, rows, :] through the rotation, fp64."""
    B, H, S, D = q.shape
    G = k.shape[1]
    g = int(attn.kv_head(h, H, G))
    rows = np.asarray(rows, dtype=np.int64)
    qr = _rot(attn._f64(q[b, h]), np.arange(S), cfg, operand_dtype)[None, None]
    kr = _rot(attn._f64(k[b, g]), np.arange(S), cfg, operand_dtype)[None, None]
    dqr = attn.backward_rows(qr, kr, attn._f64(v[b, g])[None, None], attn._f64(do[b, h])[None, None], 0, 0,
                             rows, scale, causal, window, num_sinks)
    return rope(dqr, rows, inverse=True, cfg=cfg)


def backward_keys(q, k, v, do, b: int, g: int, keys, scale=None, causal=True, window=0, num_sinks=0,
                  cfg: YarnConfig = YARN, operand_dtype=None):
    """dK[b, g, keys, :] and dV[b, g, keys, :] through the rotation, fp64."""
    B, H, S, D = q.shape
    hpg = H // k.shape[1]
    keys = np.asarray(keys, dtype=np.int64)
    qr, kr = _group_rotated(q, k, b, g, cfg, operand_dtype)
    dkr, dv = attn.backward_keys(qr, kr, attn._f64(v[b, g])[None, None],
                                 attn._f64(do[b, g * hpg:(g + 1) * hpg])[None], 0, 0, keys, scale, causal,
                                 window, num_sinks)
    return rope(dkr, keys, inverse=True, cfg=cfg), dv


def decode(q, k, v, scale=None, window=0, num_sinks=0, cfg: YarnConfig = YARN, operand_dtype=None):
    """Decode through the rotation: query row t at position Skv - Sq + t, cache key j at
    position j (the cache holds unrotated keys here; rotating them is part of the
    computation checked)."""
    Sq, Skv = q.shape[2], k.shape[2]
    qr = _rot(q, np.arange(Skv - Sq, Skv), cfg, operand_dtype)
    kr = _rot(k, np.arange(Skv), cfg, operand_dtype)
    return attn.decode(qr, kr, v, scale, window, num_sinks)
