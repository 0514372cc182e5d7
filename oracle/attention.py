"""CPU fp64 oracle for causal grouped-query attention (forward and backward).

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow definition that the
GPU library is checked against.  Only the test suite, the package's smoke
check and the benchmark's CPU-baseline leg may import it; the product path
never does, and nothing here shares code with the HIP kernels.

What it computes, and where the pages state it:

* Scores ``s_ij = scale * q_i . k_j`` with ``scale = 1/sqrt(d)``, a causal
  mask (query i sees only keys j <= i), a row softmax and ``out = attn . V``
  -- "nx_f32_gqa_gate.nx source" (nishifamily.com), header comment of the
  program (the RUNG 4 description) and its ``out1_0`` / ``softmax2``
  functions, which subtract the row maximum before exponentiating.
* Grouped-query head sharing: H query heads read G < H key/value heads and
  query head ``h`` uses kv head ``h // (H/G)`` -- same page, test T2
  ("GQA GROUPING"), heads {0,1} -> kv0 and {2,3} -> kv1 for H=4, G=2.
* Sliding window and attention sinks -- "SnapKitty Transformer 8B" model card
  (huggingface.co), Model Specifications table (Sliding Window 65,536;
  Attention Sinks 2,048) and the FlashAttention Inference example call
  ``flash_attention_fwd(Q, K, V, causal=True, sliding_window=..., num_sinks=...)``.
  Reading used here (the card gives sizes, not a formula): with window W > 0,
  query i sees key j iff j <= i and (i - W < j or j < num_sinks).  Sinks are
  key positions exempt from the window that still obey causality.
* The saved per-row log-sum-exp and the backward
  ``dS = P * (dO V^T - D)`` -- model card, Protected Inventions list
  (FlashAttention-3 Hopper backward kernel).  Reading used here:
  ``D_i = sum_j P_ij dP_ij`` and the loss is ``L = <O, dO>`` for an upstream
  gradient dO.  dK and dV of a kv head sum over the query heads that share it.

All arithmetic is IEEE fp64 through numpy (matmul, exp, log); inputs are
converted from whatever dtype they arrive in (bf16 and fp32 convert exactly).
Rows are independent in the forward, so ``forward`` may evaluate any subset of
query rows; it evaluates them in chunks only to bound memory, which does not
change any row's arithmetic.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "kv_head",
    "visible",
    "attention_weights",
    "forward",
    "forward_rows",
    "backward",
    "backward_group",
    "visible_pairs_per_head",
]

_ROW_CHUNK = 1024


def _f64(x) -> np.ndarray:
    """Convert a numpy array or a CPU torch tensor (any float dtype) to fp64."""
    if hasattr(x, "detach"):  # torch tensor: go through fp32/fp64 exactly
        import torch

        x = x.detach().to("cpu")
        if x.dtype in (torch.bfloat16, torch.float16):
            x = x.to(torch.float32)
        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def kv_head(h, H: int, G: int):
    """kv head read by query head h: contiguous groups of H/G query heads
    ("nx_f32_gqa_gate.nx source", test T2: kv(qh) = qh / (H/G))."""
    if G <= 0 or H % G != 0:
        raise ValueError(f"H={H} must be a positive multiple of G={G}")
    return np.asarray(h) // (H // G)


def visible(i, j, causal: bool = True, window: int = 0, num_sinks: int = 0):
    """Boolean visibility of key j for query i (broadcasting over arrays).

    causal: j <= i ("nx_f32_gqa_gate.nx source", header: token i attends only
    to j <= i).  window W > 0: additionally i - W < j, unless j is one of the
    first ``num_sinks`` positions (model card, Model Specifications: Sliding
    Window, Attention Sinks).
    """
    i = np.asarray(i)
    j = np.asarray(j)
    vis = np.ones(np.broadcast(i, j).shape, dtype=bool)
    if causal:
        vis &= j <= i
    if window > 0:
        vis &= (j > i - window) | (j < num_sinks)
    return vis


def _scores(q_rows, k, rows, scale, causal, window, num_sinks):
    """Masked scaled scores for the given query rows of one head: -inf where hidden."""
    s = scale * (q_rows @ k.T)
    mask = visible(rows[:, None], np.arange(k.shape[0])[None, :], causal, window, num_sinks)
    return np.where(mask, s, -np.inf)


def _softmax_rows(s):
    """Row softmax with the row maximum subtracted first ("softmax2" on the
    nx page); also returns the natural-log log-sum-exp of each row."""
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return e / l, (m + np.log(l))[:, 0]


def attention_weights(q, k, scale=None, causal=True, window=0, num_sinks=0):
    """Full attention-probability tensor P [B, H, S, S] (small inputs only)."""
    q, k = _f64(q), _f64(k)
    B, H, S, D = q.shape
    G = k.shape[1]
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    rows = np.arange(S)
    P = np.zeros((B, H, S, S))
    for b in range(B):
        for h in range(H):
            g = int(kv_head(h, H, G))
            P[b, h], _ = _softmax_rows(_scores(q[b, h], k[b, g], rows, scale, causal, window, num_sinks))
    return P


def forward_rows(q, k, v, b: int, h: int, rows, scale=None, causal=True, window=0, num_sinks=0):
    """Output rows O[b, h, rows, :] and lse[b, h, rows] of one query head.

    q [B,H,S,D], k/v [B,G,S,D].  ``rows`` is an int array of query positions.
    """
    B, H, S, D = q.shape
    G = k.shape[1]
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    g = int(kv_head(h, H, G))
    rows = np.asarray(rows, dtype=np.int64)
    kk, vv = _f64(k[b, g]), _f64(v[b, g])
    out = np.empty((rows.size, D))
    lse = np.empty(rows.size)
    for c0 in range(0, rows.size, _ROW_CHUNK):
        r = rows[c0:c0 + _ROW_CHUNK]
        p, lse[c0:c0 + r.size] = _softmax_rows(
            _scores(_f64(q[b, h, r]), kk, r, scale, causal, window, num_sinks))
        out[c0:c0 + r.size] = p @ vv
    return out, lse


def forward(q, k, v, scale=None, causal=True, window=0, num_sinks=0):
    """O [B,H,S,D] and lse [B,H,S] (natural log of the scaled scores), fp64."""
    B, H, S, D = q.shape
    out = np.empty((B, H, S, D))
    lse = np.empty((B, H, S))
    rows = np.arange(S)
    for b in range(B):
        for h in range(H):
            out[b, h], lse[b, h] = forward_rows(q, k, v, b, h, rows, scale, causal, window, num_sinks)
    return out, lse


def backward_group(q, k, v, do, b: int, g: int, scale=None, causal=True, window=0, num_sinks=0):
    """Gradients of L = <O, dO> for kv head g of batch b.

    Returns dq [H/G, S, D] for the query heads of the group (in head order),
    and dk, dv [S, D] for kv head g, all fp64.
    """
    B, H, S, D = q.shape
    G = k.shape[1]
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    hpg = H // G
    kk, vv = _f64(k[b, g]), _f64(v[b, g])
    rows = np.arange(S)
    dq = np.zeros((hpg, S, D))
    dk = np.zeros((S, D))
    dv = np.zeros((S, D))
    for t in range(hpg):
        h = g * hpg + t
        assert int(kv_head(h, H, G)) == g
        qh, doh = _f64(q[b, h]), _f64(do[b, h])
        P, _ = _softmax_rows(_scores(qh, kk, rows, scale, causal, window, num_sinks))
        dv += P.T @ doh                       # O = P V
        dP = doh @ vv.T                       # dL/dP
        Dr = (P * dP).sum(axis=1, keepdims=True)
        dS = P * (dP - Dr)                    # softmax backward
        dq[t] = scale * (dS @ kk)             # s = scale q.k
        dk += scale * (dS.T @ qh)
    return dq, dk, dv


def backward_rows(q, k, v, do, b: int, h: int, rows, scale=None, causal=True, window=0, num_sinks=0):
    """dQ[b, h, rows, :] of L = <O, dO>, fp64.

    The same formulas as ``backward_group`` for the given query rows only: a
    row's dQ needs nothing but its own row of P and dP.
    """
    B, H, S, D = q.shape
    G = k.shape[1]
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    g = int(kv_head(h, H, G))
    rows = np.asarray(rows, dtype=np.int64)
    kk, vv = _f64(k[b, g]), _f64(v[b, g])
    dq = np.empty((rows.size, D))
    for c0 in range(0, rows.size, _ROW_CHUNK):
        r = rows[c0:c0 + _ROW_CHUNK]
        P, _ = _softmax_rows(_scores(_f64(q[b, h, r]), kk, r, scale, causal, window, num_sinks))
        dP = _f64(do[b, h, r]) @ vv.T
        Dr = (P * dP).sum(axis=1, keepdims=True)
        dq[c0:c0 + r.size] = scale * ((P * (dP - Dr)) @ kk)
    return dq


def backward_keys(q, k, v, do, b: int, g: int, keys, scale=None, causal=True, window=0, num_sinks=0):
    """dK[b, g, keys, :] and dV[b, g, keys, :] of L = <O, dO>, fp64.

    The same formulas as ``backward_group``, evaluated on the query rows (of
    every head of the group) that see at least one of the given keys; each of
    those rows is taken in full, since its P needs all of its visible keys.
    """
    B, H, S, D = q.shape
    G = k.shape[1]
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    hpg = H // G
    keys = np.asarray(keys, dtype=np.int64)
    kk, vv = _f64(k[b, g]), _f64(v[b, g])
    sees = visible(np.arange(S)[:, None], keys[None, :], causal, window, num_sinks).any(axis=1)
    rows = np.nonzero(sees)[0]
    dk = np.zeros((keys.size, D))
    dv = np.zeros((keys.size, D))
    for t in range(hpg):
        h = g * hpg + t
        for c0 in range(0, rows.size, _ROW_CHUNK):
            r = rows[c0:c0 + _ROW_CHUNK]
            qh, doh = _f64(q[b, h, r]), _f64(do[b, h, r])
            P, _ = _softmax_rows(_scores(qh, kk, r, scale, causal, window, num_sinks))
            dP = doh @ vv.T
            Dr = (P * dP).sum(axis=1, keepdims=True)
            dS = P * (dP - Dr)
            dv += P[:, keys].T @ doh
            dk += scale * (dS[:, keys].T @ qh)
    return dk, dv


def backward(q, k, v, do, scale=None, causal=True, window=0, num_sinks=0):
    """dQ [B,H,S,D], dK [B,G,S,D], dV [B,G,S,D] of L = <O, dO>, fp64."""
    B, H, S, D = q.shape
    G = k.shape[1]
    hpg = H // G
    dq = np.zeros((B, H, S, D))
    dk = np.zeros((B, G, S, D))
    dv = np.zeros((B, G, S, D))
    for b in range(B):
        for g in range(G):
            dq[b, g * hpg:(g + 1) * hpg], dk[b, g], dv[b, g] = backward_group(
                q, k, v, do, b, g, scale, causal, window, num_sinks)
    return dq, dk, dv


def decode(q, k, v, scale=None, window=0, num_sinks=0):
    """Decode against a key/value cache: q [B,H,Sq,D] holds the newest Sq positions
    Skv - Sq .. Skv - 1 of a sequence whose keys and values are k, v [B,G,Skv,D]
    (the cache).  The same causal, windowed, sink-keeping attention as ``forward``
    for those rows; returns O [B,H,Sq,D] and lse [B,H,Sq], fp64.  (The model card's
    inference call over a cache: FlashAttention Inference and Text Generation
    examples, KV Cache column of the Memory Usage table.)
    """
    B, H, Sq, D = q.shape
    G, Skv = k.shape[1], k.shape[2]
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    positions = np.arange(Skv - Sq, Skv, dtype=np.int64)
    out = np.empty((B, H, Sq, D))
    lse = np.empty((B, H, Sq))
    for b in range(B):
        for h in range(H):
            g = int(kv_head(h, H, G))
            kk, vv = _f64(k[b, g]), _f64(v[b, g])
            P, lse[b, h] = _softmax_rows(_scores(_f64(q[b, h]), kk, positions, scale, True, window, num_sinks))
            out[b, h] = P @ vv
    return out, lse


def visible_pairs_per_head(S: int, causal=True, window=0, num_sinks=0) -> int:
    """Number of visible (i, j) pairs of one head, counted row by row."""
    total = 0
    j = np.arange(S)
    for i in range(S):
        total += int(visible(i, j, causal, window, num_sinks).sum())
    return total
