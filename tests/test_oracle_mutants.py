"""Each plausible mistake planted in a copy of the oracle must fail a pin.

The mistakes are planted on the CPU by patching the oracle module's helpers
for the duration of one test; the oracle's source is not changed.
"""

import numpy as np
import pytest

import oracle.attention as ref
from tests import oracle_checks as oc


def _mut_kv_interleaved(h, H, G):
    return np.asarray(h) % G


def _mut_causal_strict(i, j, causal=True, window=0, num_sinks=0):
    i, j = np.asarray(i), np.asarray(j)
    vis = np.ones(np.broadcast(i, j).shape, dtype=bool)
    if causal:
        vis &= j < i
    if window > 0:
        vis &= (j > i - window) | (j < num_sinks)
    return vis


def _mut_window_wide(i, j, causal=True, window=0, num_sinks=0):
    i, j = np.asarray(i), np.asarray(j)
    vis = np.ones(np.broadcast(i, j).shape, dtype=bool)
    if causal:
        vis &= j <= i
    if window > 0:
        vis &= (j >= i - window) | (j < num_sinks)
    return vis


def _mut_sinks_acausal(i, j, causal=True, window=0, num_sinks=0):
    i, j = np.asarray(i), np.asarray(j)
    vis = np.ones(np.broadcast(i, j).shape, dtype=bool)
    if causal:
        vis &= j <= i
    if window > 0:
        vis &= j > i - window
    return vis | (j < num_sinks)


def _mut_sinks_inclusive(i, j, causal=True, window=0, num_sinks=0):
    i, j = np.asarray(i), np.asarray(j)
    vis = np.ones(np.broadcast(i, j).shape, dtype=bool)
    if causal:
        vis &= j <= i
    if window > 0:
        vis &= (j > i - window) | (j <= num_sinks)
    return vis


def _mut_no_scale(q_rows, k, rows, scale, causal, window, num_sinks):
    s = q_rows @ k.T
    mask = ref.visible(rows[:, None], np.arange(k.shape[0])[None, :], causal, window, num_sinks)
    return np.where(mask, s, -np.inf)


def _mut_transposed_scores(q_rows, k, rows, scale, causal, window, num_sinks):
    # scores taken against the key rows in reverse order (an index slip)
    s = scale * (q_rows @ k[::-1].T)
    mask = ref.visible(rows[:, None], np.arange(k.shape[0])[None, :], causal, window, num_sinks)
    return np.where(mask, s, -np.inf)


def _mut_lse_base2(s):
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return e / l, ((m + np.log(l)) / np.log(2.0))[:, 0]


def _mut_lse_no_max(s):
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return e / l, np.log(l)[:, 0]


def _make_bwd_mutant(kind):
    def backward_group(q, k, v, do, b, g, scale=None, causal=True, window=0, num_sinks=0):
        B, H, S, D = q.shape
        G = k.shape[1]
        scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
        hpg = H // G
        kk, vv = ref._f64(k[b, g]), ref._f64(v[b, g])
        rows = np.arange(S)
        dq = np.zeros((hpg, S, D))
        dk = np.zeros((S, D))
        dv = np.zeros((S, D))
        for t in range(hpg):
            h = g * hpg + t
            qh, doh = ref._f64(q[b, h]), ref._f64(do[b, h])
            P, _ = ref._softmax_rows(ref._scores(qh, kk, rows, scale, causal, window, num_sinks))
            dv += (P @ doh) if kind == "dv_no_transpose" else (P.T @ doh)
            dP = doh @ vv.T
            if kind == "D_rowsum_dP":
                Dr = dP.sum(axis=1, keepdims=True)
            else:
                Dr = (P * dP).sum(axis=1, keepdims=True)
            dS = P * dP if kind == "no_D" else P * (dP - Dr)
            if kind == "dS_sign":
                dS = -dS
            dq[t] = (dS @ kk) if kind == "dq_no_scale" else scale * (dS @ kk)
            if kind == "dq_transposed":
                dq[t] = scale * (dS.T @ kk)
            dk += (dS.T @ qh) if kind == "dk_no_scale" else scale * (dS.T @ qh)
            if kind == "dk_last_head_only":
                dk = scale * (dS.T @ qh)
        return dq, dk, dv
    return backward_group


def _make_weights_mutant(kind):
    # attention_weights with its own index slip: heads interleaved over the kv heads, or the
    # scale left out
    def attention_weights(q, k, scale=None, causal=True, window=0, num_sinks=0):
        q, k = ref._f64(q), ref._f64(k)
        B, H, S, D = q.shape
        G = k.shape[1]
        scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
        rows = np.arange(S)
        P = np.zeros((B, H, S, S))
        for b in range(B):
            for h in range(H):
                g = h % G if kind == "interleaved" else h // (H // G)
                sc = 1.0 if kind == "no_scale" else scale
                P[b, h], _ = ref._softmax_rows(ref._scores(q[b, h], k[b, g], rows, sc, causal, window, num_sinks))
        return P
    return attention_weights


MUTANTS = {
    "kv_head_interleaved": ("kv_head", _mut_kv_interleaved),
    "causal_strict": ("visible", _mut_causal_strict),
    "window_one_wider": ("visible", _mut_window_wide),
    "sinks_ignore_causality": ("visible", _mut_sinks_acausal),
    "sinks_one_more": ("visible", _mut_sinks_inclusive),
    "scale_dropped": ("_scores", _mut_no_scale),
    "keys_reversed": ("_scores", _mut_transposed_scores),
    "lse_base2": ("_softmax_rows", _mut_lse_base2),
    "lse_without_max": ("_softmax_rows", _mut_lse_no_max),
}
MUTANTS["weights_kv_interleaved"] = ("attention_weights", _make_weights_mutant("interleaved"))
MUTANTS["weights_scale_dropped"] = ("attention_weights", _make_weights_mutant("no_scale"))
for _kind in ["dv_no_transpose", "D_rowsum_dP", "no_D", "dS_sign", "dq_no_scale", "dq_transposed",
              "dk_no_scale", "dk_last_head_only"]:
    MUTANTS["bwd_" + _kind] = ("backward_group", _make_bwd_mutant(_kind))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(ref, attr, fn)
    failed = []
    with np.errstate(all="ignore"):
        for check in oc.ALL_CHECKS:
            try:
                check(ref)
            except (AssertionError, ValueError, FloatingPointError, IndexError):
                failed.append(check.__name__)
    assert failed, f"no pin caught mutant {name}"
