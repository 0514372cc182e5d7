"""Pins for the CPU oracle: each check takes an implementation module exposing
``forward``, ``forward_rows``, ``backward``, ``attention_weights`` and raises
AssertionError when the implementation disagrees with what the pages or the
mathematics fix.  The same checks run against deliberately broken copies of
the oracle (tests/test_oracle_mutants.py) to show they catch such mistakes.

Nothing here re-types the oracle's formula: expected values come from the
worked example's closed form, from closed forms with K = 0, from exact
identities of the gradient, from finite differences, or from PyTorch's own
CPU attention routine and autograd.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# --------------------------------------------------------------------------
# 1. The gate program's worked example ("nx_f32_gqa_gate.nx source", main).
# --------------------------------------------------------------------------
def check_worked_example(impl):
    with open(os.path.join(GOLDEN, "p5_worked_example.json")) as f:
        ex = json.load(f)
    Q = np.array(ex["Q"])[None, None]
    K = np.array(ex["K"])[None, None]
    V = np.array(ex["V"])[None, None]
    scale = 1.0 / math.sqrt(ex["d"])
    O, lse = impl.forward(Q, K, V, scale=scale, causal=True)

    # Closed form: s00 = Q0.K0/sqrt2 = a, s10 = Q1.K0/sqrt2 = 0, s11 = a.
    a = 1.0 / math.sqrt(2.0)
    p10 = 1.0 / (1.0 + math.exp(a))
    p11 = math.exp(a) / (1.0 + math.exp(a))
    V0, V1 = ex["V"]
    O_exp = np.array([V0, [p10 * V0[0] + p11 * V1[0], p10 * V0[1] + p11 * V1[1]]])
    lse_exp = np.array([a, math.log(1.0 + math.exp(a))])
    assert np.allclose(O[0, 0], O_exp, rtol=0, atol=1e-12), (O[0, 0], O_exp)
    assert np.allclose(lse[0, 0], lse_exp, rtol=0, atol=1e-12), (lse[0, 0], lse_exp)
    assert abs(p10 - 0.330238450673343) < 1e-12  # value quoted in the design notes

    # Backward of L = out[1][0]: dO one-hot at (1, 0).
    dO = np.zeros_like(Q)
    dO[0, 0, 1, 0] = 1.0
    dq, dk, dv = impl.backward(Q, K, V, dO, scale=scale, causal=True)
    g = np.array([V0[0], V1[0]])              # dL/dattn[1][j] = V[j][0]
    dot = p10 * g[0] + p11 * g[1]
    ds = np.array([p10 * (g[0] - dot), p11 * (g[1] - dot)])
    dv_exp = np.array([[p10, 0.0], [p11, 0.0]])
    dq_exp = np.array([[0.0, 0.0], [scale * ds[0], scale * ds[1]]])   # K = I
    dk_exp = np.array([[0.0, scale * ds[0]], [0.0, scale * ds[1]]])   # Q1 = e1
    assert np.allclose(dv[0, 0], dv_exp, rtol=0, atol=1e-12), dv[0, 0]
    assert np.allclose(dq[0, 0], dq_exp, rtol=0, atol=1e-12), dq[0, 0]
    assert np.allclose(dk[0, 0], dk_exp, rtol=0, atol=1e-12), dk[0, 0]

    # The page's own gradchecks T3 (dL/dV[0][0]) and T4 (dL/dQ[1][0]):
    # central differences with its step h and tolerance.
    h, tol = ex["gradcheck_step_h"], ex["gradcheck_tol"]

    def out10(Qx, Vx):
        return impl.forward(Qx, K, Vx, scale=scale, causal=True)[0][0, 0, 1, 0]

    Vp, Vm = V.copy(), V.copy()
    Vp[0, 0, 0, 0] += h
    Vm[0, 0, 0, 0] -= h
    assert abs((out10(Q, Vp) - out10(Q, Vm)) / (2 * h) - dv[0, 0, 0, 0]) <= tol
    Qp, Qm = Q.copy(), Q.copy()
    Qp[0, 0, 1, 0] += h
    Qm[0, 0, 1, 0] -= h
    assert abs((out10(Qp, V) - out10(Qm, V)) / (2 * h) - dq[0, 0, 1, 0]) <= tol


# --------------------------------------------------------------------------
# 2. T0 / T1 / T2 of the gate program, computed rather than asserted.
# --------------------------------------------------------------------------
def check_rows_sum_to_one(impl):
    rng = _rng(11)
    for (B, H, G, S, D, causal, W, NS) in [(1, 4, 2, 9, 4, True, 0, 0), (2, 2, 1, 13, 3, True, 4, 2),
                                           (1, 2, 2, 6, 2, False, 0, 0)]:
        q, k = _rand(rng, B, H, S, D), _rand(rng, B, G, S, D)
        P = impl.attention_weights(q, k, causal=causal, window=W, num_sinks=NS)
        assert np.allclose(P.sum(-1), 1.0, rtol=0, atol=1e-12)
        assert (P >= 0).all()
        if causal:  # nothing above the diagonal: no future leakage
            assert np.all(np.triu(P, k=1) == 0.0)


def check_token0(impl):
    rng = _rng(12)
    for (B, H, G, S, D, W, NS) in [(2, 4, 2, 8, 5, 0, 0), (1, 6, 3, 10, 4, 3, 2), (1, 4, 1, 5, 2, 1, 0)]:
        q, k, v = _rand(rng, B, H, S, D), _rand(rng, B, G, S, D), _rand(rng, B, G, S, D)
        scale = 1.0 / math.sqrt(D)
        O, lse = impl.forward(q, k, v, scale=scale, causal=True, window=W, num_sinks=NS)
        for b in range(B):
            for h in range(H):
                g = h // (H // G)
                assert np.array_equal(O[b, h, 0], v[b, g, 0]), (b, h)
                assert abs(lse[b, h, 0] - scale * float(q[b, h, 0] @ k[b, g, 0])) < 1e-12


def check_gqa_grouping(impl):
    # H=4, G=2: heads {0,1} read kv0 and {2,3} read kv1 (test T2).  With V_g
    # constant (g+1) every output row of a head equals its kv head's constant.
    rng = _rng(13)
    B, H, G, S, D = 1, 4, 2, 7, 3
    q, k = _rand(rng, B, H, S, D), _rand(rng, B, G, S, D)
    v = np.empty((B, G, S, D))
    for g in range(G):
        v[:, g] = g + 1.0
    O, _ = impl.forward(q, k, v, causal=True)
    for h, want in zip(range(H), [1.0, 1.0, 2.0, 2.0]):
        assert np.allclose(O[0, h], want, rtol=0, atol=1e-12), (h, O[0, h, :, 0])
    # and the dV routing: gradient of kv g is fed only by heads of group g
    do = np.zeros((B, H, S, D))
    do[0, 1] = 1.0  # only head 1 (group 0) has an upstream gradient
    _, dk, dv = impl.backward(q, k, v, do, causal=True)
    assert np.abs(dv[0, 1]).max() == 0.0 and np.abs(dk[0, 1]).max() == 0.0
    assert np.allclose(dv[0, 0].sum(0), S, rtol=0, atol=1e-12)


def check_attention_weights(impl):
    """The probability tensor itself: the worked example's attention row in closed form;
    kv head 1 with K = 0 gives heads {2, 3} uniform rows 1/|vis(i)| over the visible set
    (written as index ranges) while heads {0, 1}, which read kv head 0 with random K, do
    not; and P V equals the forward's output for every head (T2's grouping, through P)."""
    with open(os.path.join(GOLDEN, "p5_worked_example.json")) as f:
        ex = json.load(f)
    a = 1.0 / math.sqrt(2.0)
    P = impl.attention_weights(np.array(ex["Q"])[None, None], np.array(ex["K"])[None, None],
                               scale=1.0 / math.sqrt(ex["d"]), causal=True)
    p10 = 1.0 / (1.0 + math.exp(a))
    assert np.allclose(P[0, 0], [[1.0, 0.0], [p10, 1.0 - p10]], rtol=0, atol=1e-12), P[0, 0]
    rng = _rng(16)
    for S, W, NS in [(37, 0, 0), (37, 5, 3), (70, 17, 5), (40, 1, 2)]:
        B, H, G, D = 1, 4, 2, 3
        q, v = _rand(rng, B, H, S, D), _rand(rng, B, G, S, D)
        k = _rand(rng, B, G, S, D) * 3.0
        k[:, 1] = 0.0
        P = impl.attention_weights(q, k, causal=True, window=W, num_sinks=NS)
        for i in range(S):
            want = np.zeros(S)
            rs = visible_ranges(i, W, NS)
            n = sum(hi - lo for lo, hi in rs)
            for lo, hi in rs:
                want[lo:hi] = 1.0 / n
            for h in (2, 3):
                assert np.allclose(P[0, h, i], want, rtol=0, atol=1e-12), (S, W, NS, h, i)
        for h in (0, 1):  # random keys: some row with several visible keys is far from uniform
            assert max(float(np.ptp(P[0, h, i][P[0, h, i] > 0])) for i in range(S)) > 0.05, (S, W, NS, h)
        O, _ = impl.forward(q, k, v, causal=True, window=W, num_sinks=NS)
        for h in range(H):
            assert np.allclose(P[0, h] @ v[0, h // 2], O[0, h], rtol=0, atol=1e-12), (S, W, NS, h)


# --------------------------------------------------------------------------
# 3. Mask semantics from the K = 0 closed form: uniform attention over the
#    visible set, so lse_i = ln |vis(i)| and O_i = mean of the visible V rows.
#    The visible set is written here as explicit index ranges.
# --------------------------------------------------------------------------
def visible_ranges(i: int, W: int, NS: int):
    """Causal visible keys of query i as half-open ranges [lo, hi)."""
    if W <= 0 or W >= i + 1:
        return [(0, i + 1)]
    lo = i - W + 1
    out = [(lo, i + 1)]
    if NS > 0:
        out.append((0, min(NS, lo)))
    return out


K0_CASES = [(1, 0, 0), (37, 0, 0), (37, 5, 0), (37, 5, 3), (37, 5, 9), (37, 1, 0), (37, 1, 2),
            (37, 37, 2), (37, 50, 4), (64, 16, 16), (70, 17, 5), (70, 17, 40)]


def check_k_zero_closed_form(impl):
    rng = _rng(14)
    for S, W, NS in K0_CASES:
        B, H, G, D = 1, 4, 2, 3
        q, v = _rand(rng, B, H, S, D), _rand(rng, B, G, S, D)
        k = np.zeros((B, G, S, D))
        O, lse = impl.forward(q, k, v, causal=True, window=W, num_sinks=NS)
        for g in range(G):
            csum = np.concatenate([np.zeros((1, D)), np.cumsum(v[0, g], axis=0)])
            for i in range(S):
                rs = visible_ranges(i, W, NS)
                n = sum(hi - lo for lo, hi in rs)
                mean = sum(csum[hi] - csum[lo] for lo, hi in rs) / n
                for h in range(g * (H // G), (g + 1) * (H // G)):
                    assert abs(lse[0, h, i] - math.log(n)) < 1e-12, (S, W, NS, i, lse[0, h, i], n)
                    assert np.allclose(O[0, h, i], mean, rtol=0, atol=1e-12), (S, W, NS, i)


def check_special_cases(impl):
    rng = _rng(15)
    B, H, G, S, D = 2, 4, 2, 19, 4
    q, k, v = _rand(rng, B, H, S, D), _rand(rng, B, G, S, D), _rand(rng, B, G, S, D)
    # W = 1 without sinks: each query sees only itself, so O_i = V_i exactly.
    O, _ = impl.forward(q, k, v, causal=True, window=1)
    for h in range(H):
        assert np.array_equal(O[:, h], v[:, h // (H // G)])
    # W >= S is no window at all.
    Oa, la = impl.forward(q, k, v, causal=True, window=S)
    Ob, lb = impl.forward(q, k, v, causal=True, window=0)
    assert np.allclose(Oa, Ob, rtol=0, atol=1e-13) and np.allclose(la, lb, rtol=0, atol=1e-13)
    # Sinks without a window change nothing.
    Oc, lc = impl.forward(q, k, v, causal=True, window=0, num_sinks=5)
    assert np.allclose(Oc, Ob, rtol=0, atol=1e-13) and np.allclose(lc, lb, rtol=0, atol=1e-13)
    # Linearity in V; lse does not depend on V.
    Od, ld = impl.forward(q, k, 2.5 * v, causal=True, window=6, num_sinks=2)
    Oe, le = impl.forward(q, k, v, causal=True, window=6, num_sinks=2)
    assert np.allclose(Od, 2.5 * Oe, rtol=0, atol=1e-12) and np.allclose(ld, le, rtol=0, atol=1e-13)
    # A row subset gives the same rows as the full evaluation.
    rows = np.array([0, 3, 7, 18])
    Or, lr = impl.forward_rows(q, k, v, 1, 3, rows, causal=True, window=6, num_sinks=2)
    assert np.allclose(Or, Oe[1, 3, rows], rtol=0, atol=1e-13) and np.allclose(lr, le[1, 3, rows], rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# 4. PyTorch's CPU attention (fp64) and autograd as an independent library.
# --------------------------------------------------------------------------
def _range_mask(S, causal, W, NS):
    m = torch.zeros(S, S, dtype=torch.bool)
    for i in range(S):
        if not causal:
            m[i, :] = True
            continue
        for lo, hi in visible_ranges(i, W, NS):
            m[i, lo:hi] = True
    return m


TORCH_CASES = [(1, 4, 2, 9, 4, True, 0, 0), (2, 8, 2, 33, 8, True, 0, 0), (1, 4, 2, 40, 5, True, 7, 3),
               (1, 6, 3, 21, 6, True, 4, 6), (2, 4, 4, 17, 3, False, 0, 0), (1, 2, 1, 64, 16, True, 16, 4)]


def check_torch_sdpa(impl):
    rng = _rng(16)
    for (B, H, G, S, D, causal, W, NS) in TORCH_CASES:
        qn, kn, vn, don = (_rand(rng, B, H, S, D), _rand(rng, B, G, S, D), _rand(rng, B, G, S, D),
                           _rand(rng, B, H, S, D))
        q, k, v = (torch.tensor(x, requires_grad=True) for x in (qn, kn, vn))
        mask = _range_mask(S, causal, W, NS)
        scale = 1.0 / math.sqrt(D)
        o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale, enable_gqa=(H != G))
        (o * torch.tensor(don)).sum().backward()
        kr = k.detach().repeat_interleave(H // G, dim=1)
        sc = scale * (q.detach() @ kr.transpose(-1, -2))
        lse_t = torch.logsumexp(sc.masked_fill(~mask, float("-inf")), dim=-1)

        O, lse = impl.forward(qn, kn, vn, scale=scale, causal=causal, window=W, num_sinks=NS)
        dq, dk, dv = impl.backward(qn, kn, vn, don, scale=scale, causal=causal, window=W, num_sinks=NS)
        tag = (B, H, G, S, D, causal, W, NS)
        assert np.allclose(O, o.detach().numpy(), rtol=0, atol=1e-11), tag
        assert np.allclose(lse, lse_t.numpy(), rtol=0, atol=1e-11), tag
        assert np.allclose(dq, q.grad.numpy(), rtol=0, atol=1e-10), tag
        assert np.allclose(dk, k.grad.numpy(), rtol=0, atol=1e-10), tag
        assert np.allclose(dv, v.grad.numpy(), rtol=0, atol=1e-10), tag


def check_sampled_backward_vs_torch(impl):
    """dQ of chosen query rows and dK/dV of chosen keys (the row/key-restricted
    oracle entry points used on the largest shapes) against autograd through
    PyTorch's attention, on the same small cases."""
    rng = _rng(19)
    for (B, H, G, S, D, causal, W, NS) in TORCH_CASES:
        qn, kn, vn, don = (_rand(rng, B, H, S, D), _rand(rng, B, G, S, D), _rand(rng, B, G, S, D),
                           _rand(rng, B, H, S, D))
        q, k, v = (torch.tensor(x, requires_grad=True) for x in (qn, kn, vn))
        mask = _range_mask(S, causal, W, NS)
        scale = 1.0 / math.sqrt(D)
        o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale, enable_gqa=(H != G))
        (o * torch.tensor(don)).sum().backward()
        kw = dict(scale=scale, causal=causal, window=W, num_sinks=NS)
        tag = (B, H, G, S, D, causal, W, NS)
        b = B - 1
        rows = np.array(sorted({0, S // 2, S - 1, min(3, S - 1)}))
        keys = np.array(sorted({0, 1, S // 3, S - 2, S - 1}))
        for h in range(H):
            dq = impl.backward_rows(qn, kn, vn, don, b, h, rows, **kw)
            assert np.allclose(dq, q.grad[b, h, rows].numpy(), rtol=0, atol=1e-10), (tag, h)
        for g in range(G):
            dk, dv = impl.backward_keys(qn, kn, vn, don, b, g, keys, **kw)
            assert np.allclose(dk, k.grad[b, g, keys].numpy(), rtol=0, atol=1e-10), (tag, g)
            assert np.allclose(dv, v.grad[b, g, keys].numpy(), rtol=0, atol=1e-10), (tag, g)


# --------------------------------------------------------------------------
# 4b. Decode against a cache: the newest Sq positions of a sequence of Skv keys.
# --------------------------------------------------------------------------
DECODE_CASES = [(1, 4, 2, 1, 1, 4, 0, 0), (2, 4, 2, 1, 37, 5, 0, 0), (1, 8, 2, 3, 40, 6, 7, 3),
                (1, 6, 3, 5, 21, 4, 4, 6), (2, 4, 4, 2, 17, 3, 0, 0), (1, 2, 1, 16, 64, 8, 16, 4),
                (1, 4, 1, 9, 9, 3, 0, 0)]


def check_decode_vs_torch(impl):
    rng = _rng(20)
    for (B, H, G, Sq, Skv, D, W, NS) in DECODE_CASES:
        q, k, v = _rand(rng, B, H, Sq, D), _rand(rng, B, G, Skv, D), _rand(rng, B, G, Skv, D)
        mask = _range_mask(Skv, True, W, NS)[Skv - Sq:]  # rows of the newest Sq positions
        scale = 1.0 / math.sqrt(D)
        qt, kt, vt = (torch.tensor(x) for x in (q, k, v))
        o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale, enable_gqa=(H != G))
        sc = scale * (qt @ kt.repeat_interleave(H // G, dim=1).transpose(-1, -2))
        lse_t = torch.logsumexp(sc.masked_fill(~mask, float("-inf")), dim=-1)
        O, lse = impl.decode(q, k, v, scale=scale, window=W, num_sinks=NS)
        tag = (B, H, G, Sq, Skv, D, W, NS)
        assert np.allclose(O, o.numpy(), rtol=0, atol=1e-11), tag
        assert np.allclose(lse, lse_t.numpy(), rtol=0, atol=1e-11), tag


def check_decode_k_zero_closed_form(impl):
    # K = 0: every visible key has score 0, so each row is the plain mean of the V rows it
    # sees and lse = ln(number of them); row t sits at position Skv - Sq + t
    rng = _rng(21)
    for Skv, W, NS in K0_CASES:
        for Sq in sorted({1, min(4, Skv), Skv}):
            B, H, G, D = 1, 4, 2, 3
            q, v = _rand(rng, B, H, Sq, D), _rand(rng, B, G, Skv, D)
            k = np.zeros((B, G, Skv, D))
            O, lse = impl.decode(q, k, v, window=W, num_sinks=NS)
            for g in range(G):
                csum = np.concatenate([np.zeros((1, D)), np.cumsum(v[0, g], axis=0)])
                for t in range(Sq):
                    rs = visible_ranges(Skv - Sq + t, W, NS)
                    n = sum(hi - lo for lo, hi in rs)
                    mean = sum(csum[hi] - csum[lo] for lo, hi in rs) / n
                    for h in range(g * (H // G), (g + 1) * (H // G)):
                        assert abs(lse[0, h, t] - math.log(n)) < 1e-12, (Skv, W, NS, Sq, t)
                        assert np.allclose(O[0, h, t], mean, rtol=0, atol=1e-12), (Skv, W, NS, Sq, t)


# --------------------------------------------------------------------------
# 5. Gradients: central differences of L = <O, dO>, and exact identities.
# --------------------------------------------------------------------------
FD_CASES = [(1, 4, 2, 6, 3, True, 0, 0), (1, 4, 2, 7, 3, True, 3, 2), (2, 2, 1, 5, 2, False, 0, 0),
            (1, 3, 3, 6, 2, True, 2, 0)]


def check_fd_gradients(impl):
    rng = _rng(17)
    h = 1e-5
    for (B, H, G, S, D, causal, W, NS) in FD_CASES:
        q, k, v, do = (_rand(rng, B, H, S, D), _rand(rng, B, G, S, D), _rand(rng, B, G, S, D),
                       _rand(rng, B, H, S, D))
        kw = dict(causal=causal, window=W, num_sinks=NS)

        def loss(qx, kx, vx):
            return float((impl.forward(qx, kx, vx, **kw)[0] * do).sum())

        grads = impl.backward(q, k, v, do, **kw)
        for which, (x, gx) in enumerate(zip((q, k, v), grads)):
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = [q, k, v]
                args_m = [q, k, v]
                args_p[which], args_m[which] = xp, xm
                fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            err = np.abs(fd - gx).max()
            assert err < 1e-7, ((B, H, G, S, D, causal, W, NS), "qkv"[which], err)


def check_grad_identities(impl):
    rng = _rng(18)
    for (B, H, G, S, D, W, NS) in [(2, 8, 2, 30, 4, 0, 0), (1, 4, 1, 45, 5, 9, 4), (1, 6, 3, 20, 3, 2, 1)]:
        q, k, v, do = (_rand(rng, B, H, S, D), _rand(rng, B, G, S, D), _rand(rng, B, G, S, D),
                       _rand(rng, B, H, S, D))
        dq, dk, dv = impl.backward(q, k, v, do, causal=True, window=W, num_sinks=NS)
        hpg = H // G
        for b in range(B):
            for g in range(G):
                # scores of a row are shift invariant, so dK sums to zero over keys
                assert np.allclose(dk[b, g].sum(0), 0.0, rtol=0, atol=1e-12)
                # rows of P sum to one, so dV sums to the group's summed dO
                want = do[b, g * hpg:(g + 1) * hpg].sum(axis=(0, 1))
                assert np.allclose(dv[b, g].sum(0), want, rtol=0, atol=1e-11)
        # dV is linear in dO
        _, _, dv2 = impl.backward(q, k, v, 3.0 * do, causal=True, window=W, num_sinks=NS)
        assert np.allclose(dv2, 3.0 * dv, rtol=0, atol=1e-12)


ALL_CHECKS = [check_worked_example, check_rows_sum_to_one, check_token0, check_gqa_grouping, check_attention_weights,
              check_k_zero_closed_form, check_special_cases, check_torch_sdpa, check_fd_gradients,
              check_grad_identities, check_sampled_backward_vs_torch, check_decode_vs_torch,
              check_decode_k_zero_closed_form]
