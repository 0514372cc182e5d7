"""Pins for the rotary-embedding oracle (``oracle.rope``): each check takes an
implementation module exposing ``rope``, ``rope_frequencies``, ``yarn_frequencies``,
``yarn_mscale``, ``forward``, ``forward_rows``, ``backward``, ``backward_group``,
``backward_rows``, ``backward_keys``, ``decode`` and the configurations ``YARN`` / ``PLAIN``, and raises
AssertionError when it disagrees with what the published methods or the mathematics fix.
tests/test_oracle_mutants.py plants mistakes in copies of the oracle to show the checks
catch them.

Expected values come from: powers of ten that the base 10000 gives for D = 64; the
complex-number form of the rotation (numpy's complex exponential); the frequency regions
of YaRN's ramp worked out by hand below; exact identities (rotation at position 0,
norms, relative positions, the inverse); PyTorch's attention routine and autograd; and
central differences.
"""

from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F

from tests.oracle_checks import _range_mask, _rand, _rng

D64 = 64


def check_plain_frequencies(impl):
    # base 10000, D = 64: theta_i = 10^(-i/8); every 8th pair is a power of ten
    th = impl.rope_frequencies(D64, 10000.0)
    assert th.shape == (32,)
    for i, want in [(0, 1.0), (8, 0.1), (16, 0.01), (24, 0.001)]:
        assert abs(th[i] - want) <= 1e-15 * max(want, 1e-300) * 8, (i, th[i])
    ratio = th[1:] / th[:-1]
    assert np.allclose(ratio, 10.0 ** (-1.0 / 8.0), rtol=1e-13, atol=0)
    # D = 4: pairs (0, 1) and (2, 3) at 1 and 1/100
    assert np.allclose(impl.rope_frequencies(4, 10000.0), [1.0, 0.01], rtol=1e-15, atol=0)
    # a factor of 1 leaves the plain frequencies
    assert np.array_equal(impl.yarn_frequencies(D64, impl.PLAIN), th)


def check_complex_form(impl):
    # pair i as z = x_{2i} + 1j x_{2i+1}: the rotation is z * exp(1j p theta_i), times m
    rng = _rng(40)
    for cfg in (impl.PLAIN, impl.YARN):
        for S, D in [(7, 4), (33, 64), (5, 64)]:
            x = _rand(rng, 2, S, D)
            pos = rng.integers(0, 204800, size=S)
            th = impl.yarn_frequencies(D, cfg)
            z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * pos[:, None] * th[None, :])
            want = np.empty_like(x)
            want[..., 0::2], want[..., 1::2] = z.real, z.imag
            want *= impl.yarn_mscale(cfg)
            got = impl.rope(x, pos, cfg=cfg)
            assert np.allclose(got, want, rtol=0, atol=1e-9), (cfg, S, D, np.abs(got - want).max())
            zi = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(-1j * pos[:, None] * th[None, :])
            wi = np.empty_like(x)
            wi[..., 0::2], wi[..., 1::2] = zi.real, zi.imag
            wi *= impl.yarn_mscale(cfg)
            assert np.allclose(impl.rope(x, pos, inverse=True, cfg=cfg), wi, rtol=0, atol=1e-9)


def check_mscale_and_identities(impl):
    # YaRN's temperature for s = 32: 0.1 ln 32 + 1 = 1 + 0.5 ln 2
    assert abs(impl.yarn_mscale(impl.YARN) - (1.0 + 0.5 * math.log(2.0))) < 1e-15
    assert impl.yarn_mscale(impl.PLAIN) == 1.0
    m = 1.0 + 0.5 * math.log(2.0)
    rng = _rng(41)
    x = _rand(rng, 3, 9, D64)
    # position 0 is no rotation
    assert np.allclose(impl.rope(x, np.zeros(9, dtype=np.int64)), m * x, rtol=0, atol=1e-14)
    assert np.allclose(impl.rope(x, np.zeros(9, dtype=np.int64), cfg=impl.PLAIN), x, rtol=0, atol=0)
    pos = np.array([0, 1, 2, 100, 6399, 6400, 65535, 131072, 204799])
    y = impl.rope(x, pos)
    # every pair keeps its length, times m
    n_in = np.hypot(x[..., 0::2], x[..., 1::2])
    n_out = np.hypot(y[..., 0::2], y[..., 1::2])
    assert np.allclose(n_out, m * n_in, rtol=1e-13, atol=0)
    # the inverse undoes the rotation: m^2 x
    assert np.allclose(impl.rope(y, pos, inverse=True), m * m * x, rtol=0, atol=1e-12)
    # R(p)^T = R(-p)
    assert np.allclose(impl.rope(x, pos, inverse=True), impl.rope(x, -pos), rtol=0, atol=1e-12)


def check_relative_position(impl):
    # <R(a) q, R(b) k> depends on a - b only: shifting both positions changes nothing, and
    # at a == b it is m^2 <q, k>
    rng = _rng(42)
    m2 = impl.yarn_mscale(impl.YARN) ** 2
    q, k = _rand(rng, 1, D64), _rand(rng, 1, D64)
    for a, b in [(0, 0), (5, 2), (6400, 17), (204799, 204000), (3, 90000)]:
        base = float((impl.rope(q, [a]) * impl.rope(k, [b])).sum())
        for t in (1, 777, 100000):
            shifted = float((impl.rope(q, [a + t]) * impl.rope(k, [b + t])).sum())
            assert abs(shifted - base) < 1e-9, (a, b, t)
        if a == b:
            assert abs(base - m2 * float((q * k).sum())) < 1e-11
    # but not on a + b: swapping the two positions changes the score in general
    s1 = float((impl.rope(q, [10]) * impl.rope(k, [3])).sum())
    s2 = float((impl.rope(q, [3]) * impl.rope(k, [10])).sum())
    assert abs(s1 - s2) > 1e-3


def check_yarn_regions(impl):
    # D = 64, base 10000, L = 6400, alpha = 1, beta = 32: pair i turns
    # r_i = 6400 * 10^(-i/8) / (2 pi) times over the original context:
    #   r_12 = 32.2 > beta  (pairs 0..12 keep theta_i),
    #   r_13 = 24.2 and r_24 = 1.019 lie inside the ramp,
    #   r_25 = 0.764 < alpha (pairs 25..31 are interpolated: theta_i / 32).
    th = impl.rope_frequencies(D64, 10000.0)
    ty = impl.yarn_frequencies(D64, impl.YARN)
    ratio = ty / th
    assert np.allclose(ratio[:13], 1.0, rtol=0, atol=1e-15)
    assert np.allclose(ratio[25:], 1.0 / 32.0, rtol=1e-15, atol=0)
    mid = ratio[13:25]
    assert (mid < 1.0).all() and (mid > 1.0 / 32.0).all() and (np.diff(mid) < 0).all()
    # at pair 24 the ramp is just above its start: gamma = (r_24 - 1) / 31, where
    # r_24 = 6400 / (2000 pi) = 1.0185916357881302
    gamma24 = (6400.0 / (2000.0 * math.pi) - 1.0) / 31.0
    assert abs(ratio[24] - (1.0 / 32.0 + gamma24 * (31.0 / 32.0))) < 1e-15
    # position interpolation: a slow pair at position 32 p turns as the plain pair at p;
    # a fast pair is the plain rotation at the same position (both times m)
    rng = _rng(43)
    x = _rand(rng, 4, D64)
    m = impl.yarn_mscale(impl.YARN)
    p = np.array([1, 200, 6399, 6400])
    y_slow = impl.rope(x, 32 * p)
    y_plain = impl.rope(x, p, cfg=impl.PLAIN)
    assert np.allclose(y_slow[:, 50:], m * y_plain[:, 50:], rtol=0, atol=1e-12)
    y_fast = impl.rope(x, 32 * p)
    y_plain_fast = impl.rope(x, 32 * p, cfg=impl.PLAIN)
    assert np.allclose(y_fast[:, :26], m * y_plain_fast[:, :26], rtol=0, atol=1e-9)


def _torch_rotate(x, pos, freqs, m):
    """m * rotation through PyTorch's complex numbers (view_as_complex, polar)."""
    xt = torch.as_tensor(x, dtype=torch.float64)
    S, D = xt.shape[-2], xt.shape[-1]
    zc = torch.view_as_complex(xt.reshape(*xt.shape[:-1], D // 2, 2).contiguous())
    ang = torch.as_tensor(np.asarray(pos, dtype=np.float64))[:, None] * torch.as_tensor(freqs)[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)
    return m * torch.view_as_real(zc * rot).reshape(xt.shape)


ROPE_TORCH_CASES = [(1, 4, 2, 9, 4, True, 0, 0), (2, 8, 2, 33, 8, True, 0, 0), (1, 4, 2, 40, 64, True, 7, 3),
                    (1, 6, 3, 21, 6, False, 0, 0)]


def check_attention_vs_torch(impl):
    # attention over q and k rotated with PyTorch's complex arithmetic (frequencies from
    # the pinned yarn_frequencies), through PyTorch's attention and autograd
    rng = _rng(44)
    for cfg in (impl.YARN, impl.PLAIN):
        for (B, H, G, S, D, causal, W, NS) in ROPE_TORCH_CASES:
            qn, kn, vn, don = (_rand(rng, B, H, S, D), _rand(rng, B, G, S, D), _rand(rng, B, G, S, D),
                               _rand(rng, B, H, S, D))
            q, k, v = (torch.tensor(x, requires_grad=True) for x in (qn, kn, vn))
            fr, m = impl.yarn_frequencies(D, cfg), impl.yarn_mscale(cfg)
            pos = np.arange(S)
            qr, kr = _torch_rotate(q, pos, fr, m), _torch_rotate(k, pos, fr, m)
            mask = _range_mask(S, causal, W, NS)
            scale = 1.0 / math.sqrt(D)
            o = F.scaled_dot_product_attention(qr, kr, v, attn_mask=mask, scale=scale, enable_gqa=(H != G))
            (o * torch.tensor(don)).sum().backward()
            sc = scale * (qr.detach() @ kr.detach().repeat_interleave(H // G, dim=1).transpose(-1, -2))
            lse_t = torch.logsumexp(sc.masked_fill(~mask, float("-inf")), dim=-1)
            kw = dict(scale=scale, causal=causal, window=W, num_sinks=NS, cfg=cfg)
            O, lse = impl.forward(qn, kn, vn, **kw)
            dq, dk, dv = impl.backward(qn, kn, vn, don, **kw)
            tag = (cfg.factor, B, H, G, S, D, causal, W, NS)
            assert np.allclose(O, o.detach().numpy(), rtol=0, atol=1e-10), tag
            assert np.allclose(lse, lse_t.numpy(), rtol=0, atol=1e-10), tag
            assert np.allclose(dq, q.grad.numpy(), rtol=0, atol=1e-9), tag
            assert np.allclose(dk, k.grad.numpy(), rtol=0, atol=1e-9), tag
            assert np.allclose(dv, v.grad.numpy(), rtol=0, atol=1e-9), tag


def check_rope_fd_gradients(impl):
    # central differences of L = <O, dO> through the rotation
    rng = _rng(45)
    h = 1e-5
    for (B, H, G, S, D, W, NS) in [(1, 2, 1, 5, 4, 0, 0), (1, 4, 2, 6, 4, 3, 1)]:
        q, k, v, do = (_rand(rng, B, H, S, D), _rand(rng, B, G, S, D), _rand(rng, B, G, S, D),
                       _rand(rng, B, H, S, D))
        kw = dict(causal=True, window=W, num_sinks=NS)

        def loss(qx, kx, vx):
            return float((impl.forward(qx, kx, vx, **kw)[0] * do).sum())

        grads = impl.backward(q, k, v, do, **kw)
        for which, (x, gx) in enumerate(zip((q, k, v), grads)):
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p, args_m = [q, k, v], [q, k, v]
                args_p[which], args_m[which] = xp, xm
                fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            err = np.abs(fd - gx).max()
            assert err < 1e-7, ((B, H, G, S, D, W, NS), "qkv"[which], err)


def check_rows_keys_and_decode(impl):
    # the row-, key- and decode-restricted entry points against the full forward/backward
    rng = _rng(46)
    B, H, G, S, D, W, NS = 2, 4, 2, 37, 64, 9, 3
    q, k, v, do = (_rand(rng, B, H, S, D), _rand(rng, B, G, S, D), _rand(rng, B, G, S, D),
                   _rand(rng, B, H, S, D))
    kw = dict(causal=True, window=W, num_sinks=NS)
    O, lse = impl.forward(q, k, v, **kw)
    dq, dk, dv = impl.backward(q, k, v, do, **kw)
    rows = np.array([0, 1, 8, 9, 20, 36])
    keys = np.array([0, 2, 3, 17, 35, 36])
    for b in range(B):
        for h in range(H):
            Or, lr = impl.forward_rows(q, k, v, b, h, rows, **kw)
            assert np.allclose(Or, O[b, h, rows], rtol=0, atol=1e-12)
            assert np.allclose(lr, lse[b, h, rows], rtol=0, atol=1e-12)
            assert np.allclose(impl.backward_rows(q, k, v, do, b, h, rows, **kw), dq[b, h, rows], rtol=0,
                               atol=1e-11)
        for g in range(G):
            dkr, dvr = impl.backward_keys(q, k, v, do, b, g, keys, **kw)
            assert np.allclose(dkr, dk[b, g, keys], rtol=0, atol=1e-11)
            assert np.allclose(dvr, dv[b, g, keys], rtol=0, atol=1e-11)
            dqg, dkg, dvg = impl.backward_group(q, k, v, do, b, g, **kw)
            hpg = H // G
            assert np.allclose(dqg, dq[b, g * hpg:(g + 1) * hpg], rtol=0, atol=1e-11)
            assert np.allclose(dkg, dk[b, g], rtol=0, atol=1e-11) and np.allclose(dvg, dv[b, g], rtol=0, atol=1e-11)
    # decode of the newest Sq rows is the forward's last Sq rows
    for Sq in (1, 4, S):
        Od, ld = impl.decode(q[:, :, S - Sq:], k, v, window=W, num_sinks=NS)
        assert np.allclose(Od, O[:, :, S - Sq:], rtol=0, atol=1e-12), Sq
        assert np.allclose(ld, lse[:, :, S - Sq:], rtol=0, atol=1e-12), Sq


def _bf16_nearest_even(x):
    """fp64 -> fp32 -> bf16, each to nearest even, by integer arithmetic on the fp32 bits
    (finite values), back in fp64."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def check_stored_operands(impl):
    # with operand_dtype = bf16 the attention runs over the bf16 roundings of the rotated
    # q and k (and nothing else is rounded): against PyTorch's attention over operands
    # rounded by the integer rule above
    rng = _rng(47)
    B, H, G, S, D, W, NS = 1, 4, 2, 40, 64, 9, 3
    qn, kn, vn, don = (_rand(rng, B, H, S, D), _rand(rng, B, G, S, D), _rand(rng, B, G, S, D),
                       _rand(rng, B, H, S, D))
    pos = np.arange(S)
    qr = torch.tensor(_bf16_nearest_even(impl.rope(qn, pos)), requires_grad=True)
    kr = torch.tensor(_bf16_nearest_even(impl.rope(kn, pos)), requires_grad=True)
    v = torch.tensor(vn)
    mask = _range_mask(S, True, W, NS)
    o = F.scaled_dot_product_attention(qr, kr, v, attn_mask=mask, scale=1.0 / 8.0, enable_gqa=True)
    (o * torch.tensor(don)).sum().backward()
    kw = dict(window=W, num_sinks=NS, operand_dtype=torch.bfloat16)
    O, _ = impl.forward(qn, kn, vn, **kw)
    dq, dk, _ = impl.backward(qn, kn, vn, don, **kw)
    assert np.allclose(O, o.detach().numpy(), rtol=0, atol=1e-11)
    # the gradients with respect to the rounded rotated operands, rotated back
    assert np.allclose(dq, impl.rope(qr.grad.numpy(), pos, inverse=True), rtol=0, atol=1e-10)
    assert np.allclose(dk, impl.rope(kr.grad.numpy(), pos, inverse=True), rtol=0, atol=1e-10)
    # and the rounding matters: the exact rotation gives a different O
    O_exact, _ = impl.forward(qn, kn, vn, window=W, num_sinks=NS)
    assert np.abs(O_exact - O).max() > 1e-4


ALL_ROPE_CHECKS = [check_plain_frequencies, check_complex_form, check_mscale_and_identities,
                   check_relative_position, check_yarn_regions, check_attention_vs_torch,
                   check_rope_fd_gradients, check_rows_keys_and_decode, check_stored_operands]
