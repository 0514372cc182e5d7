"""The C-ABI library on the host: it loads, exports every declared entry point,
validates arguments before any HIP call, and its host-side pair count agrees
with the oracle.  No kernel is launched here."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle.attention as ref
import transformer_attention_07_amd as gqa
from transformer_attention_07_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "gqa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = gqa.library()
    declared = _declared_functions()
    assert len(declared) == 19, declared
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(declared) == sorted(binding.EXPORTED)
    assert gqa.abi_version() == 1


def test_header_constants_match_the_binding():
    text = open(os.path.join(ROOT, "include", "gqa.h")).read()
    assert int(re.search(r"#define GQA_ABI_VERSION (\d+)", text).group(1)) == gqa.abi_version()
    shift = int(re.search(r"#define GQA_MAX_SEQ \(1 << (\d+)\)", text).group(1))
    assert binding.GQA_MAX_SEQ == 1 << shift
    shift = int(re.search(r"#define GQA_NOALLOC_MAX_ROWS \(1 << (\d+)\)", text).group(1))
    assert binding.GQA_NOALLOC_MAX_ROWS == 1 << shift
    for name, value in re.findall(r"\b(GQA_(?:OK|ERR_\w+)) = (\d+)", text):
        assert getattr(binding, name) == int(value), name
    for name, value in re.findall(r"\b(GQA_(?:F32|BF16|F16)) = (\d+)", text):
        assert getattr(binding, name) == int(value), name


def test_status_strings():
    for s in range(5):
        assert gqa.status_str(s).startswith("GQA_")
    assert "unknown" in gqa.status_str(99)


FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation first


def _fwd(p, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, o_lo=None):
    return gqa.library().gqa_attn_fwd(ctypes.byref(p), q, k, v, o, o_lo, lse, None)


@pytest.mark.parametrize("kw,status", [
    (dict(H=6, G=4), binding.GQA_ERR_INVALID_ARG),          # H % G != 0
    (dict(G=0), binding.GQA_ERR_INVALID_ARG),
    (dict(H=0), binding.GQA_ERR_INVALID_ARG),
    (dict(B=-1), binding.GQA_ERR_INVALID_ARG),
    (dict(S=-5), binding.GQA_ERR_INVALID_ARG),
    (dict(scale=0.0), binding.GQA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), binding.GQA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), binding.GQA_ERR_INVALID_ARG),
    (dict(window=-1), binding.GQA_ERR_INVALID_ARG),
    (dict(num_sinks=-1), binding.GQA_ERR_INVALID_ARG),
    (dict(causal=0, window=8), binding.GQA_ERR_INVALID_ARG),  # window needs causal
    (dict(causal=0, num_sinks=2), binding.GQA_ERR_INVALID_ARG),
    (dict(causal=2), binding.GQA_ERR_INVALID_ARG),
    (dict(dtype=7), binding.GQA_ERR_INVALID_ARG),
    (dict(D=128), binding.GQA_ERR_UNSUPPORTED),
    (dict(D=32), binding.GQA_ERR_UNSUPPORTED),
    (dict(S=binding.GQA_MAX_SEQ + 1), binding.GQA_ERR_UNSUPPORTED),
    (dict(S=binding.GQA_MAX_SEQ + 1, dtype=binding.GQA_F32), binding.GQA_ERR_UNSUPPORTED),
])
def test_fwd_validation(kw, status):
    args = dict(B=1, H=4, G=2, S=128, D=64, scale=0.125, causal=1, window=0, num_sinks=0, dtype=binding.GQA_BF16)
    args.update(kw)
    p = binding.gqa_problem(**args)
    assert _fwd(p) == status


def test_fwd_pointer_checks():
    p = gqa.make_problem(1, 4, 2, 128)
    assert _fwd(p, q=None) == binding.GQA_ERR_INVALID_ARG
    assert _fwd(p, lse=None) == binding.GQA_ERR_INVALID_ARG
    assert _fwd(p, v=FAKE + 2) == binding.GQA_ERR_INVALID_ARG   # misaligned
    assert _fwd(p, o=FAKE + 8) == binding.GQA_ERR_INVALID_ARG
    assert _fwd(p, o_lo=FAKE + 4) == binding.GQA_ERR_INVALID_ARG
    # the rounding residual only exists for 16-bit outputs
    p32 = gqa.make_problem(1, 4, 2, 128, dtype=binding.GQA_F32)
    assert _fwd(p32, o_lo=FAKE) == binding.GQA_ERR_INVALID_ARG


def test_empty_problem_is_a_noop():
    for B, S in [(0, 128), (2, 0)]:
        p = gqa.make_problem(B, 4, 2, S)
        assert _fwd(p, None, None, None, None, None) == binding.GQA_OK
        assert gqa.library().gqa_attn_bwd_workspace_bytes(ctypes.byref(p)) == 0


def test_bwd_validation_and_workspace():
    lib = gqa.library()
    p = gqa.make_problem(2, 8, 2, 100)
    need = lib.gqa_attn_bwd_workspace_bytes(ctypes.byref(p))
    assert need == ((2 * 8 * 100 * 4 + 255) // 256) * 256
    args = [ctypes.byref(p)] + [FAKE] * 4 + [None] + [FAKE] * 5   # o_lo = NULL
    assert lib.gqa_attn_bwd(*args, None, need, None) == binding.GQA_ERR_WORKSPACE
    assert lib.gqa_attn_bwd(*args, FAKE, need - 1, None) == binding.GQA_ERR_WORKSPACE
    bad = gqa.make_problem(2, 8, 3, 100)
    assert lib.gqa_attn_bwd(ctypes.byref(bad), *([FAKE] * 10), FAKE, need, None) == binding.GQA_ERR_INVALID_ARG
    assert lib.gqa_attn_bwd_dkdv(ctypes.byref(p), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, None) \
        == binding.GQA_ERR_INVALID_ARG
    assert lib.gqa_attn_bwd_dq(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 4, None) \
        == binding.GQA_ERR_INVALID_ARG
    assert lib.gqa_attn_bwd_grads(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None) \
        == binding.GQA_ERR_INVALID_ARG
    assert lib.gqa_attn_bwd_grads(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 8, FAKE, FAKE, None) \
        == binding.GQA_ERR_INVALID_ARG
    assert lib.gqa_attn_bwd_grads(ctypes.byref(bad), *([FAKE] * 9), None) == binding.GQA_ERR_INVALID_ARG
    assert lib.gqa_attn_bwd_preprocess(ctypes.byref(p), FAKE, None, None, FAKE, None) == binding.GQA_ERR_INVALID_ARG
    assert lib.gqa_attn_bwd_preprocess(ctypes.byref(p), FAKE, FAKE + 2, FAKE, FAKE, None) == binding.GQA_ERR_INVALID_ARG
    # sequences beyond the 32-bit in-slab addressing
    long_p = gqa.make_problem(1, 2, 1, binding.GQA_MAX_SEQ + 1)
    assert lib.gqa_attn_bwd_workspace_bytes(ctypes.byref(long_p)) == 0
    assert lib.gqa_attn_bwd(ctypes.byref(long_p), *([FAKE] * 10), FAKE, 1 << 40, None) == binding.GQA_ERR_UNSUPPORTED
    assert lib.gqa_attn_bwd_grads(ctypes.byref(long_p), *([FAKE] * 9), None) == binding.GQA_ERR_UNSUPPORTED


def test_bwd_noalloc_validation():
    # the allocation-free backward: gqa_attn_bwd's checks, and problems whose delta vector
    # does not fit the library's fixed scratch refused with GQA_ERR_WORKSPACE, all before
    # any HIP call
    lib = gqa.library()
    q, k, v, o, olo, lse, do, dq, dk, dv = (FAKE + i * (1 << 34) for i in range(10))
    ok = gqa.make_problem(1, 4, 2, 128)
    assert lib.gqa_attn_bwd_noalloc(ctypes.byref(gqa.make_problem(1, 4, 3, 128)), q, k, v, o, olo, lse, do, dq,
                                    dk, dv, None) == binding.GQA_ERR_INVALID_ARG
    assert lib.gqa_attn_bwd_noalloc(ctypes.byref(ok), q, k, v, o, olo, lse, do, q, dk, dv, None) \
        == binding.GQA_ERR_INVALID_ARG                                    # dQ over Q
    assert lib.gqa_attn_bwd_noalloc(ctypes.byref(ok), q, k, None, o, olo, lse, do, dq, dk, dv, None) \
        == binding.GQA_ERR_INVALID_ARG
    assert lib.gqa_attn_bwd_noalloc(ctypes.byref(gqa.make_problem(0, 4, 2, 128)), *([None] * 10), None) \
        == binding.GQA_OK                                                 # empty: no-op
    rows = binding.GQA_NOALLOC_MAX_ROWS
    fits, over = gqa.make_problem(1, 128, 16, rows // 128), gqa.make_problem(1, 128, 16, rows // 128 + 1)
    assert lib.gqa_attn_bwd_noalloc(ctypes.byref(over), q, k, v, o, olo, lse, do, dq, dk, dv, None) \
        == binding.GQA_ERR_WORKSPACE
    import torch
    if torch.cuda.device_count() == 0:  # valid: fails only at the device lookup (fake pointers)
        assert lib.gqa_attn_bwd_noalloc(ctypes.byref(fits), q, k, v, o, olo, lse, do, dq, dk, dv, None) \
            == binding.GQA_ERR_HIP


def _dec(p, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return gqa.library().gqa_attn_decode(ctypes.byref(p), q, k, v, o, lse, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(H=6, G=4), binding.GQA_ERR_INVALID_ARG),          # H % G != 0
    (dict(G=0), binding.GQA_ERR_INVALID_ARG),
    (dict(B=-1), binding.GQA_ERR_INVALID_ARG),
    (dict(Sq=-1), binding.GQA_ERR_INVALID_ARG),
    (dict(Skv=-1), binding.GQA_ERR_INVALID_ARG),
    (dict(Sq=9, Skv=8), binding.GQA_ERR_INVALID_ARG),      # the rows are positions of the cache
    (dict(scale=0.0), binding.GQA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), binding.GQA_ERR_INVALID_ARG),
    (dict(window=-1), binding.GQA_ERR_INVALID_ARG),
    (dict(num_sinks=-1), binding.GQA_ERR_INVALID_ARG),
    (dict(dtype=7), binding.GQA_ERR_INVALID_ARG),
    (dict(dtype=binding.GQA_F32), binding.GQA_ERR_UNSUPPORTED),
    (dict(D=128), binding.GQA_ERR_UNSUPPORTED),
    (dict(Skv=binding.GQA_MAX_SEQ + 1), binding.GQA_ERR_UNSUPPORTED),
])
def test_decode_validation(kw, status):
    args = dict(B=1, H=8, G=2, Sq=1, Skv=4096, D=64, scale=0.125, window=0, num_sinks=0, dtype=binding.GQA_BF16)
    args.update(kw)
    p = binding.gqa_decode_problem(**args)
    assert _dec(p) == status
    assert gqa.library().gqa_attn_decode_workspace_bytes(ctypes.byref(p)) == 0


def test_decode_pointers_workspace_and_empty():
    lib = gqa.library()
    p = gqa.make_decode_problem(2, 8, 2, 3, 1000, window=256, num_sinks=16)
    need = lib.gqa_attn_decode_workspace_bytes(ctypes.byref(p))
    # one partial state per split and wave: O (128 x 64 fp32) plus maximum and sum (2 x 128)
    per_part = 128 * 64 * 4 + 2 * 128 * 4
    assert need > 0 and need % 256 == 0 and need % per_part == 0
    assert _dec(p, q=None) == binding.GQA_ERR_INVALID_ARG
    assert _dec(p, lse=None) == binding.GQA_ERR_INVALID_ARG
    assert _dec(p, k=FAKE + 2) == binding.GQA_ERR_INVALID_ARG
    assert _dec(p, o=FAKE + 8) == binding.GQA_ERR_INVALID_ARG
    assert _dec(p, ws=FAKE + 4) == binding.GQA_ERR_INVALID_ARG
    assert _dec(p, ws=None, ws_bytes=need) == binding.GQA_ERR_WORKSPACE
    assert _dec(p, ws_bytes=need - 1) == binding.GQA_ERR_WORKSPACE
    for B, Sq in [(0, 1), (2, 0)]:
        e = gqa.make_decode_problem(B, 8, 2, Sq, 100)
        assert _dec(e, None, None, None, None, None, None, 0) == binding.GQA_OK
        assert lib.gqa_attn_decode_workspace_bytes(ctypes.byref(e)) == 0


@pytest.mark.parametrize("S,causal,W,NS", [(1, True, 0, 0), (50, True, 0, 0), (50, False, 0, 0), (50, True, 7, 0),
                                          (50, True, 7, 3), (50, True, 7, 12), (50, True, 60, 5), (50, True, 7, 60),
                                          (33, True, 1, 1), (200, True, 64, 64), (201, True, 65, 63)])
def test_visible_pairs_match_oracle(S, causal, W, NS):
    assert gqa.gqa_visible_pairs(S, causal, W, NS) == ref.visible_pairs_per_head(S, causal, W, NS)


def test_visible_pairs_at_workload_sizes():
    # values at the bench workloads, from the closed form n(n+1)/2 and the window sums
    assert gqa.gqa_visible_pairs(2048) == 2048 * 2049 // 2
    assert gqa.gqa_visible_pairs(16384) == 134225920
    S, W, NS = 65536, 16384, 2048
    by_rows = sum(min(i + 1, W) + min(NS, max(0, i - W + 1)) for i in range(S))
    assert gqa.gqa_visible_pairs(S, True, W, NS) == by_rows == 1038099456


# ---- rotary embedding entry points: validation only (no launch) ----
def _rope_apply(r, x=FAKE, y=FAKE, n=4, S=128, D=64, pos0=0, inverse=0, dtype=binding.GQA_BF16):
    return gqa.library().gqa_rope_apply(None if r is None else ctypes.byref(r), x, y, n, S, D, pos0, inverse, dtype,
                                        None)


@pytest.mark.parametrize("kw,status", [
    (dict(base=1.0), binding.GQA_ERR_INVALID_ARG),
    (dict(base=float("nan")), binding.GQA_ERR_INVALID_ARG),
    (dict(factor=0.5), binding.GQA_ERR_INVALID_ARG),
    (dict(factor=float("inf")), binding.GQA_ERR_INVALID_ARG),
    (dict(mscale=-1.0), binding.GQA_ERR_INVALID_ARG),
    (dict(orig_ctx=0.0), binding.GQA_ERR_INVALID_ARG),
    (dict(alpha=32.0, beta=32.0), binding.GQA_ERR_INVALID_ARG),
    (dict(alpha=float("nan")), binding.GQA_ERR_INVALID_ARG),
])
def test_rope_config_validation(kw, status):
    r = gqa.make_rope(**kw)
    assert _rope_apply(r, x=None) == status      # the configuration is checked first
    p = gqa.make_problem(1, 4, 2, 128)
    lib = gqa.library()
    assert lib.gqa_attn_fwd_rope(ctypes.byref(p), ctypes.byref(r), FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE,
                                 None) == status
    assert lib.gqa_attn_bwd_rope(ctypes.byref(p), ctypes.byref(r), *([FAKE] * 5), None, *([FAKE] * 5), FAKE,
                                 1 << 40, None) == status


def test_rope_plain_factor_ignores_ramp_fields():
    # with factor 1 the ramp is unused, so its fields are not checked (empty call: no launch)
    r = gqa.make_rope(factor=1.0, orig_ctx=0.0, alpha=5.0, beta=1.0)
    assert _rope_apply(r, n=0) == binding.GQA_OK


def test_rope_apply_argument_checks():
    r = gqa.make_rope()
    I = binding.GQA_ERR_INVALID_ARG
    assert _rope_apply(None) == I
    assert _rope_apply(r, dtype=7) == I
    assert _rope_apply(r, n=-1) == I
    assert _rope_apply(r, S=-1) == I
    assert _rope_apply(r, pos0=-1) == I
    assert _rope_apply(r, pos0=2 ** 31 - 100, S=128) == I     # positions past 2^31 - 1
    assert _rope_apply(r, inverse=2) == I
    assert _rope_apply(r, D=128) == binding.GQA_ERR_UNSUPPORTED
    assert _rope_apply(r, x=None) == I
    assert _rope_apply(r, y=FAKE + 8) == I                      # misaligned
    assert _rope_apply(r, y=FAKE + 128) == I                    # partial overlap with x
    for n, S in [(0, 128), (4, 0)]:
        assert _rope_apply(r, x=None, y=None, n=n, S=S) == binding.GQA_OK


def test_fwd_bwd_rope_argument_checks():
    lib = gqa.library()
    r = gqa.make_rope()
    p = gqa.make_problem(1, 4, 2, 128)
    I = binding.GQA_ERR_INVALID_ARG
    kbytes = 1 * 2 * 128 * 64 * 2
    base = dict(q=FAKE, k=FAKE + (1 << 24), v=FAKE + (2 << 24), o=FAKE + (3 << 24), o_lo=None,
                lse=FAKE + (4 << 24), q_rot=None, k_rot=FAKE + (5 << 24))

    def fwd(**kw):
        a = dict(base, **kw)
        return lib.gqa_attn_fwd_rope(ctypes.byref(p), ctypes.byref(r), a["q"], a["k"], a["v"], a["o"], a["o_lo"],
                                     a["lse"], a["q_rot"], a["k_rot"], None)
    assert fwd(k_rot=None) == I
    assert fwd(q_rot=FAKE + 8) == I                              # misaligned
    assert fwd(k_rot=base["k"]) == I                             # k_rot is the input k
    assert fwd(k_rot=base["k"] + kbytes - 16) == I               # k_rot overlaps k
    assert fwd(q_rot=base["k_rot"]) == I                         # q_rot overlaps k_rot
    assert lib.gqa_attn_fwd_rope(ctypes.byref(p), None, *([FAKE] * 4), None, FAKE, None, FAKE, None) == I
    e = gqa.make_problem(0, 4, 2, 128)
    assert lib.gqa_attn_fwd_rope(ctypes.byref(e), ctypes.byref(r), *([None] * 8), None) == binding.GQA_OK
    # backward: the workspace is checked as for gqa_attn_bwd
    need = lib.gqa_attn_bwd_workspace_bytes(ctypes.byref(p))
    args = [ctypes.byref(p), ctypes.byref(r)] + [FAKE] * 4 + [None] + [FAKE] * 5
    assert lib.gqa_attn_bwd_rope(*args, None, need, None) == binding.GQA_ERR_WORKSPACE
    assert lib.gqa_attn_bwd_rope(*args, FAKE, need - 1, None) == binding.GQA_ERR_WORKSPACE
    assert lib.gqa_attn_bwd_rope(ctypes.byref(e), ctypes.byref(r), *([None] * 10), None, 0, None) == binding.GQA_OK


# ---- FP8 forward: validation only (no launch) ----
def test_fp8_forward_argument_checks():
    lib = gqa.library()
    p = gqa.make_problem(1, 4, 2, 128)
    need = lib.gqa_attn_fwd_fp8_workspace_bytes(ctypes.byref(p))
    assert need == ((1 * 2 * 64 * 128 + 255) // 256) * 256
    ragged = gqa.make_problem(2, 8, 2, 100)
    assert lib.gqa_attn_fwd_fp8_workspace_bytes(ctypes.byref(ragged)) == ((2 * 2 * 64 * 128 + 255) // 256) * 256
    ok = binding.gqa_fp8_scales(0.01, 0.02, 0.03)

    def call(p=p, sc=ok, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, ws=FAKE, wsb=1 << 30):
        return lib.gqa_attn_fwd_fp8(ctypes.byref(p), None if sc is None else ctypes.byref(sc), q, k, v, o, lse, ws,
                                    wsb, None)
    I = binding.GQA_ERR_INVALID_ARG
    assert call(sc=None) == I
    assert call(sc=binding.gqa_fp8_scales(0.0, 1.0, 1.0)) == I
    assert call(sc=binding.gqa_fp8_scales(1.0, float("nan"), 1.0)) == I
    assert call(sc=binding.gqa_fp8_scales(1.0, 1.0, -2.0)) == I
    assert call(q=None) == I
    assert call(o=FAKE + 8) == I
    assert call(ws=None, wsb=need) == binding.GQA_ERR_WORKSPACE
    assert call(wsb=need - 1) == binding.GQA_ERR_WORKSPACE
    assert call(p=gqa.make_problem(1, 4, 2, 128, dtype=binding.GQA_F16)) == binding.GQA_ERR_UNSUPPORTED
    assert call(p=gqa.make_problem(1, 4, 2, 128, D=128)) == binding.GQA_ERR_UNSUPPORTED
    assert call(p=gqa.make_problem(1, 4, 2, binding.GQA_MAX_SEQ + 1)) == binding.GQA_ERR_UNSUPPORTED
    assert lib.gqa_attn_fwd_fp8_workspace_bytes(ctypes.byref(gqa.make_problem(1, 4, 2, binding.GQA_MAX_SEQ + 1))) == 0
    e = gqa.make_problem(0, 4, 2, 128)
    assert call(p=e, q=None, k=None, v=None, o=None, lse=None, ws=None, wsb=0) == binding.GQA_OK


def test_clock_probe_argument_checks():
    lib = gqa.library()
    I = binding.GQA_ERR_INVALID_ARG
    assert lib.gqa_clock_probe(None, 256, 100, None) == I
    assert lib.gqa_clock_probe(FAKE + 8, 256, 100, None) == I
    assert lib.gqa_clock_probe(FAKE, 0, 100, None) == I
    assert lib.gqa_clock_probe(FAKE, 256, 0, None) == I
    assert lib.gqa_clock_probe(FAKE, 256, 10 ** 8, None) == I


def test_outputs_overlapping_inputs_or_outputs_are_rejected():
    # distinct, far-apart fake device addresses, all 16-byte aligned: each call below differs
    # from a valid one only in the overlap, and is refused before any HIP call
    lib = gqa.library()
    I = binding.GQA_ERR_INVALID_ARG
    q, k, v, o, olo, lse, do, dq, dk, dv, ws, qr, kr = (FAKE + i * (1 << 32) for i in range(13))
    p = gqa.make_problem(1, 4, 2, 128)     # Q/O bytes 65536, K/V 32768, lse 2048
    P = ctypes.byref(p)
    big = 1 << 40
    # forward: O over K, lse inside Q, o_lo over O
    assert lib.gqa_attn_fwd(P, q, k, v, k, None, lse, None) == I
    assert lib.gqa_attn_fwd(P, q, k, v, o, None, q + 256, None) == I
    assert lib.gqa_attn_fwd(P, q, k, v, o, o + 4096, lse, None) == I
    # backward: dQ over Q, dK over dV, the delta workspace over lse
    assert lib.gqa_attn_bwd(P, q, k, v, o, olo, lse, do, q, dk, dv, ws, big, None) == I
    assert lib.gqa_attn_bwd(P, q, k, v, o, olo, lse, do, dq, dk, dk + 1024, ws, big, None) == I
    assert lib.gqa_attn_bwd(P, q, k, v, o, olo, lse, do, dq, dk, dv, lse, big, None) == I
    assert lib.gqa_attn_bwd_preprocess(P, o, olo, do, o + 512, None) == I
    assert lib.gqa_attn_bwd_dkdv(P, q, k, v, lse, do, ws, k, dv, None) == I
    assert lib.gqa_attn_bwd_dq(P, q, k, v, lse, do, ws, do, None) == I
    assert lib.gqa_attn_bwd_grads(P, q, k, v, lse, do, ws, dq, dk, ws + 16, None) == I
    # RoPE: the stored rotated Q over O, dV over V
    r = ctypes.byref(binding.make_rope())
    assert lib.gqa_attn_fwd_rope(P, r, q, k, v, o, None, lse, o + 64, kr, None) == I
    assert lib.gqa_attn_bwd_rope(P, r, qr, kr, v, o, olo, lse, do, dq, dk, v, ws, big, None) == I
    # FP8 (e4m3 Q8 is 32768 bytes): O inside Q8, the V^T workspace over V8
    sc = ctypes.byref(binding.gqa_fp8_scales(1.0, 1.0, 1.0))
    assert lib.gqa_attn_fwd_fp8(P, sc, q, k, v, q + 16384, lse, ws, big, None) == I
    assert lib.gqa_attn_fwd_fp8(P, sc, q, k, v, o, lse, v, big, None) == I
    # decode: O over K, the workspace over Q
    d = binding.gqa_decode_problem(1, 8, 2, 1, 4096, 64, 0.125, 0, 0, binding.GQA_BF16)
    D = ctypes.byref(d)
    assert lib.gqa_attn_decode(D, q, k, v, k, lse, ws, big, None) == I
    assert lib.gqa_attn_decode(D, q, k, v, o, lse, q, big, None) == I
    # control: with no GPU present, the same calls with distinct buffers pass validation and
    # fail only at the launch (never run where a device exists: the pointers are fake)
    import torch
    if torch.cuda.device_count() == 0:
        H = binding.GQA_ERR_HIP
        assert lib.gqa_attn_fwd(P, q, k, v, o, olo, lse, None) == H
        assert lib.gqa_attn_bwd(P, q, k, v, o, olo, lse, do, dq, dk, dv, ws, big, None) == H
        assert lib.gqa_attn_bwd_preprocess(P, o, olo, do, ws, None) == H
        assert lib.gqa_attn_bwd_dkdv(P, q, k, v, lse, do, ws, dk, dv, None) == H
        assert lib.gqa_attn_bwd_dq(P, q, k, v, lse, do, ws, dq, None) == H
        assert lib.gqa_attn_bwd_grads(P, q, k, v, lse, do, ws, dq, dk, dv, None) == H
        assert lib.gqa_attn_fwd_rope(P, r, q, k, v, o, None, lse, qr, kr, None) == H
        assert lib.gqa_attn_bwd_rope(P, r, qr, kr, v, o, olo, lse, do, dq, dk, dv, ws, big, None) == H
        assert lib.gqa_attn_fwd_fp8(P, sc, q, k, v, o, lse, ws, big, None) == H
        assert lib.gqa_attn_decode(D, q, k, v, o, lse, ws, big, None) == H


def test_header_serves_a_plain_c_caller(tmp_path):
    # include/gqa.h compiled as C99 with warnings as errors, linked against the built library
    import shutil
    import subprocess

    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lib_dir = os.path.join(ROOT, "transformer_attention_07_amd")
    exe = str(tmp_path / "c_abi_check")
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c_abi_check.c"), "-o", exe, "-L", lib_dir, "-lgqa",
                    f"-Wl,-rpath,{lib_dir}"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "status GQA_ERR_INVALID_ARG" in r.stdout
