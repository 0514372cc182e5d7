"""The rotary-embedding oracle against its pins, and planted mistakes against the pins
(no GPU).  Mistakes are planted on the CPU by patching the oracle module's helpers for
one test; the oracle's source is not changed."""

import numpy as np
import pytest

import oracle.rope as rr
from tests import rope_checks as rc


@pytest.mark.parametrize("check", rc.ALL_ROPE_CHECKS, ids=lambda c: c.__name__)
def test_rope_oracle_pin(check):
    check(rr)


_orig_rotate = rr._rotate_pairs
_orig_freq = rr.yarn_frequencies
_orig_mscale = rr.yarn_mscale
_orig_rope = rr.rope
_orig_rope_freq = rr.rope_frequencies


def _mut_clockwise(x, ang):
    return _orig_rotate(x, -ang)


def _mut_half_split_pairs(x, ang):
    # pairs (i, i + D/2) instead of (2i, 2i + 1)
    D = x.shape[-1]
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., :D // 2], x[..., D // 2:]
    return np.concatenate([x0 * c - x1 * s, x0 * s + x1 * c], axis=-1)


def _mut_swapped_in_pair(x, ang):
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 1::2] = x0 * c - x1 * s
    y[..., 0::2] = x0 * s + x1 * c
    return y


def _mut_freq_exponent(D, base):
    return base ** (-np.arange(D // 2, dtype=np.float64) / D)


def _mut_ramp_reversed(D, cfg=rr.YARN):
    theta = rr.rope_frequencies(D, cfg.base)
    if cfg.factor == 1.0:
        return theta
    r = cfg.orig_ctx * theta / (2.0 * np.pi)
    gamma = np.clip((r - cfg.alpha) / (cfg.beta - cfg.alpha), 0.0, 1.0)
    return gamma * theta / cfg.factor + (1.0 - gamma) * theta


def _mut_no_interpolation(D, cfg=rr.YARN):
    return rr.rope_frequencies(D, cfg.base)


def _mut_all_interpolated(D, cfg=rr.YARN):
    return rr.rope_frequencies(D, cfg.base) / cfg.factor


def _mut_ramp_wavelength(D, cfg=rr.YARN):
    # ramp on the wavelength instead of the number of rotations
    theta = rr.rope_frequencies(D, cfg.base)
    if cfg.factor == 1.0:
        return theta
    r = 2.0 * np.pi / theta
    gamma = np.clip((r - cfg.alpha) / (cfg.beta - cfg.alpha), 0.0, 1.0)
    return (1.0 - gamma) * theta / cfg.factor + gamma * theta


def _mut_no_mscale(cfg=rr.YARN):
    return 1.0


def _mut_mscale_sqrt(cfg=rr.YARN):
    return float(np.sqrt(_orig_mscale(cfg)))


def _mut_inverse_ignored(x, positions, inverse=False, cfg=rr.YARN):
    return _orig_rope(x, positions, False, cfg)


def _mut_no_mscale_on_inverse(x, positions, inverse=False, cfg=rr.YARN):
    y = _orig_rope(x, positions, inverse, cfg)
    return y / _orig_mscale(cfg) if inverse else y


def _mut_positions_from_one(x, positions, inverse=False, cfg=rr.YARN):
    # a query/key position off by one only where positions are given as a slice of rows
    pos = np.asarray(positions)
    return _orig_rope(x, pos + (1 if pos.size and pos.size < 40 and pos.min() > 0 else 0), inverse, cfg)


def _mut_rot_v_too(q, k, cfg, operand_dtype=None):
    S = q.shape[2]
    pos = np.arange(S)
    return _orig_rope(q, pos, cfg=cfg), _orig_rope(k, pos, cfg=cfg)[..., ::-1].copy()


def _mut_only_q(q, k, cfg, operand_dtype=None):
    S = q.shape[2]
    return _orig_rope(q, np.arange(S), cfg=cfg), rr.attn._f64(k)


def _mut_stored_truncated(x, operand_dtype):
    # rounding toward zero instead of to nearest
    if operand_dtype is None:
        return x
    b = x.astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    return b.view(np.float32).astype(np.float64)


def _mut_stored_ignored(x, operand_dtype):
    return x


MUTANTS = {
    "rotation_clockwise": ("_rotate_pairs", _mut_clockwise),
    "pairs_split_in_halves": ("_rotate_pairs", _mut_half_split_pairs),
    "pair_outputs_swapped": ("_rotate_pairs", _mut_swapped_in_pair),
    "frequency_exponent_halved": ("rope_frequencies", _mut_freq_exponent),
    "ramp_reversed": ("yarn_frequencies", _mut_ramp_reversed),
    "no_interpolation": ("yarn_frequencies", _mut_no_interpolation),
    "all_pairs_interpolated": ("yarn_frequencies", _mut_all_interpolated),
    "ramp_on_wavelength": ("yarn_frequencies", _mut_ramp_wavelength),
    "mscale_dropped": ("yarn_mscale", _mut_no_mscale),
    "mscale_square_root": ("yarn_mscale", _mut_mscale_sqrt),
    "backward_not_transposed": ("rope", _mut_inverse_ignored),
    "backward_without_mscale": ("rope", _mut_no_mscale_on_inverse),
    "row_positions_off_by_one": ("rope", _mut_positions_from_one),
    "keys_rotated_wrongly": ("_rot_qk", _mut_rot_v_too),
    "keys_not_rotated": ("_rot_qk", _mut_only_q),
    "stored_operands_truncated": ("_stored", _mut_stored_truncated),
    "stored_operands_not_rounded": ("_stored", _mut_stored_ignored),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_rope_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(rr, attr, fn)
    failed = []
    with np.errstate(all="ignore"):
        for check in rc.ALL_ROPE_CHECKS:
            try:
                check(rr)
            except (AssertionError, ValueError, FloatingPointError, IndexError):
                failed.append(check.__name__)
    assert failed, f"no pin caught mutant {name}"
