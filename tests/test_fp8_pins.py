"""The e4m3 facts the FP8 path and its parity bounds rest on (no GPU).

The oracle for the FP8 forward is the plain attention of ``oracle.attention`` over the
dequantised inputs (scale * code value), so what needs pinning is the decoding of OCP
e4m3 codes (PyTorch's float8_e4m3fn conversion, which both the input generator and the
oracle use) and the rounding bound the GPU parity test derives its tolerance from.
"""

import numpy as np
import torch

# OCP 8-bit floating point specification, E4M3: bias 7, no infinities, S.1111.111 = NaN
OCP_E4M3 = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x3C: 1.5,
            0x40: 2.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}


def test_e4m3_decoding_matches_the_ocp_definition():
    codes = torch.tensor(list(OCP_E4M3), dtype=torch.uint8).view(torch.float8_e4m3fn)
    got = codes.to(torch.float64).tolist()
    assert got == list(OCP_E4M3.values())
    assert torch.isnan(torch.tensor([0x7F], dtype=torch.uint8).view(torch.float8_e4m3fn).float()).all()
    # every finite code by the formula: (-1)^s 2^(e - 7) (1 + m/8), subnormals 2^-6 m/8
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue
        want = (-1) ** s * (2.0 ** (e - 7) * (1 + m / 8) if e else 2.0 ** -6 * m / 8)
        assert torch.tensor([c], dtype=torch.uint8).view(torch.float8_e4m3fn).double().item() == want


def test_e4m3_rounding_is_nearest_within_half_ulp():
    # the GPU parity bound takes |round(x) - x| <= max(2^-4 |x|, 2^-10) for |x| <= 448
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.uniform(0, 448, 100000), np.exp2(rng.uniform(-14, 8.8, 100000))]).astype(np.float32)
    r = torch.from_numpy(x).to(torch.float8_e4m3fn).double().numpy()
    err = np.abs(r - x.astype(np.float64))
    assert (err <= np.maximum(2.0 ** -4 * x, 2.0 ** -10) + 1e-12).all()
    # and it is the nearest code: no code is closer
    allv = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    nearest = np.abs(allv[None, :] - x[:2000, None].astype(np.float64)).min(axis=1)
    assert np.allclose(err[:2000], nearest, rtol=0, atol=0)
