"""Pins of the oracle's number-format codecs against the OCP specifications and torch's casts.

None of these calls the GPU library. torch's CPU casts (float8_e4m3fn, bfloat16) are library
routines independent of the oracle's C code.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLD, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_e2m1_table_matches_ocp_mx():
    for code, val in _rows("ocp_mx_fp4_e2m1.txt"):
        got = O.e2m1_value(int(code, 16))
        assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), code


def test_e4m3_landmarks_match_ofp8():
    for code, val in _rows("ocp_ofp8_e4m3.txt"):
        got = O.e4m3_value(int(code, 16))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val), code


def test_e4m3_decode_all_codes_vs_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([O.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_e4m3_encode_vs_torch_in_range():
    g = torch.Generator().manual_seed(11)
    x = torch.cat([torch.randn(20000, generator=g) * s for s in (1e-3, 0.05, 1.0, 30.0, 150.0)])
    # every code's value and every midpoint between neighbours (ties must go to even)
    vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float()
    vals = vals[torch.isfinite(vals)].unique()
    mids = (vals[1:] + vals[:-1]) / 2
    x = torch.cat([x, vals, mids, -mids]).clamp(-448, 448)
    ref = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([O.e4m3_encode(float(v)) for v in x.tolist()], dtype=np.uint8)
    # torch encodes -0.0 midpoint results with the sign bit; compare values where both are zero
    both_zero = (ref & 0x7F == 0) & (got & 0x7F == 0)
    assert np.array_equal(ref[~both_zero], got[~both_zero])


def test_e4m3_encode_saturates():
    for v in (448.0, 463.9, 464.0, 500.0, 1e9):
        assert O.e4m3_encode(v) == 0x7E
        assert O.e4m3_encode(-v) == 0xFE


def test_bf16_encode_decode_vs_torch():
    g = torch.Generator().manual_seed(12)
    x = torch.cat([torch.randn(50000, generator=g) * s for s in (1e-30, 1e-3, 1.0, 1e20)])
    ref = x.to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    got = np.array([O.bf16_encode(float(v)) for v in x.tolist()], dtype=np.uint16)
    assert np.array_equal(ref, got)
    back = torch.from_numpy(got.astype(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(back, np.array([O.bf16_value(int(b)) for b in got]))


def _nearest_e2m1_brute(v):
    """Brute-force nearest E2M1 code over the 16-entry table; ties to the even mantissa bit."""
    best = None
    for c in range(16):
        val = O.e2m1_value(c)
        d = abs(val - v)
        key = (d, c & 1)  # smaller distance first, then even mantissa
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


@pytest.mark.parametrize("amax,byte", [(float(a), int(b)) for a, b in _rows("ocp_mx_scale_rule.txt")])
def test_fp4_block_scale_rule(amax, byte):
    v = np.zeros(32)
    v[5] = amax
    v[9] = -amax / 3
    codes, scale = O.fp4_block_encode(v)
    assert scale == byte


def test_fp4_block_elements_vs_brute_force():
    rng = np.random.default_rng(5)
    for trial in range(200):
        v = rng.normal(size=32) * 10.0 ** rng.uniform(-3, 3)
        codes, scale = O.fp4_block_encode(v)
        X = 2.0 ** (scale - 127)
        for i in range(32):
            c = (codes[i // 2] >> (4 if i & 1 else 0)) & 15
            r = v[i] / X
            rr = max(-6.0, min(6.0, r))
            exp = _nearest_e2m1_brute(rr)
            # +0 and -0 are both acceptable encodings of a value that rounds to zero
            if O.e2m1_value(exp) == 0.0:
                assert O.e2m1_value(c) == 0.0
            else:
                assert c == exp, (trial, i, v[i], r)


def test_fp4_zero_block_and_saturation():
    codes, scale = O.fp4_block_encode(np.zeros(32))
    assert scale == 127 and not codes.any()
    v = np.zeros(32)
    v[0] = 7.9  # floor(log2 7.9) = 2 -> X = 1 -> 7.9 saturates to 6
    codes, scale = O.fp4_block_encode(v)
    assert scale == 127 and (codes[0] & 15) == 7


def test_row_roundtrip_formats():
    rng = np.random.default_rng(3)
    x = rng.normal(size=(7, 512))
    rows, _ = O.encode_rows(x, O.FMT_ROW_E4M3_BF16)
    assert rows.shape == (7, 576)
    y = O.decode_rows(rows, 512, O.FMT_ROW_E4M3_BF16)
    ref_n = torch.from_numpy(x[:, :448]).float().to(torch.float8_e4m3fn).double().numpy()
    ref_r = torch.from_numpy(x[:, 448:]).float().to(torch.bfloat16).double().numpy()
    assert np.array_equal(y[:, :448], ref_n)
    assert np.array_equal(y[:, 448:], ref_r)
    rows, sc = O.encode_rows(x[:, :128], O.FMT_FP4_E8M0)
    assert rows.shape == (7, 64) and sc.shape == (7, 4)
    y = O.decode_rows(rows, 128, O.FMT_FP4_E8M0, sc)
    # MX error bound: amax/X < 8, so saturation at 6 costs < 2X; inside the grid the error is at
    # most half the widest E2M1 step (2), i.e. X
    X = 2.0 ** (sc.astype(np.float64) - 127)
    err = np.abs(y - x[:, :128]).reshape(7, 4, 32)
    assert (err < 2.0 * X[:, :, None]).all()
    rows, _ = O.encode_rows(x[:, :128], O.FMT_ROW_F32)
    y = O.decode_rows(rows, 128, O.FMT_ROW_F32)
    assert np.array_equal(y, x[:, :128].astype(np.float32).astype(np.float64))
