"""Pins of the oracle's RoPE (oc_rope, oc_kv_compress_rope) against closed forms, the complex form
of the rotation and the properties that define RoPE.

The rotation follows RoFormer (Su et al., "RoFormer: Enhanced Transformer with Rotary Position
Embedding", section 3.2, general form): adjacent pairs of the last R dims, pair j turned
counter-clockwise by p * base^(-2j/R) at position p. A compressed entry sits at the position of
the last token of its group. Together the tests catch a wrong pairing (adjacent vs split halves),
a wrong direction, a wrong frequency schedule (exponent, offset, dims), a missing per-query
position step, a rotation applied before pooling and a wrong entry position.
"""
import math

import numpy as np
import pytest

import oracle as O

F32, BF16 = O.DT_F32, O.DT_BF16


def _rand(shape, seed, std=1.0):
    return (np.random.default_rng(seed).normal(size=shape) * std).astype(np.float32)


def _unit(D, d):
    x = np.zeros((1, 1, 1, D), np.float32)
    x[0, 0, 0, d] = 1.0
    return x


def _complex_rope(x, positions, R, base, sign=1.0):
    """The rotation as complex multiplication: pair (a, b) -> (a + ib) e^(i p w_j), with the R/2
    frequencies w_j spaced geometrically from 1 down towards 1/base (numpy geomspace)."""
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    w = np.geomspace(1.0, 1.0 / base, R // 2, endpoint=False)
    z = x[..., D - R::2] + 1j * x[..., D - R + 1::2]
    ang = sign * np.asarray(positions, np.float64)[..., None] * w
    z = z * np.exp(1j * ang)
    out = x.copy()
    out[..., D - R::2] = z.real
    out[..., D - R + 1::2] = z.imag
    return out


@pytest.mark.parametrize("base", [10000.0, 500000.0, 2.0])
def test_first_pair_turns_by_the_position_counter_clockwise(base):
    """theta_0 = base^0 = 1 whatever the base: at p = 1 the first rotary pair turns by one radian,
    counter-clockwise, and nothing leaves the pair."""
    D, R = 16, 8
    got = O.rope(_unit(D, D - R), np.array([1]), R, base)[0, 0, 0]
    want = np.zeros(D)
    want[D - R], want[D - R + 1] = math.cos(1.0), math.sin(1.0)
    np.testing.assert_allclose(got, want, atol=1e-15)
    got = O.rope(_unit(D, D - R + 1), np.array([1]), R, base)[0, 0, 0]
    want = np.zeros(D)
    want[D - R], want[D - R + 1] = -math.sin(1.0), math.cos(1.0)
    np.testing.assert_allclose(got, want, atol=1e-15)


def test_dims_before_the_rotary_part_are_untouched():
    x = _rand((2, 3, 4, 128), 1)
    got = O.rope(x, np.array([5, 70000]), 64)
    np.testing.assert_array_equal(got[..., :64], x[..., :64].astype(np.float64))
    assert not np.allclose(got[..., 64:], x[..., 64:])


@pytest.mark.parametrize("R,base,p,j,ang", [
    (4, 10000.0, 100, 1, 1.0),          # theta_1 = 10000^(-2/4) = 1/100
    (8, 10000.0, 1000, 3, 1.0),         # R = 8: theta_j = 10000^(-j/4) = 10^(-j)
    (8, 10000.0, 1000, 2, 10.0),
    (32, 65536.0, 1 << 9, 9, 1.0),      # base 2^16, R = 32: theta_j = 2^(-j)
    (32, 65536.0, 1 << 15, 15, 1.0),
])
def test_frequency_schedule_closed_forms(R, base, p, j, ang):
    """Pair j turns by p * base^(-2j/R); each case makes that angle a small exact number."""
    got = O.rope(_unit(R, 2 * j), np.array([p]), R, base)[0, 0, 0]
    np.testing.assert_allclose([got[2 * j], got[2 * j + 1]], [math.cos(ang), math.sin(ang)],
                               atol=1e-12)


def test_frequencies_are_a_geometric_split_of_one_to_one_over_base():
    """Recovered from the rotation of unit pairs at p = 1: w_0 = 1, a constant ratio between
    neighbours, and one more step after the last one lands on exactly 1/base."""
    D = R = 64
    base = 10000.0
    x = np.zeros((1, 1, R // 2, D), np.float32)
    for j in range(R // 2):
        x[0, 0, j, 2 * j] = 1.0
    got = O.rope(x, np.array([1]), R, base)[0, 0]
    w = np.array([math.atan2(got[j, 2 * j + 1], got[j, 2 * j]) for j in range(R // 2)])
    assert abs(w[0] - 1.0) < 1e-15
    ratio = w[1:] / w[:-1]
    np.testing.assert_allclose(ratio, ratio[0], rtol=1e-12)
    assert abs(w[-1] * ratio[0] - 1.0 / base) < 1e-15


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_rows_match_the_complex_form(dtype):
    """Every row (b, i, h) at position pos[b] + i equals complex multiplication by e^(i p w)."""
    B, Q, H, D, R = 3, 5, 4, 128, 64
    x = _rand((B, Q, H, D), 2)
    if dtype == BF16:
        bits = np.array([O.bf16_encode(float(v)) for v in x.ravel()], np.uint16).reshape(x.shape)
        xv = np.array([O.bf16_value(int(v)) for v in bits.ravel()]).reshape(x.shape)
        x_in = bits
    else:
        xv, x_in = x, x
    pos = np.array([0, 1 << 20, 987654], np.int64)
    got = O.rope(x_in, pos, R)
    positions = pos[:, None, None] + np.arange(Q)[None, :, None] + np.zeros((1, 1, H))
    want = _complex_rope(xv, positions, R, 10000.0)
    np.testing.assert_allclose(got, want, atol=1e-9, rtol=1e-9)


def test_inverse_turns_back_and_equals_the_negative_position():
    x = _rand((2, 3, 2, 64), 3)
    pos = np.array([12345, 1 << 20], np.int64)
    fwd = O.rope(x, pos, 64).astype(np.float32)
    back = O.rope(fwd, pos, 64, inverse=True)
    np.testing.assert_allclose(back, x, atol=1e-6)
    positions = pos[:, None, None] + np.arange(3)[None, :, None] + np.zeros((1, 1, 2))
    np.testing.assert_allclose(O.rope(x, pos, 64, inverse=True),
                               _complex_rope(x, positions, 64, 10000.0, sign=-1.0), atol=1e-9)


def test_pair_norms_are_preserved():
    x = _rand((1, 4, 8, 512), 4)
    got = O.rope(x, np.array([777777]), 64)
    x = x.astype(np.float64)
    n0 = np.hypot(x[..., 448::2], x[..., 449::2])
    n1 = np.hypot(got[..., 448::2], got[..., 449::2])
    np.testing.assert_allclose(n1, n0, rtol=1e-12)


def test_scores_depend_only_on_the_relative_position():
    """RoFormer's defining property: <rope(q, a), rope(k, c)> = <rope(q, a - c), k>."""
    q = _rand((1, 1, 1, 128), 5)
    k = _rand((1, 1, 1, 128), 6)
    for a, c in [(10, 3), (1 << 20, (1 << 20) - 4096), (500000, 7)]:
        lhs = np.dot(O.rope(q, np.array([a]), 64).ravel(), O.rope(k, np.array([c]), 64).ravel())
        rhs = np.dot(O.rope(q, np.array([a - c]), 64).ravel(), k.astype(np.float64).ravel())
        assert abs(lhs - rhs) < 1e-9 * (1 + abs(rhs)), (a, c, lhs, rhs)


# ----------------------------------------------------------------------------- compression
def _compress_inputs(B, T, D, m, seed):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(B, T, D)).astype(np.float32)
    w = (rng.normal(size=D) * 0.05).astype(np.float32)
    beta = (rng.normal(size=m) * 0.3).astype(np.float32)
    return x, w, beta


def test_compress_m1_rotates_each_token_at_its_own_position():
    B, T, D = 2, 40, 128
    x, w, beta = _compress_inputs(B, T, D, 1, 7)
    tok = np.array([0, 1 << 20], np.int64)
    r = O.kv_compress(x, F32, 1, w, beta, O.FMT_ROW_F32, tok_pos=tok, rope_dims=64)
    want = O.rope(x[:, :, None, :], tok, 64)[:, :, 0, :]
    np.testing.assert_allclose(r["pre"], want, atol=1e-12)


@pytest.mark.parametrize("m,span,skip", [(4, 4, 0), (128, 128, 0), (4, 8, 1)])
def test_compress_turns_the_pooled_entry_at_its_groups_last_token(m, span, skip):
    """A constant sequence pools to the constant row; each entry g is then turned by the position
    of the last token of its group, tok_pos + m(g+1) - 1, whatever the span."""
    B, G, D = 2, 6, 64
    T = G * m
    v = _rand((B, 1, D), 8)
    x = np.repeat(v, T, axis=1)
    _, w, beta = _compress_inputs(B, T, D, span, 9)
    tok = np.array([3, 100003], np.int64)
    r = O.kv_compress(x, F32, m, w, beta, O.FMT_ROW_F32, span=span, skip=skip, tok_pos=tok,
                      rope_dims=32)
    g = np.arange(skip, G)
    positions = tok[:, None] + m * (g[None, :] + 1) - 1
    want = _complex_rope(np.broadcast_to(v, (B, G - skip, D)), positions, 32, 10000.0)
    np.testing.assert_allclose(r["pre"], want, atol=1e-9)


def test_compress_pools_first_and_rotates_after():
    """The non-rotary dims equal plain compression; the rotary dims are the plain pooled values
    turned at the entry's position (so the rotation does not enter the gate or the weights)."""
    B, T, D, m = 2, 64, 512, 4
    x, w, beta = _compress_inputs(B, T, D, m, 10)
    tok = np.array([1 << 20, 5], np.int64)
    plain = O.kv_compress(x, F32, m, w, beta, O.FMT_ROW_E4M3_BF16)
    rot = O.kv_compress(x, F32, m, w, beta, O.FMT_ROW_E4M3_BF16, tok_pos=tok, rope_dims=64)
    np.testing.assert_array_equal(rot["pi"], plain["pi"])
    np.testing.assert_array_equal(rot["pre"][..., :448], plain["pre"][..., :448])
    positions = tok[:, None] + m * (np.arange(T // m)[None, :] + 1) - 1
    np.testing.assert_allclose(rot["pre"], _complex_rope(plain["pre"], positions, 64, 10000.0),
                               atol=1e-9)
    enc, _ = O.encode_rows(rot["pre"], O.FMT_ROW_E4M3_BF16)
    np.testing.assert_array_equal(enc, rot["rows"])


def test_rejects_bad_rotary_widths():
    x = _rand((1, 1, 1, 64), 11)
    for R in (0, 3, 66):
        with pytest.raises(ValueError):
            O.rope(x, np.array([1]), R)
