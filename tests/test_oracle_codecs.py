"""Pins for the oracle's number-format codecs (CPU only).

Each test checks the oracle against something other than itself: torch's own
float8_e4m3fn and bfloat16 conversions (library routines the oracle never
calls), the values printed on the pages (tests/golden/page_values.txt), exact
rational arithmetic, and exhaustive or strided sweeps of the float32 space.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import golden


def _f32_from_bits(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def _torch_e4m3(y: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(y, np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def _e4m3_table_from_torch() -> np.ndarray:
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()


# ---------------------------------------------------------------- E4M3 ----

def test_e4m3_decode_every_code_matches_torch(orc):
    ref = _e4m3_table_from_torch()
    for c in range(256):
        got = np.float32(orc.e4m3_decode(c))
        if np.isnan(ref[c]):
            assert np.isnan(got), hex(c)
            assert c in (0x7F, 0xFF)
        else:
            assert got.view(np.uint32) == ref[c].view(np.uint32), hex(c)


def test_e4m3_max_and_code_count(orc):
    # the page's FP8_MAX constant is the largest finite code
    assert orc.e4m3_decode(0x7E) == golden("e4m3_max")
    assert orc.e4m3_decode(0xFE) == -golden("e4m3_max")
    vals = [orc.e4m3_decode(c) for c in range(int(golden("e4m3_code_points")))]
    finite = [v for v in vals if not math.isnan(v)]
    # 256 code points: 2 NaN patterns, +0 and -0, and 253 distinct finite reals
    assert len(vals) - len(finite) == 2
    assert len(set(finite)) == 253
    assert max(finite) == 448.0 and min(finite) == -448.0
    # smallest subnormal 2^-9, smallest normal 2^-6
    assert orc.e4m3_decode(0x01) == 2.0 ** -9
    assert orc.e4m3_decode(0x08) == 2.0 ** -6


def _e4m3_probe_points():
    table = _e4m3_table_from_torch()
    pos = np.unique(table[(~np.isnan(table)) & (table >= 0)]).astype(np.float32)
    mids = ((pos[:-1].astype(np.float64) + pos[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (pos[:-1].astype(np.float64) + pos[1:]) / 2)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    # strided sweep over every float32 bit pattern from 0 to 448
    sweep = _f32_from_bits(np.arange(0, 0x43E00001, 4099, dtype=np.uint32))
    rng = np.random.default_rng(11)
    rand = _f32_from_bits(rng.integers(0, 0x43E00001, 200_000, dtype=np.uint32))
    tiny = np.array([2.0 ** -10, np.nextafter(np.float32(2.0 ** -10), np.float32(1)),
                     np.nextafter(np.float32(2.0 ** -10), np.float32(0)), 1e-45, 1e-30,
                     3 * 2.0 ** -11, 2.0 ** -126], np.float32)
    p = np.concatenate([pos, mids, up, dn, sweep, rand, tiny]).astype(np.float32)
    return np.concatenate([p, -p])


def test_e4m3_encode_matches_torch_cast(orc):
    y = _e4m3_probe_points()
    got = orc.e4m3_encode_array(y)
    ref = _torch_e4m3(y)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(y[i]), hex(got[i]), hex(ref[i])) for i in bad[:10]]


def test_e4m3_midpoints_go_to_even_code(orc):
    table = _e4m3_table_from_torch()
    for c in range(0, 0x7E):
        lo, hi = Fraction(float(table[c])), Fraction(float(table[c + 1]))
        mid = np.float32(float((lo + hi) / 2))
        assert Fraction(float(mid)) == (lo + hi) / 2
        want = c if c % 2 == 0 else c + 1
        assert orc.e4m3_encode(float(mid)) == want, hex(c)
        assert orc.e4m3_encode(float(np.nextafter(mid, np.float32(0)))) == c
        assert orc.e4m3_encode(float(np.nextafter(mid, np.float32(1e9)))) == c + 1


def test_e4m3_signed_zero_and_saturation(orc):
    assert orc.e4m3_encode(-0.0) == 0x80
    assert orc.e4m3_encode(0.0) == 0x00
    assert orc.e4m3_encode(-1e-30) == 0x80
    # just above 448 the nearest finite value is still 448 (the page clamps first)
    assert orc.e4m3_encode(460.0) == 0x7E


def test_e4m3_relative_error_in_normal_range(orc):
    """Outside the subnormal range the rounding error is at most half a step,
    2^-4 of the value; the deployment page puts it at about 3-6%."""
    rng = np.random.default_rng(5)
    y = np.exp(rng.uniform(np.log(2.0 ** -6), np.log(448.0), 100_000)).astype(np.float32)
    dec = _e4m3_table_from_torch()[orc.e4m3_encode_array(y)]
    rel = np.abs(dec.astype(np.float64) - y) / y
    assert rel.max() <= 2.0 ** -4
    assert rel.max() * 100 <= golden("e4m3_rel_err_max_pct")


# ---------------------------------------------------------------- E2M1 ----

def test_e2m1_value_set_matches_page(orc):
    page = golden("e2m1_values")
    assert [orc.e2m1_decode(i) for i in range(8)] == page
    assert [orc.e2m1_decode(8 + i) for i in range(8)] == [-v for v in page]
    assert math.copysign(1.0, orc.e2m1_decode(8)) == -1.0
    assert int(golden("e2m1_code_points")) == 16


def _e2m1_threshold_rule(y: np.ndarray) -> np.ndarray:
    """Independent restatement: the magnitude index counts the midpoints between
    neighbouring E2M1 values that lie strictly below |y| (a tie stays on the
    smaller value); the sign bit is set for y < 0."""
    vals = np.array(golden("e2m1_values"), np.float64)
    mids = (vals[:-1] + vals[1:]) / 2
    a = np.abs(y.astype(np.float64))
    idx = (a[:, None] > mids[None, :]).sum(axis=1)
    return (idx + 8 * (y < 0)).astype(np.uint8)


def test_e2m1_encode_strided_sweep(orc):
    # every 997th float32 bit pattern between 0 and 7 (beyond 6 the nearest is 6)
    y = _f32_from_bits(np.arange(0, 0x40E00001, 997, dtype=np.uint32))
    y = np.concatenate([y, -y])
    got = orc.e2m1_encode_array(y)
    ref = _e2m1_threshold_rule(y)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(y[i]), got[i], ref[i]) for i in bad[:10]]


def test_e2m1_ties_go_to_smaller_magnitude(orc):
    vals = golden("e2m1_values")
    for i in range(7):
        mid = (Fraction(vals[i]) + Fraction(vals[i + 1])) / 2
        m = np.float32(float(mid))
        assert Fraction(float(m)) == mid
        assert orc.e2m1_encode(float(m)) == i
        assert orc.e2m1_encode(-float(m)) == 8 + i
        assert orc.e2m1_encode(float(np.nextafter(m, np.float32(9)))) == i + 1
        assert orc.e2m1_encode(float(np.nextafter(m, np.float32(0)))) == i


def test_e2m1_sign_rule(orc):
    assert orc.e2m1_encode(-0.0) == 0        # sign(-0) = 0 -> +0
    assert orc.e2m1_encode(-0.1) == 8        # negative, rounds to zero -> -0
    assert orc.e2m1_encode(-1e-40) == 8
    assert orc.e2m1_encode(6.0) == 7 and orc.e2m1_encode(-6.0) == 15
    # the clamp to +-6 comes first: huge values saturate
    assert orc.e2m1_encode(1e30) == 7 and orc.e2m1_encode(-1e30) == 15


def test_e2m1_brute_force_exact_rationals(orc):
    """Nearest by exact rational distance, first (smaller) value on ties."""
    rng = np.random.default_rng(7)
    y = np.concatenate([rng.uniform(-6.5, 6.5, 4000),
                        rng.uniform(-1, 1, 2000) * 2.0 ** -20]).astype(np.float32)
    vals = [Fraction(v) for v in golden("e2m1_values")]
    for v in y:
        a = abs(Fraction(float(v)))
        d = [abs(a - w) for w in vals]
        want = d.index(min(d)) + (8 if v < 0 else 0)
        assert orc.e2m1_encode(float(v)) == want, float(v)


# ---------------------------------------------------------------- bf16 ----

def test_bf16_round_matches_torch(orc):
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 0x7F7F0000, 1_000_000, dtype=np.uint32)
    ties = (rng.integers(0, 0x7F7F, 20_000, dtype=np.uint32) << 16) | 0x8000
    near = np.concatenate([ties - 1, ties + 1])
    bits = np.concatenate([bits, ties, near, np.array([0, 1, 0x8000, 0x18000], np.uint32)])
    v = _f32_from_bits(bits)
    v = np.concatenate([v, -v])
    got = orc.bf16_round_array(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


# ------------------------------------------------------- uniform quantizer --

def test_uniform_quantizer_worked_example(orc):
    s = np.float32(golden("worked_scale"))
    x = np.float32(golden("worked_x"))
    q = orc.uniform_code(float(x), float(s), 0.0)
    assert q == golden("worked_q")
    xhat = np.float32(np.float32(q) * s)
    assert xhat == np.float32(golden("worked_xhat"))
    assert abs(float(xhat) - float(x)) == pytest.approx(golden("worked_err"), abs=1e-6)


def test_uniform_quantizer_rounds_half_to_even(orc):
    assert orc.uniform_code(2.5, 1.0, 0.0) == 2.0
    assert orc.uniform_code(3.5, 1.0, 0.0) == 4.0
    assert orc.uniform_code(-2.5, 1.0, 0.0) == -2.0
    assert orc.uniform_code(-0.5, 1.0, -8.0) == -8.0
    assert orc.uniform_code(1.0, 0.25, 3.0) == 7.0
