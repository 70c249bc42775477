"""Power-of-two scaling invariance of the oracle's quantizers (CPU).

Every format on the pages forms its scale from an amax or a range of the
scope, then divides by it (page "量化部署实战", section 伪量化实现; INT4 and
KIVI by the plainest reading of their pages).  Multiplying the input by 2^k multiplies
every amax and range by 2^k exactly, every correctly rounded quotient of two
such values is unchanged, and bf16 / E4M3 rounding of a scale commutes with
2^k away from the subnormal and overflow ranges.  So, for inputs far from
those ranges:
  * every element code is unchanged;
  * float32 and bf16 scales, KIVI minimums and the NVFP4 tensor scale are
    multiplied by exactly 2^k;
  * E8M0 scale bytes (MXFP4, MXFP8) grow by k;
  * NVFP4 block-scale codes and INT4 zero-points are unchanged.
These hold for any data, so they pin what the value-based tests cannot see
at every magnitude: a quantity that does not scale with the input mixed into
the path (a clamp applied to x rather than to x / s, a threshold or floor met
by unscaled values, a block scale formed against a fixed constant instead of
the tensor scale, exponent arithmetic that wraps).  Mistakes that scale with
the input (a wrong constant divisor) are left to the value pins.
"""
import numpy as np
import pytest

KS = (-7, 3, 20)


def data(shape, seed):
    r = np.random.default_rng(seed)
    x = r.standard_normal(shape).astype(np.float32)
    x[..., ::37] *= 9.0   # a few large values so scopes differ
    return x


def scaled(x, k):
    y = np.ldexp(x, k).astype(np.float32)
    assert np.array_equal(np.ldexp(y, -k).astype(np.float32), x)   # exact
    return y


@pytest.mark.parametrize("gran", ["tensor", "row", "1x128", "128x128"])
@pytest.mark.parametrize("elem", ["e4m3", "e5m2"])
def test_fp8_scopes_scale_invariant(orc, gran, elem):
    x = data((2, 256, 384), 11)
    c0, s0 = orc.fp8_quantize(x, gran, elem=elem)
    for k in KS:
        c1, s1 = orc.fp8_quantize(scaled(x, k), gran, elem=elem)
        assert np.array_equal(c0, c1), (gran, elem, k)
        assert np.array_equal(s1, np.ldexp(s0, k).astype(np.float32)), (gran, elem, k)


@pytest.mark.parametrize("gran", ["tensor", "row"])
def test_int8_scale_invariant(orc, gran):
    x = data((2, 64, 256), 12)
    c0, s0 = orc.int8_quantize(x, gran)
    for k in KS:
        c1, s1 = orc.int8_quantize(scaled(x, k), gran)
        assert np.array_equal(c0, c1) and np.array_equal(s1, np.ldexp(s0, k).astype(np.float32))


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_mx_scale_invariant(orc, fmt):
    q = orc.mxfp4_quantize if fmt == "mxfp4" else orc.mxfp8_quantize
    x = data((3, 64, 256), 13)
    c0, e0 = q(x)
    for k in KS:
        c1, e1 = q(scaled(x, k))
        assert np.array_equal(c0, c1), (fmt, k)
        assert np.array_equal(e1.astype(np.int32), e0.astype(np.int32) + k), (fmt, k)


def test_nvfp4_scale_invariant(orc):
    x = data((2, 64, 256), 14)
    x[1, :32] *= 1e-6      # blocks far below the tensor maximum (block-scale code 0)
    c0, b0, g0 = orc.nvfp4_quantize(x)
    assert (b0 == 0).any()
    for k in KS:
        c1, b1, g1 = orc.nvfp4_quantize(scaled(x, k))
        assert np.array_equal(c0, c1) and np.array_equal(b0, b1), k
        assert np.array_equal(g1, np.ldexp(g0, k).astype(np.float32)), k


def test_int4_scale_invariant(orc):
    x = data((2, 64, 512), 15)
    x[0, :4] = np.abs(x[0, :4])          # groups entirely above zero
    x[1, :4] = -np.abs(x[1, :4])         # and entirely below
    c0, s0, z0 = orc.int4_quantize(x)
    f0 = orc.bf16_bits_to_f32(s0)
    for k in KS:
        c1, s1, z1 = orc.int4_quantize(scaled(x, k))
        assert np.array_equal(c0, c1) and np.array_equal(z0, z1), k
        assert np.array_equal(orc.bf16_bits_to_f32(s1), np.ldexp(f0, k).astype(np.float32)), k


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("is_k", [True, False])
def test_kivi_scale_invariant(orc, bits, is_k):
    x = data((2, 64, 2, 64), 16)
    c0, s0, m0 = orc.kivi_quant(x, bits, is_k)
    for k in KS:
        c1, s1, m1 = orc.kivi_quant(scaled(x, k), bits, is_k)
        assert np.array_equal(c0, c1), (bits, is_k, k)
        assert np.array_equal(s1, np.ldexp(s0, k).astype(np.float32)), (bits, is_k, k)
        assert np.array_equal(m1, np.ldexp(m0, k).astype(np.float32)), (bits, is_k, k)


def test_scaling_check_catches_a_wrong_exponent(orc):
    """The E8M0 assertion above is not vacuous: MXFP4 scales of 2^k x differ
    from those of x by k, not by 0 or 2k."""
    x = data((1, 8, 64), 17)
    _, e0 = orc.mxfp4_quantize(x)
    _, e1 = orc.mxfp4_quantize(scaled(x, 3))
    assert not np.array_equal(e1, e0) and np.array_equal(e1.astype(int) - e0.astype(int), np.full(e0.shape, 3))
