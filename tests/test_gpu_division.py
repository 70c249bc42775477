"""The engine's correctly rounded division on the GPU, against IEEE division
computed by numpy on the host.

Every FP8, NVFP4, INT4, INT8 and KIVI code rests on x / s being the correctly
rounded quotient (page "量化部署实战", section 伪量化实现, divides by the scale
before rounding).  The engine forms it from the reciprocal y = RN(1/s) (the
hardware estimate and one Newton step) and one fused multiply-add correction
of x * y.  These tests check:
  - the reciprocal for every float s in [2^-64, 2^126), the range every scale
    the engine forms lies in (about 1.6e9 values);
  - the quotient for every float32 significand of x (in three binades, both
    signs) against 48 divisors spanning significands and exponents.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

LO_BITS = (127 - 64) << 23     # 2^-64
HI_BITS = (127 + 126) << 23    # 2^126
CHUNK = 1 << 28


@pytest.fixture(scope="module")
def pqb():
    import precision_quantization_block_amd as p
    p.lib()
    return p


def test_recip_every_float_in_scale_range(pqb):
    bad = 0
    first = LO_BITS
    while first < HI_BITS:
        n = min(CHUNK, HI_BITS - first)
        got = pqb.check_recip(first, n).cpu().numpy()
        s = np.arange(first, first + n, dtype=np.uint32).view(np.float32)
        ref = np.float32(1.0) / s
        bad += int(np.count_nonzero(got.view(np.uint32) != ref.view(np.uint32)))
        first += n
    assert bad == 0


def _divisors():
    rng = np.random.default_rng(5)
    sig = [1.0, 1.0 + 2.0 ** -23, 2.0 - 2.0 ** -23, 1.5, 1.25, 1.75, 4.0 / 3.0, 1.1]
    sig += list(1.0 + rng.random(16))
    sig = np.array(sig, dtype=np.float32)
    exps = np.array([-40, -3, 0, 7, 20, 60], dtype=np.int32)
    s = (sig[:, None] * np.ldexp(np.float32(1.0), exps)[None, :]).astype(np.float32).reshape(-1)
    return s[rng.permutation(s.size)[:48]]


@pytest.mark.parametrize("x_first", [
    127 << 23,                      # x in [1, 2)
    (127 - 30) << 23,               # x in [2^-30, 2^-29)
    (1 << 31) | (127 << 23),        # x in (-2, -1]
])
def test_quotient_every_significand(pqb, x_first):
    s = _divisors()
    nx = 1 << 23
    x = np.arange(x_first, x_first + nx, dtype=np.uint32).view(np.float32)
    st = torch.from_numpy(s).cuda()
    bad = 0
    for j0 in range(0, s.size, 8):
        got = pqb.check_div(st[j0:j0 + 8], x_first, nx).cpu().numpy()
        ref = x[None, :] / s[j0:j0 + 8, None]
        bad += int(np.count_nonzero(got.view(np.uint32) != ref.view(np.uint32)))
    assert bad == 0


def test_planted_error_is_seen(pqb):
    """The host reference tells the engine's quotient from the uncorrected
    product x * RN(1/s): some quotients differ, so a pass above means something."""
    s = _divisors()[:8]
    x = np.arange(127 << 23, (127 << 23) + (1 << 20), dtype=np.uint32).view(np.float32)
    y = np.float32(1.0) / s
    ref = x[None, :] / s[:, None]
    assert np.count_nonzero((x[None, :] * y[:, None]).view(np.uint32) != ref.view(np.uint32)) > 0
    got = pqb.check_div(torch.from_numpy(s).cuda(), 127 << 23, 1 << 20).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
