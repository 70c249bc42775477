"""Pins for the oracle's quantizers (CPU only).

What pins them, besides the oracle itself:
  * scopes: which elements share a scale is checked by moving one element and
    watching which scales change, and by numpy reductions over the reshapes
    that the deployment page's fake-quant module describes;
  * invariants fixed by the pages and by arithmetic: the largest element of a
    scope maps to +-448 (FP8), the MXFP4 block maximum lands on 4 or 6, the
    NVFP4 block holding the tensor maximum gets block scale 448, INT4 maps a
    group's minimum to -8, error bounds, storage per element;
  * element codes from torch's float8 cast (a library routine the oracle never
    uses) or from exact rational nearest-value search on small inputs.
"""
import math
import zlib
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import golden

E2M1 = [Fraction(v) for v in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]


def f32(v):
    return np.float32(v)


def torch_e4m3(y):
    return torch.from_numpy(np.ascontiguousarray(y, np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def torch_e4m3_decode(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn) \
        .to(torch.float32).numpy()


def torch_bf16_bits(v):
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def bf16_bits(x_f32):
    return torch_bf16_bits(x_f32)


def widen(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def nearest_e2m1(y: Fraction) -> int:
    a = abs(y)
    d = [abs(a - w) for w in E2M1]
    return d.index(min(d)) + (8 if y < 0 else 0)


def nib(codes, i):
    b = codes.reshape(-1)[i >> 1]
    return int(b >> 4) if i & 1 else int(b & 15)


def make(shape, seed, scale=1.0, dtype="bf16", outliers=0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g) * scale
    if outliers:
        idx = torch.randperm(x.numel(), generator=g)[:outliers]
        x.view(-1)[idx] *= 50
    if dtype == "bf16":
        return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16), True
    return x.numpy().astype(np.float32), False


def values(x, is_bf16):
    return widen(x) if is_bf16 else x


# ------------------------------------------------------------------ FP8 ----

def scope_amax(xv, gran):
    """amax per scope from numpy reshapes of [batch, rows, cols]."""
    b, r, c = xv.shape
    a = np.abs(xv)
    if gran == "tensor":
        return a.reshape(b, -1).max(axis=1)
    if gran == "row":
        return a.max(axis=2)
    if gran == "1x128":
        return a.reshape(b, r, c // 128, 128).max(axis=3)
    br = min(128, r)
    return a.reshape(b, r // br, br, c // 128, 128).max(axis=(2, 4))


def scope_of(gran, shape, bi, ri, ci):
    b, r, c = shape
    if gran == "tensor":
        return (bi,)
    if gran == "row":
        return (bi, ri)
    if gran == "1x128":
        return (bi, ri, ci // 128)
    br = min(128, r)
    return (bi, ri // br, ci // 128)


def expand(scales, gran, shape):
    b, r, c = shape
    if gran == "tensor":
        return np.broadcast_to(scales[:, None, None], shape)
    if gran == "row":
        return np.broadcast_to(scales[:, :, None], shape)
    if gran == "1x128":
        return np.repeat(scales, 128, axis=2)
    br = min(128, r)
    return np.repeat(np.repeat(scales, br, axis=1), 128, axis=2)


FP8_CASES = [
    ("tensor", (3, 40, 96)),
    ("row", (2, 37, 200)),
    ("1x128", (2, 33, 384)),
    ("128x128", (2, 256, 384)),
    ("128x128", (1, 64, 256)),     # rows < 128: the block is min(128, rows) tall
    ("128x128", (1, 1, 128)),
]


@pytest.mark.parametrize("gran,shape", FP8_CASES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fp8_scales_codes_and_dequant(orc, gran, shape, dtype):
    x, isb = make(shape, seed=zlib.crc32(repr((gran, shape)).encode()) % 1000, dtype=dtype,
                  outliers=5)
    xv = values(x, isb).reshape(shape)
    codes, scales = orc.fp8_quantize(x.reshape(shape), gran, bf16=isb)
    # scale = max(amax, 1e-12) / 448 for the page's scope
    amax = scope_amax(xv, gran)
    want = np.maximum(amax, f32(1e-12)).astype(np.float32) / f32(448.0)
    assert scales.dtype == np.float32 and scales.shape == want.shape
    assert np.array_equal(scales.view(np.uint32), want.astype(np.float32).view(np.uint32))
    # codes: torch's float8 cast of clamp(x / s, -448, 448)
    s_full = expand(scales, gran, shape)
    y = np.clip(xv / s_full, f32(-448), f32(448)).astype(np.float32)
    assert np.array_equal(codes, torch_e4m3(y))
    # dequant: decoded value times the scale, in float32; bf16 output is its RNE
    deq = orc.fp8_dequantize(codes, scales, gran)
    want_deq = (torch_e4m3_decode(codes) * s_full).astype(np.float32)
    assert np.array_equal(deq.view(np.uint32), want_deq.view(np.uint32))
    deq_b = orc.fp8_dequantize(codes, scales, gran, out_bf16=True)
    assert np.array_equal(deq_b, bf16_bits(want_deq))


@pytest.mark.parametrize("gran,shape", FP8_CASES)
def test_fp8_scope_max_maps_to_448(orc, gran, shape):
    x, isb = make(shape, seed=17, dtype="f32")
    codes, scales = orc.fp8_quantize(x.reshape(shape), gran)
    dec = torch_e4m3_decode(codes)
    s = expand(scales, gran, shape)
    amax = expand(scope_amax(x.reshape(shape), gran), gran, shape)
    at_max = np.abs(x.reshape(shape)) == amax
    assert np.all(np.abs(dec[at_max]) == golden("e4m3_max"))
    assert np.all(np.abs(dec) <= 448)
    # relative error bound of E4M3 in its normal range (2^-4 of the value)
    y = np.abs(x.reshape(shape) / s)
    normal = y >= 2.0 ** -6
    err = np.abs(dec * s - x.reshape(shape))[normal]
    assert np.all(err <= 2.0 ** -4 * np.abs(x.reshape(shape))[normal] * (1 + 1e-6))


@pytest.mark.parametrize("gran,shape", FP8_CASES)
def test_fp8_scope_locality(orc, gran, shape):
    """Raising one element changes exactly the one scale its scope owns."""
    x, _ = make(shape, seed=23, dtype="f32")
    x = x.reshape(shape)
    _, s0 = orc.fp8_quantize(x, gran)
    rng = np.random.default_rng(1)
    for _ in range(4):
        bi, ri, ci = (int(rng.integers(0, n)) for n in shape)
        x2 = x.copy()
        x2[bi, ri, ci] = 1000.0
        _, s1 = orc.fp8_quantize(x2, gran)
        changed = set(map(tuple, np.argwhere(s0 != s1)))
        assert changed == {scope_of(gran, shape, bi, ri, ci)}


def test_fp8_edge_values(orc):
    x = np.zeros((1, 2, 128), np.float32)
    x[0, 0, 0] = -0.0
    x[0, 1, :] = np.linspace(-3, 3, 128, dtype=np.float32)
    codes, scales = orc.fp8_quantize(x, "1x128")
    # an all-zero scope gets scale 1e-12/448 and zero codes, -0.0 keeps its sign
    assert scales[0, 0, 0] == f32(1e-12) / f32(448)
    assert codes[0, 0, 0] == 0x80 and np.all(codes[0, 0, 1:] == 0)
    assert codes[0, 1, 0] == 0xFE and codes[0, 1, 127] == 0x7E
    deq = orc.fp8_dequantize(codes, scales, "1x128")
    assert math.copysign(1, deq[0, 0, 0]) == -1


def test_fp8_rejects_shapes_the_reshape_rejects(orc):
    with pytest.raises(ValueError):
        orc.fp8_quantize(np.zeros((1, 4, 100), np.float32), "1x128")
    with pytest.raises(ValueError):
        orc.fp8_quantize(np.zeros((1, 200, 128), np.float32), "128x128")
    with pytest.raises(ValueError):
        orc.fp8_quantize(np.zeros((1, 128, 130), np.float32), "128x128")


def test_fp8_brute_force_tiny(orc):
    """Nearest E4M3 value by exact rational distance (ties to even code)."""
    x, _ = make((1, 3, 128), seed=99, scale=3.0, dtype="f32")
    codes, scales = orc.fp8_quantize(x, "row")
    table = torch_e4m3_decode(np.arange(256, dtype=np.uint8))
    finite = [(c, Fraction(float(table[c]))) for c in range(0x7F)]
    for r in range(3):
        s = scales[0, r]
        for c in range(128):
            y = Fraction(float(f32(x[0, r, c]) / s))     # float32 quotient, exact in Fraction
            a = abs(y)
            best = min(finite, key=lambda cv: (abs(a - cv[1]), cv[0] % 2))
            want = best[0] | (0x80 if y < 0 or math.copysign(1, float(y)) < 0 else 0)
            assert codes[0, r, c] == want


# ---------------------------------------------------------------- MXFP4 ----

def mx_expected_exponent(amax: float) -> int:
    a = max(float(np.float32(amax)), float(f32(1e-12)))
    m, e = math.frexp(a)           # exact: a = m * 2^e, m in [0.5, 1)
    return (e - 1) - 2


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mxfp4_scales_codes_dequant(orc, dtype):
    shape = (2, 24, 256)
    x, isb = make(shape, seed=4, scale=0.02, dtype=dtype, outliers=10)
    xv = values(x, isb).reshape(shape)
    codes, scales = orc.mxfp4_quantize(x.reshape(shape), bf16=isb)
    assert codes.shape == (2, 24, 128) and scales.shape == (2, 24, 8)
    blocks = xv.reshape(-1, 32)
    amax = np.abs(blocks).max(axis=1)
    X = np.array([mx_expected_exponent(a) for a in amax])
    assert np.array_equal(scales.reshape(-1).astype(int), X + 127)
    deq = orc.mxfp4_dequantize(codes, scales).reshape(-1, 32)
    for k in range(blocks.shape[0]):
        sc = Fraction(2) ** int(X[k])
        for j in range(32):
            i = k * 32 + j
            y = Fraction(float(blocks[k, j])) / sc            # exact: a power-of-two scale
            y = max(min(y, Fraction(6)), Fraction(-6))
            want = nearest_e2m1(y)
            assert nib(codes, i) == want
            v = E2M1[want & 7] * (-1 if want & 8 else 1) * sc
            assert Fraction(float(deq[k, j])) == v
        # the block maximum lands on 4 or 6 (index 6 or 7)
        top = int(np.argmax(np.abs(blocks[k])))
        assert nib(codes, k * 32 + top) & 7 in (6, 7)


def test_mxfp4_exponent_at_powers_of_two(orc):
    """floor(log2 amax) read exactly, including just below 2^k."""
    ks = list(range(-30, 40, 3))
    rows = []
    for k in ks:
        for a in (np.float32(2.0 ** k), np.nextafter(np.float32(2.0 ** k), np.float32(0))):
            blk = np.zeros(32, np.float32)
            blk[5] = -a
            rows.append(blk)
    x = np.stack(rows)[None]
    _, scales = orc.mxfp4_quantize(x)
    i = 0
    for k in ks:
        assert scales[0, i, 0] == k - 2 + 127
        assert scales[0, i + 1, 0] == k - 1 - 2 + 127
        i += 2


def test_mxfp4_zero_block_and_storage(orc):
    x = np.zeros((1, 2, 64), np.float32)
    codes, scales = orc.mxfp4_quantize(x)
    # all-zero block: amax clamps to 1e-12, floor(log2) = -40, E8M0 byte 85
    assert np.all(scales == 85) and np.all(codes == 0)
    n = 3072 * 1024
    bits = (n // 2 + n // 32) * 8 / n
    assert bits == golden("mxfp4_bits_per_element")
    assert codes.nbytes * 8 / x.size == 4 and scales.nbytes * 8 / x.size == 0.25


# ---------------------------------------------------------------- NVFP4 ----

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_nvfp4_two_level_scales(orc, dtype):
    shape = (2, 16, 128)
    x, isb = make(shape, seed=8, scale=0.02, dtype=dtype, outliers=6)
    xv = values(x, isb).reshape(shape)
    codes, scales, gs = orc.nvfp4_quantize(x.reshape(shape), bf16=isb)
    for b in range(shape[0]):
        amax_t = np.abs(xv[b]).max()
        want_gs = np.maximum(amax_t, f32(1e-12)) / f32(448.0 * 6.0)
        assert gs[b] == want_gs
        blocks = xv[b].reshape(-1, 16)
        amax_b = np.abs(blocks).max(axis=1).astype(np.float32)
        want_bs = torch_e4m3((amax_b / f32(6.0)) / gs[b])
        got_bs = scales[b].reshape(-1)
        assert np.array_equal(got_bs, want_bs)
        # the block holding the tensor maximum gets block scale 448 (code 0x7E)
        assert got_bs[int(np.argmax(amax_b))] == 0x7E
    deq = orc.nvfp4_dequantize(codes, scales, gs)
    bsdec = torch_e4m3_decode(scales)
    for b in range(shape[0]):
        for k in range(shape[1] * shape[2] // 16):
            s = np.maximum(bsdec[b].reshape(-1)[k], f32(1e-12)) * gs[b]
            for j in range(16):
                flat = b * shape[1] * shape[2] + k * 16 + j
                xe = xv[b].reshape(-1)[k * 16 + j]
                y = Fraction(float(np.float32(xe) / s))       # float32 quotient
                y = max(min(y, Fraction(6)), Fraction(-6))
                want = nearest_e2m1(y)
                assert nib(codes, flat) == want
                v = float(E2M1[want & 7]) * (-1 if want & 8 else 1)
                assert deq.reshape(-1)[flat] == np.float32(np.float32(v) * s)


def test_nvfp4_block_scale_underflow_follows_page(orc):
    """A block far below the tensor maximum gets block-scale code 0, and the
    1e-12 floor then sets its element scale to 1e-12 * tensor scale."""
    x = np.zeros((1, 1, 32), np.float32)
    x[0, 0, 0] = 1000.0
    x[0, 0, 16:32] = 1e-6
    codes, scales, gs = orc.nvfp4_quantize(x)
    assert scales[0, 0, 0] == 0x7E and scales[0, 0, 1] == 0
    assert nib(codes, 16) == 7                          # 1e-6 / (1e-12 * gs) clamps to 6
    deq = orc.nvfp4_dequantize(codes, scales, gs)
    assert deq[0, 0, 16] == np.float32(6.0) * (f32(1e-12) * gs[0])


def test_nvfp4_storage(orc):
    n = 28672 * 8192
    bits = (n // 2 + n // 16) * 8 / n
    assert bits == golden("nvfp4_bits_per_element")


# ----------------------------------------------------------------- INT4 ----

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_int4_groups(orc, dtype):
    shape = (2, 8, 384)
    x, isb = make(shape, seed=12, scale=0.02, dtype=dtype)
    xv = values(x, isb).reshape(shape)
    codes, scales, zeros = orc.int4_quantize(x.reshape(shape), bf16=isb)
    assert codes.shape == (2, 8, 192) and scales.shape == (2, 8, 3) and zeros.shape == (24,)
    deq = orc.int4_dequantize(codes, scales, zeros)
    G = 3
    for row in range(16):
        for g in range(G):
            grp = xv.reshape(16, 384)[row, g * 128:(g + 1) * 128]
            lo, hi = min(f32(0), grp.min()), max(f32(0), grp.max())
            # scale: bf16 of max(hi - lo, 1e-12) / 15 (torch's bf16 cast)
            s_bits = torch_bf16_bits(np.array([np.maximum(hi - lo, f32(1e-12)) / f32(15)]))[0]
            assert scales.reshape(16, G)[row, g] == s_bits
            s = widen(np.array([s_bits]))[0]
            gi = row * G + g                       # flat group index
            z_nib = int(zeros[gi // 2] >> (4 * (gi % 2))) & 15
            z = z_nib - 16 if z_nib & 8 else z_nib
            assert z == -8 - int(np.rint(lo / s))
            q = []
            for j in range(128):
                v = nib(codes, row * 384 + g * 128 + j)
                q.append(v - 16 if v & 8 else v)
            q = np.array(q)
            assert q.min() >= -8 and q.max() <= 7
            # the group minimum maps to -8 when it is below zero
            if grp.min() < 0:
                assert q[int(np.argmin(grp))] == -8
            xh = deq.reshape(16, 384)[row, g * 128:(g + 1) * 128]
            assert np.array_equal(xh, ((q - z).astype(np.float32) * s).astype(np.float32))
            assert np.all(np.abs(xh - grp) <= 0.6 * s)


def test_int4_special_groups(orc):
    x = np.zeros((1, 3, 128), np.float32)
    x[0, 1] = np.linspace(0.0, 1.5, 128, dtype=np.float32)     # all >= 0: lo = 0
    x[0, 2] = np.linspace(-1.5, 0.0, 128, dtype=np.float32)    # all <= 0: hi = 0
    codes, scales, zeros = orc.int4_quantize(x)
    deq = orc.int4_dequantize(codes, scales, zeros)
    assert np.all(deq[0, 0] == 0)
    z = [(int(zeros[r // 2]) >> (4 * (r % 2))) & 15 for r in range(3)]
    assert z[0] == 8 and z[1] == 8                   # z = -8 (nibble 0x8)
    assert nib(codes, 128 + 127) == 7                # hi -> 7
    assert nib(codes, 256) == 8                      # lo -> -8
    assert deq[0, 1, 0] == 0 and deq[0, 2, 127] == 0
    # nibble order: element 2i in the low nibble of byte i
    assert codes[0, 2, 0] & 15 == 8


def test_int4_infinite_range_group(orc):
    """A group holding values of both signs near the float32 maximum has a
    range hi - lo that overflows to inf.  The definition then gives s = inf
    (bf16 0x7F80), x / s = 0 for every finite x, so every code and the
    zero-point are -8; the engine leaves such groups unspecified (a documented
    precondition), and the neighbouring group is untouched."""
    x = np.zeros((1, 2, 128), np.float32)
    x[0, 0, ::2] = 3.0e38
    x[0, 0, 1::2] = -3.0e38
    x[0, 1] = np.linspace(-1.0, 2.0, 128, dtype=np.float32)
    codes, scales, zeros = orc.int4_quantize(x)
    assert scales[0, 0, 0] == 0x7F80
    assert all(nib(codes, i) == 8 for i in range(128))
    assert zeros[0] & 15 == 8
    c2, s2, z2 = orc.int4_quantize(x[:, 1:])
    assert scales[0, 1, 0] == s2[0, 0, 0]
    assert np.array_equal(codes[0, 1], c2[0, 0]) and zeros[0] >> 4 == z2[0] & 15


def test_int4_range_always_contains_zero(orc):
    """A group that lies entirely above (or below) zero still spans [0, hi]
    (or [lo, 0]): 0 must stay exactly representable."""
    x = np.zeros((1, 2, 128), np.float32)
    x[0, 0] = np.linspace(0.5, 1.5, 128, dtype=np.float32)
    x[0, 1] = np.linspace(-1.5, -0.5, 128, dtype=np.float32)
    codes, scales, zeros = orc.int4_quantize(x)
    s = widen(scales)[0]
    want = torch_bf16_bits(np.array([f32(1.5) / f32(15)]))[0]
    assert scales[0, 0, 0] == want and scales[0, 1, 0] == want
    assert zeros[0] & 15 == 8                                            # lo = 0: z = -8
    assert zeros[0] >> 4 == (-8 - int(np.rint(f32(-1.5) / s[1, 0]))) & 15  # = 7
    q0 = nib(codes, 0)                                                   # 0.5 / 0.1 = 5 -> -3
    assert (q0 - 16 if q0 & 8 else q0) == int(np.rint(f32(0.5) / s[0, 0])) - 8
    assert nib(codes, 128) == 8                                          # -1.5 -> -8


def test_int4_storage_matches_page(orc):
    n = 4096 * 128
    codes_scales = n // 2 + 2 * (n // 128)
    assert codes_scales / n == 0.515625
    assert round(codes_scales / n, 3) == golden("int4_g128_bytes_per_weight")
    assert (codes_scales + n // 256) / n == pytest.approx(0.51953125)


# ------------------------------------------------------------------- KV ----

def test_kv_write_one_scale_per_layer(orc):
    layers, tokens, heads, dim = 3, 16, 2, 128
    g = torch.Generator().manual_seed(31)
    bias = torch.randn(layers, 1, heads, dim, generator=g) * 2
    k = (bias + 0.1 * torch.randn(layers, tokens, heads, dim, generator=g)).to(torch.bfloat16)
    v = torch.randn(layers, tokens, heads, dim, generator=g).to(torch.bfloat16)
    kc, vc, ks, vs = orc.kv_write_fp8(k, v)
    for l in range(layers):
        for t, codes, sc in ((k, kc, ks), (v, vc, vs)):
            lay = t[l].float().numpy().reshape(-1)
            s = np.maximum(np.abs(lay).max(), f32(1e-12)) / f32(448)
            assert sc[l] == s
            assert np.array_equal(codes[l], torch_e4m3(np.clip(lay / s, -448, 448)))
    # V does not influence K's scales
    _, _, ks2, _ = orc.kv_write_fp8(k, v * 100)
    assert np.array_equal(ks, ks2)


@pytest.mark.parametrize("layers,heads,bf16_key,fp8_key", [
    (32, 8, "llama8b_kv_bytes_bf16", "llama8b_kv_bytes_fp8"),
    (28, 4, "qwen7b_kv_bytes_bf16", "qwen7b_kv_bytes_fp8"),
])
def test_kv_bytes_per_token_halve(orc, layers, heads, bf16_key, fp8_key):
    tokens, dim = 2, 128
    k = torch.randn(layers, tokens, heads, dim).to(torch.bfloat16)
    kc, vc, ks, vs = orc.kv_write_fp8(k, k)
    assert 2 * k.numel() * 2 / tokens == golden(bf16_key)
    assert (kc.nbytes + vc.nbytes) / tokens == golden(fp8_key)
