"""Pins for the oracle's FP8 KV-cache variants (per layer, per head, static
scale), page "量化部署实战", section KV Cache 量化：误差要和信号比.

The per-head expectation is rebuilt independently of the oracle: numpy's
amax over the token and head_dim axes, float32 division, numpy's clip and
torch's float8_e4m3fn cast (a library routine the oracle never calls; the
codec tests pin it as round-to-nearest-even for |y| <= 448).
"""
import zlib

import numpy as np
import pytest
import torch

import oracle


def rng(tag):
    return np.random.default_rng(zlib.crc32(tag.encode()))


def e4m3_torch(y):
    return torch.from_numpy(np.ascontiguousarray(y, np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def kv_input(L, T, H, D, tag, bf16):
    r = rng(tag)
    # every head gets its own magnitude, and K-like heads a constant bias per dim
    x = r.standard_normal((L, T, H, D)).astype(np.float32)
    x *= (2.0 ** r.integers(-6, 7, (1, 1, H, 1))).astype(np.float32)
    x += r.standard_normal((L, 1, H, D)).astype(np.float32) * 3
    if bf16:
        return torch.from_numpy(x).to(torch.bfloat16)
    return x


def as_f32(x):
    return x.float().numpy() if isinstance(x, torch.Tensor) else x


SHAPES = [(2, 5, 3, 16), (1, 1, 1, 8), (3, 17, 8, 128), (2, 9, 4, 64)]


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("shape", SHAPES)
def test_kv_head_matches_brute_force(shape, bf16):
    x = kv_input(*shape, f"head{shape}{bf16}", bf16)
    codes, scales = oracle.kv_quant_fp8(x, "head")
    xf = as_f32(x)
    amax = np.abs(xf).max(axis=(1, 3))                                   # [L, H]
    s = np.maximum(amax, np.float32(1e-12)) / np.float32(448)
    assert scales.shape == amax.shape
    assert np.array_equal(scales.view(np.uint32), s.astype(np.float32).view(np.uint32))
    y = np.clip(xf / s[:, None, :, None], -448, 448)
    assert np.array_equal(codes, e4m3_torch(y))


@pytest.mark.parametrize("bf16", [False, True])
def test_kv_layer_is_per_tensor_fp8_per_layer(bf16):
    L, T, H, D = 3, 11, 4, 32
    x = kv_input(L, T, H, D, f"layer{bf16}", bf16)
    codes, scales = oracle.kv_quant_fp8(x, "layer")
    xf = as_f32(x)
    s = np.maximum(np.abs(xf).reshape(L, -1).max(1), np.float32(1e-12)) / np.float32(448)
    assert np.array_equal(scales.view(np.uint32), s.astype(np.float32).view(np.uint32))
    y = np.clip(xf / s[:, None, None, None], -448, 448)
    assert np.array_equal(codes, e4m3_torch(y))
    tc, ts = oracle.fp8_quantize(x.reshape(L, 1, -1) if bf16 else xf.reshape(L, 1, -1), "tensor")
    assert np.array_equal(tc.reshape(codes.shape), codes) and np.array_equal(ts, scales)


def test_kv_one_head_equals_layer():
    x = kv_input(2, 7, 1, 64, "onehead", False)
    hc, hs = oracle.kv_quant_fp8(x, "head")
    lc, ls = oracle.kv_quant_fp8(x, "layer")
    assert np.array_equal(hc, lc) and np.array_equal(hs.reshape(-1), ls)


def test_kv_head_scope_locality():
    L, T, H, D = 2, 6, 4, 16
    x = kv_input(L, T, H, D, "local", False)
    c0, s0 = oracle.kv_quant_fp8(x, "head")
    x2 = x.copy()
    x2[1, 3, 2, 5] = 1e4
    c1, s1 = oracle.kv_quant_fp8(x2, "head")
    changed = np.argwhere(s0 != s1)
    assert changed.tolist() == [[1, 2]]
    diff = np.argwhere(c0 != c1)
    assert diff.size and np.all(diff[:, 0] == 1) and np.all(diff[:, 2] == 2)


def test_kv_head_max_encodes_to_448():
    x = kv_input(2, 13, 5, 32, "max448", False)
    codes, _ = oracle.kv_quant_fp8(x, "head")
    for l in range(2):
        for h in range(5):
            blk = x[l, :, h, :]
            t, d = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
            assert codes[l, t, h, d] == (0xFE if blk[t, d] < 0 else 0x7E)


def test_kv_static_with_dynamic_scale_equals_dynamic():
    x = kv_input(3, 9, 2, 64, "static_eq", False)
    lc, ls = oracle.kv_quant_fp8(x, "layer")
    sc, ss = oracle.kv_quant_fp8(x, "static", scales=ls)
    assert np.array_equal(lc, sc) and np.array_equal(ls, ss)


def test_kv_static_clamp_and_values():
    # s = 0.5: 1000/s = 2000 and 224/s = 448 saturate to +-448 (0x7E / 0xFE);
    # 0.26/s = 0.52 lies between E4M3 0.5 and 0.5625 and rounds to 0.5 (0x30);
    # 223.9/s = 447.8 rounds to 448; -0 keeps its sign; 1e-30/s underflows to +0.
    vals = np.array([1000, -1000, 224, 0.26, -0.0, 1e-30, 223.9, -0.26], np.float32)
    x = vals.reshape(1, 1, 1, 8)
    codes, _ = oracle.kv_quant_fp8(x, "static", scales=np.array([0.5], np.float32))
    assert codes.reshape(-1).tolist() == [0x7E, 0xFE, 0x7E, 0x30, 0x80, 0x00, 0x7E, 0xB0]
    # a calibrated scale half the dynamic one: the top half of the range saturates
    x = kv_input(1, 8, 2, 16, "static_half", False)
    _, ls = oracle.kv_quant_fp8(x, "layer")
    sc, _ = oracle.kv_quant_fp8(x, "static", scales=ls / 2)
    big = np.abs(x) / (ls[0] / 2) >= 448
    assert big.any()
    assert np.all((sc[big] & 0x7F) == 0x7E)


def test_kv_mode_and_shape_errors():
    L = oracle.lib()
    import ctypes
    x = np.zeros(8, np.float32)
    c = np.zeros(8, np.uint8)
    s = np.zeros(1, np.float32)
    P = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    assert L.orc_kv_quant_fp8(P(x), 0, 1, 1, 1, 8, 3, P(c), P(s)) == -2
    assert L.orc_kv_quant_fp8(P(x), 0, -1, 1, 1, 8, 0, P(c), P(s)) == -4


@pytest.mark.parametrize("mode", ["head", "layer"])
def test_kv_zero_scope_uses_the_floor(mode):
    """An all-zero scope gets max(0, 1e-12) / 448 as its scale (the page's
    clamp(min=1e-12)), and its zeros keep their signs."""
    x = kv_input(2, 4, 3, 16, "zero" + mode, False)
    x[1] = 0.0
    x[1, 2, :, 3] = -0.0
    codes, scales = oracle.kv_quant_fp8(x, mode)
    floor = np.float32(np.float32(1e-12) / np.float32(448))
    zs = scales[1] if mode == "layer" else scales[1, :]
    assert np.all(np.asarray(zs, np.float32).view(np.uint32) == floor.view(np.uint32))
    assert np.all(codes[1][np.signbit(x[1])] == 0x80)
    assert np.all(codes[1][~np.signbit(x[1])] == 0x00)
