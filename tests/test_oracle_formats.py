"""Pins for the oracle's format variants: FP8 E5M2 scopes, MXFP8 and symmetric
INT8 (format tables on the pages "14. 量化：让每一步搬更少的字节" (低位浮点格式)
and "LLM 推理优化 · 量化学习笔记" §4.2, §4.5, §5.1; W8A8 INT8 row of the format
table on "量化部署实战").

Expected values are rebuilt independently of the oracle: numpy arithmetic in
float32 plus torch's float8_e5m2 / float8_e4m3fn casts (library routines the
oracle never calls), and hand-computed values for the edge cases.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from conftest import golden


def rng(tag):
    return np.random.default_rng(zlib.crc32(tag.encode()))


def torch_cast(y, dtype):
    return torch.from_numpy(np.ascontiguousarray(y, np.float32)).to(dtype).view(torch.uint8).numpy()


# ------------------------------------------------------------------ E5M2 ---

def test_e5m2_decode_all_codes_against_torch():
    L = oracle.lib()
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).float().numpy()
    got = np.array([L.orc_e5m2_decode(int(c)) for c in codes], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_e5m2_page_values():
    L = oracle.lib()
    assert L.orc_e5m2_decode(0x7B) == golden("e5m2_max")                 # 57344
    assert L.orc_e5m2_decode(0x01) == 2.0 ** -16                        # smallest subnormal
    assert L.orc_e5m2_decode(0x04) == 2.0 ** -14                        # smallest normal
    vals = [L.orc_e5m2_decode(c) for c in range(256)]
    finite = {v for v in vals if np.isfinite(v)}
    assert len(vals) == 256 and len(finite) == 247                      # 256 codes
    assert sum(np.isinf(vals)) == 2 and sum(np.isnan(vals)) == 6


def test_e5m2_encode_probe_set_against_torch():
    table = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e5m2) \
        .float().numpy()
    pos = np.unique(table[np.isfinite(table) & (table >= 0)])
    mids = ((pos[:-1].astype(np.float64) + pos[1:]) / 2).astype(np.float32)
    r = rng("e5m2")
    y = np.concatenate([pos, mids, np.nextafter(mids, np.float32(1e9)),
                        np.nextafter(mids, np.float32(0)),
                        r.uniform(0, 57344, 200_000).astype(np.float32),
                        (2.0 ** r.uniform(-20, np.log2(57344), 200_000)).astype(np.float32),
                        np.array([1e-45, 3e-39, 2.0 ** -17, 57344.0], np.float32)])
    y = np.concatenate([y, -y]).astype(np.float32)
    assert np.all(np.abs(y) <= 57344)
    assert np.array_equal(oracle.e5m2_encode_array(y), torch_cast(y, torch.float8_e5m2))
    # Beyond 57344 (never reached after the +-57344 clamp) the oracle saturates,
    # where the cast would round to infinity above 61440.
    big = np.array([57345, 61439, 61441, 1e10, -70000], np.float32)
    assert oracle.e5m2_encode_array(big).tolist() == [0x7B, 0x7B, 0x7B, 0x7B, 0xFB]


# ------------------------------------------------------- FP8 E5M2 scopes ---

def fp8_expect(xf, gran, m, dtype):
    """Independent rebuild of the FP8 scopes for one element format."""
    b, r, c = xf.shape
    a = np.abs(xf)
    if gran == "tensor":
        amax = a.reshape(b, -1).max(1)
        s = np.maximum(amax, np.float32(1e-12)) / np.float32(m)
        full = np.broadcast_to(s[:, None, None], xf.shape)
    elif gran == "row":
        amax = a.max(2)
        s = np.maximum(amax, np.float32(1e-12)) / np.float32(m)
        full = np.broadcast_to(s[:, :, None], xf.shape)
    elif gran == "1x128":
        amax = a.reshape(b, r, c // 128, 128).max(3)
        s = np.maximum(amax, np.float32(1e-12)) / np.float32(m)
        full = np.repeat(s, 128, axis=2)
    else:
        br = min(128, r)
        amax = a.reshape(b, r // br, br, c // 128, 128).max(axis=(2, 4))
        s = np.maximum(amax, np.float32(1e-12)) / np.float32(m)
        full = np.repeat(np.repeat(s, br, axis=1), 128, axis=2)
    y = np.clip(xf / full, -m, m)
    return torch_cast(y, dtype), s.astype(np.float32)


@pytest.mark.parametrize("gran", ["tensor", "row", "1x128", "128x128"])
@pytest.mark.parametrize("bf16", [False, True])
def test_fp8_e5m2_scopes_match_rebuild(gran, bf16):
    r = rng(f"e5m2{gran}{bf16}")
    x = (r.standard_normal((2, 256, 384)) * np.exp(r.uniform(-6, 6, (2, 256, 1)))).astype(np.float32)
    if bf16:
        xt = torch.from_numpy(x).to(torch.bfloat16)
        xf = xt.float().numpy()
    else:
        xt, xf = x, x
    codes, scales = oracle.fp8_quantize(xt, gran, elem="e5m2")
    ec, es = fp8_expect(xf, gran, 57344.0, torch.float8_e5m2)
    assert np.array_equal(scales.reshape(-1).view(np.uint32), es.reshape(-1).view(np.uint32))
    assert np.array_equal(codes, ec)


def test_fp8_e5m2_scope_max_is_57344_and_dequant():
    x = rng("e5m2max").standard_normal((1, 8, 256)).astype(np.float32)
    codes, scales = oracle.fp8_quantize(x, "row", elem="e5m2")
    for i in range(8):
        j = np.argmax(np.abs(x[0, i]))
        assert codes[0, i, j] == (0xFB if x[0, i, j] < 0 else 0x7B)
    dq = oracle.fp8_dequantize(codes, scales, "row", elem="e5m2")
    dec = torch.from_numpy(codes).view(torch.float8_e5m2).float().numpy()
    assert np.array_equal(dq, (dec * scales[:, :, None]).astype(np.float32))
    # the E4M3 path is unchanged by the element parameter
    c4, s4 = oracle.fp8_quantize(x, "row", elem="e4m3")
    c4b, s4b = oracle.fp8_quantize(x, "row")
    assert np.array_equal(c4, c4b) and np.array_equal(s4, s4b)


# ---------------------------------------------------------------- MXFP8 ---

def mxfp8_expect(xf):
    b, r, c = xf.shape
    blk = xf.reshape(-1, 32)
    amax = np.maximum(np.abs(blk).max(1), np.float32(1e-12))
    _, e = np.frexp(amax)                         # amax = f * 2^e, f in [0.5, 1)
    X = (e - 1) - 8
    y = np.clip(np.ldexp(blk, -X[:, None]).astype(np.float32), -448, 448)
    codes = torch_cast(y, torch.float8_e4m3fn).reshape(b, r, c)
    return codes, (X + 127).astype(np.uint8).reshape(b, r, c // 32)


@pytest.mark.parametrize("bf16", [False, True])
def test_mxfp8_matches_rebuild(bf16):
    r = rng(f"mxfp8{bf16}")
    x = (r.standard_normal((2, 33, 128)) * np.exp(r.uniform(-20, 20, (2, 33, 1)))).astype(np.float32)
    xt = torch.from_numpy(x).to(torch.bfloat16) if bf16 else x
    xf = xt.float().numpy() if bf16 else x
    codes, scales = oracle.mxfp8_quantize(xt)
    ec, es = mxfp8_expect(xf)
    assert np.array_equal(scales, es)
    assert np.array_equal(codes, ec)


def test_mxfp8_edge_blocks():
    x = np.zeros((1, 4, 32), np.float32)
    x[0, 0, :] = np.linspace(-1, 1, 32) * 2.0 ** 5          # amax = 2^5: max maps to 256
    x[0, 1, :] = np.linspace(-1, 1, 32) * 1.9 * 2.0 ** -3   # significand 1.9: 486 clamps to 448
    x[0, 2, 5] = -0.0                                       # all-zero block
    x[0, 3, :] = np.linspace(-1, 1, 32) * 1.74 * 2.0 ** 10  # 445.4 rounds to 448 without clamping
    codes, scales = oracle.mxfp8_quantize(x)
    assert scales[0, 0, 0] == 5 - 8 + 127 and codes[0, 0, -1] == 0x78 and codes[0, 0, 0] == 0xF8
    assert scales[0, 1, 0] == -3 - 8 + 127 and codes[0, 1, -1] == 0x7E and codes[0, 1, 0] == 0xFE
    assert scales[0, 2, 0] == -40 - 8 + 127                 # floor(log2(1e-12)) = -40
    assert np.all(codes[0, 2] & 0x7F == 0) and codes[0, 2, 5] == 0x80
    assert scales[0, 3, 0] == 10 - 8 + 127 and codes[0, 3, -1] == 0x7E
    dq = oracle.mxfp8_dequantize(codes, scales)
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    X = scales.astype(np.int32) - 127
    assert np.array_equal(dq, np.ldexp(dec, np.repeat(X, 32, axis=2)).astype(np.float32))


# ----------------------------------------------------------------- INT8 ---

@pytest.mark.parametrize("gran", ["tensor", "row"])
@pytest.mark.parametrize("bf16", [False, True])
def test_int8_matches_rebuild(gran, bf16):
    r = rng(f"int8{gran}{bf16}")
    x = (r.standard_normal((3, 17, 200)) * np.exp(r.uniform(-8, 8, (3, 17, 1)))).astype(np.float32)
    xt = torch.from_numpy(x).to(torch.bfloat16) if bf16 else x
    xf = xt.float().numpy() if bf16 else x
    codes, scales = oracle.int8_quantize(xt, gran)
    if gran == "tensor":
        s = np.maximum(np.abs(xf).reshape(3, -1).max(1), np.float32(1e-12)) / np.float32(127)
        full = s[:, None, None]
    else:
        s = np.maximum(np.abs(xf).max(2), np.float32(1e-12)) / np.float32(127)
        full = s[:, :, None]
    assert np.array_equal(scales.view(np.uint32), s.astype(np.float32).view(np.uint32))
    q = np.clip(np.rint(xf / full), -128, 127).astype(np.int8)
    assert np.array_equal(codes, q)
    dq = oracle.int8_dequantize(codes, scales, gran)
    assert np.array_equal(dq, (codes.astype(np.float32) * full).astype(np.float32))


def test_int8_row_max_ties_and_zero():
    # amax 127 gives s = 1 exactly: 2.5 -> 2, 3.5 -> 4, -0.5 -> -0 (ties to even)
    x = np.zeros((1, 3, 8), np.float32)
    x[0, 0] = [127, 2.5, 3.5, -0.5, -127, 0.49, -1.5, 126.5]
    x[0, 2, 3] = -0.0                                       # all-zero row: s = 1e-12 / 127
    codes, scales = oracle.int8_quantize(x, "row")
    assert scales[0, 0] == 1.0
    assert codes[0, 0].tolist() == [127, 2, 4, 0, -127, 0, -2, 126]
    assert scales[0, 2] == np.float32(np.float32(1e-12) / np.float32(127))
    assert np.all(codes[0, 2] == 0)


def test_new_format_shape_errors():
    with pytest.raises(ValueError):
        oracle.mxfp8_quantize(np.zeros((2, 48), np.float32))
    with pytest.raises(ValueError):
        oracle.int8_quantize(np.zeros((2, 48), np.float32), "1x128")
