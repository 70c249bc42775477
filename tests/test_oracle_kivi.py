"""Pins for the oracle's KIVI-style KV quantization (K per channel over 32
tokens, V per token over 32 channels, 2- or 4-bit asymmetric codes with the
group minimum as zero-point): page "量化部署实战", KV Cache 量化 section (K per
channel with a zero-point absorbs the constant bias); "14. 量化：让每一步搬更少
的字节", 路线三 (KIVI: K per channel, V per token, 2 bits); "LLM 推理优化 ·
量化学习笔记" §5.1 (asymmetric zero-point), §7.4 (KIVI).

The expected codes are rebuilt with numpy float32 arithmetic and numpy bit
packing, independent of the oracle.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle


def rng(tag):
    return np.random.default_rng(zlib.crc32(tag.encode()))


def kv_like(L, T, H, D, tag):
    r = rng(tag)
    bias = (r.standard_normal((L, 1, H, D)) * 2).astype(np.float32)
    return (bias + 0.1 * r.standard_normal((L, T, H, D))).astype(np.float32)


def rebuild(xf, bits, is_k):
    L, T, H, D = xf.shape
    if is_k:   # groups (l, t // 32, h, d)
        g = xf.reshape(L, T // 32, 32, H, D)
        m, M = g.min(2), g.max(2)
        expand = lambda a: np.repeat(a, 32, axis=1)                  # noqa: E731
    else:      # groups (l, t, h, d // 32)
        g = xf.reshape(L, T, H, D // 32, 32)
        m, M = g.min(4), g.max(4)
        expand = lambda a: np.repeat(a, 32, axis=3)                  # noqa: E731
    qmax = np.float32(2 ** bits - 1)
    s = (np.maximum(M - m, np.float32(1e-12)) / qmax).astype(np.float32)
    q = np.clip(np.rint((xf - expand(m)) / expand(s)), 0, qmax).astype(np.uint8).reshape(-1)
    per = 8 // bits
    packed = np.zeros(q.size // per, np.uint8)
    for j in range(per):
        packed |= (q[j::per] << (bits * j)).astype(np.uint8)
    return packed.reshape(L, T, H, D * bits // 8), s, m


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("is_k", [True, False])
@pytest.mark.parametrize("bf16", [False, True])
def test_kivi_matches_rebuild(bits, is_k, bf16):
    x = kv_like(2, 64, 3, 64, f"kivi{bits}{is_k}{bf16}")
    xt = torch.from_numpy(x).to(torch.bfloat16) if bf16 else x
    xf = xt.float().numpy() if bf16 else x
    c, s, m = oracle.kivi_quant(xt, bits, is_k)
    ec, es, em = rebuild(xf, bits, is_k)
    assert np.array_equal(s.view(np.uint32), es.view(np.uint32))
    assert np.array_equal(m.view(np.uint32), em.view(np.uint32))
    assert np.array_equal(c, ec)
    # dequant is q * s + m, two float32 roundings, and stays within s / 2
    d = oracle.kivi_dequant(c, s, m, bits, is_k)
    per = 8 // bits
    q = np.stack([(c >> (bits * j)) & (2 ** bits - 1) for j in range(per)], -1).reshape(xf.shape)
    exp = lambda a: np.repeat(a, 32, axis=1) if is_k else np.repeat(a, 32, axis=3)  # noqa: E731
    want = (q.astype(np.float32) * exp(s)).astype(np.float32) + exp(m)
    assert np.array_equal(d.view(np.uint32), want.astype(np.float32).view(np.uint32))
    err = np.abs(d - xf)
    assert np.all(err <= exp(s) * np.float32(0.5 + 1e-5) + 4 * np.spacing(np.abs(xf) + np.abs(d)))


def test_kivi_packing_and_constant_groups():
    x = np.zeros((1, 32, 1, 32), np.float32)
    # V, one group per token: values chosen so that q = [3, 0, 1, 2] at the start
    x[0, 0, 0, :4] = [3, 0, 1, 2]
    x[0, 0, 0, 4:] = 0
    c, s, m = oracle.kivi_quant(x, 2, False)
    assert s[0, 0, 0, 0] == 1.0 and m[0, 0, 0, 0] == 0.0
    assert c[0, 0, 0, 0] == 0b10_01_00_11                 # element 4i + j at bits 2j
    c4, _, _ = oracle.kivi_quant(x * 5, 4, False)          # s = 1, q = [15, 0, 5, 10]
    assert c4[0, 0, 0, 0] == 0x0F and c4[0, 0, 0, 1] == 0xA5
    # K: a channel that is a constant bias reproduces exactly (q = 0, x = m)
    k = np.full((1, 32, 2, 32), 5.7, np.float32)
    k[0, :, 1, :] = -3.25
    c, s, m = oracle.kivi_quant(k, 2, True)
    assert np.all(c == 0)
    assert np.all(s == np.float32(np.float32(1e-12) / np.float32(3)))
    assert np.array_equal(oracle.kivi_dequant(c, s, m, 2, True), k)


def test_kivi_group_locality():
    x = kv_like(1, 64, 2, 64, "local")
    c0, s0, m0 = oracle.kivi_quant(x, 4, True)
    x2 = x.copy()
    x2[0, 40, 1, 17] += 100.0          # token group 1, head 1, channel 17
    c1, s1, m1 = oracle.kivi_quant(x2, 4, True)
    assert np.argwhere(s0 != s1).tolist() == [[0, 1, 1, 17]]
    assert np.array_equal(m0, m1)
    c0, s0, m0 = oracle.kivi_quant(x, 4, False)
    c1, s1, m1 = oracle.kivi_quant(x2, 4, False)
    assert np.argwhere(s0 != s1).tolist() == [[0, 40, 1, 0]]


def test_kivi_k_beats_per_tensor_fp8_on_biased_keys():
    """The page's case: K is a large per-channel constant plus a small
    variation.  Per channel with a zero-point (4 bits) reconstructs it far
    better than one FP8 scale for the whole layer (8 bits)."""
    r = rng("bias")
    L, T, H, D = 1, 256, 8, 128
    k = (r.standard_normal((L, 1, H, D)).astype(np.float32) * 5.7
         + 0.36 * r.standard_normal((L, T, H, D)).astype(np.float32))
    c, s, m = oracle.kivi_quant(k, 4, True)
    e_kivi = np.abs(oracle.kivi_dequant(c, s, m, 4, True) - k).mean()
    fc, fs = oracle.fp8_quantize(k.reshape(1, T, H * D), "tensor")
    e_fp8 = np.abs(oracle.fp8_dequantize(fc, fs, "tensor").reshape(k.shape) - k).mean()
    assert e_kivi < e_fp8 / 2


def test_kivi_argument_errors():
    x = np.zeros((1, 32, 1, 32), np.float32)
    with pytest.raises(ValueError):
        oracle.kivi_quant(x, 3, True)
    with pytest.raises(ValueError):
        oracle.kivi_quant(np.zeros((1, 33, 1, 32), np.float32), 2, True)   # K needs T % 32
    oracle.kivi_quant(np.zeros((1, 33, 1, 32), np.float32), 2, False)     # V does not
    with pytest.raises(ValueError):
        oracle.kivi_quant(np.zeros((1, 32, 1, 48), np.float32), 2, False)  # D % 32


def test_kivi_zero_minimum_is_positive_zero():
    """A group whose minimum is zero stores +0 whichever signed zeros it holds."""
    x = np.zeros((1, 32, 1, 32), np.float32)
    x[0, :, 0, 0] = -0.0
    x[0, 3, 0, 0] = 1.0
    x[0, 5, 0, 1:] = -0.0
    for is_k in (True, False):
        _, _, m = oracle.kivi_quant(x, 4, is_k)
        zero = m == 0
        assert zero.any() and not np.signbit(m[zero]).any()


def test_kivi_rounding_ties_go_to_even():
    """With m = 0 and M = 3 at 2 bits (or M = 15 at 4 bits) the step is exactly
    1, so halves are exact ties and rint sends them to the even integer."""
    x = np.zeros((1, 1, 1, 32), np.float32)
    x[0, 0, 0, :8] = [0.0, 3.0, 0.5, 1.5, 2.5, 1.0, 2.0, 0.25]
    c, s, m = oracle.kivi_quant(x, 2, False)
    assert s[0, 0, 0, 0] == 1.0 and m[0, 0, 0, 0] == 0.0
    q = [(int(c[0, 0, 0, i // 4]) >> (2 * (i % 4))) & 3 for i in range(8)]
    assert q == [0, 3, 0, 2, 2, 1, 2, 0]
    x4 = x * 5
    x4[0, 0, 0, :8] = [0.0, 15.0, 6.5, 7.5, 13.5, 14.5, 0.5, 2.5]
    c, s, m = oracle.kivi_quant(x4, 4, False)
    assert s[0, 0, 0, 0] == 1.0
    q = [(int(c[0, 0, 0, i // 2]) >> (4 * (i % 2))) & 15 for i in range(8)]
    assert q == [0, 15, 6, 8, 14, 14, 0, 2]
