"""Pins for the oracle's W4A16 product y = x @ dequant(W)^T (page "14. 量化：让
每一步搬更少的字节", 路线一: 4-bit weights unpacked and dequantized to 16 bits for
the multiply).  Expected values come from a pure-Python brute force that
decodes the nibbles itself, from integer arithmetic, and from closed forms."""
import zlib

import numpy as np
import torch

import oracle


def rng(tag):
    return np.random.default_rng(zlib.crc32(tag.encode()))


def weight(r, N, K):
    w = (0.02 * r.standard_normal((N, K))).astype(np.float32)
    return oracle.int4_quantize(w[None])


def bf16_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def nib(byte, hi):
    v = (int(byte) >> (4 * hi)) & 0xF
    return v - 16 if v >= 8 else v


def test_w4a16_matches_brute_force():
    r = rng("bf")
    M, N, K = 2, 5, 256
    codes, scales, zeros = weight(r, N, K)
    x = bf16_bits(r.standard_normal((M, K)))
    xf = oracle.bf16_bits_to_f32(x).tolist()
    sf = oracle.bf16_bits_to_f32(scales[0]).tolist()
    want = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            tot = 0.0
            for k in range(K):
                q = nib(codes[0, n, k // 2], k & 1)
                g = n * (K // 128) + k // 128
                z = nib(zeros[g // 2], g & 1)
                tot += xf[m][k] * (q - z) * sf[n][k // 128]
            want[m, n] = tot
    got = oracle.w4a16_gemv(x, codes, scales, zeros)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def test_w4a16_one_hot_rows_read_dequantized_columns():
    r = rng("hot")
    N, K = 7, 384
    codes, scales, zeros = weight(r, N, K)
    x = np.zeros((K, K), np.float32)
    x[np.arange(K), np.arange(K)] = 1.0
    got = oracle.w4a16_gemv(bf16_bits(x), codes, scales, zeros)
    w = oracle.int4_dequantize(codes, scales, zeros)[0]
    assert np.array_equal(got, w.T.astype(np.float64))


def test_w4a16_integer_case_is_exact():
    """Weights whose dequantized values are small integers (power-of-two
    scales) and integer activations: y is an integer matmul."""
    r = rng("int")
    N, K = 12, 256
    w = r.integers(-7, 8, (N, K)).astype(np.float32)
    w[:, ::128] = 7.0                      # max 7, min <= -7 per group
    w[:, 1::128] = -8.0                    # so the step is exactly 1
    codes, scales, zeros = oracle.int4_quantize(w[None])
    assert np.all(oracle.bf16_bits_to_f32(scales) == 1.0)
    x = r.integers(-20, 21, (3, K)).astype(np.float32)
    got = oracle.w4a16_gemv(bf16_bits(x), codes, scales, zeros)
    assert np.array_equal(got, x.astype(np.int64) @ w.T.astype(np.int64))


def test_w4a16_abs_sum_bounds_the_result():
    r = rng("abs")
    codes, scales, zeros = weight(r, 16, 512)
    x = bf16_bits(r.standard_normal((4, 512)))
    y, S = oracle.w4a16_gemv(x, codes, scales, zeros, abs_sum=True)
    assert np.all(np.abs(y) <= S) and np.all(S > 0)
