"""Pins for the oracle's MXFP4 x MXFP4 product C = dequant(A) @ dequant(B)^T
(page "LLM 推理优化 · 量化学习笔记" §4.5: 32-element blocks, one E8M0 scale each).
Expected values come from a pure-Python brute force that decodes nibbles and
scales itself, from integer arithmetic, and from closed forms."""
import zlib

import numpy as np

import oracle

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def rng(tag):
    return np.random.default_rng(zlib.crc32(tag.encode()))


def dec(byte, hi, scale):
    v = (int(byte) >> (4 * hi)) & 0xF
    return (-1.0 if v & 8 else 1.0) * E2M1[v & 7] * 2.0 ** (int(scale) - 127)


def test_mxgemm_matches_brute_force():
    r = rng("bf")
    M, N, K = 3, 4, 128
    a = r.integers(0, 256, (M, K // 2)).astype(np.uint8)
    b = r.integers(0, 256, (N, K // 2)).astype(np.uint8)
    sa = r.integers(110, 140, (M, K // 32)).astype(np.uint8)
    sb = r.integers(110, 140, (N, K // 32)).astype(np.uint8)
    want = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            want[m, n] = sum(dec(a[m, k // 2], k & 1, sa[m, k // 32]) * dec(b[n, k // 2], k & 1, sb[n, k // 32])
                             for k in range(K))
    assert np.array_equal(oracle.mxfp4_gemm(a, sa, b, sb), want)


def test_mxgemm_integer_case():
    """Unit scales and codes of the integers {0, 1, 2, 3, 4, 6} with signs: an
    integer matmul."""
    r = rng("int")
    M, N, K = 8, 16, 256
    idx = r.choice([0, 2, 4, 5, 6, 7], (M, K)) | (r.integers(0, 2, (M, K)) << 3)
    jdx = r.choice([0, 2, 4, 5, 6, 7], (N, K)) | (r.integers(0, 2, (N, K)) << 3)
    val = lambda t: np.where(t & 8, -1, 1) * np.array([0, 0, 1, 0, 2, 3, 4, 6])[t & 7]  # noqa: E731
    pack = lambda t: (t[:, 0::2] | (t[:, 1::2] << 4)).astype(np.uint8)  # noqa: E731
    one = lambda n: np.full((n, K // 32), 127, np.uint8)  # noqa: E731
    got = oracle.mxfp4_gemm(pack(idx), one(M), pack(jdx), one(N))
    assert np.array_equal(got, (val(idx) @ val(jdx).T).astype(np.float64))


def test_mxgemm_scale_is_per_block():
    """Raising one block scale of row m by 1 doubles exactly that block's part."""
    r = rng("blk")
    M, N, K = 4, 8, 128
    a = r.integers(0, 256, (M, K // 2)).astype(np.uint8)
    b = r.integers(0, 256, (N, K // 2)).astype(np.uint8)
    sa = np.full((M, K // 32), 127, np.uint8)
    sb = np.full((N, K // 32), 127, np.uint8)
    base = oracle.mxfp4_gemm(a, sa, b, sb)
    sa2 = sa.copy(); sa2[2, 1] += 1
    d = oracle.mxfp4_gemm(a, sa2, b, sb) - base
    assert np.all(d[[0, 1, 3]] == 0)
    part = oracle.mxfp4_gemm(a[2:3, 16:32], sa[2:3, 1:2], b[:, 16:32], sb[:, 1:2])
    assert np.array_equal(d[2], part[0])


def test_mxgemm_of_quantized_tensors_approximates_the_product():
    r = rng("e2e")
    x = r.standard_normal((32, 256)).astype(np.float32)
    w = (0.02 * r.standard_normal((64, 256))).astype(np.float32)
    ac, as_ = oracle.mxfp4_quantize(x[None])
    bc, bs = oracle.mxfp4_quantize(w[None])
    C = oracle.mxfp4_gemm(ac[0], as_[0], bc[0], bs[0])
    ref = x.astype(np.float64) @ w.T.astype(np.float64)
    assert np.median(np.abs(C - ref) / (np.abs(x) @ np.abs(w).T)) < 0.15
