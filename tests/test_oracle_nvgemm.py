"""Pins for the oracle's NVFP4 x NVFP4 product
C = float32(gsA gsB) * sum_k (V(a) dec(sa)) (V(b) dec(sb))
(page "量化部署实战", 格式速查, NVFP4 row: 16-element blocks with an E4M3 scale
each and a float32 tensor scale; page "14. 量化：让每一步搬更少的字节",
新一代低位格式: FP4 matrix units take the format directly).  Expected values
come from a pure-Python brute force that decodes nibbles and E4M3 bytes by
their bit fields, from the oracle's separate C dequantizer, from integer
arithmetic and from closed forms."""
import zlib

import numpy as np

import oracle

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def rng(tag):
    return np.random.default_rng(zlib.crc32(tag.encode()))


def e4m3_bits(b):
    """E4M3 value of a scale byte from its fields (sign 0, 4 exponent bits with
    bias 7, 3 mantissa bits; exponent field 0 is subnormal)."""
    e, m = (int(b) >> 3) & 15, int(b) & 7
    return (8 + m) * 2.0 ** (e - 10) if e else m * 2.0 ** -9


def elem(byte, hi):
    v = (int(byte) >> (4 * hi)) & 0xF
    return (-1.0 if v & 8 else 1.0) * E2M1[v & 7]


def random_operand(r, rows, K, lo=0, hi=127):
    codes = r.integers(0, 256, (rows, K // 2)).astype(np.uint8)
    scales = r.integers(lo, hi, (rows, K // 16)).astype(np.uint8)   # 0x7F (NaN) excluded
    return codes, scales


def test_nvgemm_matches_brute_force():
    r = rng("bf")
    M, N, K = 3, 5, 64
    a, sa = random_operand(r, M, K)
    b, sb = random_operand(r, N, K)
    ga, gb = np.float32(0.3), np.float32(1.7)
    g = float(np.float32(ga * gb))
    want = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            want[m, n] = g * sum(elem(a[m, k // 2], k & 1) * e4m3_bits(sa[m, k // 16]) *
                                 elem(b[n, k // 2], k & 1) * e4m3_bits(sb[n, k // 16]) for k in range(K))
    assert np.array_equal(oracle.nvfp4_gemm(a, sa, ga, b, sb, gb), want)


def test_nvgemm_integer_case():
    """Unit block scales (code 0x38 = 1.0), unit tensor scales and the integer
    codes {0, 1, 2, 3, 4, 6} with signs: an integer matmul."""
    r = rng("int")
    M, N, K = 8, 12, 128
    idx = r.choice([0, 2, 4, 5, 6, 7], (M, K)) | (r.integers(0, 2, (M, K)) << 3)
    jdx = r.choice([0, 2, 4, 5, 6, 7], (N, K)) | (r.integers(0, 2, (N, K)) << 3)
    val = lambda t: np.where(t & 8, -1, 1) * np.array([0, 0, 1, 0, 2, 3, 4, 6])[t & 7]  # noqa: E731
    pack = lambda t: (t[:, 0::2] | (t[:, 1::2] << 4)).astype(np.uint8)  # noqa: E731
    one = lambda n: np.full((n, K // 16), 0x38, np.uint8)  # noqa: E731
    got = oracle.nvfp4_gemm(pack(idx), one(M), 1.0, pack(jdx), one(N), 1.0)
    assert np.array_equal(got, (val(idx) @ val(jdx).T).astype(np.float64))


def test_nvgemm_block_scale_is_per_16_elements():
    """Changing one block scale of row m changes only row m, by exactly that
    16-element block's part; a block scale code of 0 removes the block."""
    r = rng("blk")
    M, N, K = 4, 6, 128
    a, sa = random_operand(r, M, K, 40, 70)
    b, sb = random_operand(r, N, K, 40, 70)
    base = oracle.nvfp4_gemm(a, sa, 1.0, b, sb, 1.0)
    sa2 = sa.copy()
    sa2[2, 5] = 0x38 + 8                                   # 2.0
    d = oracle.nvfp4_gemm(a, sa2, 1.0, b, sb, 1.0) - base
    assert np.all(d[[0, 1, 3]] == 0)
    ks = slice(5 * 16, 6 * 16)
    part = [sum(elem(a[2, k // 2], k & 1) * elem(b[n, k // 2], k & 1) * e4m3_bits(sb[n, k // 16])
                for k in range(ks.start, ks.stop)) for n in range(N)]
    assert np.array_equal(d[2], (2.0 - e4m3_bits(sa[2, 5])) * np.array(part))
    sa0 = sa.copy()
    sa0[1, 3] = 0
    a0 = a.copy()
    a0[1, 3 * 8:4 * 8] = 0                                 # the same block's codes zeroed
    assert np.array_equal(oracle.nvfp4_gemm(a, sa0, 1.0, b, sb, 1.0), oracle.nvfp4_gemm(a0, sa, 1.0, b, sb, 1.0))


def test_nvgemm_subnormal_scales():
    """Scale codes 1..7 are the E4M3 subnormals m * 2^-9."""
    K = 16
    a = np.full((1, K // 2), 0x22, np.uint8)               # every element 1.0
    b = np.full((1, K // 2), 0x22, np.uint8)
    for m in range(1, 8):
        got = oracle.nvfp4_gemm(a, np.full((1, 1), m, np.uint8), 1.0, b, np.full((1, 1), 0x38, np.uint8), 1.0)
        assert got[0, 0] == 16 * m * 2.0 ** -9


def test_nvgemm_tensor_scales_enter_as_their_float32_product():
    a = np.full((1, 8), 0x22, np.uint8)
    s = np.full((1, 1), 0x38, np.uint8)
    ga, gb = np.float32(1.0 / 3.0), np.float32(3.0)
    got = oracle.nvfp4_gemm(a, s, ga, a, s, gb)[0, 0]
    assert got == 16.0 * float(np.float32(ga * gb)) and float(np.float32(ga * gb)) != float(ga) * float(gb)


def test_nvgemm_equals_product_of_dequantized_operands():
    """On quantized data (no block scale code 0) the product equals the float64
    matmul of the oracle's C dequantizer output within that dequantizer's
    float32 rounding of dec(s) * gs (at most 2^-24 relative per operand)."""
    r = rng("deq")
    x = r.standard_normal((24, 256)).astype(np.float32)
    w = (0.05 * r.standard_normal((40, 256))).astype(np.float32)
    ac, as_, ag = oracle.nvfp4_quantize(x[None])
    bc, bs, bg = oracle.nvfp4_quantize(w[None])
    assert (as_ > 0).all() and (bs > 0).all()
    C, S = oracle.nvfp4_gemm(ac[0], as_[0], ag, bc[0], bs[0], bg, abs_sum=True)
    A = oracle.nvfp4_dequantize(ac, as_, ag)[0].astype(np.float64)
    B = oracle.nvfp4_dequantize(bc, bs, bg)[0].astype(np.float64)
    assert np.all(np.abs(C - A @ B.T) <= 3 * 2.0 ** -24 * np.abs(A) @ np.abs(B).T)
    assert np.all(np.abs(S - np.abs(A) @ np.abs(B).T) <= 3 * 2.0 ** -24 * S)


def test_nvgemm_of_quantized_tensors_approximates_the_product():
    r = rng("e2e")
    x = r.standard_normal((32, 256)).astype(np.float32)
    w = (0.02 * r.standard_normal((64, 256))).astype(np.float32)
    ac, as_, ag = oracle.nvfp4_quantize(x[None])
    bc, bs, bg = oracle.nvfp4_quantize(w[None])
    C = oracle.nvfp4_gemm(ac[0], as_[0], ag, bc[0], bs[0], bg)
    ref = x.astype(np.float64) @ w.T.astype(np.float64)
    assert np.median(np.abs(C - ref) / (np.abs(x) @ np.abs(w).T)) < 0.12
