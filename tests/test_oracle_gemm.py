"""Pins for the oracle's block-scaled FP8 GEMM (page "量化部署实战", exercise
section on FP8 blockwise scaling: FP8 products summed per 128-deep K block,
each block sum multiplied by that block's activation and weight scales, then
accumulated).  Expected values come from a pure-Python brute force over torch's
E4M3 decoding, from integer arithmetic, and from closed forms; none re-calls
the oracle's own arithmetic."""
import zlib

import numpy as np
import pytest
import torch

import oracle


def rng(tag):
    return np.random.default_rng(zlib.crc32(tag.encode()))


def random_codes(r, shape):
    c = r.integers(0, 256, shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38                  # no NaN codes
    return c


def torch_dec(codes):
    return torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()


def test_gemm_matches_brute_force_loops():
    r = rng("bf")
    M, N, K = 3, 128, 256
    a, b = random_codes(r, (M, K)), random_codes(r, (N, K))
    sa = r.uniform(0.1, 3, (M, K // 128)).astype(np.float32)
    sb = r.uniform(0.1, 3, (N // 128, K // 128)).astype(np.float32)
    da, db = torch_dec(a).tolist(), torch_dec(b).tolist()
    want = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            tot = 0.0
            for kb in range(K // 128):
                p = 0.0
                for k in range(128 * kb, 128 * kb + 128):
                    p += da[m][k] * db[n][k]
                tot += float(sa[m, kb]) * float(sb[n // 128, kb]) * p
            want[m, n] = tot
    got = oracle.fp8_block_gemm(a, sa, b, sb)
    assert np.allclose(got, want, rtol=1e-13, atol=1e-13 * np.abs(want).max())


def test_gemm_small_integers_are_exact():
    """Codes of small integers with power-of-two scales: C equals an integer
    matmul scaled exactly."""
    r = rng("int")
    M, N, K = 40, 256, 384
    vals = np.arange(-8, 9)
    ia = r.choice(vals, (M, K))
    ib = r.choice(vals, (N, K))
    ea = oracle.e4m3_encode_array(ia.astype(np.float32))
    eb = oracle.e4m3_encode_array(ib.astype(np.float32))
    assert np.array_equal(torch_dec(ea), ia) and np.array_equal(torch_dec(eb), ib)
    xa = r.integers(-3, 4, (M, K // 128))
    xb = r.integers(-3, 4, (N // 128, K // 128))
    got = oracle.fp8_block_gemm(ea, np.ldexp(1.0, xa).astype(np.float32), eb,
                                np.ldexp(1.0, xb).astype(np.float32))
    want = np.zeros((M, N))
    for kb in range(K // 128):
        ks = slice(128 * kb, 128 * kb + 128)
        P = ia[:, ks].astype(np.int64) @ ib[:, ks].T.astype(np.int64)
        want += np.ldexp(P.astype(np.float64), xa[:, kb, None] + np.repeat(xb[:, kb], 128)[None, :])
    assert np.array_equal(got, want)


def test_gemm_one_hot_rows_pick_weight_columns():
    """a[m, k] = 1 at k = m only: C[m, n] = dec(b[n, m]) * sa[m, m // 128] * sb[n // 128, m // 128]."""
    r = rng("hot")
    M, N, K = 256, 128, 256
    a = np.zeros((M, K), np.uint8)
    a[np.arange(M), np.arange(M)] = 0x38                     # 1.0
    b = random_codes(r, (N, K))
    sa = r.uniform(0.5, 2, (M, K // 128)).astype(np.float32)
    sb = r.uniform(0.5, 2, (N // 128, K // 128)).astype(np.float32)
    got = oracle.fp8_block_gemm(a, sa, b, sb)
    m = np.arange(M)
    want = torch_dec(b).T * sa[m, m // 128][:, None].astype(np.float64) \
        * sb[0, m // 128][:, None].astype(np.float64)
    assert np.array_equal(got, want)


def test_gemm_scales_act_per_block():
    """Doubling one activation scale sa[m, kb] adds exactly that block's term to
    row m; doubling one weight scale adds it to that 128-row group of columns."""
    r = rng("blk")
    M, N, K = 8, 256, 384
    a, b = random_codes(r, (M, K)), random_codes(r, (N, K))
    sa = np.ldexp(1.0, r.integers(-2, 3, (M, 3))).astype(np.float32)
    sb = np.ldexp(1.0, r.integers(-2, 3, (2, 3))).astype(np.float32)
    base = oracle.fp8_block_gemm(a, sa, b, sb)
    sa2 = sa.copy(); sa2[5, 1] *= 2
    d = oracle.fp8_block_gemm(a, sa2, b, sb) - base
    assert np.all(d[np.arange(M) != 5] == 0)
    P = torch_dec(a)[5, 128:256] @ torch_dec(b)[:, 128:256].T
    assert np.array_equal(d[5], P * float(sa[5, 1]) * np.repeat(sb[:, 1], 128).astype(np.float64))
    sb2 = sb.copy(); sb2[1, 2] *= 2
    d = oracle.fp8_block_gemm(a, sa, b, sb2) - base
    assert np.all(d[:, :128] == 0) and np.any(d[:, 128:] != 0)


def test_gemm_of_quantized_tensors_approximates_the_product():
    """End to end with the oracle's own quantizers: C approximates x @ w.T
    within the FP8 error (a transposed operand or a misplaced scale would
    not), and the absolute sum bounds |C|."""
    r = rng("e2e")
    x = r.standard_normal((64, 512)).astype(np.float32)
    w = (0.02 * r.standard_normal((256, 512))).astype(np.float32)
    ac, as_ = oracle.fp8_quantize(x[None], "1x128")
    bc, bs = oracle.fp8_quantize(w[None], "128x128")
    C, S = oracle.fp8_block_gemm(ac[0], as_[0], bc[0], bs[0], abs_sum=True)
    ref = x.astype(np.float64) @ w.T.astype(np.float64)
    err = np.abs(C - ref)
    assert np.all(np.abs(C) <= S)
    assert err.max() < 0.1 * np.abs(ref).max()
    assert np.median(err / (np.abs(x) @ np.abs(w).T)) < 0.03


def test_gemm_shape_errors():
    with pytest.raises(ValueError):
        oracle.fp8_block_gemm(np.zeros((4, 100), np.uint8), np.zeros((4, 1), np.float32),
                              np.zeros((128, 100), np.uint8), np.zeros((1, 1), np.float32))
    with pytest.raises(ValueError):
        oracle.fp8_block_gemm(np.zeros((4, 128), np.uint8), np.zeros((4, 1), np.float32),
                              np.zeros((100, 128), np.uint8), np.zeros((1, 1), np.float32))
