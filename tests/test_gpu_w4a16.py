"""GPU parity of the W4A16 product (pqb_gemv_w4a16) against the oracle's
float64 y = x @ dequant(W)^T, element by element, within a bound derived from
the kernel's float32 evaluation.

For each unit of 32 weights of one group, the kernel forms s * (sum x w -
(136 + z) sum x), where w = 136 + q (in 128 .. 143) is the code as an exact
bf16.  The products x w are exact.  The two 32-term sums (pairs of products
added into a float32 accumulator) round at most 32 times each, and the two
fused multiply-adds once each.  The units of a row are accumulated per lane
(at most K/2048 + 1 additions), then summed over 64 lanes (6 levels).  First
order, the error is at most
  (40 + K/2048) * 2^-24 * sum_k |s| |x| (|136 + q| + |136 + z|),
plus half a bf16 ulp of the value for bf16 output."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from precision_quantization_block_amd import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
U = 2.0 ** -24


@pytest.fixture(scope="module")
def pqb():
    import precision_quantization_block_amd as p
    p.lib()
    return p


def rng(tag):
    return np.random.default_rng(zlib.crc32(tag.encode()))


def bound(xb, codes, scales, zeros):
    """sum_k |s| |x| (|136 + q| + |136 + z|) for every (m, n)."""
    N = codes.shape[-2]
    K = codes.shape[-1] * 2
    c = codes.reshape(N, K // 2).astype(np.int32)
    q = np.empty((N, K), np.int32)
    q[:, 0::2] = c & 0xF
    q[:, 1::2] = c >> 4
    q = np.where(q >= 8, q - 16, q)
    G = K // 128
    zn = np.stack([zeros & 0xF, zeros >> 4], 1).reshape(-1)[:N * G].astype(np.int32).reshape(N, G)
    z = np.where(zn >= 8, zn - 16, zn)
    s = np.abs(oracle.bf16_bits_to_f32(scales.reshape(N, G)).astype(np.float64))
    A = np.repeat(s, 128, axis=1) * (np.abs(136 + q) + np.repeat(np.abs(136 + z), 128, axis=1))
    return np.abs(oracle.bf16_bits_to_f32(xb).astype(np.float64)) @ A.T


def bf16_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def check(pqb, xb, codes, scales, zeros, what):
    M, K = xb.shape
    N = codes.shape[-2]
    want = oracle.w4a16_gemv(xb, codes, scales, zeros)
    tol = (40 + K // 2048) * U * bound(xb, codes, scales, zeros) * 1.01 + 1e-30
    xd = torch.from_numpy(xb.view(np.int16)).to(DEV).view(torch.bfloat16)
    w = tuple(torch.from_numpy(np.ascontiguousarray(t)).to(DEV) for t in (codes, scales.view(np.int16), zeros))
    for dt in (torch.float32, torch.bfloat16):
        got = pqb.gemv_w4a16(xd, w, out_dtype=dt).float().cpu().numpy().astype(np.float64)
        b = tol if dt == torch.float32 else tol + 2.0 ** -8 * (np.abs(want) + tol)
        err = np.abs(got - want)
        bad = np.argwhere(err > b)
        assert bad.size == 0, (f"{what} {dt}: {len(bad)} outside the bound, first {bad[:3].tolist()}, "
                               f"err {err[tuple(bad[0])]:.3e} bound {b[tuple(bad[0])]:.3e}")


SHAPES = [(1, 128, 128), (1, 1000, 4096), (3, 333, 2176), (8, 64, 14336), (4, 257, 384),
          (2, 4096, 1024), (5, 9, 128 * 50), (6, 130, 512), (7, 77, 1152)]


@pytest.mark.parametrize("shape", SHAPES)
def test_w4a16_matches_oracle(pqb, shape):
    M, N, K = shape
    r = rng(f"w4{shape}")
    w = (0.02 * r.standard_normal((N, K)) * np.exp(r.uniform(-2, 2, (N, 1)))).astype(np.float32)
    codes, scales, zeros = oracle.int4_quantize(w[None])
    x = bf16_bits(r.standard_normal((M, K)) * np.exp(r.uniform(-3, 3, (1, K))))
    check(pqb, x, codes[0], scales[0], zeros, f"w4a16 {shape}")


def test_w4a16_exact_integer_case(pqb):
    """Dequantized weights that are small integers and integer activations:
    every term and every partial sum is an integer below 2^24, so the float32
    result equals the integer matmul exactly."""
    r = rng("int")
    N, K = 96, 1024
    w = r.integers(-7, 8, (N, K)).astype(np.float32)
    w[:, ::128], w[:, 1::128] = 7.0, -8.0
    codes, scales, zeros = oracle.int4_quantize(w[None])
    x = r.integers(-20, 21, (2, K)).astype(np.float32)
    xb = bf16_bits(x)
    xd = torch.from_numpy(xb.view(np.int16)).to(DEV).view(torch.bfloat16)
    wt = tuple(torch.from_numpy(np.ascontiguousarray(t)).to(DEV) for t in (codes[0], scales[0].view(np.int16), zeros))
    got = pqb.gemv_w4a16(xd, wt, out_dtype=torch.float32).cpu().numpy()
    assert np.array_equal(got.astype(np.int64), x.astype(np.int64) @ w.T.astype(np.int64))


def test_w4a16_engine_quantized_llama_weights(pqb):
    """The decode chain on the GPU: the engine quantizes Llama-3.1-8B-shaped
    weights (gate [14336 x 4096] and down [4096 x 14336] of layer 0) to INT4
    g128, byte-identical to the oracle's codes, and the product of one decode
    token against them matches the oracle."""
    r = rng("llama")
    for proj in (4, 6):
        w = synth.llama_weight(0, proj, device=DEV)
        q = pqb.quantize(w, "int4_asym", "grp128")
        N, K = w.shape
        x = bf16_bits(r.standard_normal((1, K)))
        c, s, z = q.codes.cpu().numpy().reshape(N, K // 2), q.scales.cpu().view(torch.int16).numpy() \
            .view(np.uint16).reshape(N, K // 128), q.aux.cpu().numpy()
        oc, os_, oz = oracle.int4_quantize(w.cpu()[None])
        assert np.array_equal(c, oc[0]) and np.array_equal(s, os_[0]) and np.array_equal(z, oz)
        check(pqb, x, c, s, z, f"llama proj {proj}")


def test_w4a16_batch_equals_single_calls(pqb):
    """A batch of 40 products of mixed shapes (two launches) gives, bit for bit,
    the single-call results, which match the oracle above."""
    r = rng("batch")
    shapes = [(int(r.integers(1, 300)), 128 * int(r.integers(1, 40))) for _ in range(40)]
    xs, ws = [], []
    for N, K in shapes:
        w = (0.02 * r.standard_normal((N, K))).astype(np.float32)
        codes, scales, zeros = oracle.int4_quantize(w[None])
        ws.append(tuple(torch.from_numpy(np.ascontiguousarray(t)).to(DEV)
                        for t in (codes[0], scales[0].view(np.int16), zeros)))
        xs.append(torch.from_numpy(bf16_bits(r.standard_normal((3, K))).view(np.int16)).to(DEV)
                  .view(torch.bfloat16))
    ys = pqb.gemv_w4a16_batch(xs, ws, out_dtype=torch.float32)
    for i in (0, 7, 31, 32, 39):
        one = pqb.gemv_w4a16(xs[i], ws[i], out_dtype=torch.float32)
        assert torch.equal(ys[i], one), i
    i = 33
    c, s, z = (t.cpu().numpy() for t in ws[i])
    check(pqb, xs[i].cpu().view(torch.int16).numpy().view(np.uint16), c, s.view(np.uint16), z,
          "batch job 33")


def test_w4a16_degenerate_sizes(pqb):
    """k = 0 is the empty sum (y = 0, also inside a batch beside a real job);
    m = 0 and n = 0 launch nothing."""
    for dt in (torch.float32, torch.bfloat16):
        for M, N in ((1, 5), (3, 300), (8, 70000)):
            x = torch.empty((M, 0), dtype=torch.bfloat16, device=DEV)
            codes = torch.empty((N, 0), dtype=torch.uint8, device=DEV)
            empty = (codes, torch.empty((N, 0), dtype=torch.int16, device=DEV),
                     torch.empty((0,), dtype=torch.uint8, device=DEV))
            y = pqb.gemv_w4a16(x, empty, out_dtype=dt)
            assert y.shape == (M, N) and bool((y == 0).all()), (dt, M, N)
    x = torch.randn((2, 256), device=DEV).to(torch.bfloat16)
    r = rng("deg")
    w = (0.02 * r.standard_normal((130, 256))).astype(np.float32)
    codes, scales, zeros = oracle.int4_quantize(w[None])
    wt = tuple(torch.from_numpy(np.ascontiguousarray(t)).to(DEV) for t in (codes[0], scales[0].view(np.int16), zeros))
    empty = (torch.empty((130, 0), dtype=torch.uint8, device=DEV), torch.empty((130, 0), dtype=torch.int16, device=DEV),
             torch.empty((0,), dtype=torch.uint8, device=DEV))
    ys = pqb.gemv_w4a16_batch([x, x[:, :0]], [wt, empty], out_dtype=torch.float32)
    assert torch.equal(ys[0], pqb.gemv_w4a16(x, wt, out_dtype=torch.float32))
    assert ys[1].shape == (2, 130) and bool((ys[1] == 0).all())
    assert pqb.gemv_w4a16(x[:0], wt).shape == (0, 130)
    none = (torch.empty((0, 128), dtype=torch.uint8, device=DEV), torch.empty((0, 2), dtype=torch.int16, device=DEV),
            torch.empty((0,), dtype=torch.uint8, device=DEV))
    assert pqb.gemv_w4a16(x, none).shape == (2, 0)


def test_w4a16_subnormal_activations(pqb):
    """Activations below 2^-126 (bf16 subnormals) keep their value: one row of
    x is all subnormal, one mixes subnormal and normal values."""
    r = rng("subn")
    N, K = 200, 1024
    w = (0.02 * r.standard_normal((N, K))).astype(np.float32)
    codes, scales, zeros = oracle.int4_quantize(w[None])
    x = np.empty((2, K), np.uint16)
    x[0] = r.integers(1, 0x80, K) | (r.integers(0, 2, K) << 15)          # +-subnormal
    x[1] = np.where(r.random(K) < 0.5, x[0], bf16_bits(r.standard_normal(K)))
    check(pqb, x, codes[0], scales[0], zeros, "subnormal x")


@pytest.mark.parametrize("M", range(1, 9))
def test_w4a16_large_launch_shape(pqb, M):
    """A launch of more than 65536 rows takes the 8-rows-per-wave shape at M <=
    2, the 4-row shape at M = 3 .. 5 and the 2-row shape above.  All against the
    oracle, with a ragged N."""
    r = rng(f"big{M}")
    N, K = 66001, 256
    w = (0.02 * r.standard_normal((N, K))).astype(np.float32)
    codes, scales, zeros = oracle.int4_quantize(w[None])
    x = bf16_bits(r.standard_normal((M, K)))
    check(pqb, x, codes[0], scales[0], zeros, f"large launch M={M}")


# ------------------------------------------------- matrix-core form, any M --
# pqb_gemm_w4a16 evaluates each group of 128 as s * (P - (136 + z) S), where
# P = sum x w and S = sum x are float32 matrix-core accumulations of exact
# products, 32 per instruction, four instructions per group; then the groups
# of each of four partial sums are added, and the four partial sums.  Counting
# every one of the 128 additions of a group as one rounding, and twice that
# for a matrix core that rounds each partial sum, the error is at most
#   (256 + K/64) * 2^-24 * sum_k |s| |x| (|136 + q| + |136 + z|).

def check_mfma(pqb, xb, codes, scales, zeros, what):
    M, K = xb.shape
    want = oracle.w4a16_gemv(xb, codes, scales, zeros)
    tol = (256 + K // 64) * U * bound(xb, codes, scales, zeros) * 1.01 + 1e-30
    xd = torch.from_numpy(xb.view(np.int16)).to(DEV).view(torch.bfloat16)
    w = tuple(torch.from_numpy(np.ascontiguousarray(t)).to(DEV) for t in (codes, scales.view(np.int16), zeros))
    for dt in (torch.float32, torch.bfloat16):
        got = pqb.gemm_w4a16(xd, w, out_dtype=dt).float().cpu().numpy().astype(np.float64)
        b = tol if dt == torch.float32 else tol + 2.0 ** -8 * (np.abs(want) + tol)
        err = np.abs(got - want)
        bad = np.argwhere(err > b)
        assert bad.size == 0, (f"{what} {dt}: {len(bad)} outside the bound, first {bad[:3].tolist()}, "
                               f"err {err[tuple(bad[0])]:.3e} bound {b[tuple(bad[0])]:.3e}")


MFMA_SHAPES = [(1, 128, 128), (4, 1000, 4096), (9, 333, 2176), (16, 64, 14336), (17, 257, 384),
               (32, 4096, 1024), (33, 9, 128 * 50), (100, 130, 512), (70, 77, 1152), (5, 16, 256),
               (2, 1, 128 * 3)]


@pytest.mark.parametrize("shape", MFMA_SHAPES)
def test_w4a16_matrix_cores_match_oracle(pqb, shape):
    """Several 16-row activation blocks and 32-row launch slices, ragged N (not
    a multiple of 16), odd group counts (a half-empty last chunk) and K from
    one group to 112."""
    M, N, K = shape
    r = rng(f"w4m{shape}")
    w = (0.02 * r.standard_normal((N, K)) * np.exp(r.uniform(-2, 2, (N, 1)))).astype(np.float32)
    codes, scales, zeros = oracle.int4_quantize(w[None])
    x = bf16_bits(r.standard_normal((M, K)) * np.exp(r.uniform(-3, 3, (1, K))))
    check_mfma(pqb, x, codes[0], scales[0], zeros, f"w4a16 mfma {shape}")


def test_w4a16_matrix_cores_exact_integer_case(pqb):
    """Small-integer weights and activations: every product, partial sum and
    correction is an integer below 2^24, so the result is the integer matmul."""
    r = rng("intm")
    N, K = 96, 1024
    w = r.integers(-7, 8, (N, K)).astype(np.float32)
    w[:, ::128], w[:, 1::128] = 7.0, -8.0
    codes, scales, zeros = oracle.int4_quantize(w[None])
    x = r.integers(-20, 21, (40, K)).astype(np.float32)
    xd = torch.from_numpy(bf16_bits(x).view(np.int16)).to(DEV).view(torch.bfloat16)
    wt = tuple(torch.from_numpy(np.ascontiguousarray(t)).to(DEV) for t in (codes[0], scales[0].view(np.int16), zeros))
    got = pqb.gemm_w4a16(xd, wt, out_dtype=torch.float32).cpu().numpy()
    assert np.array_equal(got.astype(np.int64), x.astype(np.int64) @ w.T.astype(np.int64))


def test_w4a16_matrix_cores_batch_equals_single_calls(pqb):
    """40 products of mixed shapes at M = 20 (two launches of jobs, one slice
    of rows) give, bit for bit, the single-call results."""
    r = rng("batchm")
    shapes = [(int(r.integers(1, 300)), 128 * int(r.integers(1, 40))) for _ in range(40)]
    xs, ws = [], []
    for N, K in shapes:
        w = (0.02 * r.standard_normal((N, K))).astype(np.float32)
        codes, scales, zeros = oracle.int4_quantize(w[None])
        ws.append(tuple(torch.from_numpy(np.ascontiguousarray(t)).to(DEV)
                        for t in (codes[0], scales[0].view(np.int16), zeros)))
        xs.append(torch.from_numpy(bf16_bits(r.standard_normal((20, K))).view(np.int16)).to(DEV)
                  .view(torch.bfloat16))
    ys = pqb.gemm_w4a16_batch(xs, ws, out_dtype=torch.float32)
    for i in (0, 7, 31, 32, 39):
        assert torch.equal(ys[i], pqb.gemm_w4a16(xs[i], ws[i], out_dtype=torch.float32)), i
    i = 33
    c, s, z = (t.cpu().numpy() for t in ws[i])
    check_mfma(pqb, xs[i].cpu().view(torch.int16).numpy().view(np.uint16), c, s.view(np.uint16), z,
               "batch job 33")


def test_w4a16_matrix_cores_rows_are_independent(pqb):
    """Row m of the output depends only on row m of x: a 70-row product equals,
    bit for bit, the products of its rows taken one at a time and in slices
    that cross the 16- and 32-row boundaries differently."""
    r = rng("rowsm")
    N, K = 200, 768
    w = (0.02 * r.standard_normal((N, K))).astype(np.float32)
    codes, scales, zeros = oracle.int4_quantize(w[None])
    wt = tuple(torch.from_numpy(np.ascontiguousarray(t)).to(DEV) for t in (codes[0], scales[0].view(np.int16), zeros))
    x = torch.from_numpy(bf16_bits(r.standard_normal((70, K))).view(np.int16)).to(DEV).view(torch.bfloat16)
    full = pqb.gemm_w4a16(x, wt, out_dtype=torch.float32)
    for m in (0, 15, 16, 31, 32, 47, 69):
        assert torch.equal(pqb.gemm_w4a16(x[m:m + 1].contiguous(), wt, out_dtype=torch.float32)[0], full[m]), m
    assert torch.equal(pqb.gemm_w4a16(x[5:42].contiguous(), wt, out_dtype=torch.float32), full[5:42])


def test_w4a16_matrix_cores_degenerate_sizes(pqb):
    """k = 0 writes zeros (also inside a batch), m = 0 and n = 0 launch nothing."""
    for dt in (torch.float32, torch.bfloat16):
        for M, N in ((1, 5), (33, 300), (8, 70000)):
            x = torch.empty((M, 0), dtype=torch.bfloat16, device=DEV)
            empty = (torch.empty((N, 0), dtype=torch.uint8, device=DEV),
                     torch.empty((N, 0), dtype=torch.int16, device=DEV),
                     torch.empty((0,), dtype=torch.uint8, device=DEV))
            y = pqb.gemm_w4a16(x, empty, out_dtype=dt)
            assert y.shape == (M, N) and bool((y == 0).all()), (dt, M, N)
    r = rng("degm")
    w = (0.02 * r.standard_normal((130, 256))).astype(np.float32)
    codes, scales, zeros = oracle.int4_quantize(w[None])
    wt = tuple(torch.from_numpy(np.ascontiguousarray(t)).to(DEV) for t in (codes[0], scales[0].view(np.int16), zeros))
    x = torch.from_numpy(bf16_bits(r.standard_normal((3, 256))).view(np.int16)).to(DEV).view(torch.bfloat16)
    empty = (torch.empty((130, 0), dtype=torch.uint8, device=DEV), torch.empty((130, 0), dtype=torch.int16, device=DEV),
             torch.empty((0,), dtype=torch.uint8, device=DEV))
    ys = pqb.gemm_w4a16_batch([x, x[:, :0]], [wt, empty], out_dtype=torch.float32)
    assert torch.equal(ys[0], pqb.gemm_w4a16(x, wt, out_dtype=torch.float32))
    assert ys[1].shape == (3, 130) and bool((ys[1] == 0).all())
    assert pqb.gemm_w4a16(x[:0], wt).shape == (0, 130)


def test_w4a16_matrix_cores_subnormal_activations(pqb):
    """bf16 subnormal activations keep their value on the matrix cores too."""
    r = rng("subnm")
    N, K = 200, 1024
    w = (0.02 * r.standard_normal((N, K))).astype(np.float32)
    codes, scales, zeros = oracle.int4_quantize(w[None])
    x = np.empty((2, K), np.uint16)
    x[0] = r.integers(1, 0x80, K) | (r.integers(0, 2, K) << 15)
    x[1] = np.where(r.random(K) < 0.5, x[0], bf16_bits(r.standard_normal(K)))
    check_mfma(pqb, x, codes[0], scales[0], zeros, "subnormal x (matrix cores)")


def test_w4a16_matrix_cores_engine_quantized_llama_weights(pqb):
    """A 16-token chunk against the engine's INT4 codes of Llama-3.1-8B-shaped
    gate [14336 x 4096] and down [4096 x 14336] weights of layer 0."""
    r = rng("llamam")
    for proj in (4, 6):
        w = synth.llama_weight(0, proj, device=DEV)
        q = pqb.quantize(w, "int4_asym", "grp128")
        N, K = w.shape
        c, s, z = q.codes.cpu().numpy().reshape(N, K // 2), q.scales.cpu().view(torch.int16).numpy() \
            .view(np.uint16).reshape(N, K // 128), q.aux.cpu().numpy()
        check_mfma(pqb, bf16_bits(r.standard_normal((16, K))), c, s, z, f"llama proj {proj} M=16")


@pytest.mark.parametrize("M", [1, 17, 40])
def test_w4a16_matrix_cores_large_launch(pqb, M):
    """A launch of 2^14 weight rows or more takes four 16-row tiles per
    workgroup (smaller launches one): a ragged N = 66001 with M in one block,
    two blocks, and two launch slices."""
    r = rng(f"bigm{M}")
    N, K = 66001, 256
    w = (0.02 * r.standard_normal((N, K))).astype(np.float32)
    codes, scales, zeros = oracle.int4_quantize(w[None])
    check_mfma(pqb, bf16_bits(r.standard_normal((M, K))), codes[0], scales[0], zeros,
               f"large launch M={M}")


@pytest.mark.parametrize("N", [16383, 16400])
@pytest.mark.parametrize("M", [3, 17, 40])
def test_w4a16_matrix_cores_launch_threshold(pqb, M, N):
    """Four tiles per workgroup from 2^14 weight rows on: N on both sides of
    that threshold (ragged above it), M in one 16-row block (3), in two (17)
    and in two launch slices (40 = 32 + 8)."""
    r = rng(f"widem{M}n{N}")
    K = 256
    w = (0.02 * r.standard_normal((N, K))).astype(np.float32)
    codes, scales, zeros = oracle.int4_quantize(w[None])
    check_mfma(pqb, bf16_bits(r.standard_normal((M, K))), codes[0], scales[0], zeros,
               f"wide launch M={M} N={N}")
