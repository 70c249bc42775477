"""GPU parity of the MXFP4 x MXFP4 product (pqb_gemm_mxfp4) on the block-scaled
matrix cores against the oracle's float64 dequant(A) @ dequant(B)^T.

Two E2M1 values multiply to at most 4 significant bits, within 8 binades of
each other.  So the matrix core's groups of 8 products (truncated only more
than 13 binades below a group's largest exponent) sum exactly.  The scales
are powers of two.  What remains are float32 additions: the 16 group sums of
an instruction, and the accumulation over K / 128 instructions.  The bound is
  (17 + K/128) * 2^-24 * sum_k |a| |b|,
plus half a bf16 ulp of the value for bf16 output.  Unit-scale integer
inputs are exact."""
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


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def check(pqb, a, sa, b, sb, what, rows=None):
    M, Kh = a.shape
    K = 2 * Kh
    sel = np.arange(M) if rows is None else np.asarray(rows)
    want, S = oracle.mxfp4_gemm(a[sel], sa[sel], b, sb, abs_sum=True)
    tol = (17 + K // 128) * U * S * 1.01 + 1e-35
    for dt in (torch.float32, torch.bfloat16):
        got = pqb.gemm_mxfp4((dev(a), dev(sa)), (dev(b), dev(sb)), out_dtype=dt)
        got = got[torch.from_numpy(sel).to(DEV)].float().cpu().numpy().astype(np.float64)
        bound = tol if dt == torch.float32 else tol + 2.0 ** -8 * (np.abs(want) + tol)
        err = np.abs(got - want)
        bad = np.argwhere(err > bound)
        assert bad.size == 0, (f"{what} {dt}: {len(bad)} outside the bound, first {bad[:3].tolist()}, "
                               f"err {err[tuple(bad[0])]:.3e} bound {bound[tuple(bad[0])]:.3e}")


SHAPES = [(128, 128, 128), (256, 384, 512), (100, 256, 384), (1, 128, 1152), (300, 640, 2048),
          (129, 128, 640), (64, 256, 0)]


@pytest.mark.parametrize("shape", SHAPES)
def test_mxgemm_random_codes_match_oracle(pqb, shape):
    M, N, K = shape
    r = rng(f"mx{shape}")
    a = r.integers(0, 256, (M, K // 2)).astype(np.uint8)
    b = r.integers(0, 256, (N, K // 2)).astype(np.uint8)
    sa = r.integers(107, 147, (M, K // 32)).astype(np.uint8)
    sb = r.integers(107, 147, (N, K // 32)).astype(np.uint8)
    if K == 0:   # the empty sum
        for dt in (torch.float32, torch.bfloat16):
            got = pqb.gemm_mxfp4((dev(a), dev(sa)), (dev(b), dev(sb)), out_dtype=dt)
            assert got.shape == (M, N) and torch.count_nonzero(got).item() == 0
        return
    check(pqb, a, sa, b, sb, f"random {shape}")


def test_mxgemm_exact_on_unit_scale_integers(pqb):
    r = rng("int")
    M, N, K = 160, 256, 896
    idx = r.choice([0, 2, 4, 5, 6, 7], (M, K)) | (r.integers(0, 2, (M, K)) << 3)
    jdx = r.choice([0, 2, 4, 5, 6, 7], (N, K)) | (r.integers(0, 2, (N, K)) << 3)
    pack = lambda t: (t[:, 0::2] | (t[:, 1::2] << 4)).astype(np.uint8)  # noqa: E731
    one = lambda n: np.full((n, K // 32), 127, np.uint8)  # noqa: E731
    a, b = pack(idx), pack(jdx)
    got = pqb.gemm_mxfp4((dev(a), dev(one(M))), (dev(b), dev(one(N))), out_dtype=torch.float32)
    assert np.array_equal(got.cpu().numpy().astype(np.float64), oracle.mxfp4_gemm(a, one(M), b, one(N)))


def test_mxgemm_of_engine_quantized_tensors(pqb):
    """The engine quantizes activations and a weight to MXFP4 (byte-identical
    to the oracle's codes), and the product of those codes matches the oracle."""
    x = synth.fp8_activation(rows=256, cols=1024, device="cpu")
    w = synth.fp8_weight(rows=384, cols=1024, device="cpu")
    qa, qw = pqb.quantize(x.to(DEV), "mxfp4"), pqb.quantize(w.to(DEV), "mxfp4")
    ac, as_ = oracle.mxfp4_quantize(x[None])
    bc, bs = oracle.mxfp4_quantize(w[None])
    assert np.array_equal(qa.codes.cpu().numpy().reshape(ac[0].shape), ac[0])
    assert np.array_equal(qw.scales.cpu().numpy().reshape(bs[0].shape), bs[0])
    check(pqb, ac[0], as_[0], bc[0], bs[0], "engine-quantized")
    got = pqb.gemm_mxfp4(qa, qw).cpu().double().numpy()
    ref = x.double().numpy() @ w.double().numpy().T
    assert np.median(np.abs(got - ref) / (np.abs(x.double().numpy()) @ np.abs(w.double().numpy()).T)) < 0.15


@pytest.mark.parametrize("shape", [(8192, 7168, 2048), (8192, 2048, 7168)])
def test_mxgemm_full_size_sampled(pqb, shape):
    """The benchmark's shapes, activations [M x K] times a weight [N x K], both
    MXFP4, bf16 output: sampled rows of every column against the oracle."""
    M, N, K = shape
    x = synth.fp8_activation(rows=M, cols=K, device=DEV)
    w = synth.fp8_weight(rows=N, cols=K, device=DEV)
    qa, qw = pqb.quantize(x, "mxfp4"), pqb.quantize(w, "mxfp4")
    c = pqb.gemm_mxfp4(qa, qw, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.sort(rng("full").choice(M, 24, replace=False))
    rows[-1] = M - 1
    a, sa = qa.codes.cpu().numpy().reshape(M, K // 2), qa.scales.cpu().numpy().reshape(M, K // 32)
    b, sb = qw.codes.cpu().numpy().reshape(N, K // 2), qw.scales.cpu().numpy().reshape(N, K // 32)
    want, S = oracle.mxfp4_gemm(a[rows], sa[rows], b, sb, abs_sum=True)
    tol = (17 + K // 128) * U * S * 1.01
    got = c[torch.from_numpy(rows).to(DEV)].float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - want) <= tol + 2.0 ** -8 * (np.abs(want) + tol))
