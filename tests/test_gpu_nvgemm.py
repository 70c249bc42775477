"""GPU parity of the NVFP4 x NVFP4 product (pqb_gemm_nvfp4) on the f16 matrix
cores against the oracle's float64 C = float32(gsA gsB) * sum_k A' B'.

Every scaled element V * dec(s) has at most 6 significant bits between 2^-10
and 2688, so it is exact in f16.  Each product of two of them is exact in
float32 as well.  What rounds are the float32 additions: at most 31 within one
32-deep matrix-core step (whatever order it sums in), one per step into the
accumulator, K/32 steps, and the final multiply by g.  That gives
  |C - C_exact| <= (34 + K/32) * 2^-24 * g * sum_k |A'| |B'|,
plus half a bf16 ulp of the value for bf16 output.  Unit-scale integer inputs
are exact."""
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


def operand(r, rows, K, lo=1, hi=127):
    codes = r.integers(0, 256, (rows, K // 2)).astype(np.uint8)
    scales = r.integers(lo, hi, (rows, K // 16)).astype(np.uint8)     # no 0x7F (NaN)
    return codes, scales


def check(pqb, a, sa, ga, b, sb, gb, what, rows=None):
    M, Kh = a.shape
    K = 2 * Kh
    sel = np.arange(M) if rows is None else np.asarray(rows)
    want, S = oracle.nvfp4_gemm(a[sel], sa[sel], ga, b, sb, gb, abs_sum=True)
    tol = (34 + K // 32) * U * S * 1.01 + 1e-38
    A = (dev(a), dev(sa), dev(np.float32([ga])))
    B = (dev(b), dev(sb), dev(np.float32([gb])))
    for dt in (torch.float32, torch.bfloat16):
        got = pqb.gemm_nvfp4(A, B, out_dtype=dt)
        got = got[torch.from_numpy(sel).to(DEV)].float().cpu().numpy().astype(np.float64)
        bound = tol if dt == torch.float32 else tol + 2.0 ** -8 * (np.abs(want) + tol)
        err = np.abs(got - want)
        bad = np.argwhere(err > bound)
        assert bad.size == 0, (f"{what} {dt}: {len(bad)} outside the bound, first {bad[:3].tolist()}, "
                               f"err {err[tuple(bad[0])]:.3e} bound {bound[tuple(bad[0])]:.3e}")


SHAPES = [(128, 128, 128), (256, 384, 512), (100, 256, 384), (1, 128, 1152), (300, 640, 2048),
          (129, 128, 640), (64, 256, 0)]


@pytest.mark.parametrize("shape", SHAPES)
def test_nvgemm_random_codes_match_oracle(pqb, shape):
    M, N, K = shape
    r = rng(f"nv{shape}")
    a, sa = operand(r, M, K, 40, 80)
    b, sb = operand(r, N, K, 40, 80)
    ga, gb = np.float32(r.uniform(0.01, 2.0)), np.float32(r.uniform(0.01, 2.0))
    if K == 0:   # the empty sum; scales are not read
        for dt in (torch.float32, torch.bfloat16):
            got = pqb.gemm_nvfp4((dev(a), dev(sa), dev(np.float32([ga]))),
                                 (dev(b), dev(sb), dev(np.float32([gb]))), out_dtype=dt)
            assert got.shape == (M, N) and torch.count_nonzero(got).item() == 0
        return
    check(pqb, a, sa, ga, b, sb, gb, f"random {shape}")


def test_nvgemm_full_scale_range(pqb):
    """Every scale code 0..126: subnormal E4M3 scales (codes 1..7), blocks with
    scale 0, and the largest scales, mixed within rows."""
    r = rng("range")
    M, N, K = 192, 256, 1024
    a, sa = operand(r, M, K, 0, 127)
    b, sb = operand(r, N, K, 0, 127)
    sa[:, ::7] = r.integers(0, 8, sa[:, ::7].shape)
    sb[5] = 0
    check(pqb, a, sa, np.float32(1.0), b, sb, np.float32(1.0), "full scale range")


def test_nvgemm_exact_on_unit_scale_integers(pqb):
    r = rng("int")
    M, N, K = 160, 256, 896
    idx = r.choice([0, 2, 4, 5, 6, 7], (M, K)) | (r.integers(0, 2, (M, K)) << 3)
    jdx = r.choice([0, 2, 4, 5, 6, 7], (N, K)) | (r.integers(0, 2, (N, K)) << 3)
    pack = lambda t: (t[:, 0::2] | (t[:, 1::2] << 4)).astype(np.uint8)  # noqa: E731
    one = lambda n: np.full((n, K // 16), 0x38, np.uint8)  # noqa: E731
    a, b = pack(idx), pack(jdx)
    got = pqb.gemm_nvfp4((dev(a), dev(one(M)), dev(np.float32([1.0]))),
                         (dev(b), dev(one(N)), dev(np.float32([1.0]))), out_dtype=torch.float32)
    assert np.array_equal(got.cpu().numpy().astype(np.float64), oracle.nvfp4_gemm(a, one(M), 1.0, b, one(N), 1.0))


def test_nvgemm_of_engine_quantized_tensors(pqb):
    """The engine quantizes activations and a weight to NVFP4 (byte-identical
    to the oracle's codes), and the product of those codes matches the oracle."""
    x = synth.fp8_activation(rows=256, cols=1024, device="cpu")
    w = synth.fp8_weight(rows=384, cols=1024, device="cpu")
    qa, qw = pqb.quantize(x.to(DEV), "nvfp4"), pqb.quantize(w.to(DEV), "nvfp4")
    ac, as_, ag = oracle.nvfp4_quantize(x[None])
    bc, bs, bg = oracle.nvfp4_quantize(w[None])
    assert np.array_equal(qa.codes.cpu().numpy().reshape(ac[0].shape), ac[0])
    assert np.array_equal(qw.scales.cpu().numpy().reshape(bs[0].shape), bs[0])
    assert np.array_equal(qw.aux.cpu().numpy(), bg)
    check(pqb, ac[0], as_[0], ag[0], bc[0], bs[0], bg[0], "engine-quantized")
    got = pqb.gemm_nvfp4(qa, qw).cpu().double().numpy()
    ref = x.double().numpy() @ w.double().numpy().T
    assert np.median(np.abs(got - ref) / (np.abs(x.double().numpy()) @ np.abs(w.double().numpy()).T)) < 0.12


@pytest.mark.parametrize("shape", [(8192, 7168, 2048), (8192, 2048, 7168)])
def test_nvgemm_full_size_sampled(pqb, shape):
    """The benchmark's shapes, activations [M x K] times a weight [N x K], both
    NVFP4, bf16 output: sampled rows of every column against the oracle."""
    M, N, K = shape
    x = synth.fp8_activation(rows=M, cols=K, device=DEV)
    w = synth.fp8_weight(rows=N, cols=K, device=DEV)
    qa, qw = pqb.quantize(x, "nvfp4"), pqb.quantize(w, "nvfp4")
    c = pqb.gemm_nvfp4(qa, qw, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.sort(rng("full").choice(M, 24, replace=False))
    rows[-1] = M - 1
    a, sa = qa.codes.cpu().numpy().reshape(M, K // 2), qa.scales.cpu().numpy().reshape(M, K // 16)
    b, sb = qw.codes.cpu().numpy().reshape(N, K // 2), qw.scales.cpu().numpy().reshape(N, K // 16)
    ga, gb = qa.aux.cpu().numpy()[0], qw.aux.cpu().numpy()[0]
    want, S = oracle.nvfp4_gemm(a[rows], sa[rows], ga, b, sb, gb, abs_sum=True)
    tol = (34 + K // 32) * U * S * 1.01
    got = c[torch.from_numpy(rows).to(DEV)].float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - want) <= tol + 2.0 ** -8 * (np.abs(want) + tol))


def test_nvgemm_scale_sign_bit_is_ignored(pqb):
    """The header reads block-scale bytes without their sign bit: setting bit 7
    of every scale byte leaves the product bit for bit unchanged."""
    r = rng("sign")
    M, N, K = 130, 256, 384
    a, sa = operand(r, M, K, 1, 127)
    b, sb = operand(r, N, K, 1, 127)
    g = dev(np.float32([0.75]))
    base = pqb.gemm_nvfp4((dev(a), dev(sa), g), (dev(b), dev(sb), g), out_dtype=torch.float32)
    signed = pqb.gemm_nvfp4((dev(a), dev(sa | 0x80), g), (dev(b), dev(sb | 0x80), g), out_dtype=torch.float32)
    assert torch.equal(base.view(torch.int32), signed.view(torch.int32))
