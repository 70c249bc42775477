"""GPU parity of the block-scaled FP8 GEMM (pqb_gemm_fp8_blockscaled) against
the oracle's float64 definition, element by element, within a bound derived
from how the kernel evaluates it.

The matrix core forms each 128-deep block sum P itself.  Two probes on
gfx950 showed how:
- It takes the products in groups of 8 consecutive K elements.
- Each product is truncated toward zero to a multiple of 2^(e - 13), where e
  is the group's largest sum of operand exponents.
- The 16 group sums are then added in float32.
A model doing exactly this reproduces 84-86% of random block sums bit for
bit; the rest differ in the rounding of the group additions.

So a block sum errs by less than sum_g 2^(e_g - 10), plus 15 float32
additions.  The kernel then adds one rounding for RN(sA sB) and one fused
multiply-add per block.  The tolerance is therefore
  sum_kb |sA sB| sum_g 2^(e_g - 10) + (21 + K/128) * 2^-24 * S,
  S = sum_kb |sA sB| sum_k |dec(a) dec(b)|,
plus half a bf16 ulp of the value for bf16 output.
"""
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


def random_codes(r, shape):
    c = r.integers(0, 256, shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E                  # no NaN codes
    return c


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


_DEC = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn) \
    .double().numpy()
_EF = (np.arange(256) >> 3) & 15
_EXP = np.where(_EF == 0, -6, _EF - 7).astype(np.float64)   # exponent field, unbiased


def tolerance(a, sa, b, sb, S):
    """The bound above for C[m, n] over all rows of a (codes) and b."""
    M, K = a.shape
    N = b.shape[0]
    sa = sa.astype(np.float64).reshape(M, K // 128)
    sb = np.repeat(sb.astype(np.float64).reshape(N // 128, K // 128), 128, axis=0)
    trunc = np.zeros((M, N))
    for kb in range(K // 128):
        for g in range(16):
            ks = slice(128 * kb + 8 * g, 128 * kb + 8 * g + 8)
            nz = (_DEC[a[:, ks]][:, None, :] * _DEC[b[:, ks]][None, :, :]) != 0
            e = np.where(nz, _EXP[a[:, ks]][:, None, :] + _EXP[b[:, ks]][None, :, :], -np.inf).max(2)
            t = np.where(np.isfinite(e), 2.0 ** (e - 10), 0.0)
            trunc += np.abs(sa[:, kb, None] * sb[None, :, kb]) * t
    return 1.01 * (trunc + (21 + K // 128) * U * S) + 1e-35


def check(pqb, a, sa, b, sb, what, rows=None):
    """GPU result in both output types against the oracle (on `rows` of A only,
    if given), within the bound above."""
    M, K = a.shape
    ad, sad, bd, sbd = to_dev(a), to_dev(sa), to_dev(b), to_dev(sb)
    sel = np.arange(M) if rows is None else np.asarray(rows)
    want, S = oracle.fp8_block_gemm(a[sel], sa[sel], b, sb, abs_sum=True)
    tol = tolerance(a[sel], sa[sel], b, sb, S)
    for dt in (torch.float32, torch.bfloat16):
        got = pqb.gemm_fp8_blockscaled(ad, sad, bd, sbd, out_dtype=dt)[torch.from_numpy(sel).to(DEV)]
        got = got.float().cpu().numpy().astype(np.float64)
        bound = tol if dt == torch.float32 else tol + 2.0 ** -8 * (np.abs(want) + tol)
        err = np.abs(got - want)
        bad = np.argwhere(err > bound)
        assert bad.size == 0, (f"{what} {dt}: {len(bad)} elements outside the bound, first "
                               f"{bad[:3].tolist()}, err {err[tuple(bad[0])]:.3e} bound "
                               f"{bound[tuple(bad[0])]:.3e}")


# (600, 768, 1152): several tiles in both directions and a ragged last row of
# tiles; (1024, 512, 384): a grid of 32 workgroups (the XCD-grouped order).
SHAPES = [(128, 128, 128), (256, 384, 512), (100, 256, 256), (1, 128, 384), (300, 640, 1152),
          (129, 128, 2048), (64, 256, 0), (600, 768, 1152), (1024, 512, 384)]


@pytest.mark.parametrize("shape", SHAPES)
def test_gemm_random_codes_match_oracle(pqb, shape):
    M, N, K = shape
    r = rng(f"gemm{shape}")
    a, b = random_codes(r, (M, K)), random_codes(r, (N, K))
    sa = (r.uniform(0.5, 2, (M, K // 128)) * 2.0 ** r.integers(-6, 6, (M, 1))).astype(np.float32)
    sb = (r.uniform(0.5, 2, (N // 128, K // 128)) * 2.0 ** -8).astype(np.float32)
    if K == 0:
        got = pqb.gemm_fp8_blockscaled(to_dev(a), to_dev(sa), to_dev(b), to_dev(sb),
                                       out_dtype=torch.float32)
        assert torch.count_nonzero(got).item() == 0
        return
    check(pqb, a, sa, b, sb, f"random {shape}")


def test_gemm_exact_on_small_integers(pqb):
    """Small-integer codes with power-of-two scales: every block sum is an
    integer below 2^24 and every promotion is exact, so the float32 result
    equals the oracle exactly."""
    r = rng("ints")
    M, N, K = 192, 256, 640
    ia, ib = r.integers(-4, 5, (M, K)), r.integers(-4, 5, (N, K))
    a = oracle.e4m3_encode_array(ia.astype(np.float32))
    b = oracle.e4m3_encode_array(ib.astype(np.float32))
    sa = np.ldexp(1.0, r.integers(-3, 4, (M, K // 128))).astype(np.float32)
    sb = np.ldexp(1.0, r.integers(-3, 4, (N // 128, K // 128))).astype(np.float32)
    got = pqb.gemm_fp8_blockscaled(to_dev(a), to_dev(sa), to_dev(b), to_dev(sb),
                                   out_dtype=torch.float32).cpu().numpy()
    want = oracle.fp8_block_gemm(a, sa, b, sb)
    assert np.array_equal(got.astype(np.float64), want)


def test_gemm_of_engine_quantized_tensors(pqb):
    """The W8A8 chain on the GPU: the engine quantizes bf16 activations (1x128)
    and a weight (128x128), the GEMM consumes the codes; the oracle repeats the
    GEMM on the codes the oracle's own quantizers give for the same inputs."""
    x = synth.fp8_activation(rows=384, cols=1024, device="cpu")
    w = synth.fp8_weight(rows=512, cols=1024, device="cpu")
    qa = pqb.quantize(x.to(DEV), "fp8_e4m3", "1x128")
    qw = pqb.quantize(w.to(DEV), "fp8_e4m3", "128x128")
    ac, as_ = oracle.fp8_quantize(x[None], "1x128")
    bc, bs = oracle.fp8_quantize(w[None], "128x128")
    assert np.array_equal(qa.codes.cpu().numpy().reshape(ac.shape), ac)
    assert np.array_equal(qw.codes.cpu().numpy().reshape(bc.shape), bc)
    check(pqb, ac[0], as_[0], bc[0], bs[0], "quantized W8A8")
    got = pqb.gemm_fp8_blockscaled(qa.codes.reshape(384, 1024), qa.scales.reshape(384, 8),
                                   qw.codes.reshape(512, 1024), qw.scales.reshape(4, 8),
                                   out_dtype=torch.float32).cpu().double().numpy()
    ref = x.double().numpy() @ w.double().numpy().T
    assert np.abs(got - ref).max() < 0.05 * np.abs(ref).max()


@pytest.mark.parametrize("K", [0, 128, 256, 384])
def test_gemm_three_per_cu_ragged(pqb, K):
    """528 tiles of 128 x 128, three or more per CU, so the kernel that runs
    three workgroups per CU computes them: a ragged last row of tiles
    (M = 4174) and 0 to 3 K blocks.  Sampled rows, the ragged tile's among
    them, against the oracle in float32 and bf16; the fused FP8 form's codes
    and scales on the same rows against the oracle quantizer of the float32
    result."""
    M, N = 4174, 2048
    r = rng(f"three{K}")
    a, b = random_codes(r, (M, K)), random_codes(r, (N, K))
    sa = (r.uniform(0.5, 2, (M, K // 128)) * 2.0 ** r.integers(-6, 6, (M, 1))).astype(np.float32)
    sb = (r.uniform(0.5, 2, (N // 128, K // 128)) * 2.0 ** -8).astype(np.float32)
    ad, sad, bd, sbd = to_dev(a), to_dev(sa), to_dev(b), to_dev(sb)
    c32 = pqb.gemm_fp8_blockscaled(ad, sad, bd, sbd, out_dtype=torch.float32)
    codes, scales = pqb.gemm_fp8_blockscaled_quant(ad, sad, bd, sbd)
    if K == 0:
        assert torch.count_nonzero(c32).item() == 0 and torch.count_nonzero(codes).item() == 0
        return
    rows = np.unique(np.concatenate([r.choice(4096, 32, replace=False),
                                     [4096, 4100, 4150, M - 2, M - 1]]))
    check(pqb, a, sa, b, sb, f"three per CU, K = {K}", rows=rows)
    sel = torch.from_numpy(rows).to(DEV)
    oc, os_ = oracle.fp8_quantize(c32[sel].cpu().numpy()[None], "1x128")
    assert np.array_equal(codes[sel].cpu().numpy().reshape(-1), oc.reshape(-1))
    assert np.array_equal(scales[sel].cpu().numpy().reshape(-1).view(np.int32), os_.reshape(-1).view(np.int32))


@pytest.mark.parametrize("seed", range(8))
def test_gemm_random_shapes(pqb, seed):
    """Seeded random shapes spanning 1 to 5 tiles per CU, so that either of
    the two kernels the launcher chooses between (two or three workgroups
    per CU) computes them: sampled rows, the last row among them, against
    the oracle in float32 and bf16, and the fused form's codes and scales on
    the same rows against the oracle quantizer of the float32 result."""
    r = rng(f"gshape{seed}")
    M = int(r.integers(1, 6001))
    N = 128 * int(r.integers(1, 33))
    K = 128 * int(r.choice([1, 2, 3, 5]))
    a, b = random_codes(r, (M, K)), random_codes(r, (N, K))
    sa = (r.uniform(0.5, 2, (M, K // 128)) * 2.0 ** r.integers(-6, 6, (M, 1))).astype(np.float32)
    sb = (r.uniform(0.5, 2, (N // 128, K // 128)) * 2.0 ** -8).astype(np.float32)
    rows = np.unique(np.concatenate([r.choice(M, min(M, 12), replace=False), [M - 1]]))
    check(pqb, a, sa, b, sb, f"random shape {(M, N, K)}", rows=rows)
    ad, sad, bd, sbd = to_dev(a), to_dev(sa), to_dev(b), to_dev(sb)
    c32 = pqb.gemm_fp8_blockscaled(ad, sad, bd, sbd, out_dtype=torch.float32)
    codes, scales = pqb.gemm_fp8_blockscaled_quant(ad, sad, bd, sbd)
    sel = torch.from_numpy(rows).to(DEV)
    oc, os_ = oracle.fp8_quantize(c32[sel].cpu().numpy()[None], "1x128")
    assert np.array_equal(codes[sel].cpu().numpy().reshape(-1), oc.reshape(-1))
    assert np.array_equal(scales[sel].cpu().numpy().reshape(-1).view(np.int32), os_.reshape(-1).view(np.int32))


BENCH_SHAPES = [(8192, 7168, 2048), (8192, 2048, 7168)]


@pytest.mark.parametrize("shape", BENCH_SHAPES)
def test_gemm_full_size_sampled(pqb, shape):
    """The benchmark's GEMMs, activations [M x K] (1x128) times the weight
    [N x K] (128x128), bf16 output: sampled rows of every column against the
    oracle."""
    M, N, K = shape
    x = synth.fp8_activation(rows=M, cols=K, device=DEV)
    w = synth.fp8_weight(rows=N, cols=K, device=DEV)
    qa = pqb.quantize(x, "fp8_e4m3", "1x128")
    qw = pqb.quantize(w, "fp8_e4m3", "128x128")
    a, sa = qa.codes.reshape(M, K), qa.scales.reshape(M, K // 128)
    b, sb = qw.codes.reshape(N, K), qw.scales.reshape(N // 128, K // 128)
    c = pqb.gemm_fp8_blockscaled(a, sa, b, sb, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.sort(rng("full").choice(M, 24, replace=False))
    rows[-1] = M - 1
    an, san = a.cpu().numpy(), sa.cpu().numpy()
    bn, sbn = b.cpu().numpy(), sb.cpu().numpy()
    want, S = oracle.fp8_block_gemm(an[rows], san[rows], bn, sbn, abs_sum=True)
    tol = tolerance(an[rows], san[rows], bn, sbn, S)
    got = c[torch.from_numpy(rows).to(DEV)].float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - want) <= tol + 2.0 ** -8 * (np.abs(want) + tol))


@pytest.mark.parametrize("shape", [(256, 384, 512), (100, 256, 256), (300, 640, 1152), (1, 128, 128),
                                   (64, 256, 0)])
def test_gemm_fused_fp8_quant_matches_oracle_quantizer(pqb, shape):
    """The fused epilogue: its codes and scales equal the oracle's FP8 1x128
    quantization of the GEMM's own float32 result (checked against the oracle
    GEMM above), byte for byte.  K = 0 quantizes the all-zero product."""
    M, N, K = shape
    r = rng(f"fused{shape}")
    a, b = random_codes(r, (M, K)), random_codes(r, (N, K))
    sa = (r.uniform(0.5, 2, (M, K // 128)) * 2.0 ** r.integers(-6, 6, (M, 1))).astype(np.float32)
    sb = (r.uniform(0.5, 2, (N // 128, K // 128)) * 2.0 ** -8).astype(np.float32)
    ad, sad, bd, sbd = to_dev(a), to_dev(sa), to_dev(b), to_dev(sb)
    c32 = pqb.gemm_fp8_blockscaled(ad, sad, bd, sbd, out_dtype=torch.float32).cpu().numpy()
    codes, scales = pqb.gemm_fp8_blockscaled_quant(ad, sad, bd, sbd)
    oc, os_ = oracle.fp8_quantize(c32[None], "1x128")
    assert np.array_equal(scales.cpu().numpy().view(np.int32).reshape(-1), os_.view(np.int32).reshape(-1))
    assert np.array_equal(codes.cpu().numpy().reshape(-1), oc.reshape(-1))
    if M <= 300 and K > 0:
        check(pqb, a, sa, b, sb, f"fused {shape} (float32 result)")


@pytest.mark.parametrize("shape", BENCH_SHAPES)
def test_gemm_fused_quant_full_size_sampled(pqb, shape):
    """Fused GEMM + 1x128 quantization at the benchmark's shapes: sampled rows of
    the codes and scales against the oracle quantizer on the GEMM's float32 rows."""
    M, N, K = shape
    x = synth.fp8_activation(rows=M, cols=K, device=DEV)
    w = synth.fp8_weight(rows=N, cols=K, device=DEV)
    qa = pqb.quantize(x, "fp8_e4m3", "1x128")
    qw = pqb.quantize(w, "fp8_e4m3", "128x128")
    args = (qa.codes.reshape(M, K), qa.scales.reshape(M, K // 128), qw.codes.reshape(N, K),
            qw.scales.reshape(N // 128, K // 128))
    codes, scales = pqb.gemm_fp8_blockscaled_quant(*args)
    c32 = pqb.gemm_fp8_blockscaled(*args, out_dtype=torch.float32)
    rows = torch.from_numpy(np.sort(rng("fq").choice(M, 32, replace=False))).to(DEV)
    oc, os_ = oracle.fp8_quantize(c32[rows].cpu().numpy()[None], "1x128")
    assert np.array_equal(codes[rows].cpu().numpy().reshape(-1), oc.reshape(-1))
    assert np.array_equal(scales[rows].cpu().numpy().reshape(-1).view(np.int32), os_.reshape(-1).view(np.int32))
