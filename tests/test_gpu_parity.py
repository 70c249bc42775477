"""GPU parity: the HIP engine (through the C ABI) against the CPU oracle.

Codes, scales, auxiliary buffers and dequantized values must match bit for
bit.  Sizes here span several tiles plus ragged tails; the full workload sizes
are covered in test_gpu_workloads.py.
"""
import numpy as np
import pytest
import torch

import oracle
from precision_quantization_block_amd import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def pqb():
    import precision_quantization_block_amd as p
    p.lib()
    return p


def host_bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy().view(np.uint32)
    return t.numpy()


def same(gpu: torch.Tensor, ref: np.ndarray, what: str):
    g = host_bits(gpu).reshape(-1)
    r = np.ascontiguousarray(ref)
    r = (r.view(np.uint32) if r.dtype == np.float32 else r).reshape(-1)
    assert g.shape == r.shape, f"{what}: shape {g.shape} vs {r.shape}"
    bad = np.nonzero(g != r)[0]
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:8]}: " \
                          f"gpu {g[bad[:8]]} oracle {r[bad[:8]]}"


def as_ref_f32(t):
    return t.float().numpy()


# ------------------------------------------------------------ codecs -------

def _f32(bits):
    return np.asarray(bits, np.uint32).view(np.float32)


def test_encode_e4m3_probe_set(pqb):
    rng = np.random.default_rng(0)
    table = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn) \
        .float().numpy()
    pos = np.unique(table[~np.isnan(table) & (table >= 0)])
    mids = ((pos[:-1].astype(np.float64) + pos[1:]) / 2).astype(np.float32)
    y = np.concatenate([
        pos, mids, np.nextafter(mids, np.float32(1e9)), np.nextafter(mids, np.float32(0)),
        _f32(np.arange(0, 0x43E00001, 977, dtype=np.uint32)),
        _f32(rng.integers(0, 0x43E00001, 300_000, dtype=np.uint32)),
        np.array([448.5, 455.9, 463.9, 2.0 ** -10, 1e-45, 3e-39], np.float32),
    ]).astype(np.float32)
    y = np.concatenate([y, -y])
    got = pqb.encode_e4m3(torch.from_numpy(y).to(DEV))
    same(got, oracle.e4m3_encode_array(y), "E4M3 encode")


def test_encode_e4m3_exhaustive_vs_torch_cast(pqb):
    """Every float32 with |y| <= 448 (both signs): the engine's E4M3 rounding
    against torch's float8_e4m3fn cast, which the oracle's tests pin."""
    top = 0x43E00000  # 448.0
    chunk = 1 << 27
    for sign in (0, 0x80000000):
        for lo in range(0, top + 1, chunk):
            hi = min(lo + chunk, top + 1)
            bits = torch.arange(lo, hi, dtype=torch.int64, device=DEV) | sign
            y = bits.to(torch.int32).view(torch.float32) if sign == 0 else \
                (bits - (1 << 32)).to(torch.int32).view(torch.float32)
            got = pqb.encode_e4m3(y)
            ref = y.cpu().to(torch.float8_e4m3fn).view(torch.uint8)
            ok = torch.equal(got.cpu(), ref)
            assert ok, f"E4M3 mismatch in bit range [{lo:#x}, {hi:#x}) sign {sign:#x}"


def test_encode_e2m1_exhaustive(pqb):
    """Every float32 in [-8, 8]: nibble = count of E2M1 midpoints strictly below
    |y| (ties to the smaller value), sign bit for y < 0; plus oracle samples."""
    mids = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    top = 0x41000000  # 8.0
    chunk = 1 << 27
    for sign in (0, 1):
        for lo in range(0, top + 1, chunk):
            hi = min(lo + chunk, top + 1)
            bits = torch.arange(lo, hi, dtype=torch.int64, device=DEV)
            if sign:
                bits = bits - (1 << 31)   # set the sign bit (as int32)
            y = bits.to(torch.int32).view(torch.float32)
            got = pqb.encode_e2m1(y).cpu()
            yc = y.cpu()
            idx = torch.searchsorted(mids, yc.abs(), right=False).to(torch.uint8)
            ref = idx | ((yc < 0).to(torch.uint8) << 3)
            assert torch.equal(got, ref), f"E2M1 mismatch in [{lo:#x}, {hi:#x}) sign {sign}"
    rng = np.random.default_rng(1)
    y = np.concatenate([rng.uniform(-7, 7, 200_000),
                        rng.uniform(-1, 1, 50_000) * 1e-38]).astype(np.float32)
    y = np.concatenate([y, np.array([0.0, -0.0, 1e30, -1e30], np.float32)])
    same(pqb.encode_e2m1(torch.from_numpy(y).to(DEV)), oracle.e2m1_encode_array(y),
         "E2M1 vs oracle")


# -------------------------------------------------------------- FP8 --------

FP8_SHAPES = {
    "tensor": [(1, 300, 512), (3, 17, 200), (2, 5, 9)],
    "row": [(1, 301, 7168), (2, 33, 200), (1, 7, 9000), (1, 9, 12)],
    "1x128": [(1, 333, 7168), (2, 7, 384), (1, 1, 128)],
    "128x128": [(1, 384, 2048), (2, 256, 384), (1, 64, 256), (3, 1, 128), (1, 128, 128)],
}


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("gran", list(FP8_SHAPES))
def test_fp8_parity(pqb, gran, dtype):
    for i, (b, r, c) in enumerate(FP8_SHAPES[gran]):
        x = synth.fp8_activation(rows=b * r, cols=c, seed=10 + i).reshape(b, r, c).to(dtype)
        q = pqb.quantize(x.to(DEV), "fp8_e4m3", gran, shape=(b, r, c))
        oc, os_ = oracle.fp8_quantize(x, gran)
        same(q.codes, oc, f"fp8 {gran} {(b, r, c)} codes")
        same(q.scales, os_, f"fp8 {gran} {(b, r, c)} scales")
        same(pqb.dequantize(q), oracle.fp8_dequantize(oc, os_, gran),
             f"fp8 {gran} {(b, r, c)} dequant f32")
        same(pqb.dequantize(q, torch.bfloat16), oracle.fp8_dequantize(oc, os_, gran, True),
             f"fp8 {gran} {(b, r, c)} dequant bf16")


# --------------------------------------------------------------- FP4 -------

MX_SHAPES = [(1, 96, 1024), (2, 33, 96), (1, 1, 32), (1, 257, 160)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_mxfp4_parity(pqb, dtype):
    for i, (b, r, c) in enumerate(MX_SHAPES):
        x = synth.mlp_weight_fp32(rows=b * r, cols=c, seed=20 + i).reshape(b, r, c).to(dtype)
        q = pqb.quantize(x.to(DEV), "mxfp4", shape=(b, r, c))
        oc, os_ = oracle.mxfp4_quantize(x)
        same(q.codes, oc, f"mx {(b, r, c)} codes")
        same(q.scales, os_, f"mx {(b, r, c)} scales")
        same(pqb.dequantize(q), oracle.mxfp4_dequantize(oc, os_), f"mx {(b, r, c)} dequant")
        same(pqb.dequantize(q, torch.bfloat16), oracle.mxfp4_dequantize(oc, os_, True),
             f"mx {(b, r, c)} dequant bf16")


NV_SHAPES = [(1, 96, 1024), (3, 33, 96), (1, 1, 16), (2, 129, 48)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_nvfp4_parity(pqb, dtype):
    for i, (b, r, c) in enumerate(NV_SHAPES):
        x = synth.heavy_tail_weight(rows=b * r, cols=c, seed=30 + i).reshape(b, r, c).to(dtype)
        q = pqb.quantize(x.to(DEV), "nvfp4", shape=(b, r, c))
        oc, os_, og = oracle.nvfp4_quantize(x)
        same(q.codes, oc, f"nv {(b, r, c)} codes")
        same(q.scales, os_, f"nv {(b, r, c)} scales")
        same(q.aux, og, f"nv {(b, r, c)} tensor scale")
        same(pqb.dequantize(q), oracle.nvfp4_dequantize(oc, os_, og), f"nv {(b, r, c)} dequant")
        same(pqb.dequantize(q, torch.bfloat16), oracle.nvfp4_dequantize(oc, os_, og, True),
             f"nv {(b, r, c)} dequant bf16")


def test_nvfp4_dequant_every_code(pqb):
    """NVFP4 dequantization of hand-made codes: every code byte at every byte
    position of a 4-byte unit, every block-scale code the quantizer can write
    (0 .. 0x7E, one per row) and three tensor scales (the smallest gs the
    quantizer forms, 1, and an arbitrary one), in float32 and bf16."""
    b, r, c = 3, 127, 2048
    byte = (np.arange(c // 2) // 4).astype(np.uint8)     # byte i = i // 4: all 256 at each position
    codes = np.broadcast_to(byte, (b, r, c // 2)).copy()
    scales = np.broadcast_to(np.arange(r, dtype=np.uint8)[:, None], (b, r, c // 16)).copy()
    gs = np.array([np.float32(1e-12) / np.float32(2688), 1.0, 3.7e-5], np.float32)
    q = pqb.Quantized(torch.from_numpy(codes).reshape(-1).to(DEV),
                      torch.from_numpy(scales).reshape(-1).to(DEV),
                      torch.from_numpy(gs).to(DEV), "nvfp4", "blk16", (b, r, c))
    same(pqb.dequantize(q), oracle.nvfp4_dequantize(codes, scales, gs), "nv dequant every code")
    same(pqb.dequantize(q, torch.bfloat16), oracle.nvfp4_dequantize(codes, scales, gs, True),
         "nv dequant bf16 every code")


# -------------------------------------------------------------- INT4 -------

INT4_SHAPES = [(1, 64, 4096), (2, 9, 384), (1, 1, 128), (1, 3, 14336)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_int4_parity(pqb, dtype):
    for i, (b, r, c) in enumerate(INT4_SHAPES):
        x = synth.fp8_weight(rows=b * r, cols=c, seed=40 + i).reshape(b, r, c).to(dtype)
        q = pqb.quantize(x.to(DEV), "int4_asym", shape=(b, r, c))
        oc, os_, oz = oracle.int4_quantize(x)
        same(q.codes, oc, f"int4 {(b, r, c)} codes")
        same(q.scales, os_, f"int4 {(b, r, c)} scales")
        same(q.aux, oz, f"int4 {(b, r, c)} zeros")
        same(pqb.dequantize(q), oracle.int4_dequantize(oc, os_, oz), f"int4 {(b, r, c)} dequant")
        same(pqb.dequantize(q, torch.bfloat16), oracle.int4_dequantize(oc, os_, oz, True),
             f"int4 {(b, r, c)} dequant bf16")


def _int4_edge_groups(rows=64, cols=4096):
    """bf16 rows of 32 groups each, many of them hand-made: exact .5 ties at
    scales 1 and 3 (lo = -8 s, hi = 7 s), ties next to the range ends, constant
    groups (zero, -0, negative, positive), one-signed groups (zero-point 7 and
    -8), rint(lo / s) = -15, tiny and huge ranges, single outliers; the rest is
    the weight recipe.  Full rows are whole 512-unit chunks, the shape on which
    bf16 quantization stages its loads through LDS."""
    g = torch.Generator().manual_seed(91)
    x = torch.randn((rows, cols), generator=g) * 0.02
    grp = x.view(rows, cols // 128, 128)
    ties1 = torch.cat([torch.tensor([-8.0, 7.0]), torch.arange(-7.5, 7.0, 1.0)])    # s = 1
    ties3 = torch.cat([torch.tensor([-24.0, 21.0]), 3 * torch.arange(-7.5, 7.0, 1.0)])  # s = 3
    for r in range(rows):
        for k in range(cols // 128):
            kind = (r * 32 + k) % 16
            if kind == 0:
                grp[r, k] = ties1.repeat(128 // ties1.numel() + 1)[:128]
            elif kind == 1:
                grp[r, k] = ties3.repeat(128 // ties3.numel() + 1)[:128]
            elif kind == 2:
                grp[r, k] = 0.0
            elif kind == 3:
                grp[r, k] = -0.0
            elif kind == 4:
                grp[r, k] = -1.25
            elif kind == 5:
                grp[r, k] = 3.0
            elif kind == 6:
                grp[r, k] = -grp[r, k].abs() - 1e-3          # all negative: z = 7
            elif kind == 7:
                grp[r, k] = grp[r, k].abs() + 1e-3           # all positive: z = -8
            elif kind == 8:
                grp[r, k] = grp[r, k].abs()
                grp[r, k, 17] = -1.0                         # lo far below: rint(lo/s) = -15
                grp[r, k, 18] = 0.0
            elif kind == 9:
                grp[r, k] = grp[r, k] * 1e-35                # subnormal-scale range
            elif kind == 10:
                grp[r, k] = grp[r, k] * 1e36                 # range near 1e35
            elif kind == 11:
                grp[r, k, (r + k) % 128] = 50.0              # one outlier
            elif kind == 12:
                grp[r, k] = torch.arange(128) % 16 - 8.0     # every code at s = 1
    return x.to(torch.bfloat16)


def test_int4_full_chunks_edge_groups(pqb):
    x = _int4_edge_groups()
    oc, os_, oz = oracle.int4_quantize(x)
    q = pqb.quantize(x.to(DEV), "int4_asym")
    same(q.codes, oc, "int4 edge groups codes")
    same(q.scales, os_, "int4 edge groups scales")
    same(q.aux, oz, "int4 edge groups zeros")
    (qb,) = pqb.quantize_batch([(x.to(DEV), "int4_asym", None)])
    same(qb.codes, oc, "int4 edge groups codes (batch)")
    same(qb.scales, os_, "int4 edge groups scales (batch)")
    same(qb.aux, oz, "int4 edge groups zeros (batch)")
    same(pqb.dequantize(q), oracle.int4_dequantize(oc, os_, oz), "int4 edge groups dequant")


@pytest.mark.parametrize("rows", [16384, 16385])
def test_two_pass_fold_threshold(pqb, rows):
    """Per-tensor FP8 and NVFP4 on bf16 [2, rows, 1024]: 16384 rows give 1024
    pass-1 partials per slice, which pass 2 reduces itself (two launches);
    16385 rows give 1025, which take the finalize launch.  Each slice has one
    planted maximum, so the oracle on sampled rows plus the maximum's row sees
    the slice's own tensor scale."""
    cols = 1024
    g = torch.Generator().manual_seed(rows)
    x = torch.randn((2, rows, cols), generator=g)
    maxpos = [(int(torch.randint(rows, (1,), generator=g)), int(torch.randint(cols, (1,), generator=g)))
              for _ in range(2)]
    for b, (r, c) in enumerate(maxpos):
        x[b, r, c] = -40.0 if b else 40.0
    x = x.to(torch.bfloat16)
    xd = x.to(DEV)
    qf = pqb.quantize(xd, "fp8_e4m3", "tensor")
    qn = pqb.quantize(xd, "nvfp4")
    fc, fs = qf.codes.reshape(2, rows, cols), qf.scales
    nc, nb = qn.codes.reshape(2, rows, cols // 2), qn.scales.reshape(2, rows, cols // 16)
    for b in range(2):
        pick = sorted({int(i) for i in torch.randint(rows, (8,), generator=g)} | {maxpos[b][0]})
        xs = x[b, pick].unsqueeze(0)
        oc, os_ = oracle.fp8_quantize(xs, "tensor")
        same(fs[b:b + 1], os_, f"fold {rows} fp8 scale {b}")
        same(fc[b, pick], oc, f"fold {rows} fp8 codes {b}")
        oc, ob, og = oracle.nvfp4_quantize(xs)
        same(qn.aux[b:b + 1], og, f"fold {rows} nvfp4 gs {b}")
        same(nc[b, pick], oc, f"fold {rows} nvfp4 codes {b}")
        same(nb[b, pick], ob, f"fold {rows} nvfp4 block scales {b}")


def test_int4_infinite_range_group_stays_local(pqb):
    """A group whose range overflows float32 (values of both signs near
    +-3e38) is outside INT4's documented input range; its own bytes are
    unspecified, but every other group must match the oracle."""
    x = synth.fp8_weight(rows=16, cols=512, seed=5).float()
    x[3, 128:256:2] = 3.0e38
    x[3, 129:256:2] = -3.0e38
    for dtype in (torch.float32, torch.bfloat16):
        xt = x.to(dtype)
        q = pqb.quantize(xt.to(DEV), "int4_asym")
        oc, os_, oz = oracle.int4_quantize(xt)
        bad_group = 3 * 4 + 1
        keep_g = np.ones(16 * 4, bool)
        keep_g[bad_group] = False
        keep_c = np.repeat(keep_g, 64)
        g_codes = host_bits(q.codes).reshape(-1)
        assert np.array_equal(g_codes[keep_c], oc.reshape(-1)[keep_c]), f"int4 codes {dtype}"
        g_s = host_bits(q.scales).reshape(-1)
        assert np.array_equal(g_s[keep_g], os_.reshape(-1)[keep_g]), f"int4 scales {dtype}"
        zn = host_bits(q.aux).reshape(-1)
        zg = np.stack([zn & 15, zn >> 4], -1).reshape(-1)
        zo = np.stack([oz & 15, oz >> 4], -1).reshape(-1)
        assert np.array_equal(zg[keep_g], zo[keep_g]), f"int4 zero-points {dtype}"


# ---------------------------------------------------------------- KV -------

def test_kv_write_parity(pqb):
    k, v = synth.kv_cache(layers=3, tokens=100, heads=8, head_dim=128)
    kc, vc, ks, vs = pqb.kv_write_fp8(k.to(DEV), v.to(DEV))
    okc, ovc, oks, ovs = oracle.kv_write_fp8(k, v)
    same(kc, okc, "kv k codes")
    same(vc, ovc, "kv v codes")
    same(ks, oks, "kv k scales")
    same(vs, ovs, "kv v scales")
    dk, dv = pqb.fp8_kv_write(k.to(DEV), v.to(DEV))
    same(dk, oracle.fp8_dequantize(okc.reshape(3, 1, -1), oks, "tensor"), "kv k dequant")


# ------------------------------------------------------------- edges -------

def _edge_tensor(rows, cols, dtype):
    g = torch.Generator().manual_seed(77)
    x = torch.randn((rows, cols), generator=g)
    x[0, :] = 0.0                                   # all-zero blocks
    x[1, :] = -0.0
    x[2, :] = torch.tensor(1e-40).expand(cols)      # subnormal block
    x[2, ::3] = -1e-41
    x[3, :] = x[3, :] * 1e-30                       # tiny block
    x[4, :] = x[4, :] * 1e30                        # huge block
    x[5, 5] = 3e38                                  # near float max
    x[6, :] = torch.arange(cols) % 7 - 3.0          # small integers: exact ties
    x[7, ::2] = 2.0 ** -126                          # smallest normal
    x[8, :] = 0.0
    x[8, 0] = -1e-45                                 # one negative subnormal in a zero block
    x[9, 1:] = 1e-42
    x[9, 0] = 100.0                                  # one large value, subnormal rest
    if dtype == torch.bfloat16:
        x = x.to(torch.bfloat16)
    return x


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_edge_values_all_formats(pqb, dtype):
    x = _edge_tensor(16, 256, dtype)
    xd = x.to(DEV)
    for gran in ("tensor", "row", "1x128", "128x128"):
        q = pqb.quantize(xd, "fp8_e4m3", gran)
        oc, os_ = oracle.fp8_quantize(x, gran)
        same(q.codes, oc, f"edge fp8 {gran} codes")
        same(q.scales, os_, f"edge fp8 {gran} scales")
        same(pqb.dequantize(q), oracle.fp8_dequantize(oc, os_, gran), f"edge fp8 {gran} deq")
    q = pqb.quantize(xd, "mxfp4")
    oc, os_ = oracle.mxfp4_quantize(x)
    same(q.codes, oc, "edge mx codes")
    same(q.scales, os_, "edge mx scales")
    same(pqb.dequantize(q), oracle.mxfp4_dequantize(oc, os_), "edge mx deq")
    for rows in (slice(0, 16), slice(0, 3), slice(8, 10), slice(3, 5)):
        xs = x[rows].contiguous()
        q = pqb.quantize(xs.to(DEV), "nvfp4")
        oc, os_, og = oracle.nvfp4_quantize(xs)
        same(q.codes, oc, f"edge nv codes {rows}")
        same(q.scales, os_, f"edge nv scales {rows}")
        same(q.aux, og, f"edge nv gs {rows}")
        same(pqb.dequantize(q), oracle.nvfp4_dequantize(oc, os_, og), f"edge nv deq {rows}")
    xi = x.clone()
    xi[4] = xi[4] * 1e-5    # keep hi - lo finite for INT4
    xi[5, 5] = 1e30
    q = pqb.quantize(xi.to(DEV), "int4_asym")
    oc, os_, oz = oracle.int4_quantize(xi)
    same(q.codes, oc, "edge int4 codes")
    same(q.scales, os_, "edge int4 scales")
    same(q.aux, oz, "edge int4 zeros")
    same(pqb.dequantize(q), oracle.int4_dequantize(oc, os_, oz), "edge int4 deq")


def test_mx_exponent_boundaries(pqb):
    rows = []
    for k in range(-30, 40):
        for a in (np.float32(2.0 ** k), np.nextafter(np.float32(2.0 ** k), np.float32(0))):
            blk = np.linspace(-1, 1, 32).astype(np.float32) * a * np.float32(0.5)
            blk[7] = -a
            rows.append(blk)
    x = torch.from_numpy(np.stack(rows))
    q = pqb.quantize(x.to(DEV), "mxfp4")
    oc, os_ = oracle.mxfp4_quantize(x)
    same(q.codes, oc, "mx boundary codes")
    same(q.scales, os_, "mx boundary scales")


def test_int4_dequant_extreme_ranges(pqb):
    """Groups whose range is the input type's largest finite value, with the
    zero-point at both ends of its range (7 when the group is all negative,
    -8 when all positive).  In float32, (z + 8) s alone would overflow while
    (q - z) s is finite for every code but the one at -max, whose value
    overflows in the oracle too."""
    for dtype in (torch.float32, torch.bfloat16):
        fmax = torch.finfo(dtype).max   # FLT_MAX itself rounds to inf in bf16
        ramp = torch.linspace(0, 1, 128).repeat(2)
        g = torch.zeros((6, 256))
        g[0] = -ramp * fmax                                   # lo = -max, hi = 0: z = 7
        g[1] = ramp * fmax                                    # lo = 0, hi = max: z = -8
        g[2, :128] = -fmax * 0.97
        g[2, 128:] = fmax * 0.45                              # one extreme group, one constant
        g[3] = torch.linspace(-1, 1, 256) * fmax * 0.49       # range just under the maximum
        g[4] = -torch.linspace(0, 1, 256) * 1e30
        g[5] = torch.linspace(-3, 5, 256)
        x = g.to(dtype)
        assert torch.isfinite(x).all()
        q = pqb.quantize(x.to(DEV), "int4_asym")
        oc, os_, oz = oracle.int4_quantize(x)
        same(q.codes, oc, f"extreme int4 codes {dtype}")
        same(q.scales, os_, f"extreme int4 scales {dtype}")
        same(q.aux, oz, f"extreme int4 zeros {dtype}")
        same(pqb.dequantize(q), oracle.int4_dequantize(oc, os_, oz), f"extreme int4 deq {dtype}")
        same(pqb.dequantize(q, torch.bfloat16), oracle.int4_dequantize(oc, os_, oz, True),
             f"extreme int4 deq bf16 {dtype}")


def test_int4_exact_ties(pqb):
    """Groups whose elements sit exactly on half-steps of the stored scale."""
    g = torch.zeros((4, 128))
    g[0] = (torch.arange(128) % 16 - 8).float() * 0.5 + 0.25   # s = 0.5 after rounding
    g[1] = torch.arange(128).float() / 127 * 15 - 7.5
    g[2] = -(torch.arange(128) % 31).float() * 0.5
    g[3] = torch.linspace(-1, 2, 128)
    q = pqb.quantize(g.to(DEV), "int4_asym")
    oc, os_, oz = oracle.int4_quantize(g)
    same(q.codes, oc, "int4 tie codes")
    same(q.aux, oz, "int4 tie zeros")


def test_empty_and_repeatable(pqb):
    e = torch.empty((0, 128), device=DEV, dtype=torch.bfloat16)
    q = pqb.quantize(e, "fp8_e4m3", "1x128")
    assert q.codes.numel() == 0
    x = synth.fp8_activation(rows=64, cols=1024, seed=3).to(DEV)
    a = pqb.quantize(x, "nvfp4")
    b = pqb.quantize(x, "nvfp4")
    assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)
