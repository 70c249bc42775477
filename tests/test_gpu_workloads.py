"""GPU parity at the full workload sizes, in the launch configuration bench.py
times.  The oracle computes sampled outputs: whole rows (blocks never cross a
row) or whole 128-row bands (128x128 tiles).  Where a scale covers the whole
tensor or slice, the sample always contains the row that holds the maximum,
so the oracle's scale is the global one.
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


def say(*a):
    print(*a, flush=True)


def u8(t):
    return t.detach().cpu().numpy()


def bits(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy().view(np.uint32)
    return t.numpy()


def f32bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def eq(a, b, what):
    a, b = np.asarray(a).reshape(-1), f32bits(b).reshape(-1)
    bad = np.nonzero(a != b)[0]
    assert a.shape == b.shape and bad.size == 0, f"{what}: {bad.size} mismatches at {bad[:8]}"


def sample_rows(nrows, k, seed, extra=()):
    rng = np.random.default_rng(seed)
    rows = set(int(r) for r in rng.choice(nrows, size=min(k, nrows), replace=False))
    rows.update(int(r) for r in extra)
    return sorted(rows)


def row_of_max(x2d: torch.Tensor) -> int:
    return int(torch.argmax(x2d.abs().float().amax(dim=1)).item())


def test_fp8_activations_1x128_full(pqb):
    a = synth.fp8_activation(device=DEV)
    say("fp8 act [8192, 7168] 1x128")
    q = pqb.quantize(a, "fp8_e4m3", "1x128")
    codes, scales = q.codes.view(8192, 7168), q.scales.view(8192, 56)
    for r in sample_rows(8192, 48, 0, [0, 8191]):
        oc, os_ = oracle.fp8_quantize(a[r:r + 1].cpu(), "1x128")
        eq(u8(codes[r]), oc, f"act codes row {r}")
        eq(bits(scales[r]), os_, f"act scales row {r}")
    # per-token variant on the same tensor
    q = pqb.quantize(a, "fp8_e4m3", "row")
    for r in sample_rows(8192, 16, 1):
        oc, os_ = oracle.fp8_quantize(a[r:r + 1].cpu(), "row")
        eq(u8(q.codes.view(8192, 7168)[r]), oc, f"per-token codes row {r}")
        eq(bits(q.scales[r:r + 1]), os_, f"per-token scale row {r}")


def test_fp8_weight_128x128_full(pqb):
    w = synth.fp8_weight(device=DEV)
    say("fp8 weight [7168, 2048] 128x128")
    q = pqb.quantize(w, "fp8_e4m3", "128x128")
    codes, scales = q.codes.view(7168, 2048), q.scales.view(56, 16)
    for band in (0, 23, 55):
        sl = slice(band * 128, band * 128 + 128)
        oc, os_ = oracle.fp8_quantize(w[sl].cpu(), "128x128")
        eq(u8(codes[sl]), oc, f"weight codes band {band}")
        eq(bits(scales[band]), os_, f"weight scales band {band}")
    dq = pqb.dequantize(q)
    oc, os_ = oracle.fp8_quantize(w[:128].cpu(), "128x128")
    eq(bits(dq[0, :128]), oracle.fp8_dequantize(oc, os_, "128x128"), "weight dequant band 0")


def test_mlp_weight_fp32_mx_nv_full(pqb):
    w = synth.mlp_weight_fp32()
    say("mlp weight [3072, 1024] f32 mx/nv (whole tensor)")
    q = pqb.quantize(w.to(DEV), "mxfp4")
    oc, os_ = oracle.mxfp4_quantize(w)
    eq(u8(q.codes), oc, "mx codes")
    eq(u8(q.scales), os_, "mx scales")
    eq(bits(pqb.dequantize(q)), oracle.mxfp4_dequantize(oc, os_), "mx dequant")
    q = pqb.quantize(w.to(DEV), "nvfp4")
    oc, os_, og = oracle.nvfp4_quantize(w)
    eq(u8(q.codes), oc, "nv codes")
    eq(u8(q.scales), os_, "nv scales")
    eq(bits(q.aux), og, "nv gs")
    eq(bits(pqb.dequantize(q)), oracle.nvfp4_dequantize(oc, os_, og), "nv dequant")


def test_heavy_tail_weight_mx_nv_full(pqb):
    w = synth.heavy_tail_weight(device=DEV)
    say("heavy-tailed [28672, 8192] bf16 mx/nv")
    rows = sample_rows(28672, 12, 2, [row_of_max(w)])
    ws = w[rows].cpu()
    qm = pqb.quantize(w, "mxfp4")
    oc, os_ = oracle.mxfp4_quantize(ws)
    eq(u8(qm.codes.view(28672, 4096)[rows]), oc, "mx codes")
    eq(u8(qm.scales.view(28672, 256)[rows]), os_, "mx scales")
    dq = pqb.dequantize(qm, torch.bfloat16)
    eq(bits(dq[0][rows]), oracle.mxfp4_dequantize(oc, os_, True), "mx dequant bf16")
    qn = pqb.quantize(w, "nvfp4")
    oc, os_, og = oracle.nvfp4_quantize(ws)        # the sample holds the tensor maximum
    eq(bits(qn.aux), og, "nv tensor scale")
    eq(u8(qn.codes.view(28672, 4096)[rows]), oc, "nv codes")
    eq(u8(qn.scales.view(28672, 512)[rows]), os_, "nv scales")
    dq = pqb.dequantize(qn, torch.bfloat16)
    eq(bits(dq[0][rows]), oracle.nvfp4_dequantize(oc, os_, og, True), "nv dequant bf16")


def test_llama_int4_all_224(pqb):
    say("llama-3.1-8b 224 weights int4 g128")
    for layer in range(synth.LLAMA_LAYERS):
        for p, (name, r, c) in enumerate(synth.LLAMA_PROJ):
            w = synth.llama_weight(layer, p, device=DEV)
            q = pqb.quantize(w, "int4_asym")
            G = c // 128
            rows = sample_rows(r, 2, 100 * layer + p)
            for row in rows:
                oc, os_, oz = oracle.int4_quantize(w[row:row + 1].cpu())
                eq(u8(q.codes.view(r, c // 2)[row]), oc, f"{name}{layer} codes row {row}")
                eq(bits(q.scales.view(r, G)[row]), os_, f"{name}{layer} scales row {row}")
                eq(u8(q.aux[row * G // 2:(row + 1) * G // 2]), oz, f"{name}{layer} zeros row {row}")
        if layer % 8 == 7:
            say(f"  layers 0..{layer} ok")
    w = synth.llama_weight(0, 4, device=DEV)
    q = pqb.quantize(w, "int4_asym")
    oc, os_, oz = oracle.int4_quantize(w[:2].cpu())
    eq(bits(pqb.dequantize(q, torch.bfloat16)[0, :2]), oracle.int4_dequantize(oc, os_, oz, True),
       "gate0 dequant bf16")


def test_kv_write_full(pqb):
    say("kv [28, 32768, 8, 128] bf16")
    k, v = synth.kv_cache(device=DEV)
    kc, vc, ks, vs = pqb.kv_write_fp8(k, v)
    for t, codes, sc, name in ((k, kc, ks, "K"), (v, vc, vs, "V")):
        for layer in (0, 13, 27):
            x = t[layer].reshape(32768, 1024)
            toks = sample_rows(32768, 3, layer, [row_of_max(x)])
            xs = x[toks].cpu().reshape(1, -1)
            oc, os_ = oracle.fp8_quantize(xs, "tensor")
            eq(bits(sc[layer:layer + 1]), os_, f"{name} scale layer {layer}")
            eq(u8(codes[layer].reshape(32768, 1024)[toks]), oc, f"{name} codes layer {layer}")


def test_sweep_1gib_all_formats(pqb):
    say("1 GiB bf16 [65536, 8192], every format")
    g = synth.gaussian(device=DEV)
    R, C = 65536, 8192
    mrow = row_of_max(g)
    rows = sample_rows(R, 6, 6, [mrow])
    gs_ = g[rows].cpu()
    for gran in ("1x128", "row", "tensor", "128x128"):
        q = pqb.quantize(g, "fp8_e4m3", gran)
        codes = q.codes.view(R, C)
        if gran == "128x128":
            band = mrow // 128
            oc, os_ = oracle.fp8_quantize(g[band * 128:(band + 1) * 128].cpu(), gran)
            eq(u8(codes[band * 128:(band + 1) * 128]), oc, "sweep 128x128 codes")
            eq(bits(q.scales.view(R // 128, C // 128)[band]), os_, "sweep 128x128 scales")
            continue
        oc, os_ = oracle.fp8_quantize(gs_, gran)
        eq(u8(codes[rows]), oc, f"sweep fp8 {gran} codes")
        if gran == "1x128":
            eq(bits(q.scales.view(R, C // 128)[rows]), os_, "sweep 1x128 scales")
        elif gran == "row":
            eq(bits(q.scales[rows]), os_, "sweep row scales")
        else:
            eq(bits(q.scales), os_, "sweep tensor scale")
    q = pqb.quantize(g, "mxfp4")
    oc, os_ = oracle.mxfp4_quantize(gs_)
    eq(u8(q.codes.view(R, C // 2)[rows]), oc, "sweep mx codes")
    q = pqb.quantize(g, "nvfp4")
    oc, os_, og = oracle.nvfp4_quantize(gs_)
    eq(bits(q.aux), og, "sweep nv gs")
    eq(u8(q.codes.view(R, C // 2)[rows]), oc, "sweep nv codes")
    eq(u8(q.scales.view(R, C // 16)[rows]), os_, "sweep nv scales")
    q = pqb.quantize(g, "int4_asym")
    oc, os_, oz = oracle.int4_quantize(gs_)
    eq(u8(q.codes.view(R, C // 2)[rows]), oc, "sweep int4 codes")
    eq(bits(q.scales.view(R, C // 128)[rows]), os_, "sweep int4 scales")


def test_past_2_31_elements(pqb):
    """A bf16 tensor [262272, 8192] holds 2^31 + 2^20 elements: its last
    128-row band lies wholly past element 2^31, where 32-bit element indexing
    would wrap.  Every one-pass and two-pass format, quantize and dequantize to
    bf16 and to float32, is compared with the oracle on three 128-row bands
    (first, middle, last);
    the tensor maximum is planted in the last band, so the per-tensor scales
    of the sample are the global ones."""
    R, C = 262272, 8192
    assert R * C > 2 ** 31 and (R - 128) * C >= 2 ** 31
    g = torch.Generator(device=DEV).manual_seed(31)
    x = torch.randn((R, C), generator=g, device=DEV).to(torch.bfloat16)
    x[R - 1, C - 1] = 40.0
    bands = list(range(0, 128)) + list(range(131072, 131200)) + list(range(R - 128, R))
    xs = x[bands].cpu()
    say("past 2^31: fp8 scopes")
    for gran in ("1x128", "128x128", "row", "tensor"):
        q = pqb.quantize(x, "fp8_e4m3", gran)
        oc, os_ = oracle.fp8_quantize(xs, gran)
        eq(u8(q.codes.view(R, C)[bands]), oc, f"fp8 {gran} codes")
        if gran == "1x128":
            eq(bits(q.scales.view(R, C // 128)[bands]), os_, "fp8 1x128 scales")
        elif gran == "row":
            eq(bits(q.scales[bands]), os_, "fp8 row scales")
        elif gran == "tensor":
            eq(bits(q.scales), os_, "fp8 tensor scale")
        else:
            tiles = [0, 1024, R // 128 - 1]
            eq(bits(q.scales.view(R // 128, C // 128)[tiles]), os_, "fp8 128x128 scales")
        dq = pqb.dequantize(q, torch.bfloat16)
        eq(bits(dq[0][bands]), oracle.fp8_dequantize(oc, os_, gran, True), f"fp8 {gran} dequant")
        del dq
        dq = pqb.dequantize(q, torch.float32)
        eq(bits(dq[0][bands]), oracle.fp8_dequantize(oc, os_, gran), f"fp8 {gran} dequant f32")
        del q, dq
    say("past 2^31: mxfp4, nvfp4, int4")
    q = pqb.quantize(x, "mxfp4")
    oc, os_ = oracle.mxfp4_quantize(xs)
    eq(u8(q.codes.view(R, C // 2)[bands]), oc, "mx codes")
    eq(u8(q.scales.view(R, C // 32)[bands]), os_, "mx scales")
    eq(bits(pqb.dequantize(q, torch.bfloat16)[0][bands]), oracle.mxfp4_dequantize(oc, os_, True), "mx dequant")
    eq(bits(pqb.dequantize(q, torch.float32)[0][bands]), oracle.mxfp4_dequantize(oc, os_), "mx dequant f32")
    del q
    q = pqb.quantize(x, "nvfp4")
    oc, os_, og = oracle.nvfp4_quantize(xs)
    eq(bits(q.aux), og, "nv tensor scale")
    eq(u8(q.codes.view(R, C // 2)[bands]), oc, "nv codes")
    eq(u8(q.scales.view(R, C // 16)[bands]), os_, "nv scales")
    eq(bits(pqb.dequantize(q, torch.bfloat16)[0][bands]), oracle.nvfp4_dequantize(oc, os_, og, True), "nv dequant")
    eq(bits(pqb.dequantize(q, torch.float32)[0][bands]), oracle.nvfp4_dequantize(oc, os_, og), "nv dequant f32")
    del q
    q = pqb.quantize(x, "int4_asym")
    oc, os_, oz = oracle.int4_quantize(xs)
    eq(u8(q.codes.view(R, C // 2)[bands]), oc, "int4 codes")
    eq(bits(q.scales.view(R, C // 128)[bands]), os_, "int4 scales")
    zb = u8(q.aux).reshape(R, C // 256)          # 64 groups per row: 32 whole bytes
    eq(zb[bands], oz, "int4 zero-points")
    eq(bits(pqb.dequantize(q, torch.bfloat16)[0][bands]), oracle.int4_dequantize(oc, os_, oz, True),
       "int4 dequant")
    eq(bits(pqb.dequantize(q, torch.float32)[0][bands]), oracle.int4_dequantize(oc, os_, oz),
       "int4 dequant f32")
    del q
    say("past 2^31: e5m2, int8, mxfp8")
    q = pqb.quantize(x, "fp8_e5m2", "1x128")
    oc, os_ = oracle.fp8_quantize(xs, "1x128", elem="e5m2")
    eq(u8(q.codes.view(R, C)[bands]), oc, "e5m2 codes")
    eq(bits(q.scales.view(R, C // 128)[bands]), os_, "e5m2 scales")
    eq(bits(pqb.dequantize(q, torch.float32)[0][bands]), oracle.fp8_dequantize(oc, os_, "1x128", elem="e5m2"),
       "e5m2 dequant f32")
    del q
    q = pqb.quantize(x, "int8_sym", "row")
    oc, os_ = oracle.int8_quantize(xs, "row")
    eq(u8(q.codes.view(R, C)[bands]), oc.view(np.uint8), "int8 codes")
    eq(bits(q.scales[bands]), os_, "int8 scales")
    eq(bits(pqb.dequantize(q, torch.float32)[0][bands]), oracle.int8_dequantize(oc, os_, "row"),
       "int8 dequant f32")
    del q
    q = pqb.quantize(x, "mxfp8")
    oc, os_ = oracle.mxfp8_quantize(xs)
    eq(u8(q.codes.view(R, C)[bands]), oc, "mxfp8 codes")
    eq(u8(q.scales.view(R, C // 32)[bands]), os_, "mxfp8 scales")
    eq(bits(pqb.dequantize(q, torch.float32)[0][bands]), oracle.mxfp8_dequantize(oc, os_), "mxfp8 dequant f32")


def test_fp8_128x128_paired_tiles(pqb):
    """Launches of 4096 or more 128x128 tiles (with an even number per tile row)
    take two adjacent tiles per workgroup.  Checked on sampled tile rows: a
    batch of 64 slices of 100 rows (short tiles, br = 100) in bf16 with E4M3,
    and a float32 [16384, 4096] tensor with E5M2."""
    g = torch.Generator(device=DEV).manual_seed(128)
    x = (torch.randn((64, 100, 8192), generator=g, device=DEV) *
         torch.exp(torch.randn((64, 100, 1), generator=g, device=DEV))).to(torch.bfloat16)
    q = pqb.quantize(x, "fp8_e4m3", "128x128")
    dq = pqb.dequantize(q, torch.bfloat16)
    for b in (0, 31, 63):
        oc, os_ = oracle.fp8_quantize(x[b:b + 1].cpu(), "128x128")
        eq(u8(q.codes.view(64, 100, 8192)[b]), oc, f"paired e4m3 codes slice {b}")
        eq(bits(q.scales.view(64, 64)[b]), os_, f"paired e4m3 scales slice {b}")
        eq(bits(dq[b]), oracle.fp8_dequantize(oc, os_, "128x128", True), f"paired e4m3 dequant {b}")
    y = torch.randn((16384, 4096), generator=g, device=DEV) * 3.0
    q = pqb.quantize(y, "fp8_e5m2", "128x128")
    for tr in (0, 77, 127):
        rows = slice(128 * tr, 128 * tr + 128)
        oc, os_ = oracle.fp8_quantize(y[rows].cpu(), "128x128", elem="e5m2")
        eq(u8(q.codes.view(16384, 4096)[rows]), oc, f"paired e5m2 codes tile row {tr}")
        eq(bits(q.scales.view(128, 32)[tr]), os_, f"paired e5m2 scales tile row {tr}")


def test_fp8_1x128_large_ragged_chunk(pqb):
    """From 2^28 elements the 1x128 quantizer takes chunks of 2 tiles per wave.
    A bf16 [32300, 8320] tensor (>= 2^28 elements, an odd number of 64-unit
    tiles) ends in a half chunk; the first rows and the last rows, which hold
    it, are compared with the oracle."""
    R, C = 32300, 8320
    assert R * C >= 2 ** 28 and (R * C // 8 // 64) % 2 == 1
    g = torch.Generator(device=DEV).manual_seed(283)
    x = torch.randn((R, C), generator=g, device=DEV).to(torch.bfloat16)
    q = pqb.quantize(x, "fp8_e4m3", "1x128")
    rows = list(range(0, 4)) + list(range(R - 40, R))
    oc, os_ = oracle.fp8_quantize(x[rows].cpu(), "1x128")
    eq(u8(q.codes.view(R, C)[rows]), oc, "1x128 codes")
    eq(bits(q.scales.view(R, C // 128)[rows]), os_, "1x128 scales")
