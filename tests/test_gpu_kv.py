"""GPU parity of the FP8 KV-cache write with a scale mode per tensor
(pqb_kv_write_fp8_ex): per layer, per head, static scale, against the oracle,
byte for byte (codes and scales)."""
import zlib

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


def bits(t):
    t = t.detach().cpu().contiguous()
    return t.view(torch.int32).numpy() if t.dtype == torch.float32 else t.numpy()


def kv_pair(L, T, H, D, tag, dtype):
    g = torch.Generator().manual_seed(zlib.crc32(tag.encode()))
    bias = torch.randn((L, 1, H, D), generator=g) * 2
    k = (bias + 0.1 * torch.randn((L, T, H, D), generator=g)).to(dtype)
    v = (torch.randn((L, T, H, D), generator=g)
         * 2.0 ** torch.randint(-4, 5, (1, 1, H, 1), generator=g)).to(dtype)
    return k, v


def check(x, codes, scales, mode, given=None, what=""):
    oc, os_ = oracle.kv_quant_fp8(x, mode, scales=given)
    got_c = codes.cpu().numpy()
    bad = np.argwhere(got_c != oc)
    assert bad.size == 0, f"{what}: {len(bad)} code mismatches, first {bad[:4].tolist()}"
    if mode != "static":
        assert np.array_equal(bits(scales), os_.view(np.int32)), f"{what}: scales differ"


SHAPES = [(3, 100, 8, 128), (2, 33, 4, 64), (1, 7, 40, 128), (2, 5, 12, 64), (1, 1, 1, 8),
          (1, 3, 256, 8), (2, 129, 2, 256)]
MODES = [("layer", "layer"), ("head", "head"), ("head", "layer"), ("layer", "head")]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", SHAPES)
def test_kv_modes_match_oracle(pqb, shape, dtype):
    k, v = kv_pair(*shape, f"modes{shape}", dtype)
    kd, vd = k.to(DEV), v.to(DEV)
    for km, vm in MODES:
        kc, vc, ks, vs = pqb.kv_write_fp8_ex(kd, vd, km, vm)
        check(k, kc, ks, km, what=f"K {km} {shape} {dtype}")
        check(v, vc, vs, vm, what=f"V {vm} {shape} {dtype}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_kv_static_scales(pqb, dtype):
    """Static per-layer scales: at the dynamic scale (same codes as LAYER), at a
    quarter of it (the clamp binds for the largest values), at 4x, and at the
    ends of the supported range."""
    L, T, H, D = 3, 40, 8, 128
    k, v = kv_pair(L, T, H, D, "static", dtype)
    kd, vd = k.to(DEV), v.to(DEV)
    _, _, ks, vs = pqb.kv_write_fp8_ex(kd, vd, "layer", "layer")
    for f in (1.0, 0.25, 4.0):
        sk, sv = ks * f, vs * f
        kc, vc, _, _ = pqb.kv_write_fp8_ex(kd, vd, "static", "static", k_scales=sk, v_scales=sv)
        check(k, kc, None, "static", sk.cpu().numpy(), f"K static x{f}")
        check(v, vc, None, "static", sv.cpu().numpy(), f"V static x{f}")
    # extreme but valid scales: everything saturates, or everything underflows
    for s in (2.0 ** -64, 2.0 ** -30, 2.0 ** 100, 2.0 ** 125):
        sk = torch.full((L,), s, dtype=torch.float32, device=DEV)
        kc, _, _, _ = pqb.kv_write_fp8_ex(kd, None, "static", k_scales=sk)
        check(k, kc, None, "static", sk.cpu().numpy(), f"K static s={s}")


def test_kv_layer_mode_equals_kv_write_fp8(pqb):
    L, T, H, D = 4, 77, 8, 128
    k, v = kv_pair(L, T, H, D, "same", torch.bfloat16)
    kd, vd = k.to(DEV), v.to(DEV)
    a = pqb.kv_write_fp8(kd, vd)
    b = pqb.kv_write_fp8_ex(kd, vd, "layer", "layer")
    for x, y in zip(a, b):
        assert torch.equal(x.reshape(-1).view(torch.uint8), y.reshape(-1).view(torch.uint8))


def test_kv_only_k_or_only_v(pqb):
    L, T, H, D = 2, 50, 4, 128
    k, v = kv_pair(L, T, H, D, "one", torch.bfloat16)
    kc, vc, ks, vs = pqb.kv_write_fp8_ex(k.to(DEV), None, "head")
    assert vc is None and vs is None
    check(k, kc, ks, "head", what="only K")
    kc, vc, ks, vs = pqb.kv_write_fp8_ex(None, v.to(DEV), v_mode="layer")
    assert kc is None and ks is None
    check(v, vc, vs, "layer", what="only V")
    sv = torch.tensor([0.01, 0.002], device=DEV)
    _, vc, _, _ = pqb.kv_write_fp8_ex(None, v.to(DEV), v_mode="static", v_scales=sv)
    check(v, vc, None, "static", sv.cpu().numpy(), "only V static")


def test_kv_edge_values(pqb):
    """Zero heads (the 1e-12 floor), signed zeros, bf16 subnormals, a huge value
    in one head and values near the E4M3 rounding boundaries."""
    L, T, H, D = 2, 9, 4, 64
    x = torch.randn((L, T, H, D)) * 0.5
    x[0, :, 1] = 0.0
    x[0, 3, 1, ::2] = -0.0
    x[1, :, 2] = torch.randn((T, D)) * 1e-39
    x[1, 4, 3, 7] = 3e38
    x[0, :, 3] = torch.linspace(-448, 448, T * D).reshape(T, D) * 2.0 ** -20
    for dtype in (torch.float32, torch.bfloat16):
        xd = x.to(dtype)
        for mode in ("layer", "head"):
            kc, _, ks, _ = pqb.kv_write_fp8_ex(xd.to(DEV), None, mode)
            check(xd, kc, ks, mode, what=f"edges {mode} {dtype}")


def test_kv_full_size_head_mode_sampled(pqb):
    """The full cache write, K and V [28 x 32768 x 8 x 128] bf16, per head:
    every scale and sampled tokens of every layer against the oracle (which
    works one (layer, head) at a time here)."""
    k, v = synth.kv_cache(device=DEV)
    L, T, H, D = 28, 32768, 8, 128
    k = k.reshape(L, T, H, D)
    v = v.reshape(L, T, H, D)
    kc, vc, ks, vs = pqb.kv_write_fp8_ex(k, v, "head", "head")
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    for x, c, s, name in ((k, kc, ks, "K"), (v, vc, vs, "V")):
        for layer in rng.choice(L, 4, replace=False):
            xl = x[layer].cpu()                            # [T, H, D]
            # the oracle on this layer alone gives its 8 per-head scales
            _, os_ = oracle.kv_quant_fp8(xl.reshape(1, T, H, D), "head")
            assert np.array_equal(bits(s[layer]), os_.reshape(-1).view(np.int32)), \
                f"{name} layer {layer} scales"
            toks = rng.choice(T, 16, replace=False)
            sub = xl[toks].reshape(16, H * D).float().numpy()
            sc = os_.reshape(H)
            y = sub.reshape(16, H, D) / sc[None, :, None]
            ref = oracle.e4m3_encode_array(np.clip(y, -448, 448).astype(np.float32).reshape(-1))
            got = c[layer][toks].cpu().numpy().reshape(-1)
            assert np.array_equal(got, ref), f"{name} layer {layer} sampled codes"
