"""GPU parity of the KIVI-style 2/4-bit KV cache (pqb_kv_write_kivi,
pqb_kv_read_kivi) against the oracle: codes byte for byte, scales and minimums
bit for bit, dequantized values bit for bit in float32 and bf16."""
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


def f32_bits(t):
    return t.detach().cpu().contiguous().view(torch.int32).numpy()


def out_bits(t):
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).numpy()


def oracle_out_bits(a):
    return a.view(np.int16) if a.dtype == np.uint16 else a.view(np.int32)


def kv_pair(L, T, H, D, tag, dtype):
    """K with a per-channel bias and a few outlier channels; V per-head scaled."""
    g = torch.Generator().manual_seed(zlib.crc32(tag.encode()))
    bias = torch.randn((L, 1, H, D), generator=g) * 2
    bias[..., ::17] *= 8
    k = (bias + 0.3 * torch.randn((L, T, H, D), generator=g)).to(dtype)
    v = (torch.randn((L, T, H, D), generator=g)
         * 2.0 ** torch.randint(-4, 5, (1, 1, H, 1), generator=g)).to(dtype)
    return k, v


def check_write(x, parts, bits, is_k, what):
    oc, os_, om = oracle.kivi_quant(x, bits, is_k)
    c, s, m = parts
    got = c.cpu().numpy().reshape(oc.shape)
    bad = np.argwhere(got != oc)
    assert bad.size == 0, f"{what}: {len(bad)} code bytes differ, first {bad[:4].tolist()}"
    assert np.array_equal(f32_bits(s).reshape(os_.shape), os_.view(np.int32)), f"{what}: scales"
    assert np.array_equal(f32_bits(m).reshape(om.shape), om.view(np.int32)), f"{what}: mins"
    return oc, os_, om


def check_read(pqb, parts, o, shape, bits, is_k, what):
    oc, os_, om = o
    for out_dtype, bf in ((torch.float32, False), (torch.bfloat16, True)):
        ref = oracle.kivi_dequant(oc, os_, om, bits, is_k, out_bf16=bf)
        args = (parts, None) if is_k else (None, parts)
        ko, vo = pqb.kv_read_kivi(*args, shape, bits, out_dtype)
        got = ko if is_k else vo
        assert (vo if is_k else ko) is None
        assert np.array_equal(out_bits(got).reshape(ref.shape), oracle_out_bits(ref)), \
            f"{what}: dequant to {out_dtype} differs"


SHAPES = [(2, 64, 8, 128), (1, 96, 3, 32), (3, 32, 1, 64), (1, 160, 5, 96), (2, 256, 2, 256),
          (1, 32, 1, 32), (1, 544, 4, 128)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("shape", SHAPES)
def test_kivi_write_and_read_match_oracle(pqb, shape, bits, dtype):
    k, v = kv_pair(*shape, f"kivi{shape}{bits}", dtype)
    kp, vp = pqb.kv_write_kivi(k.to(DEV), v.to(DEV), bits)
    tag = f"{shape} {bits}b {dtype}"
    ok = check_write(k, kp, bits, True, "K " + tag)
    ov = check_write(v, vp, bits, False, "V " + tag)
    check_read(pqb, kp, ok, shape, bits, True, "K " + tag)
    check_read(pqb, vp, ov, shape, bits, False, "V " + tag)


def test_kivi_v_only_any_token_count(pqb):
    """V alone needs no multiple of 32 tokens; K alone leaves V untouched."""
    for shape in ((2, 45, 3, 64), (1, 1, 1, 32), (3, 7, 9, 160)):
        _, v = kv_pair(*shape, f"vonly{shape}", torch.bfloat16)
        kp, vp = pqb.kv_write_kivi(None, v.to(DEV), 2)
        assert kp is None
        o = check_write(v, vp, 2, False, f"V only {shape}")
        check_read(pqb, vp, o, shape, 2, False, f"V only {shape}")
    k, _ = kv_pair(1, 64, 2, 64, "konly", torch.float32)
    kp, vp = pqb.kv_write_kivi(k.to(DEV), None, 4)
    assert vp is None
    check_write(k, kp, 4, True, "K only")


def edge_tensor():
    """Groups that are constant, all zero with signed zeros, exact rounding ties
    (s = 1), bf16 subnormals, and a range close to the float32 maximum."""
    L, T, H, D = 1, 64, 2, 64
    x = torch.randn((L, T, H, D)) * 0.5
    x[0, :, 0, 0] = 1.25                              # constant K group, V groups vary
    x[0, 0, 1, :32] = -3.0                            # constant V group
    x[0, :32, 0, 1] = -0.0                            # K group of signed zeros
    x[0, :32, 0, 1][::3] = 0.0
    x[0, 5, 1, 32:] = -0.0                            # V group of zeros
    ties = torch.tensor([0.0, 3.0, 0.5, 1.5, 2.5, 1.0, 2.0, 0.25] * 4)
    x[0, :32, 1, 2] = ties                            # K group 0..3: s = 1 at 2 bits
    x[0, 7, 0, :32] = ties                            # V group
    x[0, :, 1, 3] = torch.randn(T) * 1e-39            # subnormal K channel
    x[0, 9, 1, :32] = torch.randn(32) * 1e-39         # subnormal V group
    x[0, 40, 0, 4] = 1.5e38                           # range near the float32 maximum
    x[0, 41, 0, 4] = -1.5e38
    x[0, 11, 0, 32:] = torch.linspace(-1.5e38, 1.5e38, 32)
    return x


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_kivi_edge_groups(pqb, bits, dtype):
    x = edge_tensor().to(dtype)
    shape = tuple(x.shape)
    kp, vp = pqb.kv_write_kivi(x.to(DEV), x.to(DEV), bits)
    ok = check_write(x, kp, bits, True, f"K edges {bits}b {dtype}")
    ov = check_write(x, vp, bits, False, f"V edges {bits}b {dtype}")
    check_read(pqb, kp, ok, shape, bits, True, "K edges")
    check_read(pqb, vp, ov, shape, bits, False, "V edges")


@pytest.mark.parametrize("bits", [2, 4])
def test_kivi_full_cache_sampled(pqb, bits):
    """The full cache, K and V [28 x 32768 x 8 x 128] bf16, written and read back
    as the benchmark does; sampled 32-token windows of several layers against
    the oracle (a K group never crosses a window, a V group never a token)."""
    L, T, H, D = 28, 32768, 8, 128
    k, v = synth.kv_cache(device=DEV)
    k = k.reshape(L, T, H, D)
    v = v.reshape(L, T, H, D)
    kp, vp = pqb.kv_write_kivi(k, v, bits)
    ko, vo = pqb.kv_read_kivi(kp, vp, (L, T, H, D), bits, torch.bfloat16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11 + bits)
    per_tok = H * D * bits // 8
    for layer in rng.choice(L, 3, replace=False):
        for w in sorted(rng.choice(T // 32, 4, replace=False)):
            t0 = int(w) * 32
            sl = (slice(int(layer), int(layer) + 1), slice(t0, t0 + 32))
            for x, parts, out, is_k, name in ((k, kp, ko, True, "K"), (v, vp, vo, False, "V")):
                xs = x[sl].cpu()
                oc, os_, om = oracle.kivi_quant(xs, bits, is_k)
                c, s, m = parts
                b0 = (int(layer) * T + t0) * per_tok
                got_c = c[b0:b0 + 32 * per_tok].cpu().numpy()
                assert np.array_equal(got_c, oc.reshape(-1)), f"{name} codes layer {layer} t0 {t0}"
                gs = s[int(layer), t0 // 32] if is_k else s[int(layer), t0:t0 + 32]
                gm = m[int(layer), t0 // 32] if is_k else m[int(layer), t0:t0 + 32]
                assert np.array_equal(f32_bits(gs).reshape(-1), os_.view(np.int32).reshape(-1))
                assert np.array_equal(f32_bits(gm).reshape(-1), om.view(np.int32).reshape(-1))
                ref = oracle.kivi_dequant(oc, os_, om, bits, is_k, out_bf16=True)
                assert np.array_equal(out_bits(out[sl]).reshape(ref.shape), ref.view(np.int16)), \
                    f"{name} dequant layer {layer} t0 {t0}"
