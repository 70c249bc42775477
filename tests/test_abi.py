"""The C ABI on the CPU: the library loads, exports what include/pqb.h
declares, sizes its buffers as the pages' storage arithmetic says, and turns
bad arguments into status codes before anything reaches the GPU."""
import ctypes
import os
import re

import pytest

from conftest import ROOT, golden

HEADER = os.path.join(ROOT, "include", "pqb.h")

import precision_quantization_block_amd as pqb  # noqa: E402


@pytest.fixture(scope="module")
def L():
    return pqb.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pqb_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol(L):
    names = declared_functions()
    assert "pqb_quantize" in names and "pqb_dequantize" in names and "pqb_kv_write_fp8" in names
    for n in names:
        assert hasattr(L, n), n
    assert pqb.abi_version() == 1


def test_source_hash_is_checked(L, monkeypatch):
    """The library carries the digest of the sources it was built from, and the
    binding refuses one that no longer matches them."""
    from precision_quantization_block_amd import _build
    assert L.pqb_source_hash().decode() == _build.source_hash()
    pqb.pqb.check_source_hash(L)
    monkeypatch.setattr(_build, "source_hash", lambda: "0000000000000000")
    with pytest.raises(RuntimeError, match="other sources"):
        pqb.pqb.check_source_hash(L)


def test_status_strings(L):
    for code in range(0, -9, -1):
        assert pqb.status_string(code) not in ("", "unknown status")
    assert pqb.status_string(5) == "unknown status"


def test_sizes_match_storage_arithmetic():
    n = 28672 * 8192
    mx = pqb.query_sizes("mxfp4", "blk32", 1, 28672, 8192)
    assert (mx["codes"] + mx["scales"]) * 8 / n == golden("mxfp4_bits_per_element")
    nv = pqb.query_sizes("nvfp4", "blk16", 1, 28672, 8192)
    assert (nv["codes"] + nv["scales"]) * 8 / n == golden("nvfp4_bits_per_element")
    assert nv["aux"] == 4 and nv["workspace"] > 0
    i4 = pqb.query_sizes("int4_asym", "grp128", 1, 4096, 4096)
    per = (i4["codes"] + i4["scales"]) / (4096 * 4096)
    assert per == 0.515625 and round(per, 3) == golden("int4_g128_bytes_per_weight")
    assert i4["aux"] == 4096 * 4096 // 256
    f8 = pqb.query_sizes("fp8_e4m3", "1x128", 1, 8192, 7168)
    assert f8 == {"codes": 58720256, "scales": 1835008, "aux": 0, "workspace": 0}
    f8w = pqb.query_sizes("fp8_e4m3", "128x128", 1, 7168, 2048)
    assert f8w["scales"] == 4 * 56 * 16
    f8s = pqb.query_sizes("fp8_e4m3", "128x128", 1, 64, 256)
    assert f8s["scales"] == 4 * 1 * 2


def test_llama8b_int4_total_is_about_3_6_gb():
    """32 decoder layers of the Llama-3.1-8B linear shapes at INT4 g128:
    packed codes plus 2-byte scales come to about 3.6 GB."""
    shapes = [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096),
              (14336, 4096), (14336, 4096), (4096, 14336)]
    total = params = 0
    for r, c in shapes:
        s = pqb.query_sizes("int4_asym", "grp128", 1, r, c)
        total += s["codes"] + s["scales"]
        params += r * c
    total *= 32
    params *= 32
    assert total == 3_598_712_832
    assert round(total / 1e9, 1) == golden("llama8b_int4_gb")
    assert round(params / 1e9, 1) == 7.0


def test_kv_workspace_and_bytes():
    assert pqb.lib().pqb_kv_workspace_bytes(28, 32768 * 8 * 128) > 0
    assert pqb.lib().pqb_kv_workspace_bytes(0, 10) == 0


@pytest.mark.parametrize("fmt,gran,shape,status", [
    ("fp8_e4m3", "blk32", (1, 8, 32), -3),
    ("mxfp4", "1x128", (1, 8, 128), -3),
    ("fp8_e4m3", "1x128", (1, 8, 100), -4),
    ("fp8_e4m3", "128x128", (1, 200, 128), -4),
    ("fp8_e4m3", "128x128", (1, 128, 130), -4),
    ("mxfp4", "blk32", (1, 8, 48), -4),
    ("nvfp4", "blk16", (1, 8, 24), -4),
    ("int4_asym", "grp128", (1, 8, 64), -4),
    ("fp8_e4m3", "row", (-1, 8, 64), -4),
])
def test_query_sizes_rejects(fmt, gran, shape, status):
    with pytest.raises(pqb.PqbError) as e:
        pqb.query_sizes(fmt, gran, *shape)
    assert e.value.status == status


def test_quantize_argument_errors_before_launch(L):
    """Every case below must fail validation, so no kernel is ever enqueued."""
    P = ctypes.c_void_p
    fake = P(0x10000)          # aligned, never dereferenced
    odd = P(0x10001)
    q = L.pqb_quantize
    # unknown enums
    assert q(fake, 7, 1, 8, 128, 0, 2, fake, fake, None, None, 0, None) == -2
    assert q(fake, 1, 1, 8, 128, 9, 2, fake, fake, None, None, 0, None) == -2
    assert q(fake, 1, 1, 8, 128, 0, 9, fake, fake, None, None, 0, None) == -2
    # bad pairing and shapes
    assert q(fake, 1, 1, 8, 128, 0, 4, fake, fake, None, None, 0, None) == -3
    assert q(fake, 1, 1, 8, 100, 0, 2, fake, fake, None, None, 0, None) == -4
    # null pointers
    assert q(None, 1, 1, 8, 128, 0, 2, fake, fake, None, None, 0, None) == -1
    assert q(fake, 1, 1, 8, 128, 0, 2, None, fake, None, None, 0, None) == -1
    assert q(fake, 1, 1, 8, 128, 2, 5, fake, fake, None, fake, 1 << 20, None) == -1   # NV aux
    assert q(fake, 1, 1, 8, 128, 3, 6, fake, fake, None, None, 0, None) == -1        # INT4 aux
    assert q(fake, 1, 1, 8, 128, 0, 0, fake, fake, None, None, 0, None) == -1        # workspace
    # workspace too small
    assert q(fake, 1, 1, 8, 128, 0, 0, fake, fake, None, fake, 0, None) == -6
    # alignment
    assert q(odd, 1, 1, 8, 128, 0, 2, fake, fake, None, None, 0, None) == -5
    assert q(fake, 1, 1, 8, 128, 0, 2, odd, fake, None, None, 0, None) == -5
    # empty tensors succeed without touching anything
    assert q(None, 1, 0, 8, 128, 0, 2, None, None, None, None, 0, None) == 0


def test_dequantize_and_kv_errors(L):
    P = ctypes.c_void_p
    fake, odd = P(0x10000), P(0x10002)
    d = L.pqb_dequantize
    assert d(fake, fake, None, 0, 2, 1, 8, 128, 5, fake, None) == -2
    assert d(None, fake, None, 0, 2, 1, 8, 128, 0, fake, None) == -1
    assert d(fake, fake, None, 2, 5, 1, 8, 128, 0, fake, None) == -1       # NV needs gs
    assert d(fake, fake, None, 0, 2, 1, 8, 128, 0, odd, None) == -5
    kv = L.pqb_kv_write_fp8
    assert kv(fake, fake, 1, 2, 1024, fake, fake, fake, fake, fake, 0, None) == -6
    assert kv(None, fake, 1, 2, 1024, fake, fake, fake, fake, fake, 1 << 20, None) == -1
    assert kv(fake, fake, 4, 2, 1024, fake, fake, fake, fake, fake, 1 << 20, None) == -2
    assert kv(fake, fake, 1, 0, 1024, None, None, None, None, None, 0, None) == 0
    assert L.pqb_encode_e4m3(None, 4, fake, None) == -1
    assert L.pqb_encode_e2m1(fake, -1, fake, None) == -4


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        pqb.quantize(torch.zeros(4, 128), "fp8_e4m3", "1x128")


def test_quantize_batch_errors_before_launch(L):
    J = pqb.pqb._Job
    fake = 0x10000

    def job(**kw):
        d = dict(x=fake, codes=fake, scales=fake, aux=None, batch=1, rows=128, cols=256,
                 dtype=1, fmt=0, gran=2, reserved=0)
        d.update(kw)
        return J(**d)

    def run(*jobs):
        return L.pqb_quantize_batch((J * len(jobs))(*jobs), len(jobs), None)

    # a bad job anywhere fails the whole call before anything is enqueued
    assert run(job(), job(gran=0)) == -3                 # per-tensor FP8 needs two passes
    assert run(job(fmt=2, gran=5), job()) == -3          # so does NVFP4
    assert run(job(), job(reserved=1)) == -2
    assert run(job(), job(fmt=7)) == -2
    assert run(job(), job(dtype=3)) == -2
    assert run(job(), job(x=None)) == -1
    assert run(job(fmt=3, gran=6)) == -1                 # INT4 needs its zero-point buffer
    assert run(job(), job(cols=100)) == -4
    assert run(job(), job(rows=-1)) == -4
    assert run(job(), job(codes=fake + 2)) == -5
    assert L.pqb_quantize_batch(None, -1, None) == -4
    assert L.pqb_quantize_batch(None, 1, None) == -1
    assert L.pqb_quantize_batch(None, 0, None) == 0
    # empty jobs are accepted and launch nothing (no device is touched)
    assert run(job(rows=0), job(batch=0, fmt=3, gran=6, aux=fake)) == 0


def test_quantize_batch_launch_plan(L):
    """How many launches a batch takes (no device work), and the grid limit:
    a launch of more than 2^32 - 1 threads is refused before anything runs."""
    J = pqb.pqb._Job
    fake = 0x10000

    def job(**kw):
        d = dict(x=fake, codes=fake, scales=fake, aux=None, batch=1, rows=128, cols=256,
                 dtype=1, fmt=0, gran=2, reserved=0)
        d.update(kw)
        return J(**d)

    def launches(*jobs):
        return L.pqb_quantize_batch_launches((J * len(jobs))(*jobs), len(jobs))

    int4 = dict(fmt=3, gran=6, aux=fake)
    assert launches(job(), job(gran=3)) == 1                       # 1x128 and 128x128 share one
    assert launches(job(), job(gran=3), job(gran=1)) == 2          # a per-row job is its own
    assert launches(*[job(**int4)] * 72) == 1                      # up to 72 jobs per launch
    assert launches(*[job(**int4)] * 73) == 2
    assert launches(*[job(**int4)] * 224) == 4                     # the Llama-3.1-8B decoder
    assert launches(job(), job(fmt=1, gran=4), job(**int4)) == 3   # one launch per family
    assert launches(job(rows=0)) == 0
    assert launches(job(gran=0)) == -3
    # 2^36 elements of 1x128 FP8 need 2^23 workgroups of 512 threads: one too many
    assert launches(job(rows=1 << 20, cols=1 << 16)) == -4
    assert launches(job(rows=(1 << 20) - 1, cols=1 << 16)) == 1
    assert L.pqb_quantize_batch((J * 1)(job(rows=1 << 20, cols=1 << 16)), 1, None) == -4
    # one wave per row, 4 rows per 256-thread workgroup
    assert launches(job(gran=1, rows=4 * (0xFFFFFFFF // 256) + 1, cols=8)) == -4
    assert launches(job(gran=1, rows=4 * (0xFFFFFFFF // 256), cols=8)) == 1


def test_division_check_errors_before_launch(L):
    fake = 0x10000
    assert L.pqb_check_recip(0, -1, fake, None) == -4
    assert L.pqb_check_recip(0xFFFFFFFF, 2, fake, None) == -4     # past the last pattern
    assert L.pqb_check_recip(5, 0, None, None) == 0
    assert L.pqb_check_recip(5, 3, None, None) == -1
    assert L.pqb_check_recip(5, 3, fake + 2, None) == -5
    assert L.pqb_check_div(fake, -1, 0, 4, fake, None) == -4
    assert L.pqb_check_div(fake, 1, 0xFFFFFFF0, 17, fake, None) == -4
    assert L.pqb_check_div(fake, 1 << 40, 0, 1 << 30, fake, None) == -4
    assert L.pqb_check_div(None, 2, 0, 4, fake, None) == -1
    assert L.pqb_check_div(fake, 2, 0, 4, fake + 1, None) == -5
    assert L.pqb_check_div(fake, 0, 0, 4, fake, None) == 0


def test_quantize_noalloc_errors_before_launch(L):
    """The no-allocation entry point validates like pqb_quantize and refuses a
    shape whose workspace exceeds its fixed scratch, before any GPU call."""
    fake = 0x10000
    P = pqb.lib().pqb_quantize_noalloc
    # a per-tensor FP8 slice of 2^33 float32 elements needs > 1 MiB of partials
    assert pqb.query_sizes("fp8_e4m3", "tensor", 1, 1 << 17, 1 << 16)["workspace"] > 1 << 20
    assert P(fake, 0, 1, 1 << 17, 1 << 16, 0, 0, fake, fake, None, None) == -8
    assert P(fake, 1, 1, 1 << 17, 1 << 16, 2, 5, fake, fake, fake, None) == -8   # NVFP4
    assert P(fake, 1, 1, 8, 100, 0, 2, fake, fake, None, None) == -4            # 1x128 shape
    assert P(None, 1, 1, 8, 128, 0, 0, fake, fake, None, None) == -1
    assert P(fake, 1, 1, 8, 128, 2, 5, fake, fake, None, None) == -1            # NVFP4 needs aux
    assert P(fake + 2, 1, 1, 8, 128, 0, 0, fake, fake, None, None) == -5
    assert P(fake, 1, 1, 8, 128, 9, 0, fake, fake, None, None) == -2
    assert P(fake, 1, 1, 0, 128, 0, 0, None, None, None, None) == 0               # empty
    assert pqb.status_string(-8) != "unknown status"


def test_dequantize_batch_errors_before_launch(L):
    J = pqb.pqb._DqJob
    fake = 0x10000

    def job(**kw):
        d = dict(codes=fake, scales=fake, aux=None, out=fake, batch=1, rows=128, cols=256, fmt=0,
                 gran=2, out_dtype=1, reserved=0)
        d.update(kw)
        return J(**d)

    def run(*jobs):
        return L.pqb_dequantize_batch((J * len(jobs))(*jobs), len(jobs), None)

    assert run(job(), job(reserved=1)) == -2
    assert run(job(), job(out_dtype=5)) == -2
    assert run(job(), job(fmt=1, gran=5)) == -3
    assert run(job(), job(fmt=3, gran=6)) == -1          # INT4 needs its zero-points
    assert run(job(), job(fmt=2, gran=5)) == -1          # NVFP4 needs its tensor scales
    assert run(job(), job(cols=100)) == -4
    assert run(job(), job(out=fake + 8)) == -5
    assert L.pqb_dequantize_batch(None, -1, None) == -4
    assert L.pqb_dequantize_batch(None, 0, None) == 0
    assert run(job(rows=0), job(batch=0, fmt=3, gran=6)) == 0   # empty: nothing launched


def test_kv_write_ex_errors_before_launch(L):
    P = ctypes.c_void_p
    fake, odd = P(0x10000), P(0x10002)
    ws = L.pqb_kv_workspace_bytes_ex
    f = L.pqb_kv_write_fp8_ex
    big = 1 << 30

    def kv(k=fake, v=fake, dt=1, shape=(2, 16, 8, 128), km=0, vm=0, kc=fake, vc=fake,
           ks=fake, vs=fake, w=fake, wb=big):
        return f(k, v, dt, *shape, km, vm, kc, vc, ks, vs, w, wb, None)

    assert ws(2, 16, 8, 128) > 0
    assert ws(2, 16, 8, 100) == 0                     # head_dim % 8
    assert kv(dt=5) == -2
    assert kv(km=3) == -2 and kv(vm=-1) == -2
    assert kv(shape=(2, 16, 8, 100)) == -4
    assert kv(shape=(-1, 16, 8, 128)) == -4
    assert kv(shape=(2, 16, 300, 128), km=1) == -4    # more heads than the per-head limit
    assert kv(shape=(2, 16, 256, 8 * 4096), km=1) == -4  # heads * (head_dim/8)^2 = 2^32
    assert kv(k=None, v=None) == -1
    assert kv(kc=None) == -1 and kv(vs=None) == -1
    assert kv(w=None) == -1
    assert kv(wb=ws(2, 16, 8, 128) - 1) == -6
    assert kv(k=odd) == -5 and kv(vc=odd) == -5 and kv(w=odd) == -5
    # static modes need no workspace; empty shapes launch nothing
    assert kv(shape=(0, 16, 8, 128)) == 0
    assert kv(shape=(2, 0, 8, 128), km=1, vm=1, w=None, wb=0) == 0
    assert kv(k=None, kc=None, ks=None, shape=(2, 0, 8, 128)) == 0


def test_kivi_errors_before_launch(L):
    P = ctypes.c_void_p
    fake, odd, odd8 = P(0x10000), P(0x10002), P(0x10008)
    w = L.pqb_kv_write_kivi
    r = L.pqb_kv_read_kivi

    def wr(k=fake, v=fake, dt=1, shape=(2, 64, 8, 128), bits=2, kc=fake, vc=fake, ks=fake,
           km=fake, vs=fake, vm=fake):
        return w(k, v, dt, *shape, bits, kc, vc, ks, km, vs, vm, None)

    def rd(kc=fake, vc=fake, ks=fake, km=fake, vs=fake, vm=fake, shape=(2, 64, 8, 128), bits=4,
           dt=0, ko=fake, vo=fake):
        return r(kc, vc, ks, km, vs, vm, *shape, bits, dt, ko, vo, None)

    for f in (wr, rd):
        assert f(dt=2) == -2
        assert f(bits=3) == -2 and f(bits=8) == -2 and f(bits=0) == -2
        assert f(shape=(2, 64, 8, 96 + 8)) == -4           # head_dim % 32
        assert f(shape=(2, 48, 8, 128)) == -4              # K needs tokens % 32
        assert f(shape=(-2, 64, 8, 128)) == -4
        assert f(shape=(1 << 20, 1 << 10, 1 << 4, 128)) == -4   # 2^41 elements
        assert f(shape=(1 << 30, 1 << 30, 1 << 30, 1 << 30)) == -4  # product overflows int64
    assert wr(k=None, v=None) == -1 and rd(kc=None, vc=None) == -1
    assert wr(kc=None) == -1 and wr(km=None) == -1 and wr(vm=None) == -1
    assert rd(ks=None) == -1 and rd(vo=None) == -1 and rd(ko=None) == -1
    assert wr(k=odd) == -5 and wr(vc=odd8) == -5 and wr(ks=odd8) == -5 and wr(vm=odd8) == -5
    assert rd(kc=odd8) == -5 and rd(vs=odd8) == -5 and rd(ko=odd8) == -5
    # empty shapes launch nothing; V alone does not need tokens % 32
    assert wr(shape=(0, 64, 8, 128)) == 0 and rd(shape=(2, 64, 0, 128)) == 0
    assert wr(k=None, kc=None, ks=None, km=None, shape=(2, 0, 8, 128)) == 0
    assert wr(k=None, shape=(2, 48, 8, 128), v=fake, vc=None) == -1   # V checks still run
    assert rd(kc=None, shape=(0, 48, 8, 128)) == 0


def test_gemm_errors_before_launch(L):
    P = ctypes.c_void_p
    fake, odd = P(0x10000), P(0x10008)
    g = L.pqb_gemm_fp8_blockscaled

    def gm(a=fake, sa=fake, b=fake, sb=fake, m=256, n=256, k=512, dt=1, c=fake):
        return g(a, sa, b, sb, m, n, k, dt, c, None)

    assert gm(dt=3) == -2
    assert gm(k=500) == -4 and gm(n=200) == -4 and gm(m=-1) == -4 and gm(k=-128) == -4
    assert gm(m=1 << 31) == -4 and gm(k=1 << 31) == -4
    assert gm(m=(1 << 31) - 1, n=(1 << 30)) == -4          # too many tiles
    assert gm(a=None) == -1 and gm(sb=None) == -1 and gm(c=None) == -1
    assert gm(a=odd) == -5 and gm(b=odd) == -5 and gm(c=odd) == -5 and gm(sa=P(0x10002)) == -5
    assert gm(m=0) == 0 and gm(n=0, c=None) == 0               # nothing to do
    gq = L.pqb_gemm_fp8_blockscaled_quant

    def gmq(a=fake, sa=fake, b=fake, sb=fake, m=256, n=256, k=512, c=fake, cs=fake):
        return gq(a, sa, b, sb, m, n, k, c, cs, None)

    assert gmq(k=500) == -4 and gmq(n=200) == -4
    assert gmq(cs=None) == -1 and gmq(c=None) == -1 and gmq(a=None) == -1
    assert gmq(cs=P(0x10002)) == -5 and gmq(c=odd) == -5
    assert gmq(m=0) == 0


def test_gemm_mxfp4_errors_before_launch(L):
    P = ctypes.c_void_p
    fake = P(0x10000)
    g = L.pqb_gemm_mxfp4

    def gm(a=fake, sa=fake, b=fake, sb=fake, m=256, n=256, k=512, dt=0, c=fake):
        return g(a, sa, b, sb, m, n, k, dt, c, None)

    assert gm(dt=2) == -2
    assert gm(k=500) == -4 and gm(n=200) == -4 and gm(m=-1) == -4
    assert gm(sa=None) == -1 and gm(b=None) == -1 and gm(c=None) == -1
    assert gm(a=P(0x10008)) == -5 and gm(sb=P(0x10002)) == -5 and gm(c=P(0x10004)) == -5
    assert gm(m=0) == 0


def test_gemm_nvfp4_errors_before_launch(L):
    P = ctypes.c_void_p
    fake = P(0x10000)
    g = L.pqb_gemm_nvfp4

    def gm(a=fake, sa=fake, ga=fake, b=fake, sb=fake, gb=fake, m=256, n=256, k=512, dt=0, c=fake):
        return g(a, sa, ga, b, sb, gb, m, n, k, dt, c, None)

    assert gm(dt=2) == -2
    assert gm(k=500) == -4 and gm(n=200) == -4 and gm(m=-1) == -4 and gm(k=1 << 31) == -4
    assert gm(sa=None) == -1 and gm(ga=None) == -1 and gm(gb=None) == -1 and gm(b=None) == -1
    assert gm(c=None) == -1
    assert gm(a=P(0x10008)) == -5 and gm(sb=P(0x10002)) == -5 and gm(gb=P(0x10002)) == -5
    assert gm(c=P(0x10004)) == -5
    assert gm(m=0) == 0 and gm(n=0, c=None) == 0


def test_stream_reference_errors_before_launch(L):
    P = ctypes.c_void_p
    fake = P(0x10000)
    f = L.pqb_stream_reference
    assert f(fake, 8192, 3, 8, fake, None) == -2 and f(fake, 8192, 0, 8, fake, None) == -2
    assert f(fake, 8192, 1, 2, fake, None) == -2 and f(fake, 8192, 4, 16, fake, None) == -2
    assert f(fake, 8000, 1, 8, fake, None) == -4 and f(fake, -8192, 1, 4, fake, None) == -4
    assert f(fake, (1 << 38) + 8192, 1, 8, fake, None) == -4
    assert f(None, 8192, 1, 8, fake, None) == -1 and f(fake, 8192, 2, 4, None, None) == -1
    assert f(P(0x10008), 8192, 1, 8, fake, None) == -5 and f(fake, 8192, 4, 4, P(0x10004), None) == -5
    assert f(None, 0, 1, 8, None, None) == 0


def test_w4a16_errors_before_launch(L):
    P = ctypes.c_void_p
    fake, odd = P(0x10000), P(0x10008)
    f = L.pqb_gemv_w4a16

    def gv(x=fake, m=1, c=fake, s=fake, z=fake, n=256, k=512, dt=0, y=fake):
        return f(x, m, c, s, z, n, k, dt, y, None)

    assert gv(dt=4) == -2
    assert gv(m=9) == -4 and gv(m=-1) == -4 and gv(k=500) == -4 and gv(n=-1) == -4
    assert gv(n=1 << 30, k=1 << 20) == -4          # n * k / 128 over 2^31
    assert gv(x=None) == -1 and gv(z=None) == -1 and gv(y=None) == -1
    assert gv(x=odd) == -5 and gv(c=odd) == -5 and gv(s=P(0x10001)) == -5 and gv(y=P(0x10002)) == -5
    assert gv(m=0) == 0 and gv(n=0, y=None) == 0
    from precision_quantization_block_amd.pqb import _W4Job
    fb = L.pqb_gemv_w4a16_batch
    J = lambda **kw: _W4Job(**{**dict(x=0x10000, codes=0x10000, scales=0x10000, zeros=0x10000,  # noqa: E731
                                      y=0x10000, n=256, k=512), **kw})
    arr = lambda *js: (_W4Job * len(js))(*js)  # noqa: E731
    assert fb(arr(J(), J(k=500)), 2, 1, 0, None) == -4        # second job bad: nothing launched
    assert fb(arr(J(), J(y=None)), 2, 1, 0, None) == -1
    assert fb(arr(J(x=0x10008)), 1, 1, 0, None) == -5
    assert fb(arr(J()), 1, 9, 0, None) == -4 and fb(arr(J()), 1, 1, 3, None) == -2
    assert fb(None, 1, 1, 0, None) == -1 and fb(None, 0, 1, 0, None) == 0
    assert fb(arr(J(n=0, y=None)), 1, 1, 0, None) == 0


def test_w4a16_matrix_core_errors_before_launch(L):
    P = ctypes.c_void_p
    fake, odd = P(0x10000), P(0x10008)
    f = L.pqb_gemm_w4a16

    def gm(x=fake, m=1, c=fake, s=fake, z=fake, n=256, k=512, dt=0, y=fake):
        return f(x, m, c, s, z, n, k, dt, y, None)

    assert gm(dt=4) == -2
    assert gm(m=-1) == -4 and gm(m=1 << 31) == -4 and gm(k=500) == -4 and gm(n=-1) == -4
    assert gm(n=1 << 30, k=1 << 20) == -4
    assert gm(x=None) == -1 and gm(z=None) == -1 and gm(y=None) == -1
    assert gm(m=9, x=odd) == -5 and gm(c=odd) == -5 and gm(s=P(0x10001)) == -5 and gm(y=P(0x10002)) == -5
    assert gm(m=0) == 0 and gm(m=100, n=0, y=None) == 0
    from precision_quantization_block_amd.pqb import _W4Job
    fb = L.pqb_gemm_w4a16_batch
    J = lambda **kw: _W4Job(**{**dict(x=0x10000, codes=0x10000, scales=0x10000, zeros=0x10000,  # noqa: E731
                                      y=0x10000, n=256, k=512), **kw})
    arr = lambda *js: (_W4Job * len(js))(*js)  # noqa: E731
    assert fb(arr(J(), J(k=500)), 2, 40, 0, None) == -4       # second job bad: nothing launched
    assert fb(arr(J(), J(y=None)), 2, 40, 0, None) == -1
    assert fb(arr(J(x=0x10008)), 1, 40, 0, None) == -5
    assert fb(arr(J()), 1, -1, 0, None) == -4 and fb(arr(J()), 1, 1, 3, None) == -2
    assert fb(None, 1, 1, 0, None) == -1 and fb(None, 0, 1, 0, None) == 0
    assert fb(arr(J(n=0, y=None)), 1, 40, 0, None) == 0


def test_head_index_by_multiply_high_is_exact():
    """Per-head kernels find the head of a column c < heads * hu (hu = head_dim
    / 8 units) as the high 32 bits of c * ceil(2^32 / hu).  The ABI admits
    heads * hu^2 < 2^32; check every column at the edges of that rule."""
    import numpy as np

    def heads_of(c, hu):
        # the kernel's arithmetic: a 32-bit multiplier, 0 meaning "the column itself"
        magic = 0 if hu == 1 else ((0xFFFFFFFF // hu) + 1)
        assert magic < 1 << 32
        if magic == 0:
            return c.copy()
        return (c.astype(np.uint64) * np.uint64(magic)) >> np.uint64(32)

    for heads, hu in ((256, 4095), (256, 1), (1, 65535), (255, 4103), (3, 37837), (8, 16),
                      (40, 16), (12, 8)):
        assert heads * hu * hu < 1 << 32
        c = np.arange(heads * hu, dtype=np.uint64)
        assert np.array_equal(heads_of(c, hu), c // np.uint64(hu)), (heads, hu)
    # just past the rule the shortcut does fail somewhere, so the bound is needed
    heads, hu = 65536, 65535
    c = np.arange(heads * hu - 100000, heads * hu, dtype=np.uint64)
    assert not np.array_equal(heads_of(c, hu), c // np.uint64(hu))


def test_variant_sizes_and_pairs(L):
    # E5M2 sizes equal E4M3's; INT8 has per-tensor and per-row scopes only;
    # MXFP8 stores one byte per element and one E8M0 byte per 32
    for gran in ("tensor", "row", "1x128", "128x128"):
        assert pqb.query_sizes("fp8_e5m2", gran, 2, 256, 384) == \
            pqb.query_sizes("fp8_e4m3", gran, 2, 256, 384)
    assert pqb.query_sizes("int8_sym", "row", 2, 3, 40) == \
        {"codes": 240, "scales": 24, "aux": 0, "workspace": 0}
    assert pqb.query_sizes("mxfp8", "blk32", 1, 4, 64) == \
        {"codes": 256, "scales": 8, "aux": 0, "workspace": 0}
    S = pqb.pqb._Sizes()
    assert L.pqb_query_sizes(6, 2, 1, 8, 128, ctypes.byref(S)) == -3   # INT8 x 1x128
    assert L.pqb_query_sizes(5, 5, 1, 8, 128, ctypes.byref(S)) == -3   # MXFP8 x blk16
    assert L.pqb_query_sizes(5, 4, 1, 8, 48, ctypes.byref(S)) == -4    # MXFP8 needs c % 32
    assert L.pqb_query_sizes(7, 0, 1, 8, 128, ctypes.byref(S)) == -2   # unknown format
    # per-tensor INT8 and E5M2 need workspace, so the batch call refuses them
    J = pqb.pqb._Job
    fake = 0x10000
    jobs = (J * 1)(J(fake, fake, fake, None, 1, 8, 128, 1, 6, 0, 0))
    assert L.pqb_quantize_batch(jobs, 1, None) == -3
    jobs = (J * 1)(J(fake, fake, fake, None, 1, 8, 128, 1, 4, 0, 0))
    assert L.pqb_quantize_batch(jobs, 1, None) == -3
    assert L.pqb_encode_e5m2(None, 4, fake, None) == -1
