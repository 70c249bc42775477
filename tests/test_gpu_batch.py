"""GPU parity of the fused batch entry point (pqb_quantize_batch).

Every job of a mixed batch must give exactly what the oracle gives for that
tensor alone (and so what pqb_quantize gives): codes, scales and zero-points
bit for bit.  The batches mix every one-pass kind, both input dtypes, ragged
shapes and empty tensors, and run past the per-launch job limit so that the
split into several launches is exercised.
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


def host_bits(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).reshape(-1)
    if t.dtype == torch.float32:
        return t.numpy().view(np.uint32).reshape(-1)
    return t.numpy().reshape(-1)


def ref_bits(a):
    a = np.ascontiguousarray(a)
    return (a.view(np.uint32) if a.dtype == np.float32 else a).reshape(-1)


def oracle_of(x, fmt, gran):
    if fmt == "fp8_e4m3":
        return oracle.fp8_quantize(x, gran)
    if fmt == "mxfp4":
        return oracle.mxfp4_quantize(x)
    return oracle.int4_quantize(x)


def check(q, ref, what):
    outs = [q.codes, q.scales] + ([q.aux] if len(ref) > 2 else [])
    for name, g, r in zip(("codes", "scales", "aux"), outs, ref):
        g, r = host_bits(g), ref_bits(r)
        assert g.shape == r.shape, f"{what} {name}: shape {g.shape} vs {r.shape}"
        bad = np.nonzero(g != r)[0]
        assert bad.size == 0, f"{what} {name}: {bad.size} mismatches, first at {bad[:8]}"


MIXED = [
    ("fp8_e4m3", "128x128", (1, 384, 2048)),
    ("fp8_e4m3", "1x128", (1, 333, 7168)),
    ("mxfp4", None, (2, 33, 96)),
    ("int4_asym", None, (1, 3, 14336)),
    ("fp8_e4m3", "row", (2, 33, 200)),
    ("fp8_e4m3", "128x128", (2, 64, 256)),
    ("fp8_e4m3", "1x128", (1, 0, 128)),          # empty
    ("mxfp4", None, (1, 257, 160)),
    ("int4_asym", None, (2, 9, 384)),
    ("fp8_e4m3", "128x128", (3, 1, 128)),
    ("fp8_e4m3", "row", (1, 7, 9000)),
    ("fp8_e4m3", "1x128", (2, 7, 384)),
    ("mxfp4", None, (1, 1, 32)),
    ("int4_asym", None, (1, 1, 128)),
]


def _inputs(specs, seed0):
    xs = []
    for i, (fmt, gran, (b, r, c)) in enumerate(specs):
        dtype = torch.bfloat16 if i % 2 == 0 else torch.float32
        x = synth.fp8_activation(rows=max(b * r, 1), cols=c, seed=seed0 + i)[: b * r]
        xs.append(x.reshape(b, r, c).to(dtype))
    return xs


@pytest.mark.parametrize("repeat", [1, 3])
def test_batch_matches_oracle(pqb, repeat):
    """`repeat` copies of the mixed list (14 or 42 jobs)."""
    specs = MIXED * repeat
    xs = _inputs(specs, 100)
    outs = pqb.quantize_batch([(x.to(DEV), f, g) for x, (f, g, _) in zip(xs, specs)])
    assert len(outs) == len(specs)
    for i, (x, (fmt, gran, shp), q) in enumerate(zip(xs, specs, outs)):
        check(q, oracle_of(x, fmt, gran or pqb.pqb.DEFAULT_GRAN[fmt]),
              f"job {i} {fmt} {gran} {shp} {x.dtype}")


def test_batch_equals_single_calls(pqb):
    specs = MIXED
    xs = [x.to(DEV) for x in _inputs(specs, 300)]
    outs = pqb.quantize_batch([(x, f, g) for x, (f, g, _) in zip(xs, specs)])
    for i, (x, (fmt, gran, shp), q) in enumerate(zip(xs, specs, outs)):
        s = pqb.quantize(x, fmt, gran)
        for name in ("codes", "scales", "aux"):
            a, b = getattr(q, name), getattr(s, name)
            assert (a is None) == (b is None)
            if a is not None:
                assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"job {i} {name}"


def test_batch_decoder_int4_weights(pqb):
    """The seven projections of one decoder layer (4096 hidden, 14336 MLP,
    8 KV heads of 128) as INT4 g128, in one call."""
    shapes = [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096),
              (14336, 4096), (14336, 4096), (4096, 14336)]
    ws = [synth.fp8_weight(rows=r, cols=c, seed=500 + i).to(torch.bfloat16)
          for i, (r, c) in enumerate(shapes)]
    outs = pqb.quantize_batch([(w.to(DEV), "int4_asym", None) for w in ws])
    rng = np.random.default_rng(7)
    for i, (w, q) in enumerate(zip(ws, outs)):
        # sampled rows, checked against the oracle one row at a time
        r, c = w.shape
        for row in rng.choice(r, 6, replace=False):
            oc, os_, oz = oracle.int4_quantize(w[row:row + 1])
            g = c // 128
            assert np.array_equal(host_bits(q.codes[row * c // 2:(row + 1) * c // 2]),
                                  ref_bits(oc)), f"proj {i} row {row} codes"
            assert np.array_equal(host_bits(q.scales[row * g:(row + 1) * g]),
                                  ref_bits(os_)), f"proj {i} row {row} scales"
            # zero-points of one row: g nibbles starting at flat group row*g (g even)
            zb = host_bits(q.aux[row * g // 2:(row * g + g) // 2])
            assert np.array_equal(zb, ref_bits(oz)), f"proj {i} row {row} zeros"


def test_batch_many_jobs_several_launches(pqb):
    """300 small ragged jobs: 150 FP8 (1x128 and 128x128), 75 MXFP4 and 75
    INT4, so each family is split over several launches (FP8 3, MXFP4 2,
    INT4 2) and the workgroup-to-job search crosses every job boundary."""
    rng = np.random.default_rng(11)
    specs = []
    for i in range(300):
        k = i % 4
        if k in (0, 1):
            gran = "1x128" if k == 0 else "128x128"
            rows = int(rng.integers(1, 6)) if k == 0 else int(rng.choice([1, 3, 64, 128, 256]))
            specs.append(("fp8_e4m3", gran, (1, rows, 128 * int(rng.integers(1, 4)))))
        elif k == 2:
            specs.append(("mxfp4", None, (1, int(rng.integers(1, 9)), 32 * int(rng.integers(1, 6)))))
        else:
            specs.append(("int4_asym", None, (1, int(rng.integers(1, 5)), 128 * int(rng.integers(1, 4)))))
    xs = _inputs(specs, 700)
    items = [(x.to(DEV), f, g) for x, (f, g, _) in zip(xs, specs)]
    outs = pqb.quantize_batch(items)
    for i, (x, (fmt, gran, shp), q) in enumerate(zip(xs, specs, outs)):
        check(q, oracle_of(x, fmt, gran or pqb.pqb.DEFAULT_GRAN[fmt]),
              f"job {i} {fmt} {gran} {shp} {x.dtype}")


DQ_SPECS = [("fp8_e4m3", "1x128", (1, 33, 384)), ("fp8_e5m2", "1x128", (2, 5, 128)),
            ("mxfp4", "blk32", (1, 17, 96)), ("mxfp8", "blk32", (3, 4, 64)),
            ("nvfp4", "blk16", (3, 7, 48)), ("int4_asym", "grp128", (2, 9, 384)),
            ("fp8_e4m3", "tensor", (2, 10, 40)), ("fp8_e4m3", "row", (1, 6, 200)),
            ("fp8_e4m3", "128x128", (1, 256, 256)), ("int8_sym", "row", (1, 3, 24)),
            ("int4_asym", "grp128", (1, 0, 128))]


@pytest.mark.parametrize("repeat", [1, 9])
def test_dequantize_batch_equals_single_calls(pqb, repeat):
    """Mixed formats and scopes, both output dtypes, NVFP4 with several slices
    and an empty job; 9 copies make 90 fused jobs (NVFP4 slices counted one by
    one: 108), so the float32 and bf16 launches each split in two."""
    qs = []
    for i, (fmt, gran, shp) in enumerate(DQ_SPECS * repeat):
        b, r, c = shp
        x = synth.fp8_activation(rows=max(b * r, 1), cols=c, seed=900 + i)[: b * r].reshape(b, r, c)
        qs.append((pqb.quantize(x.to(DEV), fmt, gran), torch.bfloat16 if i % 2 else torch.float32))
    outs = pqb.dequantize_batch(qs)
    for i, ((q, dt), o) in enumerate(zip(qs, outs)):
        ref = pqb.dequantize(q, dt)
        assert o.dtype == ref.dtype and o.shape == ref.shape
        assert torch.equal(o.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                           ref.view(torch.int16 if dt == torch.bfloat16 else torch.int32)), \
            f"job {i} {q.fmt} {q.gran} {q.shape} {dt}"


def test_batch_empty_list(pqb):
    assert pqb.quantize_batch([]) == []
