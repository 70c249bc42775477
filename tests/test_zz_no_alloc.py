"""pqb_quantize_noalloc (the entry point for callers that cannot allocate)
against pqb_quantize with a caller-supplied workspace: the same bytes for the
two-pass formats that use its fixed scratch, two calls in a row with the
second on a smaller input (the scratch keeps the first call's contents), and
for a one-pass format that needs no scratch."""
import ctypes

import numpy as np
import pytest
import torch

from precision_quantization_block_amd import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
DTYPES = {torch.float32: 0, torch.bfloat16: 1}


@pytest.fixture(scope="module")
def pqb():
    import precision_quantization_block_amd as p
    p.lib()
    return p


def _outputs(pqb, fmt, gran, shape):
    s = pqb.query_sizes(fmt, gran, *shape)
    return {k: torch.zeros((max(v, 16),), dtype=torch.uint8, device=DEV) for k, v in s.items()}, s


def _noalloc(pqb, x, fmt, gran, shape):
    out, s = _outputs(pqb, fmt, gran, shape)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    rc = pqb.lib().pqb_quantize_noalloc(P(x), DTYPES[x.dtype], *shape, pqb.FORMATS[fmt],
                                        pqb.GRANS[gran], P(out["codes"]), P(out["scales"]),
                                        P(out["aux"]) if s["aux"] else None,
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, pqb.status_string(rc)
    return out, s


def _same(out, s, q, what):
    for name in ("codes", "scales", "aux"):
        ref = getattr(q, name)
        if not s[name]:
            continue
        got = out[name][: s[name]].cpu().numpy()
        exp = ref.view(torch.uint8).reshape(-1).cpu().numpy()
        assert got.shape == exp.shape and np.array_equal(got, exp), f"{what} {name}"


@pytest.mark.parametrize("fmt,gran", [("fp8_e4m3", "tensor"), ("nvfp4", "blk16"),
                                      ("fp8_e5m2", "tensor"), ("int8_sym", "tensor")])
def test_noalloc_equals_workspace_entry_point(pqb, fmt, gran):
    # the first call covers more scratch than the second
    for i, (shape, dtype) in enumerate((((3, 1000, 384), torch.bfloat16),
                                        ((2, 33, 128), torch.float32))):
        x = synth.fp8_activation(rows=shape[0] * shape[1], cols=shape[2], seed=60 + i)
        x = x.reshape(shape).to(dtype).to(DEV)
        q = pqb.quantize(x, fmt, gran)
        out, s = _noalloc(pqb, x, fmt, gran, shape)
        torch.cuda.synchronize()
        _same(out, s, q, f"{fmt} {shape} call {i}")


def test_noalloc_one_pass_format_and_empty(pqb):
    x = synth.fp8_weight(rows=256, cols=512, seed=3).to(DEV)
    q = pqb.quantize(x, "int4_asym")
    out, s = _noalloc(pqb, x, "int4_asym", "grp128", (1, 256, 512))
    torch.cuda.synchronize()
    _same(out, s, q, "int4 through noalloc")
    e = torch.empty((0,), dtype=torch.bfloat16, device=DEV)
    _noalloc(pqb, e, "nvfp4", "blk16", (1, 0, 16))


def test_noalloc_largest_slice_that_fits(pqb):
    """One per-tensor slice of 2^31 - 8192 bf16 elements (4 GiB) needs exactly
    the 1 MiB scratch (8192 more do not fit); checked on the scale and a sample
    of codes against the workspace form."""
    rows, cols = (1 << 18) - 1, 1 << 13
    need = pqb.query_sizes("fp8_e4m3", "tensor", 1, rows, cols)["workspace"]
    assert need == (1 << 20)
    assert pqb.query_sizes("fp8_e4m3", "tensor", 1, rows + 1, cols)["workspace"] > (1 << 20)
    x = torch.randn((rows, cols), device=DEV, dtype=torch.bfloat16)
    q = pqb.quantize(x, "fp8_e4m3", "tensor")
    out, s = _noalloc(pqb, x, "fp8_e4m3", "tensor", (1, rows, cols))
    torch.cuda.synchronize()
    assert torch.equal(out["scales"][:4], q.scales.view(torch.uint8))
    idx = torch.randint(0, rows * cols, (1 << 20,), device=DEV)
    assert torch.equal(out["codes"][idx], q.codes.view(torch.uint8).reshape(-1)[idx])
