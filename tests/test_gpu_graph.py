"""The library's calls captured in a HIP graph (through torch.cuda.CUDAGraph) and
replayed: one-pass MXFP4, two-pass NVFP4 (its workspace partials rewritten on
every call) and an INT4 batch call.  Every replay, with the program's own eager
work and a synchronization between replays, must reproduce the eager call's
bytes exactly (the library issues kernel launches only, no memset or copy)."""
import ctypes

import pytest
import torch

from precision_quantization_block_amd import synth

pytestmark = pytest.mark.gpu


def _calls(p, xs, fmt, gran, shape, bufs, stream):
    L = p.lib()
    out = []
    for x, b in zip(xs, bufs):
        ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
        args = (ptr(x), 1 if x.dtype == torch.bfloat16 else 0, *shape, p.FORMATS[fmt], p.GRANS[gran],
                ptr(b["codes"]), ptr(b["scales"]), ptr(b["aux"]), ptr(b["workspace"]),
                b["sizes"]["workspace"], ctypes.c_void_p(stream))
        out.append(lambda args=args: L.pqb_quantize(*args))
    return out


def _alloc(p, fmt, gran, shape):
    s = p.query_sizes(fmt, gran, *shape)
    mk = lambda n: torch.zeros((max(n, 16),), dtype=torch.uint8, device="cuda") if n else None  # noqa: E731
    return {"codes": mk(s["codes"]), "scales": mk(s["scales"]), "aux": mk(s["aux"]),
            "workspace": mk(s["workspace"]), "sizes": s}


@pytest.mark.parametrize("fmt,gran", [("mxfp4", "blk32"), ("nvfp4", "blk16")])
def test_graph_replay_matches_eager(fmt, gran):
    import precision_quantization_block_amd as p
    shape = (1, 3072, 1024)
    xs = [synth.mlp_weight_fp32(seed=s, device="cuda").reshape(shape) for s in range(3)]
    eager = [_alloc(p, fmt, gran, shape) for _ in xs]
    for c in _calls(p, xs, fmt, gran, shape, eager, torch.cuda.current_stream().cuda_stream):
        assert c() == 0
    torch.cuda.synchronize()
    bufs = [_alloc(p, fmt, gran, shape) for _ in xs]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=side):
        for c in _calls(p, xs, fmt, gran, shape, bufs, side.cuda_stream):
            assert c() == 0
    for rep in range(3):
        for b in bufs:                      # eager work between replays
            b["codes"].zero_()
            b["scales"].zero_()
            if b["aux"] is not None:
                b["aux"].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for e, b in zip(eager, bufs):
            for k in ("codes", "scales", "aux"):
                if e[k] is not None:
                    assert torch.equal(e[k], b[k]), (fmt, rep, k)


def test_graph_replay_int4_batch_matches_eager():
    import precision_quantization_block_amd as p
    from precision_quantization_block_amd.synth import LLAMA_PROJ
    ws = [synth.llama_weight(0, j, device="cuda") for j in range(len(LLAMA_PROJ))]
    want = [p.quantize(w, "int4_asym") for w in ws]
    torch.cuda.synchronize()
    outs = [p.quantize(w, "int4_asym") for w in ws]     # buffers of the right shapes
    J = p.pqb._Job
    jobs = (J * len(ws))(*[J(w.data_ptr(), o.codes.data_ptr(), o.scales.data_ptr(), o.aux.data_ptr(), 1,
                             w.shape[0], w.shape[1], 1, p.FORMATS["int4_asym"], p.GRANS["grp128"], 0)
                           for w, o in zip(ws, outs)])
    L = p.lib()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=side):
        assert L.pqb_quantize_batch(jobs, len(ws), ctypes.c_void_p(side.cuda_stream)) == 0
    for rep in range(3):
        for o in outs:
            o.codes.zero_()
            o.scales.zero_()
            o.aux.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(want, outs):
            assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales) and torch.equal(a.aux, b.aux), rep
