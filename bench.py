"""Throughput of the quantize-pack path on one MI355X.

Headline workload: INT4 group-128 asymmetric conversion of a whole
Llama-3.1-8B-shaped decoder, 32 layers x {q [4096x4096], k and v [1024x4096],
o [4096x4096], gate and up [14336x4096], down [4096x14336]} bf16 weights
(6,979,321,856 weights, 13.96 GB in, 3.63 GB of codes, bf16 scales and
zero-point nibbles out).  One step = one pqb_quantize_batch call over all 224
weights.  value = (bytes read + bytes written) per step / time, in GB/s; the
inputs sit in HBM before timing starts, and one step touches 17.6 GB, far more
than the 256 MB Infinity Cache, so nothing is served from it.

The last stdout line is the headline record (one compact JSON object).  Every
other workload gets one `record <name> <json>` line on stderr (and, with
--records FILE, a JSON file holding all of them): the FP8 W8A8 step, MXFP4 /
NVFP4 on the float32 [3072, 1024] MLP weight and on the bf16 [28672, 8192]
heavy-tailed weight, the FP8 KV write of [28 x 32768 x 8 x 128] K and V,
every format on a 1 GiB bf16 tensor, the GEMMs and W4A16.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras]
       [--no-cpu] [--copy-probe] [--reps R] [--only NAME] [--records FILE]
       [--headline-only]
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP8_MFMA_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 matrix peak (no sparsity)
FP4_MFMA_PEAK_TFLOPS = 10100.0      # MI355X dense FP4 / FP6 matrix peak
BF16_MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 / f16 matrix peak
METRIC = "quantize-pack GB/s (bytes in+out) and % of HBM peak, per format"
HEADLINE_KERNEL = "k_multi<INT4> (fused INT4 g128 batch kernel)"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "k_multi_int4_llama8b_224w_counters.json")
KERNEL_SOURCES = ["precision_quantization_block_amd/csrc/k_multi.hip",
                  "precision_quantization_block_amd/csrc/quant.h",
                  "precision_quantization_block_amd/csrc/device.h"]
_RECORDS = {}


def record(name, rec_):
    """One non-headline result: a stderr line now, the --records file at the end."""
    _RECORDS[name] = rec_
    print(f"record {name} {json.dumps(rec_, separators=(',', ':'))}", file=sys.stderr,
          flush=True)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class Engine:
    """Direct C-ABI calls on preallocated buffers (no allocation while timing)."""

    def __init__(self, torch, pqb):
        self.torch, self.pqb, self.L = torch, pqb, pqb.lib()
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def alloc(self, fmt, gran, shape, device):
        t = self.torch
        s = self.pqb.query_sizes(fmt, gran, *shape)
        buf = {k: (t.empty((max(v, 16),), dtype=t.uint8, device=device) if v else None)
               for k, v in s.items()}
        buf["sizes"] = s
        return buf

    def quantize(self, x, fmt, gran, shape, buf):
        P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
        s = buf["sizes"]
        rc = self.L.pqb_quantize(P(x), 1 if x.dtype == self.torch.bfloat16 else 0, *shape,
                                 self.pqb.FORMATS[fmt], self.pqb.GRANS[gran], P(buf["codes"]),
                                 P(buf["scales"]), P(buf["aux"]), P(buf["workspace"]),
                                 s["workspace"], self.stream)
        if rc != 0:
            raise RuntimeError(f"pqb_quantize {fmt}/{gran}: status {rc}")

    def quantize_call(self, x, fmt, gran, shape, buf, stream=None):
        """pqb_quantize on `x` into `buf` with its arguments marshalled once: the
        returned call costs one ctypes call, so that a loop of small tensors times
        the library rather than Python.  `stream` (a raw handle) defaults to the
        engine's stream."""
        ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
        st = self.stream if stream is None else ctypes.c_void_p(stream)
        args = (ptr(x), 1 if x.dtype == self.torch.bfloat16 else 0, *shape,
                self.pqb.FORMATS[fmt], self.pqb.GRANS[gran], ptr(buf["codes"]), ptr(buf["scales"]),
                ptr(buf["aux"]), ptr(buf["workspace"]), buf["sizes"]["workspace"], st)
        f = self.L.pqb_quantize

        def call():
            rc = f(*args)
            if rc != 0:
                raise RuntimeError(f"pqb_quantize {fmt}/{gran}: status {rc}")
        return call

    def dequantize_call(self, buf, fmt, gran, shape, out, stream=None):
        """pqb_dequantize of `buf` into `out`, arguments marshalled once."""
        ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
        st = self.stream if stream is None else ctypes.c_void_p(stream)
        args = (ptr(buf["codes"]), ptr(buf["scales"]), ptr(buf["aux"]), self.pqb.FORMATS[fmt],
                self.pqb.GRANS[gran], *shape, 1 if out.dtype == self.torch.bfloat16 else 0,
                ptr(out), st)
        f = self.L.pqb_dequantize

        def call():
            rc = f(*args)
            if rc != 0:
                raise RuntimeError(f"pqb_dequantize {fmt}/{gran}: status {rc}")
        return call

    def jobs(self, items):
        """A prebuilt pqb_job array for `items` = [(x, fmt, gran, shape, buf)]."""
        J = self.pqb.pqb._Job
        arr = (J * len(items))()
        for j, (x, fmt, gran, shape, buf) in zip(arr, items):
            j.x, j.codes, j.scales = x.data_ptr(), buf["codes"].data_ptr(), \
                buf["scales"].data_ptr()
            j.aux = buf["aux"].data_ptr() if buf["aux"] is not None else None
            j.batch, j.rows, j.cols = shape
            j.dtype = 1 if x.dtype == self.torch.bfloat16 else 0
            j.fmt, j.gran = self.pqb.FORMATS[fmt], self.pqb.GRANS[gran]
        return arr, len(items)

    def batch(self, jobs):
        rc = self.L.pqb_quantize_batch(jobs[0], jobs[1], self.stream)
        if rc != 0:
            raise RuntimeError(f"pqb_quantize_batch: status {rc}")

    def dequantize(self, buf, fmt, gran, shape, out):
        P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
        rc = self.L.pqb_dequantize(P(buf["codes"]), P(buf["scales"]), P(buf["aux"]),
                                   self.pqb.FORMATS[fmt], self.pqb.GRANS[gran], *shape,
                                   1 if out.dtype == self.torch.bfloat16 else 0, P(out),
                                   self.stream)
        if rc != 0:
            raise RuntimeError(f"pqb_dequantize {fmt}/{gran}: status {rc}")

    def dq_jobs(self, items):
        """A prebuilt pqb_dq_job array for `items` = [(buf, fmt, gran, shape, out)]."""
        J = self.pqb.pqb._DqJob
        arr = (J * len(items))()
        for j, (buf, fmt, gran, shape, out) in zip(arr, items):
            j.codes, j.scales = buf["codes"].data_ptr(), buf["scales"].data_ptr()
            j.aux = buf["aux"].data_ptr() if buf["aux"] is not None else None
            j.out = out.data_ptr()
            j.batch, j.rows, j.cols = shape
            j.fmt, j.gran = self.pqb.FORMATS[fmt], self.pqb.GRANS[gran]
            j.out_dtype = 1 if out.dtype == self.torch.bfloat16 else 0
        return arr, len(items)

    def dequantize_batch(self, jobs):
        rc = self.L.pqb_dequantize_batch(jobs[0], jobs[1], self.stream)
        if rc != 0:
            raise RuntimeError(f"pqb_dequantize_batch: status {rc}")

    def kv(self, k, v, kc, vc, ks, vs, ws):
        P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        layers = k.shape[0]
        rc = self.L.pqb_kv_write_fp8(P(k), P(v), 1, layers, k.numel() // layers, P(kc), P(vc),
                                     P(ks), P(vs), P(ws), ws.numel(), self.stream)
        if rc != 0:
            raise RuntimeError(f"pqb_kv_write_fp8: status {rc}")


def out_bytes(sizes):
    return sizes["codes"] + sizes["scales"] + sizes["aux"]


def time_loop(torch, fn, reps, warmup):
    """Average time (ms) per call over `reps` back-to-back calls on the current
    stream, bracketed by two events."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(reps):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def time_reps(torch, fn, reps, warmup):
    """(loop mean, median, min) in ms.  The mean comes from `reps` back-to-back
    calls bracketed by two events; median and min from a second run of `reps`
    calls with an event between consecutive calls (each such event adds a small
    gap, so per-repeat times run slightly above the back-to-back mean)."""
    mean = time_loop(torch, fn, reps, warmup)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        fn(i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    t = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))
    mid = reps // 2
    med = t[mid] if reps % 2 else 0.5 * (t[mid - 1] + t[mid])
    return mean, med, t[0]


def rec(bytes_moved, times, two_pass_read=0, **kw):
    """One result record; `times` = (mean, median, min) in ms.  GB/s (Form 1)
    counts the input once plus every output; for two-pass formats
    `two_pass_read` is the second input read, added in the *_incl_pass1
    figures."""
    mean, med, mn = times
    gbs = bytes_moved / (mean * 1e-3) / 1e9
    d = {"bytes": int(bytes_moved), "ms": round(mean, 5), "ms_median": round(med, 5),
         "ms_min": round(mn, 5), "gbs": round(gbs, 1),
         "gbs_median": round(bytes_moved / (med * 1e-3) / 1e9, 1),
         "gbs_at_min": round(bytes_moved / (mn * 1e-3) / 1e9, 1),
         "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    if two_pass_read:
        tb = bytes_moved + two_pass_read
        d["bytes_incl_pass1"] = int(tb)
        d["gbs_incl_pass1"] = round(tb / (mean * 1e-3) / 1e9, 1)
        d["frac_hbm_peak_incl_pass1"] = round(tb / (mean * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    d.update(kw)
    return d


# ----------------------------------------------------------------------------
# headline: INT4 g128 over the 224 Llama-3.1-8B-shaped decoder weights
# ----------------------------------------------------------------------------

def llama_int4_set(torch, eng, synth, dev):
    """The 224 bf16 weights (seed 3000 + 7 layer + proj) and their INT4 outputs."""
    from precision_quantization_block_amd.synth import LLAMA_LAYERS, LLAMA_PROJ
    xs, bufs, shapes = [], [], []
    nb = 0
    for layer in range(LLAMA_LAYERS):
        for p, (_, r, c) in enumerate(LLAMA_PROJ):
            x = synth.llama_weight(layer, p, device=dev)
            b = eng.alloc("int4_asym", "grp128", (1, r, c), dev)
            xs.append(x)
            bufs.append(b)
            shapes.append((1, r, c))
            nb += x.numel() * 2 + out_bytes(b["sizes"])
    return xs, bufs, shapes, nb


def bench_headline(torch, eng, synth, steps, warmup):
    dev = torch.device("cuda:0")
    xs, bufs, shapes, step_bytes = llama_int4_set(torch, eng, synth, dev)
    jobs = eng.jobs([(x, "int4_asym", "grp128", shp, b) for x, shp, b in zip(xs, shapes, bufs)])
    launches = eng.L.pqb_quantize_batch_launches(jobs[0], jobs[1])

    def step(i):
        eng.batch(jobs)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region: K steps back to back on the stream the kernels are launched
    # on (the current stream, which eng.stream is), events only at the ends.
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    wall0 = time.perf_counter()
    ev[0].record()
    for k in range(steps):
        step(k)
    ev[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = ev[0].elapsed_time(ev[1])
    log(f"headline: {steps} steps of INT4 g128 over 224 weights, {ms_total / steps:.4f} ms per "
        f"step, {launches} launches per step (wall {wall * 1e3:.1f} ms)")
    return {"ms_per_step": ms_total / steps, "step_bytes": step_bytes, "launches": launches,
            "wall_s": wall, "xs": xs, "bufs": bufs, "shapes": shapes}


def int4_records_extra(torch, eng, h, reps=5):
    """The same 224 weights quantized with one pqb_quantize call each, and
    dequantized back to bf16, one call each and as one batch call."""
    dev = torch.device("cuda:0")
    xs, bufs, shapes = h["xs"], h["bufs"], h["shapes"]

    qcalls = [eng.quantize_call(x, "int4_asym", "grp128", shp, b)
              for x, shp, b in zip(xs, shapes, bufs)]

    def one_by_one(i):
        for c in qcalls:
            c()

    t = time_reps(torch, one_by_one, reps, 1)
    record("llama8b_224w_bf16_int4_g128_per_tensor",
           rec(h["step_bytes"], t, op="INT4 g128 asym, 224 weights, one pqb_quantize call each",
               launches=224))
    # leave the batch call's outputs in place for the parity check
    eng.batch(eng.jobs([(x, "int4_asym", "grp128", shp, b)
                        for x, shp, b in zip(xs, shapes, bufs)]))
    outs = [torch.empty(shp, dtype=torch.bfloat16, device=dev) for shp in shapes]
    nbd = sum(out_bytes(b["sizes"]) + o.numel() * 2 for b, o in zip(bufs, outs))

    dcalls = [eng.dequantize_call(b, "int4_asym", "grp128", shp, o)
              for shp, b, o in zip(shapes, bufs, outs)]

    def dq_all(i):
        for c in dcalls:
            c()

    t = time_reps(torch, dq_all, reps, 1)
    record("llama8b_224w_bf16_int4_g128_dequant",
           rec(nbd, t, op="dequantize INT4 -> bf16, 224 weights, one call each", launches=224))
    if hasattr(eng.L, "pqb_dequantize_batch"):
        djobs = eng.dq_jobs([(b, "int4_asym", "grp128", shp, o)
                             for shp, b, o in zip(shapes, bufs, outs)])
        t = time_reps(torch, lambda i: eng.dequantize_batch(djobs), reps, 1)
        record("llama8b_224w_bf16_int4_g128_dequant_batch",
               rec(nbd, t, op="dequantize INT4 -> bf16, 224 weights, one batch call"))
    del outs
    torch.cuda.synchronize()


# ----------------------------------------------------------------------------
# secondary: the FP8 E4M3 W8A8 step (weight 128x128 + activations 1x128)
# ----------------------------------------------------------------------------

def bench_w8a8(torch, eng, synth, steps, warmup, nsets):
    """bf16 weight [7168, 2048] with 128x128 block scales plus bf16 activations
    [8192, 7168] with 1x128 block scales, one pqb_quantize_batch call (one fused
    launch) per step, rotated over `nsets` buffer sets (> 1 GiB in all)."""
    dev = torch.device("cuda:0")
    wshape, ashape = (1, 7168, 2048), (1, 8192, 7168)
    sets = []
    for i in range(nsets):
        w = synth.fp8_weight(seed=1 + 1000 * i, device=dev)
        a = synth.fp8_activation(seed=2 + 1000 * i, device=dev)
        sets.append((w, a, eng.alloc("fp8_e4m3", "128x128", wshape, dev),
                     eng.alloc("fp8_e4m3", "1x128", ashape, dev)))
    w_bytes = 7168 * 2048 * 2 + out_bytes(sets[0][2]["sizes"])
    a_bytes = 8192 * 7168 * 2 + out_bytes(sets[0][3]["sizes"])
    step_bytes = w_bytes + a_bytes
    jobs = [eng.jobs([(a, "fp8_e4m3", "1x128", ashape, ab), (w, "fp8_e4m3", "128x128", wshape, wb)])
            for w, a, wb, ab in sets]

    def step(i):
        eng.batch(jobs[i % nsets])

    pairs = [(eng.quantize_call(a, "fp8_e4m3", "1x128", ashape, ab),
              eng.quantize_call(w, "fp8_e4m3", "128x128", wshape, wb)) for w, a, wb, ab in sets]

    def two_launches(i):
        qa, qw = pairs[i % nsets]
        qa()
        qw()

    t = time_reps(torch, step, steps, warmup)
    ms_two = time_loop(torch, two_launches, steps, warmup)
    r = rec(step_bytes, t, op="FP8 E4M3 W8A8 step: weight [7168x2048] 128x128 + "
            "activations [8192x7168] 1x128, one fused launch", rotated_sets=nsets)
    r["two_launch_ms"] = round(ms_two, 5)
    r["two_launch_gbs"] = round(step_bytes / (ms_two * 1e-3) / 1e9, 1)
    record("w8a8_fp8_7168x2048_128x128_8192x7168_1x128", r)
    del sets, jobs
    torch.cuda.empty_cache()
    return r


# ----------------------------------------------------------------------------
# other workloads
# ----------------------------------------------------------------------------

def bench_extras(torch, eng, synth, reps, only=None):
    """Every other workload; `only` keeps the ones whose name contains it."""
    dev = torch.device("cuda:0")
    out = {}

    def want(*names):
        return only is None or any(only in n for n in names)

    def graph_time(r, nb, nsets, make_calls):
        """The same calls (one per buffer set) captured once in a HIP graph and
        replayed: GPU time per call without the host's launch cost, added to
        record `r`.  The library issues kernel launches only, so a replay
        rewrites exactly what the eager calls wrote."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        calls = make_calls(side.cuda_stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for c in calls:
                c()
        t = time_loop(torch, lambda i: g.replay(), max(4, reps // 2), 2) / nsets
        r["graph_ms_per_call"] = round(t, 5)
        r["graph_gbs"] = round(nb / (t * 1e-3) / 1e9, 1)
        del g

    def one(name, x, fmt, gran, shape, dq_dtype=None):
        """Quantize (and dequantize) `x`, rotating over enough buffer sets that
        the Infinity Cache cannot serve repeated reads: at least 4 sets and
        more than 1 GiB in all for tensors under 1 GiB."""
        if not want(name):
            return
        in_bytes = x.numel() * x.element_size()
        set_bytes = in_bytes + out_bytes(eng.pqb.query_sizes(fmt, gran, *shape))
        if dq_dtype is not None:
            set_bytes += x.numel() * torch.empty((), dtype=dq_dtype).element_size()
        nsets = 1 if in_bytes >= 1 << 30 else max(4, -(-(1 << 30) // set_bytes) + 1)
        xs = [x] + [x.clone() for _ in range(nsets - 1)]
        bufs = [eng.alloc(fmt, gran, shape, dev) for _ in range(nsets)]
        nb = in_bytes + out_bytes(bufs[0]["sizes"])
        two_pass = fmt == "nvfp4" or gran == "tensor"
        qcalls = [eng.quantize_call(xs[i], fmt, gran, shape, bufs[i]) for i in range(nsets)]
        t = time_reps(torch, lambda i: qcalls[i % nsets](), reps, 3)
        out[name] = rec(nb, t, in_bytes if two_pass else 0, op=f"quantize {fmt}/{gran}",
                        shape=list(shape), dtype=str(x.dtype).replace("torch.", ""),
                        rotated_sets=nsets)
        if in_bytes < (64 << 20):
            graph_time(out[name], nb, nsets,
                       lambda st: [eng.quantize_call(xs[i], fmt, gran, shape, bufs[i], st)
                                   for i in range(nsets)])
        if dq_dtype is not None:
            o = [torch.empty(shape, dtype=dq_dtype, device=dev) for _ in range(nsets)]
            nbd = out_bytes(bufs[0]["sizes"]) + o[0].numel() * o[0].element_size()
            dcalls = [eng.dequantize_call(bufs[i], fmt, gran, shape, o[i]) for i in range(nsets)]
            t = time_reps(torch, lambda i: dcalls[i % nsets](), reps, 3)
            out[name + "_dequant"] = rec(nbd, t, op=f"dequantize {fmt} -> "
                                         f"{str(dq_dtype).replace('torch.', '')}",
                                         shape=list(shape), rotated_sets=nsets)
            if in_bytes < (64 << 20):
                graph_time(out[name + "_dequant"], nbd, nsets,
                           lambda st: [eng.dequantize_call(bufs[i], fmt, gran, shape, o[i], st)
                                       for i in range(nsets)])
        log(f"{name}: {out[name]['gbs']} GB/s over {nsets} buffer sets"
            + (f", {out[name]['graph_gbs']} GB/s replayed from a graph" if "graph_gbs" in out[name] else ""))
        del xs, bufs
        torch.cuda.empty_cache()

    # float32 MLP weight, MXFP4 and NVFP4
    if want("mlp3072x1024"):
        w = synth.mlp_weight_fp32(device=dev)
        one("mlp3072x1024_f32_mxfp4", w, "mxfp4", "blk32", (1, 3072, 1024), torch.float32)
        one("mlp3072x1024_f32_nvfp4", w, "nvfp4", "blk16", (1, 3072, 1024), torch.float32)
        del w
    # heavy-tailed [28672, 8192] bf16 weight
    if want("w28672x8192"):
        w = synth.heavy_tail_weight(device=dev)
        one("w28672x8192_bf16_mxfp4", w, "mxfp4", "blk32", (1, 28672, 8192), torch.bfloat16)
        one("w28672x8192_bf16_nvfp4", w, "nvfp4", "blk16", (1, 28672, 8192), torch.bfloat16)
        del w
    # FP8 weight alone (128x128 tiles)
    if want("w7168x2048"):
        w = synth.fp8_weight(device=dev)
        one("w7168x2048_bf16_fp8_128x128", w, "fp8_e4m3", "128x128", (1, 7168, 2048))
        del w
    # 1 GiB bf16 tensor, every format
    sweep = (("fp8_e4m3", "1x128", torch.bfloat16), ("fp8_e4m3", "128x128", torch.bfloat16),
             ("fp8_e4m3", "row", torch.bfloat16), ("fp8_e4m3", "tensor", torch.bfloat16),
             ("mxfp4", "blk32", torch.bfloat16), ("nvfp4", "blk16", torch.bfloat16),
             ("int4_asym", "grp128", torch.bfloat16), ("fp8_e5m2", "1x128", torch.bfloat16),
             ("int8_sym", "row", torch.bfloat16), ("mxfp8", "blk32", torch.bfloat16))
    names = [f"sweep1GiB_bf16_{f}_{g}" for f, g, _ in sweep]
    if want(*names):
        g = synth.gaussian(device=dev)
        for name, (fmt, gran, dq) in zip(names, sweep):
            one(name, g, fmt, gran, (1, 65536, 8192), dq)
        del g
    torch.cuda.empty_cache()
    if want("kv28x32768x8x128_bf16_fp8", "kv28x32768x8x128_bf16_kivi"):
        out.update(bench_kv(torch, eng, synth, reps))
    if want("gemm_fp8_bs_8192x7168x2048_bf16", "gemm_fp8_bs_8192x2048x7168_bf16"):
        out.update(bench_gemm(torch, eng, synth, reps))
    if want("llama8b_224w_int4_g128_w4a16_decode_m1_one_batch",
            "llama8b_224w_int4_g128_w4a16_mfma_m16_one_batch"):
        out.update(bench_w4a16(torch, eng, synth, reps))
    return out


def bench_kv(torch, eng, synth, reps):
    """FP8 KV write of K and V [28, 32768, 8, 128] bf16, one scale per slice."""
    dev = torch.device("cuda:0")
    out = {}
    k, v = synth.kv_cache(device=dev)
    kc = torch.empty(k.shape, dtype=torch.uint8, device=dev)
    vc = torch.empty_like(kc)
    ks = torch.empty((28,), dtype=torch.float32, device=dev)
    vs = torch.empty_like(ks)
    ws = torch.empty((eng.L.pqb_kv_workspace_bytes(28, 32768 * 1024),), dtype=torch.uint8,
                     device=dev)
    nb = 2 * k.numel() * 2 + 2 * k.numel() + 2 * 28 * 4
    t = time_reps(torch, lambda i: eng.kv(k, v, kc, vc, ks, vs, ws), max(5, reps // 2), 2)
    out["kv28x32768x8x128_bf16_fp8"] = rec(nb, t, 2 * k.numel() * 2,
                                           op="FP8 KV write (per-layer scales)",
                                           shape=[28, 32768, 8, 128])
    log(f"kv: {out['kv28x32768x8x128_bf16_fp8']['gbs']} GB/s")
    # the same cache with a scale per (layer, head), and with static per-layer scales
    L_, T_, H_, D_ = 28, 32768, 8, 128
    ksh = torch.empty((L_, H_), dtype=torch.float32, device=dev)
    vsh = torch.empty_like(ksh)
    wsx = torch.empty((eng.L.pqb_kv_workspace_bytes_ex(L_, T_, H_, D_),), dtype=torch.uint8,
                      device=dev)
    P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731

    def kv_ex(km, vm, ks_, vs_):
        rc = eng.L.pqb_kv_write_fp8_ex(P(k), P(v), 1, L_, T_, H_, D_, km, vm, P(kc), P(vc),
                                       P(ks_), P(vs_), P(wsx), wsx.numel(), eng.stream)
        if rc != 0:
            raise RuntimeError(f"pqb_kv_write_fp8_ex: status {rc}")

    t = time_reps(torch, lambda i: kv_ex(1, 1, ksh, vsh), max(5, reps // 2), 2)
    out["kv28x32768x8x128_bf16_fp8_per_head"] = rec(nb - 2 * 28 * 4 + 2 * 28 * 8 * 4, t,
                                                    2 * k.numel() * 2,
                                                    op="FP8 KV write, scale per (layer, head)",
                                                    shape=[28, 32768, 8, 128])
    t = time_reps(torch, lambda i: kv_ex(2, 2, ks, vs), max(5, reps // 2), 2)
    out["kv28x32768x8x128_bf16_fp8_static"] = rec(nb, t, op="FP8 KV write, static per-layer "
                                                  "scales (one pass)", shape=[28, 32768, 8, 128])
    log(f"kv per head: {out['kv28x32768x8x128_bf16_fp8_per_head']['gbs']} GB/s, static: "
        f"{out['kv28x32768x8x128_bf16_fp8_static']['gbs']} GB/s")
    del kc, vc
    # KIVI-style 2/4-bit cache of the same K and V: K per channel over 32 tokens,
    # V per token over 32 channels; float32 scale and minimum per group.
    n = k.numel()
    for bits in (2, 4):
        cb = n * bits // 8
        kcb = torch.empty((cb,), dtype=torch.uint8, device=dev)
        vcb = torch.empty_like(kcb)
        kpar = torch.empty((2, L_, T_ // 32, H_, D_), dtype=torch.float32, device=dev)
        vpar = torch.empty((2, L_, T_, H_, D_ // 32), dtype=torch.float32, device=dev)

        def kivi_w(i, bits=bits, kcb=kcb, vcb=vcb, kpar=kpar, vpar=vpar):
            rc = eng.L.pqb_kv_write_kivi(P(k), P(v), 1, L_, T_, H_, D_, bits, P(kcb), P(vcb),
                                         P(kpar[0]), P(kpar[1]), P(vpar[0]), P(vpar[1]),
                                         eng.stream)
            if rc != 0:
                raise RuntimeError(f"pqb_kv_write_kivi: status {rc}")

        t = time_reps(torch, kivi_w, max(5, reps // 2), 2)
        key = f"kv28x32768x8x128_bf16_kivi{bits}"
        out[key] = rec(2 * n * 2 + 2 * cb + 2 * (n // 32) * 8, t,
                       op=f"KIVI {bits}-bit KV write (K per channel, V per token, groups of 32)",
                       shape=[28, 32768, 8, 128], launches=2)
        ko = torch.empty_like(k)
        vo = torch.empty_like(v)

        def kivi_r(i, bits=bits, kcb=kcb, vcb=vcb, kpar=kpar, vpar=vpar):
            rc = eng.L.pqb_kv_read_kivi(P(kcb), P(vcb), P(kpar[0]), P(kpar[1]), P(vpar[0]),
                                        P(vpar[1]), L_, T_, H_, D_, bits, 1, P(ko), P(vo),
                                        eng.stream)
            if rc != 0:
                raise RuntimeError(f"pqb_kv_read_kivi: status {rc}")

        t = time_reps(torch, kivi_r, max(5, reps // 2), 2)
        out[key + "_read"] = rec(2 * n * 2 + 2 * cb + 2 * (n // 32) * 8, t,
                                 op=f"KIVI {bits}-bit KV read to bf16", shape=[28, 32768, 8, 128],
                                 launches=2)
        log(f"kivi{bits}: write {out[key]['gbs']} GB/s, read {out[key + '_read']['gbs']} GB/s")
        del kcb, vcb, kpar, vpar, ko, vo
    del k, v
    torch.cuda.empty_cache()
    return out


def bench_gemm(torch, eng, synth, reps):
    """Block-scaled FP8 GEMM on codes the engine wrote: activations [M, K] with
    1x128 scales times a weight [N, K] with 128x128 scales, bf16 output."""
    dev = torch.device("cuda:0")
    out = {}
    for (M, N, K) in ((8192, 7168, 2048), (8192, 2048, 7168)):
        x = synth.fp8_activation(rows=M, cols=K, device=dev)
        w = synth.fp8_weight(rows=N, cols=K, device=dev)
        qa = eng.pqb.quantize(x, "fp8_e4m3", "1x128")
        qw = eng.pqb.quantize(w, "fp8_e4m3", "128x128")
        a, sa = qa.codes.reshape(M, K), qa.scales.reshape(M, K // 128)
        b, sb = qw.codes.reshape(N, K), qw.scales.reshape(N // 128, K // 128)
        c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731

        def run(i):
            rc = eng.L.pqb_gemm_fp8_blockscaled(P(a), P(sa), P(b), P(sb), M, N, K, 1, P(c),
                                                eng.stream)
            if rc != 0:
                raise RuntimeError(f"pqb_gemm_fp8_blockscaled: status {rc}")

        mean, med, mn = time_reps(torch, run, max(10, reps), 3)
        flops = 2 * M * N * K
        tf = flops / (mean * 1e-3) / 1e12
        key = f"gemm_fp8_bs_{M}x{N}x{K}_bf16"
        out[key] = {"flops": flops, "ms": round(mean, 5), "ms_median": round(med, 5),
                    "ms_min": round(mn, 5), "tflops": round(tf, 1),
                    "tflops_at_min": round(flops / (mn * 1e-3) / 1e12, 1),
                    "frac_fp8_mfma_peak": round(tf / FP8_MFMA_PEAK_TFLOPS, 4),
                    "op": "C = A (1x128 scales) x W^T (128x128 scales), scales promoted per "
                          "128-deep K block, bf16 out",
                    "bytes_in_out": M * K + N * K + 4 * (M + N // 128) * (K // 128) + 2 * M * N}
        log(f"{key}: {out[key]['tflops']} TFLOP/s ({out[key]['frac_fp8_mfma_peak'] * 100:.1f}% "
            f"of {FP8_MFMA_PEAK_TFLOPS:.0f})")
        # the next layer's FP8 1x128 activation quantization fused into the
        # epilogue, against the same GEMM with bf16 output followed by the
        # 1x128 quantizer on that output
        cc = torch.empty((M, N), dtype=torch.uint8, device=dev)
        cs = torch.empty((M, N // 128), dtype=torch.float32, device=dev)
        qbuf = eng.alloc("fp8_e4m3", "1x128", (1, M, N), dev)

        def fused(i):
            rc = eng.L.pqb_gemm_fp8_blockscaled_quant(P(a), P(sa), P(b), P(sb), M, N, K, P(cc),
                                                      P(cs), eng.stream)
            if rc != 0:
                raise RuntimeError(f"pqb_gemm_fp8_blockscaled_quant: status {rc}")

        def unfused(i):
            run(i)
            eng.quantize(c, "fp8_e4m3", "1x128", (1, M, N), qbuf)

        fm = time_reps(torch, fused, max(10, reps), 3)
        um = time_reps(torch, unfused, max(10, reps), 3)
        out[key + "_fused_fp8_1x128"] = {
            "ms": round(fm[0], 5), "ms_median": round(fm[1], 5),
            "tflops": round(flops / (fm[0] * 1e-3) / 1e12, 1),
            "unfused_ms": round(um[0], 5), "unfused_ms_median": round(um[1], 5),
            "op": "the same GEMM with its float32 result quantized to FP8 E4M3 1x128 in the "
                  "epilogue; unfused = bf16 GEMM output, then the 1x128 quantizer on it"}
        log(f"{key} fused fp8 1x128: {fm[0] * 1e3:.1f} us vs unfused {um[0] * 1e3:.1f} us")
        # the same shapes with both operands in MXFP4, on the block-scaled matrix cores
        ma, mw = eng.pqb.quantize(x, "mxfp4"), eng.pqb.quantize(w, "mxfp4")

        def run_mx(i):
            rc = eng.L.pqb_gemm_mxfp4(P(ma.codes), P(ma.scales), P(mw.codes), P(mw.scales), M, N, K,
                                      1, P(c), eng.stream)
            if rc != 0:
                raise RuntimeError(f"pqb_gemm_mxfp4: status {rc}")

        mean, med, mn = time_reps(torch, run_mx, max(10, reps), 3)
        tf = flops / (mean * 1e-3) / 1e12
        mkey = f"gemm_mxfp4_{M}x{N}x{K}_bf16"
        out[mkey] = {"flops": flops, "ms": round(mean, 5), "ms_median": round(med, 5),
                     "ms_min": round(mn, 5), "tflops": round(tf, 1),
                     "frac_fp4_mfma_peak": round(tf / FP4_MFMA_PEAK_TFLOPS, 4),
                     "op": "C = dequant(A) x dequant(W)^T, both MXFP4 (E2M1 + E8M0 per 32), "
                           "scales applied by the matrix core, bf16 out"}
        log(f"{mkey}: {tf:.1f} TFLOP/s ({tf / FP4_MFMA_PEAK_TFLOPS * 100:.1f}% of "
            f"{FP4_MFMA_PEAK_TFLOPS:.0f})")
        # both operands in NVFP4: E2M1 times E4M3 block scales widened to f16
        # per wave, f16 matrix cores, tensor scales applied once
        na, nw = eng.pqb.quantize(x, "nvfp4"), eng.pqb.quantize(w, "nvfp4")

        def run_nv(i):
            rc = eng.L.pqb_gemm_nvfp4(P(na.codes), P(na.scales), P(na.aux), P(nw.codes),
                                      P(nw.scales), P(nw.aux), M, N, K, 1, P(c), eng.stream)
            if rc != 0:
                raise RuntimeError(f"pqb_gemm_nvfp4: status {rc}")

        mean, med, mn = time_reps(torch, run_nv, max(10, reps), 3)
        tf = flops / (mean * 1e-3) / 1e12
        nkey = f"gemm_nvfp4_{M}x{N}x{K}_bf16"
        out[nkey] = {"flops": flops, "ms": round(mean, 5), "ms_median": round(med, 5),
                     "ms_min": round(mn, 5), "tflops": round(tf, 1),
                     "frac_f16_mfma_peak": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                     "op": "C = g sum_k (V dec(sA)) (V dec(sB)), both NVFP4 (E2M1 + E4M3 per 16, "
                           "float32 per tensor), widened exactly to f16, bf16 out"}
        log(f"{nkey}: {tf:.1f} TFLOP/s ({tf / BF16_MFMA_PEAK_TFLOPS * 100:.1f}% of the f16 peak "
            f"{BF16_MFMA_PEAK_TFLOPS:.0f})")
        del x, w, qa, qw, a, b, c, cc, cs, qbuf, ma, mw, na, nw
    torch.cuda.empty_cache()
    return out


def bench_w4a16(torch, eng, synth, reps):
    """W4A16 over the 224 Llama-3.1-8B-shaped weights in INT4 g128, every weight
    read once per step (once per 32 rows on the matrix cores): the decode
    kernel at M = 1 and 4, and the matrix-core kernel at M = 1, 4, 16 and 64."""
    dev = torch.device("cuda:0")
    from precision_quantization_block_amd.synth import LLAMA_LAYERS, LLAMA_PROJ
    ws, wbytes = [], 0
    for layer in range(LLAMA_LAYERS):
        for p, (_, r, c) in enumerate(LLAMA_PROJ):
            w = synth.llama_weight(layer, p, device=dev)
            b = eng.alloc("int4_asym", "grp128", (1, r, c), dev)
            eng.quantize(w, "int4_asym", "grp128", (1, r, c), b)
            ws.append((r, c, b))
            wbytes += out_bytes(b["sizes"])
            del w
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    J = eng.pqb.pqb._W4Job
    out = {}
    per_layer = len(LLAMA_PROJ)
    for M in (1, 4, 16, 64):
        g = torch.Generator(device=dev).manual_seed(77)
        xs = {K: torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
              for K in sorted({c for _, c, _ in ws})}
        ys = [torch.empty((M, r), dtype=torch.bfloat16, device=dev) for r, _, _ in ws]
        jobs = [J(xs[c].data_ptr(), b["codes"].data_ptr(), b["scales"].data_ptr(),
                  b["aux"].data_ptr(), y.data_ptr(), r, c) for (r, c, b), y in zip(ws, ys)]

        def batch(js, fn):
            arr = (J * len(js))(*js)
            return lambda: fn(arr, len(js), M, 1, eng.stream)

        nb = wbytes + sum(2 * M * c + 2 * M * r for r, c, _ in ws)
        flops = 2 * M * sum(r * c for r, c, _ in ws)
        kinds = [("mfma", eng.L.pqb_gemm_w4a16_batch)]
        if M <= 8:
            kinds.insert(0, ("decode", eng.L.pqb_gemv_w4a16_batch))
        for kind, fn in kinds:
            # one step three ways: every weight its own launch; per layer the
            # projections that share an input together (q k v | o | gate up |
            # down); all 224 weights in one batch call (7 launches of up to 32)
            single = [batch([j], fn) for j in jobs]
            grouped = []
            for L0 in range(0, len(jobs), per_layer):
                lj = jobs[L0:L0 + per_layer]
                grouped += [batch(lj[0:3], fn), batch(lj[3:4], fn), batch(lj[4:6], fn),
                            batch(lj[6:7], fn)]
            whole = [batch(jobs, fn)]
            ways = (("per_weight", single), ("per_layer_groups", grouped), ("one_batch", whole))
            if kind == "mfma" and M > 8:
                ways = ways[1:]
            for name, calls in ways:
                def step(i, calls=calls):
                    for f in calls:
                        rc = f()
                        if rc != 0:
                            raise RuntimeError(f"W4A16 batch call: status {rc}")

                t = time_reps(torch, step, max(5, reps // 4), 2)
                key = f"llama8b_224w_int4_g128_w4a16_{kind}_m{M}_{name}"
                out[key] = rec(nb, t, op=f"W4A16 product ({'matrix cores' if kind == 'mfma' else 'decode kernel'}), "
                                         f"M = {M}, all 224 weights, {name}", calls=len(calls))
                out[key]["ms_per_step"] = round(t[0], 4)
                out[key]["tflops"] = round(flops / (t[0] * 1e-3) / 1e12, 1)
                log(f"w4a16 {kind} M={M} {name}: {t[0]:.3f} ms per step, {out[key]['gbs']} GB/s")
    del ws
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the headline workload
# ----------------------------------------------------------------------------

def cpu_baseline_int4(torch, h, st_layers=1, mt_layers=8, threads=None, chunk_rows=512):
    """The INT4 oracle on the host cores, on host copies of the headline's own
    inputs: single-threaded over the first `st_layers` layers' weights, then
    one thread per core over row chunks of the first `mt_layers` layers
    (ctypes releases the GIL inside the C oracle).  Returns the record and the
    oracle's outputs (codes, scales, zero-points per weight) of the threaded leg."""
    import numpy as np
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    from precision_quantization_block_amd.synth import LLAMA_PROJ
    threads = threads or min(16, os.cpu_count() or 1)
    oracle.lib()
    P = len(LLAMA_PROJ)
    xs = [x.cpu() for x in h["xs"][: P * mt_layers]]

    def nbytes(x):
        n = x.numel()
        return 2 * n + n // 2 + 2 * (n // 128) + n // 256

    t0 = time.perf_counter()
    for x in xs[: P * st_layers]:
        oracle.int4_quantize(x)
    dt1 = time.perf_counter() - t0
    nb1 = sum(nbytes(x) for x in xs[: P * st_layers])
    # row chunks; every chunk holds an even number of groups (32 or 112 per row),
    # so its zero-point nibbles start on a byte and the pieces concatenate
    jobs = [(i, x[r:r + chunk_rows]) for i, x in enumerate(xs)
            for r in range(0, x.shape[0], chunk_rows)]
    with ThreadPoolExecutor(threads) as ex:
        t0 = time.perf_counter()
        res = list(ex.map(lambda j: oracle.int4_quantize(j[1].contiguous()), jobs))
        dtn = time.perf_counter() - t0
    outs = [([], [], []) for _ in xs]
    for (i, _), (c, s, z) in zip(jobs, res):
        outs[i][0].append(c.reshape(-1))
        outs[i][1].append(s.reshape(-1))
        outs[i][2].append(z.reshape(-1))
    outs = [tuple(np.concatenate(p) for p in o) for o in outs]
    nbn = sum(nbytes(x) for x in xs)
    r = {"value": round(nbn / dtn / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
         "sample": f"INT4 g128 of the first {mt_layers} of 32 layers (56 of 224 weights, "
                   f"{nbn / 1e9:.2f} GB in+out), {threads} threads over {chunk_rows}-row "
                   f"chunks: {dtn:.2f} s",
         "single_thread": {"value": round(nb1 / dt1 / 1e9, 4), "cores": 1,
                           "sample": f"layer 0's 7 weights: {dt1:.2f} s for {nb1 / 1e6:.0f} MB"},
         "host_cpu": _cpu_model(), "host_cores_available": os.cpu_count()}
    return r, outs


def parity_int4(torch, h, outs):
    """Byte-compare the GPU's INT4 codes, bf16 scales and zero-point nibbles with
    the oracle's for the weights the threaded CPU leg quantized."""
    import numpy as np
    mism, total = 0, 0
    for b, (c, s, z) in zip(h["bufs"], outs):
        for name, ref in (("codes", c), ("scales", s), ("aux", z)):
            ref = ref.view(np.uint8).reshape(-1)
            got = b[name][: b["sizes"][name]].cpu().numpy()
            mism += int(np.count_nonzero(got != ref)) if got.shape == ref.shape \
                else max(got.size, ref.size)
            total += ref.size
    return {"checked": f"every code, scale and zero-point byte of the first {len(outs)} weights "
                       f"of the last batch call against the oracle on the same inputs",
            "bytes_compared": total, "mismatches": mism}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def hbm_reference(torch, reps=10):
    """Bandwidth of plain torch kernels over bf16 buffers, by read:write ratio
    (copy_ and neg 1:1, add 2:1, addcmul 3:1; 1 GiB written by copy_ and neg,
    512 MiB by the others): the measured copy ceiling beside the 8 TB/s
    published peak."""
    n = 1 << 29  # bf16 elements = 1 GiB
    a = torch.ones((n,), dtype=torch.bfloat16, device="cuda:0")
    b = torch.ones((n,), dtype=torch.bfloat16, device="cuda:0")
    c = torch.empty((n,), dtype=torch.bfloat16, device="cuda:0")
    h = n // 2
    res = {}
    t = time_loop(torch, lambda i: c.copy_(a), reps, 2)
    res["copy_1r1w_gbs"] = round(2 * n * 2 / (t * 1e-3) / 1e9, 1)
    t = time_loop(torch, lambda i: torch.neg(a, out=c), reps, 2)
    res["neg_1r1w_gbs"] = round(2 * n * 2 / (t * 1e-3) / 1e9, 1)
    t = time_loop(torch, lambda i: torch.add(a[:h], b[:h], out=c[:h]), reps, 2)
    res["add_2r1w_gbs"] = round(3 * h * 2 / (t * 1e-3) / 1e9, 1)
    t = time_loop(torch, lambda i: torch.addcmul(a[:h], b[:h], a[h:], out=c[:h]), reps, 2)
    res["addcmul_3r1w_gbs"] = round(4 * h * 2 / (t * 1e-3) / 1e9, 1)
    del a, b, c
    torch.cuda.empty_cache()
    log(f"hbm reference: {res}")
    return res


def stream_ceiling(torch, eng, reps=12):
    """pqb_stream_reference over a 1 GiB source: the quantizers' own 16-byte
    non-temporal loads and stores with nothing computed, at 1, 2 and 4 bytes
    read per byte written (the INT4 headline reads 3.85 per byte written), in
    chunks of 8 tiles per wave (the quantizers' shape) and of 4; the faster of
    the two shapes is the ceiling at each mix.  The calls rotate over 1 GiB of
    output (R slices of 1/R GiB), so that no output stays in the 256 MB
    Infinity Cache between calls."""
    n = 1 << 30
    src = torch.ones((n,), dtype=torch.uint8, device="cuda:0")
    out = torch.empty((n,), dtype=torch.uint8, device="cuda:0")
    ps = ctypes.c_void_p(src.data_ptr())
    res = {}
    for r in (1, 2, 4):
        pds = [ctypes.c_void_p(out.data_ptr() + j * (n // r)) for j in range(r)]
        for tiles in (8, 4):
            def run(i, r=r, tiles=tiles, pds=pds):
                rc = eng.L.pqb_stream_reference(ps, n, r, tiles, pds[i % r], eng.stream)
                if rc != 0:
                    raise RuntimeError(f"pqb_stream_reference: status {rc}")

            t = time_loop(torch, run, reps, 4)
            res[f"r{r}_t{tiles}_gbs"] = round((n + n // r) / (t * 1e-3) / 1e9, 1)
        res[f"r{r}_gbs"] = max(res[f"r{r}_t8_gbs"], res[f"r{r}_t4_gbs"])
    del src, out
    torch.cuda.empty_cache()
    log(f"stream reference: {res}")
    return res


def copy_probe(torch, reps=3):
    """A plain elementwise kernel of known traffic (1 GiB read + 1 GiB written),
    for scaling rocprof's FETCH_SIZE / WRITE_SIZE."""
    x = torch.ones((1 << 28,), dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(reps):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    log(f"copy probe: {reps} x torch.neg on {x.numel() * 4} bytes")


# ----------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--sets", type=int, default=6,
                    help="rotated buffer sets of the W8A8 step (> 1 GiB in all)")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="time the headline only (no CPU baseline, no other workloads)")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--records", default=None, help="write every record to this JSON file")
    ap.add_argument("--only", default=None,
                    help="run only the format workloads whose name contains this string, or "
                         "'w8a8' (the FP8 W8A8 step), or 'llama8b_224w_int4' (the headline set "
                         "with its per-tensor and dequantization records), or 'stream_reference' "
                         "(the copy ceiling); no headline line, prints the records as JSON")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the quantizers shard by rows or blocks without communication; a per-tensor scale would need one MAX all-reduce of the pass-1 maxima).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import precision_quantization_block_amd as pqb
    from precision_quantization_block_amd import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    eng = Engine(torch, pqb)

    if args.copy_probe:
        copy_probe(torch)
    if args.only == "w8a8":
        print(json.dumps(bench_w8a8(torch, eng, synth, args.steps, args.warmup, args.sets)),
              flush=True)
        return
    if args.only == "llama8b_224w_int4":
        h = bench_headline(torch, eng, synth, args.steps, args.warmup)
        int4_records_extra(torch, eng, h, args.reps)
        print(json.dumps(_RECORDS), flush=True)
        return
    if args.only == "stream_reference":
        print(json.dumps({"stream_reference": stream_ceiling(torch, eng),
                          "hbm_reference": hbm_reference(torch)}), flush=True)
        return
    if args.only is not None:
        print(json.dumps(bench_extras(torch, eng, synth, args.reps, args.only)), flush=True)
        return

    h = bench_headline(torch, eng, synth, args.steps, args.warmup)
    value = h["step_bytes"] / (h["ms_per_step"] * 1e-3) / 1e9
    # k_multi<INT4> is the only kernel of a step: its average launch duration
    # is the step time over the launches, and its bytes per launch the step's
    # bytes over the launches, so achieved = step bytes / step time
    avg_launch_ms = h["ms_per_step"] / h["launches"]
    achieved = (h["step_bytes"] / h["launches"]) / (avg_launch_ms * 1e-3) / 1e9
    traffic = None
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
        if c.get("kernel_hash") == kernel_hash():
            traffic = c.get("traffic_bytes_per_launch")
    except (OSError, ValueError):
        pass
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(h["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16->int4 g128 (fp32 arithmetic)",
        "data": "synthetic (seeded; precision_quantization_block_amd/synth.py)",
        "config": {"workload": "INT4 g128 asymmetric, 224 Llama-3.1-8B-shaped bf16 weights "
                               "(32 layers x q,k,v,o,gate,up,down), one pqb_quantize_batch call",
                   "weights": sum(x.numel() for x in h["xs"]), "step_bytes": h["step_bytes"],
                   "launches_per_step": h["launches"],
                   "frac_hbm_peak": round(value / HBM_PEAK_GBS, 4)},
        "roofline": {"bound": "hbm", "kernel": HEADLINE_KERNEL, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": h["step_bytes"] // h["launches"],
                     "avg_launch_ms": round(avg_launch_ms, 5)},
        "cpu_baseline": None, "parity": None,
    }
    if not args.headline_only:
        int4_records_extra(torch, eng, h)
        if not args.no_cpu:
            line["cpu_baseline"], outs = cpu_baseline_int4(torch, h)
            line["parity"] = parity_int4(torch, h, outs)
            del outs
        del h
        torch.cuda.empty_cache()
        w8 = bench_w8a8(torch, eng, synth, args.steps, args.warmup, args.sets)
        sec = {"w8a8_fp8_step_gbs": w8["gbs"], "w8a8_fp8_step_frac": w8["frac_hbm_peak"]}
        if "llama8b_224w_bf16_int4_g128_dequant_batch" in _RECORDS:
            sec["int4_224w_dequant_batch_gbs"] = \
                _RECORDS["llama8b_224w_bf16_int4_g128_dequant_batch"]["gbs"]
        if not args.no_extras:
            for k, v in bench_extras(torch, eng, synth, args.reps).items():
                record(k, v)
        ref = hbm_reference(torch)
        record("hbm_reference", ref)
        sc = stream_ceiling(torch, eng)
        record("stream_reference", sc)
        line["copy_ceiling"] = {"kernel": "pqb_stream_reference (16-byte nt loads/stores, no arithmetic; 1 GiB "
                                          "read, outputs rotated); rN = GB/s at N bytes read per byte written",
                                "r1_gbs": sc["r1_gbs"], "r2_gbs": sc["r2_gbs"], "r4_gbs": sc["r4_gbs"],
                                "headline_frac_of_r4": round(value / sc["r4_gbs"], 4),
                                "torch_best_gbs": max(ref.values())}
        line["secondary"] = sec
    if args.records:
        with open(args.records, "w") as f:
            json.dump({"headline": line, "records": _RECORDS}, f, indent=1)
    print(json.dumps(line, separators=(",", ":")), flush=True)
    if line["parity"] is not None and line["parity"]["mismatches"]:
        log(f"PARITY FAILURE: {line['parity']['mismatches']} bytes differ from the oracle")
        sys.exit(3)


if __name__ == "__main__":
    main()
