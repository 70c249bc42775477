"""Thin Python binding over libpqb.so (argument marshalling only).

Every step of quantization runs in the HIP kernels behind the C ABI of
include/pqb.h.  Torch supplies device memory and the current stream; there is
no CPU fallback: if libpqb.so is missing or a tensor is not on the GPU, the
call raises.

Page-named fake-quant helpers (fp8_per_tensor, fp8_per_row, fp8_blockwise,
mxfp4, nvfp4, fp8_kv_write) mirror the fake-quant module on the page "量化部署
实战" (section 伪量化实现): quantize, then dequantize, returning float32 of the
input's shape.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpqb.so")

F32, BF16 = 0, 1
FORMATS = {"fp8_e4m3": 0, "mxfp4": 1, "nvfp4": 2, "int4_asym": 3, "fp8_e5m2": 4, "mxfp8": 5,
           "int8_sym": 6}
GRANS = {"tensor": 0, "row": 1, "1x128": 2, "128x128": 3, "blk32": 4, "blk16": 5, "grp128": 6}
DEFAULT_GRAN = {"mxfp4": "blk32", "nvfp4": "blk16", "int4_asym": "grp128", "mxfp8": "blk32",
                "int8_sym": "row"}

_lib = None


class PqbError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


class _Job(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("aux", ctypes.c_void_p), ("batch", ctypes.c_int64), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("dtype", ctypes.c_int32), ("fmt", ctypes.c_int32),
                ("gran", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class _DqJob(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("aux", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("batch", ctypes.c_int64), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("fmt", ctypes.c_int32), ("gran", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class _W4Job(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("zeros", ctypes.c_void_p), ("y", ctypes.c_void_p), ("n", ctypes.c_int64),
                ("k", ctypes.c_int64)]


class _Sizes(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_size_t), ("scales", ctypes.c_size_t),
                ("aux", ctypes.c_size_t), ("workspace", ctypes.c_size_t)]


def lib():
    """Load libpqb.so (built by __graft_entry__.build() or _build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        L.pqb_source_hash.restype = ctypes.c_char_p
        check_source_hash(L)
        L.pqb_abi_version.restype = I
        L.pqb_status_string.argtypes, L.pqb_status_string.restype = [I], ctypes.c_char_p
        L.pqb_query_sizes.argtypes = [I, I, I64, I64, I64, ctypes.POINTER(_Sizes)]
        L.pqb_quantize.argtypes = [P, I, I64, I64, I64, I, I, P, P, P, P, SZ, P]
        L.pqb_quantize_noalloc.argtypes = [P, I, I64, I64, I64, I, I, P, P, P, P]
        L.pqb_dequantize.argtypes = [P, P, P, I, I, I64, I64, I64, I, P, P]
        L.pqb_dequantize_batch.argtypes = [ctypes.POINTER(_DqJob), I64, P]
        L.pqb_quantize_batch.argtypes = [ctypes.POINTER(_Job), I64, P]
        L.pqb_quantize_batch_launches.argtypes = [ctypes.POINTER(_Job), I64]
        L.pqb_quantize_batch_launches.restype = I64
        L.pqb_kv_workspace_bytes.argtypes, L.pqb_kv_workspace_bytes.restype = [I64, I64], SZ
        L.pqb_kv_write_fp8.argtypes = [P, P, I, I64, I64, P, P, P, P, P, SZ, P]
        L.pqb_kv_workspace_bytes_ex.argtypes = [I64, I64, I64, I64]
        L.pqb_kv_workspace_bytes_ex.restype = SZ
        L.pqb_kv_write_fp8_ex.argtypes = [P, P, I, I64, I64, I64, I64, I, I, P, P, P, P, P, SZ, P]
        L.pqb_kv_write_kivi.argtypes = [P, P, I, I64, I64, I64, I64, I, P, P, P, P, P, P, P]
        L.pqb_kv_read_kivi.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, I, I, P, P, P]
        L.pqb_gemm_fp8_blockscaled.argtypes = [P, P, P, P, I64, I64, I64, I, P, P]
        L.pqb_gemm_fp8_blockscaled_quant.argtypes = [P, P, P, P, I64, I64, I64, P, P, P]
        L.pqb_gemv_w4a16.argtypes = [P, I64, P, P, P, I64, I64, I, P, P]
        L.pqb_gemm_mxfp4.argtypes = [P, P, P, P, I64, I64, I64, I, P, P]
        L.pqb_gemm_nvfp4.argtypes = [P, P, P, P, P, P, I64, I64, I64, I, P, P]
        L.pqb_stream_reference.argtypes = [P, I64, I, I, P, P]
        L.pqb_gemv_w4a16_batch.argtypes = [ctypes.POINTER(_W4Job), I64, I64, I, P]
        L.pqb_gemm_w4a16.argtypes = [P, I64, P, P, P, I64, I64, I, P, P]
        L.pqb_gemm_w4a16_batch.argtypes = [ctypes.POINTER(_W4Job), I64, I64, I, P]
        L.pqb_encode_e4m3.argtypes = [P, I64, P, P]
        L.pqb_encode_e5m2.argtypes = [P, I64, P, P]
        L.pqb_encode_e2m1.argtypes = [P, I64, P, P]
        L.pqb_check_recip.argtypes = [ctypes.c_uint32, I64, P, P]
        L.pqb_check_div.argtypes = [P, I64, ctypes.c_uint32, I64, P, P]
        for f in ("pqb_query_sizes", "pqb_quantize", "pqb_quantize_noalloc", "pqb_quantize_batch",
                  "pqb_dequantize", "pqb_dequantize_batch",
                  "pqb_kv_write_fp8", "pqb_kv_write_fp8_ex", "pqb_kv_write_kivi",
                  "pqb_kv_read_kivi", "pqb_gemm_fp8_blockscaled",
                  "pqb_gemm_fp8_blockscaled_quant", "pqb_gemv_w4a16",
                  "pqb_gemv_w4a16_batch", "pqb_gemm_mxfp4", "pqb_gemm_nvfp4", "pqb_stream_reference", "pqb_gemm_w4a16",
                  "pqb_gemm_w4a16_batch",
                  "pqb_encode_e4m3", "pqb_encode_e5m2", "pqb_encode_e2m1",
                  "pqb_check_recip", "pqb_check_div"):
            getattr(L, f).restype = I
        _lib = L
    return _lib


def check_source_hash(L) -> None:
    """Refuse a libpqb.so built from other sources than the csrc/ beside it
    (a stale build would run old kernels without any sign of it)."""
    from . import _build
    if not os.path.isdir(_build.CSRC):
        return
    built, here = L.pqb_source_hash().decode(), _build.source_hash()
    if built != here:
        raise RuntimeError(f"{LIB_PATH} was built from other sources (hash {built}, sources now "
                           f"{here}); rebuild it with __graft_entry__.build()")


def status_string(status: int) -> str:
    return lib().pqb_status_string(status).decode()


def abi_version() -> int:
    return lib().pqb_abi_version()


def _check(status: int, what: str):
    if status != 0:
        raise PqbError(status, what)


def _fmt(fmt) -> int:
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def _gran(gran) -> int:
    return GRANS[gran] if isinstance(gran, str) else int(gran)


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev_tensor(x: torch.Tensor, name: str, dtypes=(torch.float32, torch.bfloat16)):
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if x.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype in {dtypes}, got {x.dtype}")
    return x.contiguous()


def query_sizes(fmt, gran, batch: int, rows: int, cols: int) -> dict:
    s = _Sizes()
    _check(lib().pqb_query_sizes(_fmt(fmt), _gran(gran), batch, rows, cols, ctypes.byref(s)),
           "query_sizes")
    return {"codes": s.codes, "scales": s.scales, "aux": s.aux, "workspace": s.workspace}


@dataclass
class Quantized:
    """Packed codes, encoded scales and the format's auxiliary buffer."""
    codes: torch.Tensor
    scales: torch.Tensor
    aux: torch.Tensor | None
    fmt: str
    gran: str
    shape: tuple   # (batch, rows, cols)


def _scale_dtype(fmt: str):
    return {"fp8_e4m3": torch.float32, "fp8_e5m2": torch.float32, "int8_sym": torch.float32,
            "mxfp4": torch.uint8, "mxfp8": torch.uint8, "nvfp4": torch.uint8,
            "int4_asym": torch.bfloat16}[fmt]


def _bytes(n: int, dtype, device):
    esize = torch.empty((), dtype=dtype).element_size()
    return torch.empty((n // esize,), dtype=dtype, device=device)


def quantize(x: torch.Tensor, fmt: str, gran: str | None = None, *, shape=None,
             workspace: torch.Tensor | None = None) -> Quantized:
    """Quantize x viewed as [batch, rows, cols] (default: leading dims are the
    batch, the last two are rows and cols)."""
    gran = gran or DEFAULT_GRAN[fmt]
    x = _dev_tensor(x, "x")
    b, r, c = shape if shape is not None else _bcr(x.shape)
    if b * r * c != x.numel():
        raise ValueError("shape does not match the tensor")
    dev = x.device
    sz, codes, scales, aux = _alloc_outputs(fmt, gran, b, r, c, dev)
    if sz["workspace"] and (workspace is None or workspace.numel() * workspace.element_size()
                            < sz["workspace"]):
        workspace = torch.empty((sz["workspace"] // 4,), dtype=torch.float32, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().pqb_quantize(_ptr(x), BF16 if x.dtype == torch.bfloat16 else F32, b, r, c,
                              _fmt(fmt), _gran(gran), _ptr(codes), _ptr(scales), _ptr(aux),
                              _ptr(workspace), ws_bytes, _stream(dev)), "quantize")
    return Quantized(codes, scales, aux, fmt, gran, (b, r, c))


def _alloc_outputs(fmt, gran, b, r, c, dev):
    sz = query_sizes(fmt, gran, b, r, c)
    codes = torch.empty((sz["codes"],), dtype=torch.uint8, device=dev)
    scales = _bytes(sz["scales"], _scale_dtype(fmt), dev)
    aux = None
    if sz["aux"]:
        aux = (torch.empty((b,), dtype=torch.float32, device=dev) if fmt == "nvfp4"
               else torch.empty((sz["aux"],), dtype=torch.uint8, device=dev))
    return sz, codes, scales, aux


def quantize_batch(items) -> list:
    """Quantize several tensors with fused launches (one-pass formats only).
    `items`: sequence of (x, fmt, gran) or (x, fmt, gran, shape) tuples.
    Returns one Quantized per item, identical to quantize() on each."""
    outs, jobs = [], []
    dev = None
    for it in items:
        x, fmt, gran = it[0], it[1], it[2] or DEFAULT_GRAN[it[1]]
        x = _dev_tensor(x, "x")
        dev = x.device if dev is None else dev
        b, r, c = it[3] if len(it) > 3 and it[3] is not None else _bcr(x.shape)
        if b * r * c != x.numel():
            raise ValueError("shape does not match the tensor")
        _, codes, scales, aux = _alloc_outputs(fmt, gran, b, r, c, x.device)
        outs.append((x, Quantized(codes, scales, aux, fmt, gran, (b, r, c))))
        jobs.append(_Job(x.data_ptr(), codes.data_ptr(), scales.data_ptr(),
                         aux.data_ptr() if aux is not None else None, b, r, c,
                         BF16 if x.dtype == torch.bfloat16 else F32, _fmt(fmt), _gran(gran), 0))
    if not jobs:
        return []
    arr = (_Job * len(jobs))(*jobs)
    _check(lib().pqb_quantize_batch(arr, len(jobs), _stream(dev)), "quantize_batch")
    return [q for _, q in outs]


def dequantize(q: Quantized, out_dtype=torch.float32) -> torch.Tensor:
    b, r, c = q.shape
    out = torch.empty((b, r, c), dtype=out_dtype, device=q.codes.device)
    _check(lib().pqb_dequantize(_ptr(q.codes), _ptr(q.scales), _ptr(q.aux), _fmt(q.fmt),
                                _gran(q.gran), b, r, c,
                                BF16 if out_dtype == torch.bfloat16 else F32, _ptr(out),
                                _stream(out.device)), "dequantize")
    return out


def dequantize_batch(items) -> list:
    """Dequantize several Quantized results with fused launches.  `items`:
    sequence of Quantized or (Quantized, out_dtype) pairs (float32 by default).
    Returns one tensor per item, identical to dequantize() on each."""
    outs, jobs, dev = [], [], None
    for it in items:
        q, out_dtype = (it, torch.float32) if isinstance(it, Quantized) else (it[0], it[1])
        b, r, c = q.shape
        out = torch.empty((b, r, c), dtype=out_dtype, device=q.codes.device)
        dev = out.device
        outs.append(out)
        jobs.append(_DqJob(_ptr(q.codes), _ptr(q.scales), _ptr(q.aux), _ptr(out), b, r, c,
                           _fmt(q.fmt), _gran(q.gran), BF16 if out_dtype == torch.bfloat16 else F32,
                           0))
    if not jobs:
        return []
    arr = (_DqJob * len(jobs))(*jobs)
    _check(lib().pqb_dequantize_batch(arr, len(jobs), _stream(dev)), "dequantize_batch")
    return outs


def kv_write_fp8(k: torch.Tensor, v: torch.Tensor, workspace: torch.Tensor | None = None):
    """K and V shaped [layers, ...]; one FP8 scale per layer for each.
    Returns (k_codes, v_codes, k_scales, v_scales) with codes shaped like the input."""
    k = _dev_tensor(k, "k")
    v = _dev_tensor(v, "v")
    if k.shape != v.shape or k.dtype != v.dtype:
        raise ValueError("K and V must share shape and dtype")
    layers = k.shape[0]
    per = k.numel() // layers if layers else 0
    dev = k.device
    kc = torch.empty(k.shape, dtype=torch.uint8, device=dev)
    vc = torch.empty(v.shape, dtype=torch.uint8, device=dev)
    ks = torch.empty((layers,), dtype=torch.float32, device=dev)
    vs = torch.empty((layers,), dtype=torch.float32, device=dev)
    need = lib().pqb_kv_workspace_bytes(layers, per)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty((max(need, 4) // 4,), dtype=torch.float32, device=dev)
    _check(lib().pqb_kv_write_fp8(_ptr(k), _ptr(v), BF16 if k.dtype == torch.bfloat16 else F32,
                                  layers, per, _ptr(kc), _ptr(vc), _ptr(ks), _ptr(vs),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _stream(dev)), "kv_write_fp8")
    return kc, vc, ks, vs


KV_MODES = {"layer": 0, "head": 1, "static": 2}


def kv_write_fp8_ex(k: torch.Tensor | None, v: torch.Tensor | None, k_mode="layer",
                    v_mode="layer", k_scales: torch.Tensor | None = None,
                    v_scales: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """FP8 KV write with a scale mode per tensor; K and V are [layers, tokens,
    heads, head_dim] (either may be None).  Modes: "layer" (scales [layers]),
    "head" (scales [layers, heads]) or "static" (the given float32 scales
    [layers] are used).  Returns (k_codes, v_codes, k_scales, v_scales); the
    entries of a tensor passed as None are None."""
    xs = [k, v]
    modes = [KV_MODES.get(k_mode, k_mode), KV_MODES.get(v_mode, v_mode)]
    given = [k_scales, v_scales]
    ref = next((t for t in xs if t is not None), None)
    if ref is None:
        raise ValueError("pass K, V or both")
    if ref.dim() != 4:
        raise ValueError("K and V must be [layers, tokens, heads, head_dim]")
    L, T, H, D = ref.shape
    dev = ref.device
    codes, scales = [None, None], [None, None]
    for i, x in enumerate(xs):
        if x is None:
            continue
        x = _dev_tensor(x, "kv"[i])
        if x.shape != ref.shape or x.dtype != ref.dtype:
            raise ValueError("K and V must share shape and dtype")
        xs[i] = x
        codes[i] = torch.empty(x.shape, dtype=torch.uint8, device=dev)
        if modes[i] == 2:
            if given[i] is None:
                raise ValueError("a static mode needs its scales")
            scales[i] = _dev_tensor(given[i], "scales", (torch.float32,)).reshape(L)
        else:
            scales[i] = torch.empty((L, H) if modes[i] == 1 else (L,), dtype=torch.float32,
                                    device=dev)
    need = lib().pqb_kv_workspace_bytes_ex(L, T, H, D)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty((max(need, 4) // 4,), dtype=torch.float32, device=dev)
    _check(lib().pqb_kv_write_fp8_ex(
        _ptr(xs[0]), _ptr(xs[1]), BF16 if ref.dtype == torch.bfloat16 else F32, L, T, H, D,
        modes[0], modes[1], _ptr(codes[0]), _ptr(codes[1]), _ptr(scales[0]), _ptr(scales[1]),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev)),
        "kv_write_fp8_ex")
    return codes[0], codes[1], scales[0], scales[1]


def kivi_layouts(L, T, H, D, bits):
    """Shapes of (codes, K scales / mins, V scales / mins) for a KIVI cache of
    [L, T, H, D]: codes pack 8 / bits elements per byte along the flat index."""
    return (L * T * H * D * bits // 8,), (L, T // 32, H, D), (L, T, H, D // 32)


def kv_write_kivi(k: torch.Tensor | None, v: torch.Tensor | None, bits: int = 2):
    """KIVI-style KV write: K quantized per channel over groups of 32 tokens, V
    per token over groups of 32 channels, both asymmetric at `bits` (2 or 4).
    K and V are [layers, tokens, heads, head_dim] (either may be None).  Returns
    ((k_codes, k_scales, k_mins), (v_codes, v_scales, v_mins)), None for a
    tensor passed as None."""
    xs = [k, v]
    ref = next((t for t in xs if t is not None), None)
    if ref is None:
        raise ValueError("pass K, V or both")
    if ref.dim() != 4:
        raise ValueError("K and V must be [layers, tokens, heads, head_dim]")
    L, T, H, D = ref.shape
    dev = ref.device
    shapes = kivi_layouts(L, T, H, D, bits)
    outs = [None, None]
    for i, x in enumerate(xs):
        if x is None:
            continue
        x = _dev_tensor(x, "kv"[i])
        if x.shape != ref.shape or x.dtype != ref.dtype:
            raise ValueError("K and V must share shape and dtype")
        xs[i] = x
        sshape = shapes[1 + i]
        outs[i] = (torch.empty(shapes[0], dtype=torch.uint8, device=dev),
                   torch.empty(sshape, dtype=torch.float32, device=dev),
                   torch.empty(sshape, dtype=torch.float32, device=dev))
    kc, ks, km = outs[0] if outs[0] else (None, None, None)
    vc, vs, vm = outs[1] if outs[1] else (None, None, None)
    _check(lib().pqb_kv_write_kivi(
        _ptr(xs[0]), _ptr(xs[1]), BF16 if ref.dtype == torch.bfloat16 else F32, L, T, H, D, bits,
        _ptr(kc), _ptr(vc), _ptr(ks), _ptr(km), _ptr(vs), _ptr(vm), _stream(dev)),
        "kv_write_kivi")
    return outs[0], outs[1]


def kv_read_kivi(k_parts, v_parts, shape, bits: int = 2, out_dtype=torch.bfloat16):
    """Dequantize a KIVI cache written by kv_write_kivi back to `shape` =
    (layers, tokens, heads, head_dim) in out_dtype.  k_parts / v_parts are the
    (codes, scales, mins) triples (either may be None).  Returns (k, v)."""
    L, T, H, D = shape
    parts = [k_parts, v_parts]
    ref = next((p for p in parts if p is not None), None)
    if ref is None:
        raise ValueError("pass K, V or both")
    dev = ref[0].device
    outs, args = [None, None], [[None] * 3, [None] * 3]
    for i, p in enumerate(parts):
        if p is None:
            continue
        c, s, m = p
        args[i] = [_dev_tensor(c, "codes", (torch.uint8,)),
                   _dev_tensor(s, "scales", (torch.float32,)),
                   _dev_tensor(m, "mins", (torch.float32,))]
        outs[i] = torch.empty(tuple(shape), dtype=out_dtype, device=dev)
    _check(lib().pqb_kv_read_kivi(
        _ptr(args[0][0]), _ptr(args[1][0]), _ptr(args[0][1]), _ptr(args[0][2]),
        _ptr(args[1][1]), _ptr(args[1][2]), L, T, H, D, bits,
        BF16 if out_dtype == torch.bfloat16 else F32, _ptr(outs[0]), _ptr(outs[1]), _stream(dev)),
        "kv_read_kivi")
    return outs[0], outs[1]


def gemm_fp8_blockscaled(a_codes: torch.Tensor, a_scales: torch.Tensor, b_codes: torch.Tensor,
                         b_scales: torch.Tensor, out_dtype=torch.bfloat16,
                         out: torch.Tensor | None = None) -> torch.Tensor:
    """C [M, N] = the block-scaled FP8 product of activation codes [M, K] with
    1x128 scales [M, K/128] and weight codes [N, K] with 128x128 scales
    [N/128, K/128] (the layouts quantize() writes for "1x128" and "128x128")."""
    a = _dev_tensor(a_codes, "a_codes", (torch.uint8,))
    b = _dev_tensor(b_codes, "b_codes", (torch.uint8,))
    sa = _dev_tensor(a_scales, "a_scales", (torch.float32,))
    sb = _dev_tensor(b_scales, "b_scales", (torch.float32,))
    M, K = a.shape[-2], a.shape[-1]
    N = b.shape[-2]
    if b.shape[-1] != K or a.numel() != M * K or b.numel() != N * K:
        raise ValueError("a must be [M, K] and b [N, K]")
    if sa.numel() != M * (K // 128) or sb.numel() != (N // 128) * (K // 128):
        raise ValueError("scales must be [M, K/128] and [N/128, K/128]")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    elif out.shape != (M, N) or out.dtype != out_dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [M, N] tensor of out_dtype")
    _check(lib().pqb_gemm_fp8_blockscaled(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), M, N, K,
                                          BF16 if out_dtype == torch.bfloat16 else F32,
                                          _ptr(out), _stream(a.device)), "gemm_fp8_blockscaled")
    return out


def gemm_fp8_blockscaled_quant(a_codes: torch.Tensor, a_scales: torch.Tensor,
                               b_codes: torch.Tensor, b_scales: torch.Tensor):
    """The block-scaled FP8 GEMM with its float32 result quantized to FP8 E4M3
    1x128 in the epilogue.  Returns (codes u8 [M, N], scales f32 [M, N/128])."""
    a = _dev_tensor(a_codes, "a_codes", (torch.uint8,))
    b = _dev_tensor(b_codes, "b_codes", (torch.uint8,))
    sa = _dev_tensor(a_scales, "a_scales", (torch.float32,))
    sb = _dev_tensor(b_scales, "b_scales", (torch.float32,))
    M, K = a.shape[-2], a.shape[-1]
    N = b.shape[-2]
    if b.shape[-1] != K or a.numel() != M * K or b.numel() != N * K:
        raise ValueError("a must be [M, K] and b [N, K]")
    if sa.numel() != M * (K // 128) or sb.numel() != (N // 128) * (K // 128):
        raise ValueError("scales must be [M, K/128] and [N/128, K/128]")
    codes = torch.empty((M, N), dtype=torch.uint8, device=a.device)
    scales = torch.empty((M, N // 128), dtype=torch.float32, device=a.device)
    _check(lib().pqb_gemm_fp8_blockscaled_quant(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), M, N, K,
                                                _ptr(codes), _ptr(scales), _stream(a.device)),
           "gemm_fp8_blockscaled_quant")
    return codes, scales


def gemm_mxfp4(a, b, out_dtype=torch.float32) -> torch.Tensor:
    """C = dequant(A) @ dequant(B)^T for two MXFP4 operands, each a Quantized
    from quantize(x, "mxfp4") or a (codes [rows, K/2], E8M0 scales [rows, K/32])
    pair, on the block-scaled matrix cores."""
    ac, as_ = (a.codes, a.scales) if isinstance(a, Quantized) else a
    bc, bs = (b.codes, b.scales) if isinstance(b, Quantized) else b
    K = a.shape[-1] if isinstance(a, Quantized) else 2 * ac.shape[-1]
    ac, bc = _dev_tensor(ac, "a codes", (torch.uint8,)), _dev_tensor(bc, "b codes", (torch.uint8,))
    as_, bs = _dev_tensor(as_, "a scales", (torch.uint8,)), _dev_tensor(bs, "b scales", (torch.uint8,))
    def rows(q, codes):   # leading rows of a Quantized, else of 2-D codes (or flat, K > 0)
        if isinstance(q, Quantized):
            return math.prod(q.shape[:-1])
        return codes.shape[0] if codes.dim() == 2 else (codes.numel() // (K // 2) if K else 0)

    M, N = rows(a, ac), rows(b, bc)
    if K % 128 or ac.numel() != M * (K // 2) or bc.numel() != N * (K // 2) \
            or as_.numel() != M * (K // 32) or bs.numel() != N * (K // 32):
        raise ValueError("codes must be [rows, K/2] and scales [rows, K/32]")
    c = torch.empty((M, N), dtype=out_dtype, device=ac.device)
    _check(lib().pqb_gemm_mxfp4(_ptr(ac), _ptr(as_), _ptr(bc), _ptr(bs), M, N, K,
                                BF16 if out_dtype == torch.bfloat16 else F32, _ptr(c),
                                _stream(ac.device)), "gemm_mxfp4")
    return c


def gemm_nvfp4(a, b, out_dtype=torch.float32) -> torch.Tensor:
    """C = float32(gsA gsB) * sum_k A'[m, k] B'[n, k] for two NVFP4 operands
    (A' = E2M1 value times the E4M3 block scale), each a Quantized from
    quantize(x, "nvfp4") of one [rows, K] tensor or a (codes [rows, K/2],
    E4M3 scales [rows, K/16], float32 tensor scale [1]) triple, on the f16
    matrix cores."""
    ac, as_, ag = (a.codes, a.scales, a.aux) if isinstance(a, Quantized) else a
    bc, bs, bg = (b.codes, b.scales, b.aux) if isinstance(b, Quantized) else b
    K = a.shape[-1] if isinstance(a, Quantized) else 2 * ac.shape[-1]
    ac, bc = _dev_tensor(ac, "a codes", (torch.uint8,)), _dev_tensor(bc, "b codes", (torch.uint8,))
    as_, bs = _dev_tensor(as_, "a scales", (torch.uint8,)), _dev_tensor(bs, "b scales", (torch.uint8,))
    ag, bg = _dev_tensor(ag, "a tensor scale", (torch.float32,)), _dev_tensor(bg, "b tensor scale", (torch.float32,))
    def rows(q, codes):
        if isinstance(q, Quantized):
            return math.prod(q.shape[:-1])
        return codes.shape[0] if codes.dim() == 2 else (codes.numel() // (K // 2) if K else 0)

    M, N = rows(a, ac), rows(b, bc)
    if K % 128 or ac.numel() != M * (K // 2) or bc.numel() != N * (K // 2) \
            or as_.numel() != M * (K // 16) or bs.numel() != N * (K // 16):
        raise ValueError("codes must be [rows, K/2] and scales [rows, K/16]")
    if ag.numel() != 1 or bg.numel() != 1:
        raise ValueError("each operand needs exactly one tensor scale (quantize one [rows, K] tensor)")
    c = torch.empty((M, N), dtype=out_dtype, device=ac.device)
    _check(lib().pqb_gemm_nvfp4(_ptr(ac), _ptr(as_), _ptr(ag), _ptr(bc), _ptr(bs), _ptr(bg), M, N, K,
                                BF16 if out_dtype == torch.bfloat16 else F32, _ptr(c),
                                _stream(ac.device)), "gemm_nvfp4")
    return c


def stream_reference(src: torch.Tensor, reads_per_write: int, dst: torch.Tensor | None = None,
                     tiles_per_wave: int = 8) -> torch.Tensor:
    """The quantizers' memory pattern with nothing computed (a bandwidth
    reference): reads all of src (a multiple of 8192 bytes) and writes
    src.nbytes / reads_per_write bytes, each 1 KiB output tile the XOR of
    reads_per_write consecutive 1 KiB source tiles of its chunk of
    tiles_per_wave tiles."""
    if not isinstance(src, torch.Tensor) or src.device.type != "cuda" or not src.is_contiguous():
        raise ValueError("src must be a contiguous GPU tensor")
    nb = src.numel() * src.element_size()
    if dst is None:
        dst = torch.empty((nb // reads_per_write,), dtype=torch.uint8, device=src.device)
    _check(lib().pqb_stream_reference(_ptr(src), nb, reads_per_write, tiles_per_wave, _ptr(dst),
                                      _stream(src.device)),
           "stream_reference")
    return dst


def _w4_rows(codes: torch.Tensor, K: int) -> int:
    """N of an INT4 weight [N, K] from its codes (2-D [N, K / 2], or flat when K > 0)."""
    N = codes.shape[0] if codes.dim() == 2 else (codes.numel() * 2 // K if K else 0)
    if K % 128 or codes.numel() != N * K // 2:
        raise ValueError("codes must hold N x K / 2 bytes with K a multiple of 128")
    return N


def _w4_one(fn, x, weight, out_dtype):
    x = _dev_tensor(x, "x", (torch.bfloat16,))
    if isinstance(weight, Quantized):
        codes, scales, zeros = weight.codes, weight.scales, weight.aux
    else:
        codes, scales, zeros = weight
    codes = _dev_tensor(codes, "codes", (torch.uint8,))
    scales = _dev_tensor(scales, "scales", (torch.bfloat16, torch.int16, torch.uint8))
    zeros = _dev_tensor(zeros, "zeros", (torch.uint8,))
    M, K = (1, x.shape[0]) if x.dim() == 1 else (x.shape[-2], x.shape[-1])
    N = _w4_rows(codes, K)
    y = torch.empty((M, N), dtype=out_dtype, device=x.device)
    _check(getattr(lib(), fn)(_ptr(x), M, _ptr(codes), _ptr(scales), _ptr(zeros), N, K,
                              BF16 if out_dtype == torch.bfloat16 else F32, _ptr(y),
                              _stream(x.device)), fn[4:])
    return y


def _w4_batch(fn, xs, weights, out_dtype):
    keep, ys = [], []
    arr = (_W4Job * len(xs))()
    for i, (x, wgt) in enumerate(zip(xs, weights)):
        x = _dev_tensor(x, "x", (torch.bfloat16,))
        c, s, z = (wgt.codes, wgt.scales, wgt.aux) if isinstance(wgt, Quantized) else wgt
        M, K = (1, x.shape[0]) if x.dim() == 1 else (x.shape[-2], x.shape[-1])
        N = _w4_rows(c, K)
        y = torch.empty((M, N), dtype=out_dtype, device=x.device)
        keep += [x, c, s, z]
        ys.append(y)
        arr[i] = _W4Job(x.data_ptr(), c.data_ptr(), s.data_ptr(), z.data_ptr(), y.data_ptr(), N, K)
    M = ys[0].shape[0] if ys else 0
    if any(y.shape[0] != M for y in ys):
        raise ValueError("all jobs must share M")
    _check(getattr(lib(), fn)(arr, len(xs), M, BF16 if out_dtype == torch.bfloat16 else F32,
                              _stream(ys[0].device) if ys else None), fn[4:])
    return ys


def gemv_w4a16(x: torch.Tensor, weight, out_dtype=torch.float32) -> torch.Tensor:
    """y = x @ dequant(W)^T for bf16 activations x [M, K] (M <= 8) and an INT4
    group-128 weight: a Quantized from quantize(w, "int4_asym") or a
    (codes, scales, zeros) triple in that layout, W being [N, K]."""
    return _w4_one("pqb_gemv_w4a16", x, weight, out_dtype)


def gemv_w4a16_batch(xs, weights, out_dtype=torch.float32):
    """Several W4A16 products in as few launches as possible: xs[i] (bf16 [M, K_i],
    one M for all) times weights[i] (Quantized INT4 g128, or (codes, scales,
    zeros)).  Returns the list of outputs [M, N_i]."""
    return _w4_batch("pqb_gemv_w4a16_batch", xs, weights, out_dtype)


def gemm_w4a16(x: torch.Tensor, weight, out_dtype=torch.float32) -> torch.Tensor:
    """gemv_w4a16 on the matrix cores, for any M."""
    return _w4_one("pqb_gemm_w4a16", x, weight, out_dtype)


def gemm_w4a16_batch(xs, weights, out_dtype=torch.float32):
    """gemv_w4a16_batch on the matrix cores, for any M."""
    return _w4_batch("pqb_gemm_w4a16_batch", xs, weights, out_dtype)


def encode_e5m2(y: torch.Tensor) -> torch.Tensor:
    y = _dev_tensor(y, "y", (torch.float32,))
    out = torch.empty(y.shape, dtype=torch.uint8, device=y.device)
    _check(lib().pqb_encode_e5m2(_ptr(y), y.numel(), _ptr(out), _stream(y.device)), "encode_e5m2")
    return out


def encode_e4m3(y: torch.Tensor) -> torch.Tensor:
    y = _dev_tensor(y, "y", (torch.float32,))
    out = torch.empty(y.shape, dtype=torch.uint8, device=y.device)
    _check(lib().pqb_encode_e4m3(_ptr(y), y.numel(), _ptr(out), _stream(y.device)), "encode_e4m3")
    return out


def encode_e2m1(y: torch.Tensor) -> torch.Tensor:
    y = _dev_tensor(y, "y", (torch.float32,))
    out = torch.empty(y.shape, dtype=torch.uint8, device=y.device)
    _check(lib().pqb_encode_e2m1(_ptr(y), y.numel(), _ptr(out), _stream(y.device)), "encode_e2m1")
    return out


def check_recip(first_bits: int, n: int, device="cuda") -> torch.Tensor:
    """The engine's RN(1/s) for the n floats whose bit patterns start at first_bits."""
    out = torch.empty((n,), dtype=torch.float32, device=device)
    _check(lib().pqb_check_recip(first_bits, n, _ptr(out), _stream(out.device)), "check_recip")
    return out


def check_div(s: torch.Tensor, x_first_bits: int, nx: int) -> torch.Tensor:
    """The engine's RN(x / s[j]) for the nx floats x whose bit patterns start at
    x_first_bits; returns [len(s), nx]."""
    s = _dev_tensor(s, "s", (torch.float32,)).contiguous()
    out = torch.empty((s.numel(), nx), dtype=torch.float32, device=s.device)
    _check(lib().pqb_check_div(_ptr(s), s.numel(), x_first_bits, nx, _ptr(out), _stream(s.device)),
           "check_div")
    return out


# --------------------------------------------------------------------------
# page-named fake-quant helpers: quantize then dequantize, float32 out
# --------------------------------------------------------------------------

def _bcr(shape):
    if len(shape) == 0:
        return 1, 1, 1
    if len(shape) == 1:
        return 1, 1, shape[0]
    return math.prod(shape[:-2]), shape[-2], shape[-1]


def _fake(x, fmt, gran, shape):
    return dequantize(quantize(x, fmt, gran, shape=shape)).reshape(x.shape)


def fp8_per_tensor(x):
    return _fake(x, "fp8_e4m3", "tensor", (1, math.prod(x.shape[:-1]), x.shape[-1]))


def fp8_per_row(x):
    return _fake(x, "fp8_e4m3", "row", (1, math.prod(x.shape[:-1]), x.shape[-1]))


def fp8_blockwise(x, block=(128, 128)):
    if tuple(block) == (128, 128):
        return _fake(x, "fp8_e4m3", "128x128", _bcr(x.shape))
    if tuple(block) == (1, 128):
        return _fake(x, "fp8_e4m3", "1x128", (1, math.prod(x.shape[:-1]), x.shape[-1]))
    raise ValueError("block must be (128, 128) or (1, 128)")


def mxfp4(w, block=32):
    if block != 32:
        raise ValueError("MXFP4 blocks are 32 elements")
    return _fake(w, "mxfp4", "blk32", (1, math.prod(w.shape[:-1]), w.shape[-1]))


def nvfp4(w, block=16):
    if block != 16:
        raise ValueError("NVFP4 blocks are 16 elements")
    return _fake(w, "nvfp4", "blk16", (1, math.prod(w.shape[:-1]), w.shape[-1]))


def fp8_kv_write(k, v):
    """FP8 KV-cache write with one scale per layer: returns dequantized (k, v)."""
    kc, vc, ks, vs = kv_write_fp8(k, v)
    layers = k.shape[0]
    outs = []
    for codes, sc in ((kc, ks), (vc, vs)):
        q = Quantized(codes.reshape(-1), sc, None, "fp8_e4m3", "tensor",
                      (layers, 1, codes.numel() // max(layers, 1)))
        outs.append(dequantize(q).reshape(k.shape))
    return tuple(outs)
