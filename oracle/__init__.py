"""Scalar CPU oracle for block-scaled quantization -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU engine never does, and the two
share no code: this wrapper loads ``liborc.so``, built by gcc from
``oracle.c`` alone.

Inputs are numpy arrays shaped ``[rows, cols]`` or ``[batch, rows, cols]``:
float32 values, or bf16 given as their raw ``uint16`` bit patterns (pass
``bf16=True``).  Torch CPU tensors are accepted too and converted losslessly.
Outputs follow the layouts documented in ``oracle.h``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.environ.get("PQB_ORACLE_LIB") or os.path.join(_HERE, "liborc.so")

F32, BF16 = 0, 1
TENSOR, ROW, BLK_1x128, BLK_128x128 = 0, 1, 2, 3
GRANS = {"tensor": TENSOR, "row": ROW, "1x128": BLK_1x128, "128x128": BLK_128x128}

_lib = None


def build(verbose: bool = False) -> str:
    """Compile oracle.c with gcc (IEEE binary32, no contraction, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", _LIB_PATH, _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return _LIB_PATH


def lib():
    """Load liborc.so, building it first if it is missing or older than its source."""
    global _lib
    if _lib is None:
        if (not os.path.exists(_LIB_PATH)
                or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.orc_e4m3_decode.argtypes, L.orc_e4m3_decode.restype = [ctypes.c_uint8], ctypes.c_float
        L.orc_e4m3_encode.argtypes, L.orc_e4m3_encode.restype = [ctypes.c_float], ctypes.c_uint8
        L.orc_e2m1_decode.argtypes, L.orc_e2m1_decode.restype = [ctypes.c_uint8], ctypes.c_float
        L.orc_e5m2_decode.argtypes, L.orc_e5m2_decode.restype = [ctypes.c_uint8], ctypes.c_float
        L.orc_e5m2_encode.argtypes, L.orc_e5m2_encode.restype = [ctypes.c_float], ctypes.c_uint8
        L.orc_e2m1_encode.argtypes, L.orc_e2m1_encode.restype = [ctypes.c_float], ctypes.c_uint8
        L.orc_bf16_round.argtypes, L.orc_bf16_round.restype = [ctypes.c_float], ctypes.c_uint16
        L.orc_bf16_to_f32.argtypes, L.orc_bf16_to_f32.restype = [ctypes.c_uint16], ctypes.c_float
        L.orc_uniform_code.argtypes = [ctypes.c_float] * 3
        L.orc_uniform_code.restype = ctypes.c_float
        for name in ("orc_fp8_quantize", "orc_fp8_dequantize", "orc_mxfp4_quantize",
                     "orc_mxfp4_dequantize", "orc_nvfp4_quantize", "orc_nvfp4_dequantize",
                     "orc_int4_quantize", "orc_int4_dequantize", "orc_kv_write_fp8",
                     "orc_kv_quant_fp8", "orc_fp8x_quantize", "orc_fp8x_dequantize",
                     "orc_mxfp8_quantize", "orc_mxfp8_dequantize", "orc_int8_quantize",
                     "orc_int8_dequantize", "orc_kivi_quant", "orc_kivi_dequant"):
            getattr(L, name).restype = I
        for name in ("orc_e4m3_encode_n", "orc_e5m2_encode_n", "orc_e2m1_encode_n",
                     "orc_bf16_round_n"):
            getattr(L, name).argtypes = [P, I64, P]
            getattr(L, name).restype = None
        L.orc_fp8_quantize.argtypes = [P, I, I64, I64, I64, I, P, P]
        L.orc_fp8_dequantize.argtypes = [P, P, I64, I64, I64, I, I, P]
        L.orc_mxfp4_quantize.argtypes = [P, I, I64, I64, I64, P, P]
        L.orc_fp8x_quantize.argtypes = [P, I, I64, I64, I64, I, I, P, P]
        L.orc_fp8x_dequantize.argtypes = [P, P, I64, I64, I64, I, I, I, P]
        L.orc_mxfp8_quantize.argtypes = [P, I, I64, I64, I64, P, P]
        L.orc_mxfp8_dequantize.argtypes = [P, P, I64, I64, I64, I, P]
        L.orc_int8_quantize.argtypes = [P, I, I64, I64, I64, I, P, P]
        L.orc_int8_dequantize.argtypes = [P, P, I64, I64, I64, I, I, P]
        L.orc_mxfp4_dequantize.argtypes = [P, P, I64, I64, I64, I, P]
        L.orc_nvfp4_quantize.argtypes = [P, I, I64, I64, I64, P, P, P]
        L.orc_nvfp4_dequantize.argtypes = [P, P, P, I64, I64, I64, I, P]
        L.orc_int4_quantize.argtypes = [P, I, I64, I64, I64, P, P, P]
        L.orc_int4_dequantize.argtypes = [P, P, P, I64, I64, I64, I, P]
        L.orc_kv_write_fp8.argtypes = [P, P, I, I64, I64, P, P, P, P]
        L.orc_kv_quant_fp8.argtypes = [P, I, I64, I64, I64, I64, I, P, P]
        L.orc_kivi_quant.argtypes = [P, I, I64, I64, I64, I64, I, I, P, P, P]
        L.orc_kivi_dequant.argtypes = [P, P, P, I64, I64, I64, I64, I, I, I, P]
        _lib = L
    return _lib


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------

def _as_input(x, bf16: bool | None):
    """Return (contiguous numpy array, dtype code, batch, rows, cols)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                x, bf16 = x.view(torch.int16).numpy().view(np.uint16), True
            else:
                x, bf16 = x.to(torch.float32).numpy(), False
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    if bf16 is None:
        bf16 = x.dtype == np.uint16
    if bf16:
        if x.dtype != np.uint16:
            raise TypeError("bf16 input must be given as uint16 bit patterns")
    elif x.dtype != np.float32:
        raise TypeError("input must be float32 or bf16 bits")
    if x.ndim == 2:
        batch, rows, cols = 1, x.shape[0], x.shape[1]
    elif x.ndim == 3:
        batch, rows, cols = x.shape
    else:
        raise ValueError("input must be [rows, cols] or [batch, rows, cols]")
    return x, (BF16 if bf16 else F32), batch, rows, cols


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: shape rejected (status {rc})")


def _out(shape, out_bf16: bool):
    return np.empty(shape, dtype=np.uint16 if out_bf16 else np.float32)


# --------------------------------------------------------------------------
# scalar codecs
# --------------------------------------------------------------------------

def e4m3_decode(code: int) -> float:
    return lib().orc_e4m3_decode(code)


def e4m3_encode(y: float) -> int:
    return lib().orc_e4m3_encode(y)


def e2m1_decode(nibble: int) -> float:
    return lib().orc_e2m1_decode(nibble)


def e2m1_encode(y: float) -> int:
    return lib().orc_e2m1_encode(y)


def bf16_round(v: float) -> int:
    return lib().orc_bf16_round(v)


def uniform_code(x: float, s: float, z: float) -> float:
    return lib().orc_uniform_code(x, s, z)


def e4m3_encode_array(y) -> np.ndarray:
    y = np.ascontiguousarray(y, np.float32)
    out = np.empty(y.shape, np.uint8)
    lib().orc_e4m3_encode_n(_p(y), y.size, _p(out))
    return out


def e5m2_encode_array(y) -> np.ndarray:
    y = np.ascontiguousarray(y, np.float32)
    out = np.empty(y.shape, np.uint8)
    lib().orc_e5m2_encode_n(_p(y), y.size, _p(out))
    return out


def e2m1_encode_array(y) -> np.ndarray:
    y = np.ascontiguousarray(y, np.float32)
    out = np.empty(y.shape, np.uint8)
    lib().orc_e2m1_encode_n(_p(y), y.size, _p(out))
    return out


def bf16_round_array(v) -> np.ndarray:
    v = np.ascontiguousarray(v, np.float32)
    out = np.empty(v.shape, np.uint16)
    lib().orc_bf16_round_n(_p(v), v.size, _p(out))
    return out


# --------------------------------------------------------------------------
# quantizers
# --------------------------------------------------------------------------

def _fp8_nscales(gran, batch, rows, cols):
    if gran == TENSOR:
        return (batch,)
    if gran == ROW:
        return (batch, rows)
    if gran == BLK_1x128:
        return (batch, rows, cols // 128)
    br = min(128, rows)
    return (batch, rows // br if br else 0, cols // 128)


ELEMS = {"e4m3": 0, "e5m2": 1}


def fp8_quantize(x, gran, bf16=None, elem="e4m3"):
    """-> (codes u8 [batch, rows, cols], scales f32 in the scope layout).
    elem: "e4m3" (scale amax/448) or "e5m2" (scale amax/57344)."""
    gran = GRANS.get(gran, gran)
    elem = ELEMS.get(elem, elem)
    x, dt, b, r, c = _as_input(x, bf16)
    codes = np.empty((b, r, c), np.uint8)
    br = min(128, r)
    if gran == BLK_128x128 and (c % 128 or (br and r % br)):
        _check(-4, "fp8_quantize")
    if gran == BLK_1x128 and c % 128:
        _check(-4, "fp8_quantize")
    scales = np.empty(_fp8_nscales(gran, b, r, c), np.float32)
    _check(lib().orc_fp8x_quantize(_p(x), dt, b, r, c, gran, elem, _p(codes), _p(scales)),
           "fp8_quantize")
    return codes, scales


def fp8_dequantize(codes, scales, gran, out_bf16=False, elem="e4m3"):
    gran = GRANS.get(gran, gran)
    elem = ELEMS.get(elem, elem)
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.float32)
    b, r, c = codes.shape
    out = _out((b, r, c), out_bf16)
    _check(lib().orc_fp8x_dequantize(_p(codes), _p(scales), b, r, c, gran, elem, int(out_bf16),
                                     _p(out)), "fp8_dequantize")
    return out


def mxfp8_quantize(x, bf16=None):
    """-> (codes u8 E4M3 [batch, rows, cols], scales u8 E8M0 [batch, rows, cols/32])."""
    x, dt, b, r, c = _as_input(x, bf16)
    if c % 32:
        _check(-4, "mxfp8_quantize")
    codes = np.empty((b, r, c), np.uint8)
    scales = np.empty((b, r, c // 32), np.uint8)
    _check(lib().orc_mxfp8_quantize(_p(x), dt, b, r, c, _p(codes), _p(scales)), "mxfp8_quantize")
    return codes, scales


def mxfp8_dequantize(codes, scales, out_bf16=False):
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    b, r, c = codes.shape
    out = _out((b, r, c), out_bf16)
    _check(lib().orc_mxfp8_dequantize(_p(codes), _p(scales), b, r, c, int(out_bf16), _p(out)),
           "mxfp8_dequantize")
    return out


def int8_quantize(x, gran, bf16=None):
    """Symmetric INT8, gran "tensor" or "row".
    -> (codes i8 [batch, rows, cols], scales f32 [batch] or [batch, rows])."""
    gran = GRANS.get(gran, gran)
    x, dt, b, r, c = _as_input(x, bf16)
    if gran not in (TENSOR, ROW):
        _check(-4, "int8_quantize")
    codes = np.empty((b, r, c), np.int8)
    scales = np.empty((b,) if gran == TENSOR else (b, r), np.float32)
    _check(lib().orc_int8_quantize(_p(x), dt, b, r, c, gran, _p(codes), _p(scales)),
           "int8_quantize")
    return codes, scales


def int8_dequantize(codes, scales, gran, out_bf16=False):
    gran = GRANS.get(gran, gran)
    codes = np.ascontiguousarray(codes, np.int8)
    scales = np.ascontiguousarray(scales, np.float32)
    b, r, c = codes.shape
    out = _out((b, r, c), out_bf16)
    _check(lib().orc_int8_dequantize(_p(codes), _p(scales), b, r, c, gran, int(out_bf16), _p(out)),
           "int8_dequantize")
    return out


def mxfp4_quantize(x, bf16=None):
    """-> (codes u8 [batch, rows, cols/2], scales u8 E8M0 [batch, rows, cols/32])."""
    x, dt, b, r, c = _as_input(x, bf16)
    if c % 32:
        _check(-4, "mxfp4_quantize")
    codes = np.zeros((b, r, c // 2), np.uint8)
    scales = np.empty((b, r, c // 32), np.uint8)
    _check(lib().orc_mxfp4_quantize(_p(x), dt, b, r, c, _p(codes), _p(scales)), "mxfp4_quantize")
    return codes, scales


def mxfp4_dequantize(codes, scales, out_bf16=False):
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    b, r, c2 = codes.shape
    out = _out((b, r, 2 * c2), out_bf16)
    _check(lib().orc_mxfp4_dequantize(_p(codes), _p(scales), b, r, 2 * c2, int(out_bf16), _p(out)),
           "mxfp4_dequantize")
    return out


def nvfp4_quantize(x, bf16=None):
    """-> (codes u8 [b, r, c/2], block scales u8 E4M3 [b, r, c/16], tensor scale f32 [b])."""
    x, dt, b, r, c = _as_input(x, bf16)
    if c % 16:
        _check(-4, "nvfp4_quantize")
    codes = np.zeros((b, r, c // 2), np.uint8)
    scales = np.empty((b, r, c // 16), np.uint8)
    gs = np.empty((b,), np.float32)
    _check(lib().orc_nvfp4_quantize(_p(x), dt, b, r, c, _p(codes), _p(scales), _p(gs)),
           "nvfp4_quantize")
    return codes, scales, gs


def nvfp4_dequantize(codes, scales, gs, out_bf16=False):
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    gs = np.ascontiguousarray(gs, np.float32)
    b, r, c2 = codes.shape
    out = _out((b, r, 2 * c2), out_bf16)
    _check(lib().orc_nvfp4_dequantize(_p(codes), _p(scales), _p(gs), b, r, 2 * c2, int(out_bf16),
                                      _p(out)), "nvfp4_dequantize")
    return out


def int4_quantize(x, bf16=None):
    """-> (codes u8 [b, r, c/2], scales bf16-bits u16 [b, r, c/128],
    zeros u8 [ceil(b*r*c/128 / 2)]: two signed nibbles per byte over the flat group index)."""
    x, dt, b, r, c = _as_input(x, bf16)
    if c % 128:
        _check(-4, "int4_quantize")
    codes = np.zeros((b, r, c // 2), np.uint8)
    scales = np.empty((b, r, c // 128), np.uint16)
    zeros = np.zeros(((b * r * (c // 128) + 1) // 2,), np.uint8)
    _check(lib().orc_int4_quantize(_p(x), dt, b, r, c, _p(codes), _p(scales), _p(zeros)),
           "int4_quantize")
    return codes, scales, zeros


def int4_dequantize(codes, scales, zeros, out_bf16=False):
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint16)
    zeros = np.ascontiguousarray(zeros, np.uint8)
    b, r, c2 = codes.shape
    out = _out((b, r, 2 * c2), out_bf16)
    _check(lib().orc_int4_dequantize(_p(codes), _p(scales), _p(zeros), b, r, 2 * c2,
                                     int(out_bf16), _p(out)), "int4_dequantize")
    return out


def kv_write_fp8(k, v, bf16=None):
    """K, V shaped [layers, ...]; one scale per layer for each.
    -> (k_codes, v_codes, k_scales [layers], v_scales [layers])."""
    k2, dtk, *_ = _as_input(k.reshape(k.shape[0], -1), bf16)
    v2, dtv, *_ = _as_input(v.reshape(v.shape[0], -1), bf16)
    if dtk != dtv or k2.shape != v2.shape:
        raise ValueError("K and V must share dtype and shape")
    layers, per = k2.shape
    kc = np.empty((layers, per), np.uint8)
    vc = np.empty((layers, per), np.uint8)
    ks = np.empty((layers,), np.float32)
    vs = np.empty((layers,), np.float32)
    _check(lib().orc_kv_write_fp8(_p(k2), _p(v2), dtk, layers, per, _p(kc), _p(vc), _p(ks),
                                  _p(vs)), "kv_write_fp8")
    return kc, vc, ks, vs


KV_MODES = {"layer": 0, "head": 1, "static": 2}


def kv_quant_fp8(x, mode, scales=None, bf16=None):
    """FP8 KV-cache variant on x [layers, tokens, heads, head_dim].
    mode "layer" -> scales [layers]; "head" -> [layers, heads]; "static" uses
    the given float32 scales [layers].  -> (codes u8 of x's shape, scales)."""
    mode = KV_MODES.get(mode, mode)
    L, T, H, D = x.shape
    x2, dt, *_ = _as_input(x.reshape(L, -1), bf16)
    codes = np.empty((L, T, H, D), np.uint8)
    if mode == 2:
        sc = np.ascontiguousarray(np.asarray(scales, np.float32).reshape(L))
    else:
        sc = np.empty((L, H) if mode == 1 else (L,), np.float32)
    _check(lib().orc_kv_quant_fp8(_p(x2), dt, L, T, H, D, mode, _p(codes), _p(sc)),
           "kv_quant_fp8")
    return codes, sc


def kivi_quant(x, bits, is_k, bf16=None):
    """KIVI-style KV quantization of x [layers, tokens, heads, head_dim].
    -> (codes u8 [L, T, H, D * bits / 8], scales f32, mins f32) with groups
    [L, T/32, H, D] for K and [L, T, H, D/32] for V."""
    L_, T, H, D = x.shape
    x2, dt, *_ = _as_input(x.reshape(L_, -1), bf16)
    gshape = (L_, T // 32, H, D) if is_k else (L_, T, H, D // 32)
    codes = np.zeros((L_, T, H, D * bits // 8), np.uint8)
    scales = np.empty(gshape, np.float32)
    mins = np.empty(gshape, np.float32)
    _check(lib().orc_kivi_quant(_p(x2), dt, L_, T, H, D, bits, int(is_k), _p(codes), _p(scales),
                                _p(mins)), "kivi_quant")
    return codes, scales, mins


def kivi_dequant(codes, scales, mins, bits, is_k, out_bf16=False):
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.float32)
    mins = np.ascontiguousarray(mins, np.float32)
    L_, T, H, Db = codes.shape
    D = Db * 8 // bits
    out = _out((L_, T, H * D), out_bf16).reshape(L_, T, H, D)
    _check(lib().orc_kivi_dequant(_p(codes), _p(scales), _p(mins), L_, T, H, D, bits, int(is_k),
                                  int(out_bf16), _p(out)), "kivi_dequant")
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# block-scaled FP8 GEMM (a consumer of the 1x128 and 128x128 codes)
# --------------------------------------------------------------------------

def _e4m3_table() -> np.ndarray:
    return np.array([e4m3_decode(c) for c in range(256)], np.float64)


def fp8_block_gemm(a_codes, a_scales, b_codes, b_scales, abs_sum=False):
    """Block-scaled FP8 GEMM, page "量化部署实战", exercise section on FP8
    blockwise scaling: inside each 128-deep block of K the FP8 products are
    summed, that block sum is multiplied by the block's activation scale and
    weight scale, and the results are added into the float32 output.

        C[m, n] = sum_kb sA[m, kb] * sB[n // 128, kb] * P[m, n, kb],
        P[m, n, kb] = sum_{k in kb} dec(a[m, k]) * dec(b[n, k]).

    a_codes u8 E4M3 [M, K] with a_scales f32 [M, K/128] (the 1x128 layout);
    b_codes u8 E4M3 [N, K] with b_scales f32 [N/128, K/128] (the 128x128
    layout); K and N multiples of 128.  Written out in float64: every block sum
    P is exact there (its terms are multiples of 2^-18 below 2^18, fewer than
    2^8 of them), so the only roundings are the float64 scale products and
    additions, far below float32 resolution.

    Returns C as float64 [M, N]; with abs_sum, also the same sum taken over
    absolute values (sum_kb |sA sB| sum_k |dec(a) dec(b)|), which sets the
    scale of any float32 evaluation's rounding error."""
    a_codes = np.ascontiguousarray(a_codes, np.uint8)
    b_codes = np.ascontiguousarray(b_codes, np.uint8)
    M, K = a_codes.shape
    N, Kb = b_codes.shape
    if K != Kb or K % 128 or N % 128:
        raise ValueError("need a [M, K], b [N, K] with K and N multiples of 128")
    sa = np.asarray(a_scales, np.float32).astype(np.float64).reshape(M, K // 128)
    sb = np.asarray(b_scales, np.float32).astype(np.float64).reshape(N // 128, K // 128)
    dec = _e4m3_table()
    a = dec[a_codes]
    b = dec[b_codes]
    C = np.zeros((M, N), np.float64)
    S = np.zeros((M, N), np.float64) if abs_sum else None
    for kb in range(K // 128):
        ks = slice(128 * kb, 128 * kb + 128)
        P = a[:, ks] @ b[:, ks].T                                # exact block sums
        s = sa[:, kb, None] * np.repeat(sb[:, kb], 128)[None, :]
        C += s * P
        if abs_sum:
            S += np.abs(s) * (np.abs(a[:, ks]) @ np.abs(b[:, ks]).T)
    return (C, S) if abs_sum else C


# --------------------------------------------------------------------------
# W4A16 product (a consumer of the INT4 group-128 codes)
# --------------------------------------------------------------------------

def w4a16_gemv(x, codes, scales, zeros, abs_sum=False):
    """y = x @ dequant(W)^T for bf16 activations x [M, K] and an INT4 group-128
    asymmetric weight W [N, K] in the engine's layout (codes [N, K/2], bf16
    scales [N, K/128], zero-point nibbles over the flat group index): page "14.
    量化：让每一步搬更少的字节", 路线一 (W4A16: 4-bit weights read from memory,
    unpacked and dequantized to 16 bits, then multiplied; the Marlin role).

    The dequantized weights are the oracle's own int4_dequantize values, (q -
    z) * s, exact in float32; x is widened from bf16 exactly; the product is
    the float64 matmul (every term is exact in float64, the sums round at
    2^-53).  Returns y as float64 [M, N]; with abs_sum, also sum_k |x| |w|,
    which sets the scale of a float32 evaluation's error.  x may be a torch
    bf16 tensor or raw bf16 bits (uint16)."""
    if hasattr(x, "dtype") and str(x.dtype) == "torch.bfloat16":
        xb = x.contiguous().view(__import__("torch").int16).numpy().view(np.uint16)
    else:
        xb = np.ascontiguousarray(x, np.uint16)
    M, K = xb.shape
    codes = np.ascontiguousarray(codes, np.uint8)
    N = codes.size * 2 // K
    w = int4_dequantize(codes.reshape(1, N, K // 2), scales, zeros)[0].astype(np.float64)
    xf = bf16_bits_to_f32(xb).astype(np.float64)
    y = xf @ w.T
    return (y, np.abs(xf) @ np.abs(w).T) if abs_sum else y


# --------------------------------------------------------------------------
# MXFP4 x MXFP4 product (a consumer of the MXFP4 codes)
# --------------------------------------------------------------------------

def mxfp4_gemm(a_codes, a_scales, b_codes, b_scales, abs_sum=False):
    """C = dequant(A) @ dequant(B)^T for two MXFP4 operands in the engine's
    layout (E2M1 codes [rows, K/2], element 2i in the low nibble of byte i;
    E8M0 scales [rows, K/32]): the product an MX-capable matrix core computes
    from the codes and block scales directly (page "LLM 推理优化 · 量化学习笔记"
    §4.5: MXFP4 is 32-element blocks with a shared E8M0 scale, and FP4 tensor
    cores consume it natively).  The dequantized values are the oracle's own
    mxfp4_dequantize results (+-V * 2^X, exact); the product is the float64
    matmul.  Returns C [M, N] as float64; with abs_sum, also sum_k |a| |b|."""
    a_codes = np.ascontiguousarray(a_codes, np.uint8)
    b_codes = np.ascontiguousarray(b_codes, np.uint8)
    M, Kh = a_codes.shape
    N = b_codes.shape[0]
    K = 2 * Kh
    if b_codes.shape[1] != Kh or K % 32:
        raise ValueError("need a [M, K/2], b [N, K/2] codes with K a multiple of 32")
    a = mxfp4_dequantize(a_codes.reshape(1, M, Kh), np.asarray(a_scales, np.uint8).reshape(1, M, K // 32))[0]
    b = mxfp4_dequantize(b_codes.reshape(1, N, Kh), np.asarray(b_scales, np.uint8).reshape(1, N, K // 32))[0]
    a = a.astype(np.float64)
    b = b.astype(np.float64)
    C = a @ b.T
    return (C, np.abs(a) @ np.abs(b).T) if abs_sum else C


# --------------------------------------------------------------------------
# NVFP4 x NVFP4 product (a consumer of the NVFP4 codes)
# --------------------------------------------------------------------------

_E2M1_MAG = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _nvfp4_scaled_elements(codes, scales, rows, K):
    """V(code) * dec(block scale) for every element, float64 [rows, K]: the
    nibble's E2M1 value (element 2i in the low nibble of byte i) times the
    E4M3 value of its 16-element block's scale byte."""
    codes = np.ascontiguousarray(codes, np.uint8).reshape(rows, K // 2)
    nib = np.empty((rows, K), np.uint8)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    val = np.where(nib & 8, -1.0, 1.0) * np.array(_E2M1_MAG)[nib & 7]
    dec = _e4m3_table()[np.asarray(scales, np.uint8).reshape(rows, K // 16)]
    return val * np.repeat(dec, 16, axis=1)


def nvfp4_gemm(a_codes, a_scales, a_gs, b_codes, b_scales, b_gs, abs_sum=False):
    """C = g * sum_k A'[m, k] B'[n, k] for two NVFP4 operands in the engine's
    layout (E2M1 codes [rows, K/2], E4M3 block scales [rows, K/16], one float32
    tensor scale each), the product a matrix core forms from the format (page
    "14. 量化：让每一步搬更少的字节", section 新一代低位格式：FP8、FP4 与微缩放:
    FP4 matrix units take NVFP4 operands directly; page "量化部署实战", 格式速查,
    NVFP4 row: 16-element blocks, an E4M3 scale per block and a float32 scale
    per tensor):

        A'[m, k] = V(a[m, k]) * dec(sa[m, k // 16]),  B' likewise,
        g = float32(gsA * gsB).

    Each block scale enters as its E4M3 value, so a block whose scale code is
    0 contributes 0 (pqb_dequantize's 1e-12 floor only keeps the quantizer's
    division finite); the two tensor scales enter once, as their float32
    product.  Every A' and B' value has at most 6 significant bits between
    2^-10 and 2688, so every product is exact in float64 and the matmul rounds
    only at 2^-53.  Returns C as float64 [M, N]; with abs_sum, also
    g * sum_k |A'| |B'|, which sets the scale of a float32 evaluation's error."""
    a_codes = np.asarray(a_codes, np.uint8)
    b_codes = np.asarray(b_codes, np.uint8)
    M, N = a_codes.shape[0], b_codes.shape[0]
    K = 2 * a_codes.shape[1]
    if b_codes.shape[1] != K // 2 or K % 16:
        raise ValueError("need a [M, K/2], b [N, K/2] codes with K a multiple of 16")
    A = _nvfp4_scaled_elements(a_codes, a_scales, M, K)
    B = _nvfp4_scaled_elements(b_codes, b_scales, N, K)
    g = float(np.float32(np.float32(a_gs).reshape(-1)[0]) * np.float32(np.float32(b_gs).reshape(-1)[0]))
    C = g * (A @ B.T)
    return (C, g * (np.abs(A) @ np.abs(B).T)) if abs_sum else C
