"""MI355X (gfx950) block-scaled quantization engine.

FP8 E4M3 and E5M2 (per tensor, per row, 1x128, 128x128), symmetric INT8 (per
tensor, per row), MXFP4, MXFP8, NVFP4, INT4 group-128 asymmetric and the FP8
KV-cache write (per layer, per head or static scale) and the KIVI-style
2/4-bit KV cache (K per channel, V per token), plus the block-scaled FP8
GEMM that consumes 1x128 / 128x128 codes on the matrix cores, the MXFP4
product, and the W4A16 product on INT4 codes (decode rows on the vector
units, any number of rows on the matrix cores), as HIP kernels behind
the C ABI in include/pqb.h.  The binding is loaded on first use so that the input
generators in `synth` import without the engine.
"""
_EXPORTS = {
    "quantize", "quantize_batch", "dequantize", "dequantize_batch", "query_sizes", "kv_write_fp8", "kv_write_fp8_ex",
    "KV_MODES", "kv_write_kivi", "kv_read_kivi", "kivi_layouts", "gemm_fp8_blockscaled", "gemm_fp8_blockscaled_quant",
    "gemv_w4a16", "gemv_w4a16_batch", "gemm_w4a16", "gemm_w4a16_batch", "gemm_mxfp4", "gemm_nvfp4", "stream_reference", "encode_e4m3", "encode_e5m2", "encode_e2m1",
    "check_recip", "check_div",
    "fp8_per_tensor", "fp8_per_row", "fp8_blockwise", "mxfp4", "nvfp4", "fp8_kv_write",
    "Quantized", "PqbError", "abi_version", "status_string", "lib", "FORMATS", "GRANS",
    "LIB_PATH",
}


def __getattr__(name):
    if name in _EXPORTS:
        from . import pqb
        return getattr(pqb, name)
    raise AttributeError(name)
