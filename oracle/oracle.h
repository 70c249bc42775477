/*
 * Scalar CPU oracle for block-scaled quantization.  TEST INFRASTRUCTURE ONLY.
 *
 * This library is the independent checker of the GPU engine.  Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header, table or constant with the HIP engine.
 *
 * Every routine computes in IEEE binary32 with round-to-nearest-even: the
 * fake-quant code on the page "量化部署实战" (section 伪量化实现) works on
 * float32 tensors and returns float32.  bf16 inputs are widened exactly.
 * Build with -O2 -ffp-contract=off and without fast-math.
 *
 * Layouts (row-major, "tensor" = one batch slice of [rows, cols]):
 *   FP8 codes      u8  [batch, rows, cols]
 *   4-bit codes    u8  [batch, rows, cols/2], element 2i in the low nibble
 *   FP8 scales     f32 TENSOR [batch]; ROW [batch, rows];
 *                      1x128 [batch, rows, cols/128];
 *                      128x128 [batch, rows/br, cols/128] with br = min(128, rows)
 *   MXFP4 scales   u8 E8M0 [batch, rows, cols/32]
 *   NVFP4 scales   u8 E4M3 [batch, rows, cols/16] plus f32 tensor scale [batch]
 *   INT4 scales    bf16 bits [batch, rows, cols/128]; zero-points as signed
 *                  nibbles, two per byte over the flat group index
 *                  (ceil(batch*rows*cols/128 / 2) bytes)
 *
 * Return value of the quantizers: 0 on success, -4 for a shape that the
 * pages' reshape would reject.
 */
#ifndef PQB_ORACLE_H
#define PQB_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1 };
enum { ORC_TENSOR = 0, ORC_ROW = 1, ORC_BLK_1x128 = 2, ORC_BLK_128x128 = 3 };
enum { ORC_E4M3 = 0, ORC_E5M2 = 1 };

/* number formats */
float    orc_e4m3_decode(uint8_t code);
uint8_t  orc_e4m3_encode(float y);
float    orc_e5m2_decode(uint8_t code);
uint8_t  orc_e5m2_encode(float y);
float    orc_e2m1_decode(uint8_t nibble);
uint8_t  orc_e2m1_encode(float y);
uint16_t orc_bf16_round(float v);
float    orc_bf16_to_f32(uint16_t h);
void     orc_e4m3_encode_n(const float* y, int64_t n, uint8_t* out);
void     orc_e5m2_encode_n(const float* y, int64_t n, uint8_t* out);
void     orc_e2m1_encode_n(const float* y, int64_t n, uint8_t* out);
void     orc_bf16_round_n(const float* v, int64_t n, uint16_t* out);

/* uniform-quantizer primitive q = round(x/s) + z, unclamped */
float    orc_uniform_code(float x, float s, float z);

/* FP8 E4M3 with four scopes */
int orc_fp8_quantize(const void* x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                     int gran, uint8_t* codes, float* scales);
int orc_fp8_dequantize(const uint8_t* codes, const float* scales, int64_t batch, int64_t rows,
                       int64_t cols, int gran, int out_dtype, void* out);

/* MXFP4: E2M1 in 32-element blocks, E8M0 power-of-two scale */
/* FP8 scopes with E4M3 (max 448) or E5M2 (max 57344) elements; returns -2
 * for an unknown element format. */
int orc_fp8x_quantize(const void* x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                      int gran, int elem, uint8_t* codes, float* scales);
int orc_fp8x_dequantize(const uint8_t* codes, const float* scales, int64_t batch, int64_t rows,
                        int64_t cols, int gran, int elem, int out_dtype, void* out);
/* MXFP8: E4M3 codes u8 [batch, rows, cols], E8M0 scales u8 [batch, rows, cols/32]. */
int orc_mxfp8_quantize(const void* x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                       uint8_t* codes, uint8_t* scales);
int orc_mxfp8_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t batch,
                         int64_t rows, int64_t cols, int out_dtype, void* out);
/* Symmetric INT8, TENSOR or ROW: codes i8 [batch, rows, cols], scales f32. */
int orc_int8_quantize(const void* x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                      int gran, int8_t* codes, float* scales);
int orc_int8_dequantize(const int8_t* codes, const float* scales, int64_t batch, int64_t rows,
                        int64_t cols, int gran, int out_dtype, void* out);
int orc_mxfp4_quantize(const void* x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                       uint8_t* codes, uint8_t* scales);
int orc_mxfp4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t batch,
                         int64_t rows, int64_t cols, int out_dtype, void* out);

/* NVFP4: E2M1 in 16-element blocks, E4M3 block scale, f32 tensor scale */
int orc_nvfp4_quantize(const void* x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                       uint8_t* codes, uint8_t* scales, float* tensor_scale);
int orc_nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                         int64_t batch, int64_t rows, int64_t cols, int out_dtype, void* out);

/* INT4 group-128 asymmetric */
int orc_int4_quantize(const void* x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                      uint8_t* codes, uint16_t* scales, uint8_t* zeros);
int orc_int4_dequantize(const uint8_t* codes, const uint16_t* scales, const uint8_t* zeros,
                        int64_t batch, int64_t rows, int64_t cols, int out_dtype, void* out);

/* FP8 KV-cache write: one per-tensor scale per layer, separately for K and V */
/* FP8 KV-cache variants on [layers, tokens, heads, head_dim]: one scale per
 * layer (LAYER), per (layer, head) over tokens x head_dim (HEAD), or a given
 * per-layer scale (STATIC, scales read).  Returns -2 for an unknown mode. */
enum { ORC_KV_LAYER = 0, ORC_KV_HEAD = 1, ORC_KV_STATIC = 2 };
int orc_kv_quant_fp8(const void* x, int dtype, int64_t layers, int64_t tokens, int64_t heads,
                     int64_t head_dim, int mode, uint8_t* codes, float* scales);
/* KIVI-style b-bit (2 or 4) asymmetric KV quantization on [layers, tokens,
 * heads, head_dim]: K (is_k = 1) per channel over groups of 32 tokens, V per
 * token over groups of 32 channels; float32 scales and minimums per group. */
int orc_kivi_quant(const void* x, int dtype, int64_t layers, int64_t tokens, int64_t heads,
                   int64_t head_dim, int bits, int is_k, uint8_t* codes, float* scales,
                   float* mins);
int orc_kivi_dequant(const uint8_t* codes, const float* scales, const float* mins, int64_t layers,
                     int64_t tokens, int64_t heads, int64_t head_dim, int bits, int is_k,
                     int out_dtype, void* out);
int orc_kv_write_fp8(const void* k, const void* v, int dtype, int64_t layers,
                     int64_t elems_per_layer, uint8_t* k_codes, uint8_t* v_codes,
                     float* k_scales, float* v_scales);

#ifdef __cplusplus
}
#endif
#endif
