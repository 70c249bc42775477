/*
 * Scalar CPU oracle for block-scaled quantization.  TEST INFRASTRUCTURE ONLY:
 * the test suite, the smoke check and the benchmark's CPU-baseline leg are its
 * only users.  It is deliberately slow and literal, and it shares no code with
 * the HIP engine.
 *
 * Sources (page title, section):
 *   [DEPLOY]   "量化部署实战" (quantization deployment in practice):
 *              sections 格式速查 (format table) and 伪量化实现 (the fake-quant
 *              module that quantizes and immediately dequantizes in float32).
 *   [BYTES]    "14. 量化：让每一步搬更少的字节": sections 量化在做什么
 *              (uniform quantizer and its worked example) and the table of new
 *              low-bit formats (FP8 / FP4 / micro-scaling).
 *   [NOTES]    "LLM 推理优化 · 量化（Quantization）系统学习笔记": §4.2 (bit
 *              layouts) and §5.1 (symmetric and asymmetric formulas).
 *
 * All arithmetic is IEEE binary32, round-to-nearest-even, with subnormals,
 * exactly as [DEPLOY] computes on float32 tensors.  Every division is a true
 * IEEE division.  Build with -O2 -ffp-contract=off, no fast-math.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

/* E4M3 [DEPLOY 格式速查; NOTES §4.2]: 1 sign, 4 exponent, 3 mantissa bits, no
 * infinities and a single NaN pattern per sign (exponent and mantissa all
 * ones), largest finite value 448.  448 = 1.75 * 2^8 fixes the exponent bias at
 * 7; exponent field 0 holds the subnormals m * 2^-9. */
float orc_e4m3_decode(uint8_t code) {
  int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
  float mag;
  if (e == 15 && m == 7) return sign ? -NAN : NAN;
  if (e == 0)
    mag = ldexpf((float)m, -9);
  else
    mag = ldexpf((float)(8 + m), e - 10);
  return sign ? -mag : mag;
}

/* E4M3 rounding: the nearest finite E4M3 value, ties to the code with an even
 * mantissa (round-to-nearest-even), sign bit copied from y.  This is the
 * float32 -> float8_e4m3fn cast that [DEPLOY 伪量化实现] applies after clamping
 * to +-448.  The search runs over every non-negative finite code.  Distances
 * are taken in double: for the two codes that bracket |y| the difference is
 * exact, which is all the decision needs. */
uint8_t orc_e4m3_encode(float y) {
  double a = fabs((double)y);
  int best = 0;
  double bestd = a; /* distance to code 0 (value 0) */
  for (int c = 1; c <= 0x7E; ++c) {
    double d = fabs(a - (double)orc_e4m3_decode((uint8_t)c));
    if (d < bestd || (d == bestd && (c & 1) == 0)) {
      best = c;
      bestd = d;
    }
  }
  return (uint8_t)((signbit(y) ? 0x80 : 0x00) | best);
}

/* E5M2 [BYTES 低位浮点格式 table; NOTES §4.2]: 1 sign, 5 exponent, 2 mantissa
 * bits, largest finite value 57344 = 1.75 * 2^15, which fixes the bias at 15.
 * Exponent field 31 holds the infinities (mantissa 0) and NaNs; field 0 holds
 * the subnormals m * 2^-16. */
float orc_e5m2_decode(uint8_t code) {
  int sign = code >> 7, e = (code >> 2) & 31, m = code & 3;
  float mag;
  if (e == 31) return m ? (sign ? -NAN : NAN) : (sign ? -INFINITY : INFINITY);
  if (e == 0)
    mag = ldexpf((float)m, -16);
  else
    mag = ldexpf((float)(4 + m), e - 17);
  return sign ? -mag : mag;
}

/* E5M2 rounding: the nearest finite E5M2 value, ties to the code with an even
 * mantissa (round-to-nearest-even), sign bit copied from y; the search runs
 * over every non-negative finite code (0x00..0x7B). */
uint8_t orc_e5m2_encode(float y) {
  double a = fabs((double)y);
  int best = 0;
  double bestd = a;
  for (int c = 1; c <= 0x7B; ++c) {
    double d = fabs(a - (double)orc_e5m2_decode((uint8_t)c));
    if (d < bestd || (d == bestd && (c & 1) == 0)) {
      best = c;
      bestd = d;
    }
  }
  return (uint8_t)((signbit(y) ? 0x80 : 0x00) | best);
}

/* E2M1 [DEPLOY 格式速查, 伪量化实现; BYTES 新格式]: the non-negative values are
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6.  The nibble holds the sign in bit 3 and the index
 * into this list in bits 0..2 (with exponent bias 1 the index is exactly the
 * 3-bit exponent:mantissa field). */
static const float E2M1_VALUES[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

float orc_e2m1_decode(uint8_t nibble) {
  float v = E2M1_VALUES[nibble & 7];
  return (nibble & 8) ? -v : v;
}

/* E2M1 rounding as [DEPLOY 伪量化实现] defines it: y is clamped to [-6, 6],
 * then the float32 distance from |y| to each of the eight values is taken and
 * the first index of the smallest distance wins (so ties go to the smaller
 * magnitude); the sign is that of y with sign(0) = 0, so -0.0 gives +0 and a
 * small negative y gives -0. */
uint8_t orc_e2m1_encode(float y) {
  float a = fabsf(fminf(fmaxf(y, -6.0f), 6.0f));
  int best = 0;
  float bestd = fabsf(a - E2M1_VALUES[0]);
  for (int i = 1; i < 8; ++i) {
    float d = fabsf(a - E2M1_VALUES[i]);
    if (d < bestd) {
      best = i;
      bestd = d;
    }
  }
  return (uint8_t)(((y < 0.0f) ? 8 : 0) | best);
}

/* bf16 [NOTES §4.2]: the upper 16 bits of a binary32.  Rounding: of the two
 * bf16 values that bracket v (the truncation and its successor in magnitude)
 * take the nearer, on a tie the one with an even last bit. */
uint16_t orc_bf16_round(float v) {
  uint32_t b;
  memcpy(&b, &v, 4);
  uint32_t lo = b & 0xFFFF0000u, rem = b & 0x0000FFFFu;
  if (rem > 0x8000u || (rem == 0x8000u && (lo & 0x00010000u))) lo += 0x00010000u;
  return (uint16_t)(lo >> 16);
}

float orc_bf16_to_f32(uint16_t h) {
  uint32_t b = (uint32_t)h << 16;
  float f;
  memcpy(&f, &b, 4);
  return f;
}

/* Uniform quantizer [BYTES 量化在做什么; NOTES §5.1]: the stored integer is the
 * rounded quotient x/s, shifted by the zero-point z in the asymmetric form.
 * Rounding is IEEE round-to-nearest-even on the float32 quotient. */
float orc_uniform_code(float x, float s, float z) { return rintf(x / s) + z; }

/* ------------------------------------------------------------------------ */
/* Helpers                                                                   */
/* ------------------------------------------------------------------------ */

static float ld(const void* x, int dtype, int64_t i) {
  if (dtype == ORC_BF16) return orc_bf16_to_f32(((const uint16_t*)x)[i]);
  return ((const float*)x)[i];
}

static void st(void* out, int dtype, int64_t i, float v) {
  if (dtype == ORC_BF16)
    ((uint16_t*)out)[i] = orc_bf16_round(v);
  else
    ((float*)out)[i] = v;
}

static float clampf(float v, float lo, float hi) { return fminf(fmaxf(v, lo), hi); }

static void put_nibble(uint8_t* buf, int64_t i, uint8_t v) {
  uint8_t* p = buf + (i >> 1);
  if (i & 1)
    *p = (uint8_t)((*p & 0x0F) | ((v & 0x0F) << 4));
  else
    *p = (uint8_t)((*p & 0xF0) | (v & 0x0F));
}

static uint8_t get_nibble(const uint8_t* buf, int64_t i) {
  uint8_t b = buf[i >> 1];
  return (i & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 0x0F);
}

static int bad_dims(int64_t batch, int64_t rows, int64_t cols) {
  return batch < 0 || rows < 0 || cols < 0;
}

/* ------------------------------------------------------------------------ */
/* FP8 E4M3 [DEPLOY 伪量化实现]                                              */
/* ------------------------------------------------------------------------ */

/* One scope: its scale is max(amax, 1e-12) / 448, each element becomes the
 * E4M3 code of clamp(x / scale, -448, 448).  With E5M2 elements the same steps
 * use E5M2's largest value, 57344, in place of 448. */
static float fp8_scale(float amax) { return fmaxf(amax, 1e-12f) / 448.0f; }

static uint8_t fp8_code(float x, float s) { return orc_e4m3_encode(clampf(x / s, -448.0f, 448.0f)); }

static float fp8x_max(int elem) { return elem == ORC_E5M2 ? 57344.0f : 448.0f; }

static float fp8x_scale(float amax, int elem) { return fmaxf(amax, 1e-12f) / fp8x_max(elem); }

static uint8_t fp8x_code(float x, float s, int elem) {
  float m = fp8x_max(elem);
  float y = clampf(x / s, -m, m);
  return elem == ORC_E5M2 ? orc_e5m2_encode(y) : orc_e4m3_encode(y);
}

static float fp8x_decode(uint8_t code, int elem) {
  return elem == ORC_E5M2 ? orc_e5m2_decode(code) : orc_e4m3_decode(code);
}

/* Index of the scale that element (b, r, c) uses; -1 for a rejected shape. */
static int64_t fp8_scale_index(int gran, int64_t rows, int64_t cols, int64_t b, int64_t r,
                               int64_t c) {
  switch (gran) {
    case ORC_TENSOR:
      return b;
    case ORC_ROW:
      return b * rows + r;
    case ORC_BLK_1x128:
      return (b * rows + r) * (cols / 128) + c / 128;
    case ORC_BLK_128x128: {
      int64_t br = rows < 128 ? rows : 128;
      return (b * (rows / br) + r / br) * (cols / 128) + c / 128;
    }
  }
  return -1;
}

static int fp8_shape_ok(int gran, int64_t rows, int64_t cols) {
  switch (gran) {
    case ORC_TENSOR:
    case ORC_ROW:
      return 1;
    case ORC_BLK_1x128:
      return cols % 128 == 0;
    case ORC_BLK_128x128: {
      int64_t br = rows < 128 ? rows : 128;
      return cols % 128 == 0 && (rows == 0 || rows % br == 0);
    }
  }
  return 0;
}

static int64_t fp8_num_scales(int gran, int64_t batch, int64_t rows, int64_t cols) {
  switch (gran) {
    case ORC_TENSOR:
      return batch;
    case ORC_ROW:
      return batch * rows;
    case ORC_BLK_1x128:
      return batch * rows * (cols / 128);
    case ORC_BLK_128x128: {
      int64_t br = rows < 128 ? rows : 128;
      return rows == 0 ? 0 : batch * (rows / br) * (cols / 128);
    }
  }
  return 0;
}

int orc_fp8_quantize(const void* x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                     int gran, uint8_t* codes, float* scales) {
  return orc_fp8x_quantize(x, dtype, batch, rows, cols, gran, ORC_E4M3, codes, scales);
}

int orc_fp8_dequantize(const uint8_t* codes, const float* scales, int64_t batch, int64_t rows,
                       int64_t cols, int gran, int out_dtype, void* out) {
  return orc_fp8x_dequantize(codes, scales, batch, rows, cols, gran, ORC_E4M3, out_dtype, out);
}

int orc_fp8x_quantize(const void* x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                      int gran, int elem, uint8_t* codes, float* scales) {
  if (elem != ORC_E4M3 && elem != ORC_E5M2) return -2;
  if (bad_dims(batch, rows, cols) || gran < ORC_TENSOR || gran > ORC_BLK_128x128) return -4;
  if (!fp8_shape_ok(gran, rows, cols)) return -4;
  int64_t ns = fp8_num_scales(gran, batch, rows, cols);
  /* pass 1: amax of every scope (|x| >= 0, so 0 is the neutral element) */
  for (int64_t i = 0; i < ns; ++i) scales[i] = 0.0f;
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t r = 0; r < rows; ++r)
      for (int64_t c = 0; c < cols; ++c) {
        int64_t si = fp8_scale_index(gran, rows, cols, b, r, c);
        scales[si] = fmaxf(scales[si], fabsf(ld(x, dtype, (b * rows + r) * cols + c)));
      }
  for (int64_t i = 0; i < ns; ++i) scales[i] = fp8x_scale(scales[i], elem);
  /* pass 2: codes */
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t r = 0; r < rows; ++r)
      for (int64_t c = 0; c < cols; ++c) {
        int64_t i = (b * rows + r) * cols + c;
        codes[i] = fp8x_code(ld(x, dtype, i), scales[fp8_scale_index(gran, rows, cols, b, r, c)],
                             elem);
      }
  return 0;
}

/* Dequantization is the decoded E4M3 (E5M2) value times its scope's scale. */
int orc_fp8x_dequantize(const uint8_t* codes, const float* scales, int64_t batch, int64_t rows,
                        int64_t cols, int gran, int elem, int out_dtype, void* out) {
  if (elem != ORC_E4M3 && elem != ORC_E5M2) return -2;
  if (bad_dims(batch, rows, cols) || gran < ORC_TENSOR || gran > ORC_BLK_128x128) return -4;
  if (!fp8_shape_ok(gran, rows, cols)) return -4;
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t r = 0; r < rows; ++r)
      for (int64_t c = 0; c < cols; ++c) {
        int64_t i = (b * rows + r) * cols + c;
        float s = scales[fp8_scale_index(gran, rows, cols, b, r, c)];
        st(out, out_dtype, i, fp8x_decode(codes[i], elem) * s);
      }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* MXFP4 [DEPLOY 伪量化实现; BYTES 新格式]                                   */
/* ------------------------------------------------------------------------ */

/* Each run of 32 elements along the last dimension shares the scale
 * 2^(floor(log2(max(amax, 1e-12))) - 2): E2M1's largest exponent is 2, so the
 * block maximum lands in [4, 8) before the clamp to 6.  floor(log2 a) is read
 * exactly from the binary exponent (frexp gives a = f * 2^e, f in [0.5, 1)).
 * The E8M0 byte stores the exponent with bias 127. */
int orc_mxfp4_quantize(const void* x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                       uint8_t* codes, uint8_t* scales) {
  if (bad_dims(batch, rows, cols) || cols % 32 != 0) return -4;
  int64_t nblk = batch * rows * (cols / 32);
  for (int64_t k = 0; k < nblk; ++k) {
    float amax = 0.0f;
    for (int64_t j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(ld(x, dtype, k * 32 + j)));
    int e;
    frexpf(fmaxf(amax, 1e-12f), &e);
    int X = (e - 1) - 2;
    float scale = ldexpf(1.0f, X);
    scales[k] = (uint8_t)(X + 127);
    for (int64_t j = 0; j < 32; ++j) {
      float y = clampf(ld(x, dtype, k * 32 + j) / scale, -6.0f, 6.0f);
      put_nibble(codes, k * 32 + j, orc_e2m1_encode(y));
    }
  }
  return 0;
}

int orc_mxfp4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t batch,
                         int64_t rows, int64_t cols, int out_dtype, void* out) {
  if (bad_dims(batch, rows, cols) || cols % 32 != 0) return -4;
  int64_t n = batch * rows * cols;
  for (int64_t i = 0; i < n; ++i) {
    float scale = ldexpf(1.0f, (int)scales[i / 32] - 127);
    st(out, out_dtype, i, orc_e2m1_decode(get_nibble(codes, i)) * scale);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* NVFP4 [DEPLOY 伪量化实现; BYTES 新格式]                                   */
/* ------------------------------------------------------------------------ */

/* Two levels.  The tensor scale is max(amax_tensor, 1e-12) / (448 * 6).  Each
 * run of 16 elements stores the E4M3 code of (amax_block / 6) / tensor_scale
 * (two divisions, in that order).  The elements are rounded to E2M1 against
 * max(decoded block scale, 1e-12) * tensor_scale. */
static float nv_effective_scale(uint8_t code, float gs) {
  return fmaxf(orc_e4m3_decode(code), 1e-12f) * gs;
}

int orc_nvfp4_quantize(const void* x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                       uint8_t* codes, uint8_t* scales, float* tensor_scale) {
  if (bad_dims(batch, rows, cols) || cols % 16 != 0) return -4;
  int64_t per = rows * cols;
  for (int64_t b = 0; b < batch; ++b) {
    const int64_t base = b * per;
    float amax_t = 0.0f;
    for (int64_t i = 0; i < per; ++i) amax_t = fmaxf(amax_t, fabsf(ld(x, dtype, base + i)));
    float gs = fmaxf(amax_t, 1e-12f) / (448.0f * 6.0f);
    tensor_scale[b] = gs;
    for (int64_t k = 0; k < per / 16; ++k) {
      const int64_t e0 = base + k * 16;
      float amax_b = 0.0f;
      for (int64_t j = 0; j < 16; ++j) amax_b = fmaxf(amax_b, fabsf(ld(x, dtype, e0 + j)));
      uint8_t bs = orc_e4m3_encode(amax_b / 6.0f / gs);
      scales[e0 / 16] = bs;
      float s = nv_effective_scale(bs, gs);
      for (int64_t j = 0; j < 16; ++j) {
        float y = clampf(ld(x, dtype, e0 + j) / s, -6.0f, 6.0f);
        put_nibble(codes, e0 + j, orc_e2m1_encode(y));
      }
    }
  }
  return 0;
}

int orc_nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                         int64_t batch, int64_t rows, int64_t cols, int out_dtype, void* out) {
  if (bad_dims(batch, rows, cols) || cols % 16 != 0) return -4;
  int64_t per = rows * cols;
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t i = 0; i < per; ++i) {
      int64_t g = b * per + i;
      float s = nv_effective_scale(scales[g / 16], tensor_scale[b]);
      st(out, out_dtype, g, orc_e2m1_decode(get_nibble(codes, g)) * s);
    }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* INT4 group-128 asymmetric [DEPLOY 格式速查; BYTES 量化在做什么; NOTES §5.1] */
/* ------------------------------------------------------------------------ */

/* Integers -8..7, one 2-byte (bf16) scale and one zero-point per run of 128
 * elements.  The range [lo, hi] of a group is widened to contain 0; its 15
 * steps give s = bf16(max(hi - lo, 1e-12) / 15), and the rounded s is the one
 * used.  The zero-point maps lo to -8: z = -8 - round(lo / s).  An element
 * becomes clamp(round(x / s) + z, -8, 7) and reads back as (q - z) * s. */
int orc_int4_quantize(const void* x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                      uint8_t* codes, uint16_t* scales, uint8_t* zeros) {
  if (bad_dims(batch, rows, cols) || cols % 128 != 0) return -4;
  const int64_t G = cols / 128, ngroups = batch * rows * G;
  for (int64_t i = 0; i < (ngroups + 1) / 2; ++i) zeros[i] = 0;
  for (int64_t row = 0; row < batch * rows; ++row) {
    for (int64_t g = 0; g < G; ++g) {
      const int64_t gi = row * G + g, e0 = gi * 128;
      float lo = 0.0f, hi = 0.0f;
      for (int64_t j = 0; j < 128; ++j) {
        float v = ld(x, dtype, e0 + j);
        lo = fminf(lo, v);
        hi = fmaxf(hi, v);
      }
      uint16_t sb = orc_bf16_round(fmaxf(hi - lo, 1e-12f) / 15.0f);
      float s = orc_bf16_to_f32(sb);
      float z = clampf(-8.0f - rintf(lo / s), -8.0f, 7.0f);
      scales[gi] = sb;
      put_nibble(zeros, gi, (uint8_t)((int)z & 0x0F));
      for (int64_t j = 0; j < 128; ++j) {
        float q = clampf(orc_uniform_code(ld(x, dtype, e0 + j), s, z), -8.0f, 7.0f);
        put_nibble(codes, e0 + j, (uint8_t)((int)q & 0x0F));
      }
    }
  }
  return 0;
}

static int sext4(uint8_t v) { return (v & 8) ? (int)v - 16 : (int)v; }

int orc_int4_dequantize(const uint8_t* codes, const uint16_t* scales, const uint8_t* zeros,
                        int64_t batch, int64_t rows, int64_t cols, int out_dtype, void* out) {
  if (bad_dims(batch, rows, cols) || cols % 128 != 0) return -4;
  const int64_t n = batch * rows * cols;
  for (int64_t i = 0; i < n; ++i) {
    const int64_t gi = i / 128;
    int q = sext4(get_nibble(codes, i));
    int z = sext4(get_nibble(zeros, gi));
    float s = orc_bf16_to_f32(scales[gi]);
    st(out, out_dtype, i, (float)(q - z) * s);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* FP8 KV-cache write [DEPLOY 伪量化实现, the FP8 KV cache class]             */
/* ------------------------------------------------------------------------ */

/* Each write quantizes K and V with the per-tensor FP8 rule, so every layer
 * gets one scale of its own for K and one for V, set by the data written. */
int orc_kv_write_fp8(const void* k, const void* v, int dtype, int64_t layers,
                     int64_t elems_per_layer, uint8_t* k_codes, uint8_t* v_codes,
                     float* k_scales, float* v_scales) {
  int rc = orc_fp8_quantize(k, dtype, layers, 1, elems_per_layer, ORC_TENSOR, k_codes, k_scales);
  if (rc) return rc;
  return orc_fp8_quantize(v, dtype, layers, 1, elems_per_layer, ORC_TENSOR, v_codes, v_scales);
}

/* ------------------------------------------------------------------------ */
/* MXFP8 [NOTES §4.1, §4.2, §4.5; BYTES 低位浮点格式]                         */
/* ------------------------------------------------------------------------ */

/* Blocks of 32 share an E8M0 power-of-two scale; the elements are E4M3.  By
 * the same rule as MXFP4 (whose scale exponent is floor(log2 amax) minus
 * E2M1's largest exponent, 2), the scale is 2^X with X = floor(log2(max(amax,
 * 1e-12))) - 8, 8 being E4M3's largest exponent.  Each element is the E4M3
 * code of clamp(x / 2^X, -448, 448); the block maximum lands in [256, 512), so
 * the clamp binds for blocks whose maximum has a significand of 1.75 or more.
 * The stored byte is X + 127. */
int orc_mxfp8_quantize(const void* x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                       uint8_t* codes, uint8_t* scales) {
  if (bad_dims(batch, rows, cols) || cols % 32) return -4;
  int64_t nblk = batch * rows * cols / 32;
  for (int64_t k = 0; k < nblk; ++k) {
    float amax = 0.0f;
    for (int64_t j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(ld(x, dtype, k * 32 + j)));
    int e;
    frexpf(fmaxf(amax, 1e-12f), &e); /* max(amax, 1e-12) = f * 2^e, f in [0.5, 1) */
    int X = (e - 1) - 8;
    scales[k] = (uint8_t)(X + 127);
    for (int64_t j = 0; j < 32; ++j) {
      float y = clampf(ldexpf(ld(x, dtype, k * 32 + j), -X), -448.0f, 448.0f);
      codes[k * 32 + j] = orc_e4m3_encode(y);
    }
  }
  return 0;
}

int orc_mxfp8_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t batch,
                         int64_t rows, int64_t cols, int out_dtype, void* out) {
  if (bad_dims(batch, rows, cols) || cols % 32) return -4;
  int64_t n = batch * rows * cols;
  for (int64_t i = 0; i < n; ++i)
    st(out, out_dtype, i, ldexpf(orc_e4m3_decode(codes[i]), (int)scales[i / 32] - 127));
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Symmetric INT8 [DEPLOY 格式速查; BYTES 量化在做什么; NOTES §5.1]          */
/* ------------------------------------------------------------------------ */

/* W8A8 INT8 is per channel (a weight row) and per token (an activation row);
 * per tensor is also offered.  The scale is max(amax, 1e-12) / 127 (the INT8
 * form of the symmetric scale) and q = clamp(rint(x / s), -128, 127). */
int orc_int8_quantize(const void* x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                      int gran, int8_t* codes, float* scales) {
  if (bad_dims(batch, rows, cols) || (gran != ORC_TENSOR && gran != ORC_ROW)) return -4;
  int64_t ns = gran == ORC_TENSOR ? batch : batch * rows;
  int64_t per = gran == ORC_TENSOR ? rows * cols : cols;
  for (int64_t k = 0; k < ns; ++k) {
    float amax = 0.0f;
    for (int64_t j = 0; j < per; ++j) amax = fmaxf(amax, fabsf(ld(x, dtype, k * per + j)));
    float s = fmaxf(amax, 1e-12f) / 127.0f;
    scales[k] = s;
    for (int64_t j = 0; j < per; ++j)
      codes[k * per + j] = (int8_t)clampf(rintf(ld(x, dtype, k * per + j) / s), -128.0f, 127.0f);
  }
  return 0;
}

int orc_int8_dequantize(const int8_t* codes, const float* scales, int64_t batch, int64_t rows,
                        int64_t cols, int gran, int out_dtype, void* out) {
  if (bad_dims(batch, rows, cols) || (gran != ORC_TENSOR && gran != ORC_ROW)) return -4;
  int64_t per = gran == ORC_TENSOR ? rows * cols : cols;
  int64_t n = batch * rows * cols;
  for (int64_t i = 0; i < n; ++i) st(out, out_dtype, i, (float)codes[i] * scales[i / per]);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* FP8 KV-cache variants [DEPLOY KV Cache 量化：误差要和信号比]               */
/* ------------------------------------------------------------------------ */

/* The page quantizes K and V with quantizers chosen independently: per tensor
 * (one scale for the layer's whole cache), or per head (its per_head function:
 * the amax over the token and head_dim axes, so every (layer, head) gets
 * max(amax, 1e-12) / 448).  For deployment it recommends scales computed
 * offline from calibration data; with such a static scale s the write is
 * E4M3(clamp(x / s, -448, 448)) and the clamp can bind.
 * Layout: x is [layers, tokens, heads, head_dim], row-major (token-major, as a
 * paged cache stores it); the per-head scope of (l, h) is x[l, :, h, :].
 * Scales: LAYER [layers]; HEAD [layers, heads]; STATIC [layers], read. */
static int64_t kv_scope(int mode, int64_t heads, int64_t l, int64_t h) {
  return mode == ORC_KV_HEAD ? l * heads + h : l;
}

int orc_kv_quant_fp8(const void* x, int dtype, int64_t layers, int64_t tokens, int64_t heads,
                     int64_t head_dim, int mode, uint8_t* codes, float* scales) {
  if (layers < 0 || tokens < 0 || heads < 0 || head_dim < 0) return -4;
  if (mode < ORC_KV_LAYER || mode > ORC_KV_STATIC) return -2;
  int64_t nscopes = mode == ORC_KV_HEAD ? layers * heads : layers;
  if (mode != ORC_KV_STATIC) {
    /* pass 1: the amax of every scope */
    for (int64_t i = 0; i < nscopes; ++i) scales[i] = 0.0f;
    for (int64_t l = 0; l < layers; ++l)
      for (int64_t t = 0; t < tokens; ++t)
        for (int64_t h = 0; h < heads; ++h)
          for (int64_t d = 0; d < head_dim; ++d) {
            int64_t i = ((l * tokens + t) * heads + h) * head_dim + d;
            int64_t si = kv_scope(mode, heads, l, h);
            scales[si] = fmaxf(scales[si], fabsf(ld(x, dtype, i)));
          }
    for (int64_t i = 0; i < nscopes; ++i) scales[i] = fp8_scale(scales[i]);
  }
  /* pass 2: codes, with the clamp of the page's fp8 helper */
  for (int64_t l = 0; l < layers; ++l)
    for (int64_t t = 0; t < tokens; ++t)
      for (int64_t h = 0; h < heads; ++h)
        for (int64_t d = 0; d < head_dim; ++d) {
          int64_t i = ((l * tokens + t) * heads + h) * head_dim + d;
          codes[i] = fp8_code(ld(x, dtype, i), scales[kv_scope(mode, heads, l, h)]);
        }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* KIVI-style KV quantization [DEPLOY KV Cache 量化：误差要和信号比; BYTES   */
/* 路线三; NOTES §5.1, §7.4]                                                 */
/* ------------------------------------------------------------------------ */

/* K per channel, grouped over tokens; V per token, grouped over channels;
 * b = 2 or 4 bits, asymmetric.  The zero-point absorbs a channel's constant
 * bias: for a group with minimum m and maximum M,
 *   s = max(M - m, 1e-12) / (2^b - 1),  q = clamp(rint((x - m) / s), 0, 2^b - 1),
 *   dequant x = q * s + m,
 * with a zero minimum taken as +0 (the pages give no sign for min(-0, +0)),
 * the form the KIVI method uses (the zero-point kept as the real minimum, not
 * an integer, which could not hold a large bias in b bits).  Groups are 32
 * tokens (K) or 32 channels (V).  Layout [layers, tokens, heads, head_dim];
 * codes packed along the flat index, element i at bits b * (i % (8 / b)) of
 * byte i * b / 8.  Scales and minimums are float32:
 *   K [layers, tokens / 32, heads, head_dim]   (tokens % 32 == 0)
 *   V [layers, tokens, heads, head_dim / 32]   (head_dim % 32 == 0) */
static int64_t kivi_group(int is_k, int64_t T, int64_t H, int64_t D, int64_t l, int64_t t,
                          int64_t h, int64_t d) {
  if (is_k) return ((l * (T / 32) + t / 32) * H + h) * D + d;
  return ((l * T + t) * H + h) * (D / 32) + d / 32;
}

static void put_bits(uint8_t* buf, int64_t i, int bits, unsigned v) {
  int per = 8 / bits;
  int sh = bits * (int)(i % per);
  uint8_t mask = (uint8_t)(((1u << bits) - 1) << sh);
  buf[i / per] = (uint8_t)((buf[i / per] & ~mask) | ((v << sh) & mask));
}

static unsigned get_bits(const uint8_t* buf, int64_t i, int bits) {
  int per = 8 / bits;
  return (buf[i / per] >> (bits * (int)(i % per))) & ((1u << bits) - 1);
}

int orc_kivi_quant(const void* x, int dtype, int64_t layers, int64_t tokens, int64_t heads,
                   int64_t head_dim, int bits, int is_k, uint8_t* codes, float* scales,
                   float* mins) {
  if (bits != 2 && bits != 4) return -2;
  if (layers < 0 || tokens < 0 || heads < 0 || head_dim < 0 || head_dim % 32) return -4;
  if (is_k && tokens % 32) return -4;
  int64_t ng = is_k ? layers * (tokens / 32) * heads * head_dim
                    : layers * tokens * heads * (head_dim / 32);
  float* mx = (float*)malloc((size_t)(ng > 0 ? ng : 1) * sizeof(float));
  if (!mx) return -1;
  for (int64_t g = 0; g < ng; ++g) {
    mins[g] = INFINITY;
    mx[g] = -INFINITY;
  }
  for (int64_t l = 0; l < layers; ++l)
    for (int64_t t = 0; t < tokens; ++t)
      for (int64_t h = 0; h < heads; ++h)
        for (int64_t d = 0; d < head_dim; ++d) {
          int64_t i = ((l * tokens + t) * heads + h) * head_dim + d;
          int64_t g = kivi_group(is_k, tokens, heads, head_dim, l, t, h, d);
          float v = ld(x, dtype, i);
          mins[g] = fminf(mins[g], v);
          mx[g] = fmaxf(mx[g], v);
        }
  float qmax = (float)((1 << bits) - 1);
  for (int64_t g = 0; g < ng; ++g) {
    mins[g] = mins[g] + 0.0f; /* a zero minimum is +0, whichever zeros the group holds */
    scales[g] = fmaxf(mx[g] - mins[g], 1e-12f) / qmax;
  }
  free(mx);
  for (int64_t l = 0; l < layers; ++l)
    for (int64_t t = 0; t < tokens; ++t)
      for (int64_t h = 0; h < heads; ++h)
        for (int64_t d = 0; d < head_dim; ++d) {
          int64_t i = ((l * tokens + t) * heads + h) * head_dim + d;
          int64_t g = kivi_group(is_k, tokens, heads, head_dim, l, t, h, d);
          float q = clampf(rintf((ld(x, dtype, i) - mins[g]) / scales[g]), 0.0f, qmax);
          put_bits(codes, i, bits, (unsigned)q);
        }
  return 0;
}

int orc_kivi_dequant(const uint8_t* codes, const float* scales, const float* mins, int64_t layers,
                     int64_t tokens, int64_t heads, int64_t head_dim, int bits, int is_k,
                     int out_dtype, void* out) {
  if (bits != 2 && bits != 4) return -2;
  if (layers < 0 || tokens < 0 || heads < 0 || head_dim < 0 || head_dim % 32) return -4;
  if (is_k && tokens % 32) return -4;
  for (int64_t l = 0; l < layers; ++l)
    for (int64_t t = 0; t < tokens; ++t)
      for (int64_t h = 0; h < heads; ++h)
        for (int64_t d = 0; d < head_dim; ++d) {
          int64_t i = ((l * tokens + t) * heads + h) * head_dim + d;
          int64_t g = kivi_group(is_k, tokens, heads, head_dim, l, t, h, d);
          float prod = (float)get_bits(codes, i, bits) * scales[g];
          st(out, out_dtype, i, prod + mins[g]);
        }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Array forms of the codecs (for exhaustive tests)                          */
/* ------------------------------------------------------------------------ */

void orc_e4m3_encode_n(const float* y, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(y[i]);
}

void orc_e5m2_encode_n(const float* y, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e5m2_encode(y[i]);
}

void orc_e2m1_encode_n(const float* y, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e2m1_encode(y[i]);
}

void orc_bf16_round_n(const float* v, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_round(v[i]);
}
