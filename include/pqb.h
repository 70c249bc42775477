/*
 * pqb -- block-scaled quantize-pack / dequantize engine for MI355X (gfx950).
 *
 * C ABI.  Every pointer named x, codes, scales, aux, out, k, v, workspace is a
 * device pointer owned by the caller; the library never allocates, frees or
 * synchronizes.  Every call enqueues its kernels on `stream` (a hipStream_t,
 * NULL for the default stream) and returns at once; results are ready when
 * the stream reaches that point.  Calls are thread-safe: apart from the fixed
 * scratch of pqb_quantize_noalloc, the library keeps no mutable global state.
 *
 * Formats and the passages that define them (page title, section):
 *   "量化部署实战" (quantization deployment in practice), section 伪量化实现
 *   (fake-quant implementation): FP8 E4M3 with per-tensor, per-row and
 *   block (128x128 or 1x128) scales, each scale max(amax, 1e-12)/448;
 *   MXFP4 (32-element blocks, scale 2^(floor(log2 max(amax,1e-12)) - 2));
 *   NVFP4 (16-element blocks, E4M3 block scale of (amax_block/6)/gs with tensor
 *   scale gs = max(amax_tensor, 1e-12)/(448*6)); the FP8 KV cache that
 *   quantizes K and V per tensor on every write.  Same page, 格式速查 (format
 *   table): INT4 integers -8..7 with one scale (+ zero-point) per 128.
 *   "14. 量化：让每一步搬更少的字节", section 量化在做什么: the uniform
 *   quantizer q = round(x/s) and its 2-byte scale per 128 weights.
 *   "LLM 推理优化 · 量化（Quantization）系统学习笔记" §5.1: asymmetric
 *   q = clamp(round(x/s) + z, qmin, qmax); §4.2 and §4.5: FP8 E5M2 (max 57344)
 *   and MXFP8 (32-element blocks, E8M0 scale, E4M3 elements).  "14. 量化：让
 *   每一步搬更少的字节", 量化在做什么 and the low-precision float table:
 *   symmetric INT8 with s = max|x| / 127, and E5M2's largest value 57344.
 *
 * Arithmetic: IEEE binary32 with round-to-nearest-even and subnormals; bf16
 * inputs are widened exactly.  Every quotient x/s is the correctly rounded
 * one.  Element rounding: E4M3 round-to-nearest-even after the clamp to +-448;
 * E5M2 round-to-nearest-even (max 57344); E2M1 to the nearest of {0, .5, 1,
 * 1.5, 2, 3, 4, 6} with ties to the smaller magnitude, sign bit set for negative
 * values (so -0.0 gives +0); INT4 q = clamp(rint(x/s) + z, -8, 7); INT8
 * q = clamp(rint(x/s), -128, 127).  Inputs must be finite.
 *
 * Shapes.  A tensor is [batch, rows, cols], contiguous and row-major.
 * "Per tensor" (FP8 TENSOR, the NVFP4 tensor scale) means per batch slice.
 *
 * Valid (format, granularity) pairs and the layouts they produce:
 *   FP8_E4M3 x TENSOR     codes u8 [b, r, c]      scales f32 [b]
 *   FP8_E4M3 x ROW        codes u8 [b, r, c]      scales f32 [b, r]
 *   FP8_E4M3 x BLK_1x128  codes u8 [b, r, c]      scales f32 [b, r, c/128]
 *   FP8_E4M3 x BLK_128x128 codes u8 [b, r, c]     scales f32 [b, r/br, c/128],
 *                                                 br = min(128, r)
 *   FP8_E5M2 x the same four scopes, same layouts; s = max(amax, 1e-12)/57344
 *   INT8_SYM x TENSOR / ROW: codes i8 [b, r, c], scales f32 [b] / [b, r];
 *                                                 s = max(amax, 1e-12)/127
 *   MXFP8 x BLK_32        codes u8 E4M3 [b, r, c] scales u8 E8M0 [b, r, c/32]
 *                                                 (X + 127, X = floor(log2
 *                                                 max(amax,1e-12)) - 8; codes
 *                                                 E4M3(clamp(x/2^X, +-448)))
 *   MXFP4 x BLK_32        codes u8 [b, r, c/2]    scales u8 E8M0 [b, r, c/32]
 *                                                 (exponent + 127)
 *   NVFP4 x BLK_16        codes u8 [b, r, c/2]    scales u8 E4M3 [b, r, c/16]
 *                                                 aux f32 tensor scale [b]
 *   INT4_ASYM x GRP_128   codes u8 [b, r, c/2]    scales bf16 [b, r, c/128]
 *                                                 aux u8 zero-points, two per
 *                                                 byte over the flat group
 *                                                 index (ceil(b*r*c/256) bytes)
 * 4-bit codes: element 2i in the low nibble of byte i.  INT4 codes and
 * zero-points are two's-complement nibbles; dequant is (q - z) * s.  INT4
 * also needs each group's range max(0, max x) - min(0, min x) to be finite in
 * float32 (values of both signs beyond about +-1.7e38 in one group overflow
 * it); such a group's codes, scale and zero-point are unspecified, and no
 * other group is affected.
 *
 * Shape rules: 1x128 and GRP_128 need c % 128 == 0; 128x128 needs c % 128 == 0
 * and r <= 128 or r % 128 == 0; BLK_32 needs c % 32 == 0; BLK_16 needs
 * c % 16 == 0; ROW needs b * r <= 4 * (2^32 - 1) / 256 (one wave per row).
 * An empty tensor (b*r*c == 0) is accepted and launches nothing.
 *
 * Alignment: x, codes and out must be 16-byte aligned; scales and aux 4-byte
 * aligned (2-byte for INT4 scales, 1 for byte scales and zero-points);
 * workspace 16-byte aligned.
 *
 * Errors: host-detectable problems return a negative status before anything
 * is enqueued.  A failed launch returns PQB_ERR_HIP.  Faults inside a kernel
 * surface at the caller's next synchronization.
 */
#ifndef PQB_H
#define PQB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PQB_ABI_VERSION 1

typedef enum pqb_status {
  PQB_OK = 0,
  PQB_ERR_NULL = -1,      /* a required pointer is NULL */
  PQB_ERR_ENUM = -2,      /* unknown dtype, format or granularity */
  PQB_ERR_COMBO = -3,     /* format and granularity do not go together */
  PQB_ERR_SHAPE = -4,     /* negative size, or a shape the block rules reject */
  PQB_ERR_ALIGN = -5,     /* a pointer breaks the alignment rules */
  PQB_ERR_WORKSPACE = -6, /* workspace smaller than pqb_query_sizes asks */
  PQB_ERR_HIP = -7,       /* the HIP runtime refused a launch */
  PQB_ERR_SCRATCH = -8    /* pqb_quantize_noalloc: needs more than its fixed scratch */
} pqb_status;

typedef enum pqb_dtype { PQB_F32 = 0, PQB_BF16 = 1 } pqb_dtype;

typedef enum pqb_format {
  PQB_FP8_E4M3 = 0,
  PQB_MXFP4 = 1,
  PQB_NVFP4 = 2,
  PQB_INT4_ASYM = 3,
  PQB_FP8_E5M2 = 4,
  PQB_MXFP8 = 5,
  PQB_INT8_SYM = 6
} pqb_format;

typedef enum pqb_gran {
  PQB_TENSOR = 0,
  PQB_ROW = 1,
  PQB_BLK_1x128 = 2,
  PQB_BLK_128x128 = 3,
  PQB_BLK_32 = 4,
  PQB_BLK_16 = 5,
  PQB_GRP_128 = 6
} pqb_gran;

/* Byte sizes of the buffers a (format, granularity, shape) needs.  `aux` is 0
 * when unused; `workspace` is the scratch that pqb_quantize needs (0 for the
 * one-pass formats).  Sizes do not depend on the input dtype. */
typedef struct pqb_sizes {
  size_t codes, scales, aux, workspace;
} pqb_sizes;

pqb_status pqb_query_sizes(pqb_format fmt, pqb_gran gran, int64_t batch, int64_t rows,
                           int64_t cols, pqb_sizes* out);

/* Quantize x ([batch, rows, cols] of `dtype`) into codes, scales and aux with
 * the layouts above.  The two-pass formats (FP8 TENSOR, NVFP4) first reduce the
 * per-tensor amax into `workspace` (at least pqb_query_sizes().workspace
 * bytes; its contents on entry do not matter and are overwritten). */
pqb_status pqb_quantize(const void* x, pqb_dtype dtype, int64_t batch, int64_t rows, int64_t cols,
                        pqb_format fmt, pqb_gran gran, void* codes, void* scales, void* aux,
                        void* workspace, size_t workspace_bytes, void* stream);

/* pqb_quantize for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments and results without `workspace`.  The two-pass formats
 * (FP8 / E5M2 / INT8 TENSOR, NVFP4) use instead a scratch array of
 * PQB_NOALLOC_SCRATCH_BYTES (1 MiB) that the library holds on each GPU it runs
 * on until the process ends; its address is looked up once per device, on the
 * first call with that device current.  The call allocates and frees nothing
 * (no hipMalloc, no allocating library routine).  A shape whose workspace
 * (pqb_query_sizes) exceeds the scratch returns PQB_ERR_SCRATCH before
 * anything is enqueued: e.g. one per-tensor slice of up to 2^31 - 8192 elements
 * fits.
 * `stream` must belong to the current device (else PQB_ERR_HIP, before
 * anything is enqueued).  Every call on one GPU shares
 * that GPU's scratch, and each call overwrites what it uses before reading it:
 * calls that overlap on one GPU (other streams, other host threads) race, so
 * order them.  Every other rule and error is pqb_quantize's. */
#define PQB_NOALLOC_SCRATCH_BYTES (1u << 20)
pqb_status pqb_quantize_noalloc(const void* x, pqb_dtype dtype, int64_t batch, int64_t rows,
                                int64_t cols, pqb_format fmt, pqb_gran gran, void* codes,
                                void* scales, void* aux, void* stream);

/* One tensor of a fused batch: the arguments of one pqb_quantize call. */
typedef struct pqb_job {
  const void* x;    /* input [batch, rows, cols] of `dtype` */
  void* codes;      /* outputs, laid out as for pqb_quantize */
  void* scales;
  void* aux;        /* INT4 zero-points; NULL for the other formats */
  int64_t batch, rows, cols;
  int32_t dtype;    /* pqb_dtype */
  int32_t fmt;      /* pqb_format */
  int32_t gran;     /* pqb_gran */
  int32_t reserved; /* must be 0 (else PQB_ERR_ENUM) */
} pqb_job;

/* Quantize several tensors with as few launches as possible: jobs of one
 * family share fused launches of up to 72 jobs each (FP8 E4M3/E5M2 1x128 and
 * 128x128 together; MXFP4 with MXFP8; INT4), a family's jobs split as evenly
 * as possible over its launches; per-row jobs (FP8, INT8) get a launch each.
 * Each job's outputs are exactly those of pqb_quantize on the same arguments.
 * Only the one-pass pairs qualify; a per-tensor job (FP8, INT8) or an NVFP4
 * job returns PQB_ERR_COMBO.  Every job is validated (same rules and codes as
 * pqb_quantize) and every launch is planned before anything is enqueued; a
 * launch that would exceed the grid limit of 2^32 - 1 threads returns
 * PQB_ERR_SHAPE.  Outputs of different jobs must not overlap each other or any
 * input.  `jobs` is a host array and may be reused once the call returns. */
pqb_status pqb_quantize_batch(const pqb_job* jobs, int64_t njobs, void* stream);

/* The number of kernel launches pqb_quantize_batch makes for these jobs
 * (after the same validation; no GPU work), or a negative pqb_status. */
int64_t pqb_quantize_batch_launches(const pqb_job* jobs, int64_t njobs);

/* Inverse of pqb_quantize: out[b, r, c] = decoded code times its scale(s),
 * as float32 or rounded to bf16 (round-to-nearest-even) by `out_dtype`.
 * FP8 (E4M3, E5M2): dec(code) * s.  INT8: q * s.  MXFP4: +-V * 2^(e8m0 - 127)
 * and MXFP8: dec(code) * 2^(e8m0 - 127) (both exact).  NVFP4:
 * +-V * (max(dec(block scale), 1e-12) * gs).  INT4: (q - z) * s (exact). */
pqb_status pqb_dequantize(const void* codes, const void* scales, const void* aux, pqb_format fmt,
                          pqb_gran gran, int64_t batch, int64_t rows, int64_t cols,
                          pqb_dtype out_dtype, void* out, void* stream);

/* One tensor of a fused dequantization batch: the arguments of one
 * pqb_dequantize call. */
typedef struct pqb_dq_job {
  const void* codes;  /* codes, scales and aux as pqb_quantize wrote them */
  const void* scales;
  const void* aux;    /* INT4 zero-points or NVFP4 tensor scales; NULL otherwise */
  void* out;          /* [batch, rows, cols] of out_dtype */
  int64_t batch, rows, cols;
  int32_t fmt;        /* pqb_format */
  int32_t gran;       /* pqb_gran */
  int32_t out_dtype;  /* pqb_dtype */
  int32_t reserved;   /* must be 0 (else PQB_ERR_ENUM) */
} pqb_dq_job;

/* Dequantize several tensors with as few launches as possible: FP8 E4M3 / E5M2
 * 1x128, MXFP4, MXFP8, NVFP4 (each batch slice counts as one job) and INT4
 * jobs share fused launches of up to 72 jobs, one kernel per output dtype;
 * the other scopes (FP8 / E5M2 / INT8 per tensor and per row, FP8 128x128)
 * get a pqb_dequantize launch each.  Each job's output is exactly that of
 * pqb_dequantize on the same arguments.  Every job is validated (same rules
 * and codes as pqb_dequantize) and the fused launches are planned before
 * anything is enqueued; a launch that would exceed 2^32 - 1 threads returns
 * PQB_ERR_SHAPE.  Outputs must not overlap each other or any input.  `jobs`
 * is a host array and may be reused once the call returns. */
pqb_status pqb_dequantize_batch(const pqb_dq_job* jobs, int64_t njobs, void* stream);

/* FP8 KV-cache write: K and V are [layers, elems_per_layer] of `dtype`.  Each
 * (layer, K) and (layer, V) slice gets its own per-tensor FP8 scale (written
 * to k_scales[layer], v_scales[layer]) and its E4M3 codes (k_codes, v_codes,
 * same layout as the input).  Workspace: pqb_kv_workspace_bytes(). */
size_t pqb_kv_workspace_bytes(int64_t layers, int64_t elems_per_layer);
pqb_status pqb_kv_write_fp8(const void* k, const void* v, pqb_dtype dtype, int64_t layers,
                            int64_t elems_per_layer, uint8_t* k_codes, uint8_t* v_codes,
                            float* k_scales, float* v_scales, void* workspace,
                            size_t workspace_bytes, void* stream);

/* FP8 KV-cache write with a scale mode chosen for K and for V separately
 * (page "量化部署实战", section KV Cache 量化：误差要和信号比: K and V get
 * independent quantizers; per_head takes the amax over the token and head_dim
 * axes; calibrated scales computed offline are recommended for deployment).
 *
 * K and V are [layers, tokens, heads, head_dim] of `dtype`, token-major (the
 * layout of a paged cache); codes have the same layout, one byte each.
 *   PQB_KV_LAYER   one dynamic scale per layer: scales [layers] (written);
 *                  identical to pqb_kv_write_fp8.
 *   PQB_KV_HEAD    one dynamic scale per (layer, head) over tokens x head_dim:
 *                  scales [layers, heads] (written).
 *   PQB_KV_STATIC  a given scale per layer (calibrated offline): scales
 *                  [layers] are READ; codes are E4M3(clamp(x / s, -448, 448)),
 *                  where the clamp can bind.  Each s must lie in [2^-64, 2^126)
 *                  (results for other s are unspecified).
 * Dynamic scales are max(amax, 1e-12) / 448.  Pass k = NULL (or v = NULL) to
 * write only the other; its codes and scales pointers are then ignored.
 * Shape rules: head_dim % 8 == 0; for PQB_KV_HEAD also heads <= 256 and
 * heads * (head_dim / 8)^2 < 2^32 (any head_dim up to 32760 with 256 heads).
 * Workspace (only when a dynamic mode is used): pqb_kv_workspace_bytes_ex(),
 * 16-byte aligned.  Alignment: k, v and codes 16 bytes, scales 4 bytes.
 * Errors: PQB_ERR_ENUM for an unknown dtype or mode, PQB_ERR_SHAPE for shapes
 * breaking the rules above, PQB_ERR_NULL if both k and v are NULL or a needed
 * pointer is NULL, PQB_ERR_WORKSPACE, PQB_ERR_ALIGN; all before any launch. */
typedef enum pqb_kv_mode { PQB_KV_LAYER = 0, PQB_KV_HEAD = 1, PQB_KV_STATIC = 2 } pqb_kv_mode;
size_t pqb_kv_workspace_bytes_ex(int64_t layers, int64_t tokens, int64_t heads, int64_t head_dim);
pqb_status pqb_kv_write_fp8_ex(const void* k, const void* v, pqb_dtype dtype, int64_t layers,
                               int64_t tokens, int64_t heads, int64_t head_dim,
                               pqb_kv_mode k_mode, pqb_kv_mode v_mode, uint8_t* k_codes,
                               uint8_t* v_codes, float* k_scales, float* v_scales,
                               void* workspace, size_t workspace_bytes, void* stream);

/* KIVI-style 2- or 4-bit KV cache (page "量化部署实战", section KV Cache 量化:
 * K carries a per-channel bias, so per-channel scales with a zero-point suit
 * it; page "14. 量化：让每一步搬更少的字节", 路线三: KIVI quantizes K per
 * channel and V per token, at 2 bits).
 *
 * K and V are [layers, tokens, heads, head_dim] of `dtype`, token-major.  The
 * quantizer is asymmetric over groups of 32: a K group is 32 consecutive
 * tokens of one (layer, head, channel), a V group 32 consecutive channels of
 * one (layer, token, head).  For a group with minimum m (a zero minimum is
 * stored as +0) and maximum M, in float32 with round-to-nearest-even:
 *   s = max(M - m, 1e-12) / (2^bits - 1),
 *   q = clamp(rint((x - m) / s), 0, 2^bits - 1)   (the quotient correctly rounded),
 *   dequantized x = q * s + m                      (product and sum rounded separately;
 *                                                   then bf16 RNE for a bf16 output).
 * Layouts: codes u8 [n * bits / 8] over the flat element index
 * i = ((layer * tokens + token) * heads + head) * head_dim + channel, element i
 * at bits bits * (i % (8 / bits)) of byte i * bits / 8; K scales and mins f32
 * [layers, tokens / 32, heads, head_dim]; V scales and mins f32 [layers, tokens,
 * heads, head_dim / 32].
 * pqb_kv_write_kivi quantizes k and v; pqb_kv_read_kivi dequantizes codes,
 * scales and mins back into k_out and v_out (same layout as the input, of
 * out_dtype).  Pass NULL for k (k_codes for the read) to handle V only, or for
 * v (v_codes) to handle K only; that tensor's other pointers are then ignored.
 * Shape rules: bits is 2 or 4; head_dim % 32 == 0; tokens % 32 == 0 when K is
 * handled; layers * tokens * heads * head_dim < 2^36.  Inputs must be finite
 * and each group's range M - m below the float32 overflow threshold.
 * Alignment: k, v, codes, scales, mins and outputs 16 bytes.
 * Errors, all before any launch: PQB_ERR_ENUM for an unknown dtype or bits,
 * PQB_ERR_SHAPE for shapes breaking the rules above, PQB_ERR_NULL if both
 * tensors are NULL or a needed pointer is NULL, PQB_ERR_ALIGN. */
pqb_status pqb_kv_write_kivi(const void* k, const void* v, pqb_dtype dtype, int64_t layers,
                             int64_t tokens, int64_t heads, int64_t head_dim, int bits,
                             uint8_t* k_codes, uint8_t* v_codes, float* k_scales, float* k_mins,
                             float* v_scales, float* v_mins, void* stream);
pqb_status pqb_kv_read_kivi(const uint8_t* k_codes, const uint8_t* v_codes,
                            const float* k_scales, const float* k_mins, const float* v_scales,
                            const float* v_mins, int64_t layers, int64_t tokens, int64_t heads,
                            int64_t head_dim, int bits, pqb_dtype out_dtype, void* k_out,
                            void* v_out, void* stream);

/* Block-scaled FP8 GEMM, the consumer of the codes above (page "量化部署实战",
 * exercise section on FP8 blockwise scaling: within each 128-deep block of K
 * the FP8 products are summed on the matrix cores, the block sum is multiplied
 * by that block's activation and weight scales, and the result is accumulated
 * in float32):
 *   C[m, n] = sum_kb RN(a_scales[m, kb] * b_scales[n / 128, kb]) * P[m, n, kb],
 *   P[m, n, kb] = sum over the block of dec(a[m, k]) * dec(b[n, k]),
 * one fused multiply-add per block into a float32 accumulator (bf16 output is
 * its RNE rounding).  P is formed by the matrix core in float32; the
 * evaluation error against exact arithmetic is at most about (130 + K/128)
 * * 2^-24 * sum_kb |sA sB| sum_k |dec(a) dec(b)|.
 * a: E4M3 codes [M, K] with a_scales f32 [M, K/128] (the FP8 BLK_1x128 layout
 * of a [1, M, K] tensor); b: E4M3 codes [N, K] with b_scales f32 [N/128, K/128]
 * (the BLK_128x128 layout of a [1, N, K] weight); c: [M, N] row-major of
 * out_dtype.  Shape rules: K % 128 == 0, N % 128 == 0, M, N, K < 2^31 and
 * ceil(M/128) * (N/128) < 2^31; M = 0 or N = 0 does nothing; K = 0 writes zeros.
 * Codes must not be NaN (0x7F, 0xFF), as the quantizers never write them.
 * Alignment: a, b and c 16 bytes, scales 4 bytes.  Errors, before any launch:
 * PQB_ERR_ENUM (out_dtype), PQB_ERR_SHAPE, PQB_ERR_NULL, PQB_ERR_ALIGN. */
pqb_status pqb_gemm_fp8_blockscaled(const uint8_t* a, const float* a_scales, const uint8_t* b,
                                    const float* b_scales, int64_t m, int64_t n, int64_t k,
                                    pqb_dtype out_dtype, void* c, void* stream);

/* The same GEMM with the next layer's activation quantization fused into its
 * epilogue (same page and section: the (1, 128) activation scales should be
 * computed at the end of the kernel that produces the activations, so that
 * the activations are not written and read back once more).  The float32
 * accumulators C[m, n] (as pqb_gemm_fp8_blockscaled computes them) are
 * quantized like pqb_quantize FP8_E4M3 x BLK_1x128 of a [1, M, N] tensor:
 * c_scales[m, j] = max(amax over C[m, 128 j .. 128 j + 127], 1e-12) / 448,
 * c_codes[m, n] = E4M3(clamp(C[m, n] / c_scales[m, n / 128], -448, 448)).
 * c_codes u8 [M, N] (16-byte aligned), c_scales f32 [M, N/128] (4-byte
 * aligned).  Shape rules and errors as for pqb_gemm_fp8_blockscaled; a NULL
 * c_scales is PQB_ERR_NULL. */
pqb_status pqb_gemm_fp8_blockscaled_quant(const uint8_t* a, const float* a_scales,
                                          const uint8_t* b, const float* b_scales, int64_t m,
                                          int64_t n, int64_t k, uint8_t* c_codes,
                                          float* c_scales, void* stream);

/* MXFP4 x MXFP4 product on the block-scaled matrix cores (page "LLM 推理优化
 * · 量化学习笔记" §4.5: MXFP4 is 32-element blocks sharing one E8M0 scale, the
 * format FP4 tensor cores consume directly):
 *   C[m, n] = sum_k dec(a[m, k]) 2^(sa[m, k/32] - 127) dec(b[n, k]) 2^(sb[n, k/32] - 127).
 * a, b: E2M1 codes [m, k/2] and [n, k/2] (element 2i in the low nibble of
 * byte i), sa, sb: E8M0 scales [m, k/32] and [n, k/32], exactly as
 * pqb_quantize writes MXFP4 x BLK_32 for [1, m, k] and [1, n, k]; c: [m, n]
 * row-major of out_dtype.  The matrix core applies the scales; products of
 * two E2M1 values sum exactly in groups of 8, and the float32 additions
 * bound the error by about (17 + k/128) * 2^-24 * sum_k |a| |b|.  Shape
 * rules: k % 128 == 0, n % 128 == 0, m, n, k < 2^31; m = 0 or n = 0 does
 * nothing; k = 0 writes zeros.  Alignment: a, b and c 16 bytes, scales 4.
 * Errors, before any launch: PQB_ERR_ENUM, PQB_ERR_SHAPE, PQB_ERR_NULL,
 * PQB_ERR_ALIGN. */
pqb_status pqb_gemm_mxfp4(const uint8_t* a, const uint8_t* a_scales, const uint8_t* b,
                          const uint8_t* b_scales, int64_t m, int64_t n, int64_t k,
                          pqb_dtype out_dtype, void* c, void* stream);

/* NVFP4 x NVFP4 product on the matrix cores (page "14. 量化：让每一步搬更少的
 * 字节", section 新一代低位格式：FP8、FP4 与微缩放: FP4 matrix units take
 * NVFP4 operands; page "量化部署实战", 格式速查, NVFP4 row: 16-element blocks,
 * one E4M3 scale each, and a float32 scale per tensor):
 *   C[m, n] = g * sum_k (V(a[m, k]) dec(sa[m, k/16])) (V(b[n, k]) dec(sb[n, k/16])),
 *   g = float32(a_gs[0] * b_gs[0]),
 * with V the E2M1 value of a nibble and dec the E4M3 value of a scale byte,
 * so a block whose scale code is 0 contributes 0.  a, b: E2M1 codes [m, k/2]
 * and [n, k/2] (element 2i in the low nibble of byte i); sa, sb: E4M3 scales
 * [m, k/16] and [n, k/16]; a_gs, b_gs: one float32 each in device memory;
 * exactly what pqb_quantize writes for NVFP4 x BLK_16 of [1, m, k] and
 * [1, n, k].  Scale bytes are read without their sign bit and must not be
 * 0x7F (NaN), as the quantizer never writes either.  c: [m, n] row-major of
 * out_dtype.  Each scaled element V dec(s) is exact in f16, the products are
 * exact, and the float32 sums bound the error against exact arithmetic by
 * about (34 + k/32) * 2^-24 * g * sum_k |V dec(sa)| |V dec(sb)|, plus half an
 * ulp of the result (float32, or bf16 for bf16 output).  Shape rules: k % 128 == 0,
 * n % 128 == 0, m, n, k < 2^31; m = 0 or n = 0 does nothing; k = 0 writes
 * zeros (and reads neither scale).  Alignment: a, b and c 16 bytes, scales and
 * tensor scales 4.  Errors, before any launch: PQB_ERR_ENUM, PQB_ERR_SHAPE,
 * PQB_ERR_NULL, PQB_ERR_ALIGN. */
pqb_status pqb_gemm_nvfp4(const uint8_t* a, const uint8_t* a_scales, const float* a_gs,
                          const uint8_t* b, const uint8_t* b_scales, const float* b_gs, int64_t m,
                          int64_t n, int64_t k, pqb_dtype out_dtype, void* c, void* stream);

/* W4A16 product, the consumer of the INT4 group-128 codes (page "14. 量化：让
 * 每一步搬更少的字节", 路线一: 4-bit weights read from memory, unpacked and
 * dequantized to 16 bits, then multiplied):
 *   y[m, n] = sum_k x[m, k] * (q[n, k] - z[n, k/128]) * s[n, k/128].
 * x: bf16 activations [m, k] (decode batch, 1 <= m <= 8); codes / scales /
 * zeros: the INT4_ASYM x GRP_128 layout pqb_quantize writes for a [1, n, k]
 * weight (codes u8 [n, k/2], bf16 scales [n, k/128], zero-point nibbles over
 * the flat group index); y: [m, n] row-major of out_dtype.  Evaluated in
 * float32: per 32 weights of one group, s * (sum x w - (136 + z) * sum x)
 * with w = 136 + q as exact bf16 products summed in float32, then a sum over
 * the units; the error against exact arithmetic is at most about
 * (40 + k/2048) * 2^-24 * sum_k |s| |x| (|136 + q| + |136 + z|).
 * Shape rules: k % 128 == 0, m <= 8, n * (k/128) < 2^31, k < 2^31; m = 0 or
 * n = 0 does nothing; k = 0 writes zeros.  Alignment: x and codes 16 bytes,
 * scales 2, y 4.
 * Errors, before any launch: PQB_ERR_ENUM (out_dtype), PQB_ERR_SHAPE,
 * PQB_ERR_NULL, PQB_ERR_ALIGN. */
pqb_status pqb_gemv_w4a16(const void* x, int64_t m, const uint8_t* codes, const void* scales,
                          const uint8_t* zeros, int64_t n, int64_t k, pqb_dtype out_dtype,
                          void* y, void* stream);

/* Several W4A16 products in as few launches as possible (up to 32 per
 * launch), e.g. the projections of a layer that share their input.  Each job
 * is one pqb_gemv_w4a16 call (same rules); all jobs share m and out_dtype.
 * Every job is validated before anything is enqueued.  `jobs` is a host array
 * and may be reused once the call returns; outputs must not overlap. */
typedef struct pqb_w4a16_job {
  const void* x;        /* bf16 [m, k] */
  const uint8_t* codes; /* INT4 group-128 weight [n, k] */
  const void* scales;
  const uint8_t* zeros;
  void* y;              /* [m, n] of out_dtype */
  int64_t n, k;
} pqb_w4a16_job;
pqb_status pqb_gemv_w4a16_batch(const pqb_w4a16_job* jobs, int64_t njobs, int64_t m,
                                pqb_dtype out_dtype, void* stream);

/* The W4A16 product of pqb_gemv_w4a16 on the matrix cores, for any number of
 * activation rows (decode batches and prefill chunks alike; the activations
 * are taken 32 rows per launch and the weight is read once per 32 rows):
 *   y[m, n] = sum_k x[m, k] * (q[n, k] - z[n, k/128]) * s[n, k/128],
 * same layouts, ownership and alignment as pqb_gemv_w4a16, and m >= 0 with
 * m < 2^31.  Evaluated in float32: for each group of 128, s * (P - (136 + z)
 * * S), where P = sum x w with w = 136 + q and S = sum x are matrix-core
 * float32 accumulations of exact bf16 products (32 per instruction), then a
 * sum over the groups of each of four partial sums and a sum of the four;
 * the error against exact arithmetic is at most about
 * (256 + k/64) * 2^-24 * sum_k |s| |x| (|136 + q| + |136 + z|).
 * Shape rules as pqb_gemv_w4a16 without the bound on m; m = 0 or n = 0 does
 * nothing; k = 0 writes zeros.  On Llama-3.1-8B-shaped weights it is the
 * faster of the two from m = 4; at m = 1 pqb_gemv_w4a16 is.
 * Errors, before any launch: PQB_ERR_ENUM (out_dtype), PQB_ERR_SHAPE,
 * PQB_ERR_NULL, PQB_ERR_ALIGN. */
pqb_status pqb_gemm_w4a16(const void* x, int64_t m, const uint8_t* codes, const void* scales,
                          const uint8_t* zeros, int64_t n, int64_t k, pqb_dtype out_dtype,
                          void* y, void* stream);
/* Several such products in as few launches as possible (up to 32 jobs per
 * launch and 32 activation rows): the job list of pqb_gemv_w4a16_batch, with
 * any m >= 0. */
pqb_status pqb_gemm_w4a16_batch(const pqb_w4a16_job* jobs, int64_t njobs, int64_t m,
                                pqb_dtype out_dtype, void* stream);

/* Element codecs exposed for testing the rounding rules on arrays of float32:
 * E4M3 of y (round-to-nearest-even; |y| must not exceed 464) into one byte
 * per element; E2M1 of y (ties to the smaller magnitude, saturating at 6)
 * into one nibble per byte (low 4 bits). */
pqb_status pqb_encode_e4m3(const float* y, int64_t n, uint8_t* out, void* stream);
/* E5M2 of y (round-to-nearest-even; |y| must not exceed 57344) into one byte
 * per element. */
pqb_status pqb_encode_e5m2(const float* y, int64_t n, uint8_t* out, void* stream);
pqb_status pqb_encode_e2m1(const float* y, int64_t n, uint8_t* out, void* stream);

/* The engine's division routines on generated arguments, exposed for testing
 * them against IEEE division over whole ranges of floats (every quantizer
 * code above rests on x / s being the correctly rounded quotient; page
 * "量化部署实战", section 伪量化实现, divides by the scale before rounding).
 * pqb_check_recip: out[i] = the engine's RN(1 / s) for s = the float whose
 *   bit pattern is first_bits + i, i < n; needs first_bits + n <= 2^32.
 * pqb_check_div: out[j * nx + i] = the engine's RN(x / s[j]) for x = the
 *   float whose bit pattern is x_first_bits + i, i < nx, j < ns, formed as the
 *   quantizers form it (from y = RN(1 / s[j]) and one correction); needs
 *   x_first_bits + nx <= 2^32.
 * s and out are device arrays (4-byte aligned) of ns and n (ns * nx) floats.
 * Errors, before any launch: PQB_ERR_SHAPE, PQB_ERR_NULL, PQB_ERR_ALIGN. */
pqb_status pqb_check_recip(uint32_t first_bits, int64_t n, float* out, void* stream);
pqb_status pqb_check_div(const float* s, int64_t ns, uint32_t x_first_bits, int64_t nx,
                         float* out, void* stream);

/* Measurement reference, not a quantizer: the memory pattern of the
 * quantizers with nothing computed, so that their bandwidth can be set beside
 * what the same loads and stores reach at the same read:write mix.  Reads
 * read_bytes from src and writes read_bytes / reads_per_write to dst, in
 * chunks of T = tiles_per_wave tiles of 1 KiB per wave: output tile j of chunk
 * c (at dst + c * 1024 * T / reads_per_write + 1024 j) is the bytewise XOR of
 * the chunk's source tiles reads_per_write * j .. reads_per_write * (j + 1) -
 * 1, loaded and stored 16 bytes per lane with non-temporal hints as the
 * quantizers' bf16 loads and code stores are.  reads_per_write is 1, 2 or 4;
 * tiles_per_wave 4 or 8 (the quantizers take 8); read_bytes a multiple of
 * 8192, at most 2^38; src and dst 16-byte aligned device buffers that do not
 * overlap.  Errors, before any launch: PQB_ERR_ENUM, PQB_ERR_SHAPE,
 * PQB_ERR_NULL, PQB_ERR_ALIGN. */
pqb_status pqb_stream_reference(const void* src, int64_t read_bytes, int reads_per_write,
                                int tiles_per_wave, void* dst, void* stream);

const char* pqb_status_string(pqb_status s);
int pqb_abi_version(void);
/* A digest of the sources the library was built from (16 hex digits; the
 * build computes it over csrc/ and this header), so that a loader can refuse
 * a library that no longer matches its sources. */
const char* pqb_source_hash(void);

#ifdef __cplusplus
}
#endif
#endif /* PQB_H */
