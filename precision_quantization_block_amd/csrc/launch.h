// Internal launch interface between the C ABI (abi.hip) and the kernel files.
// Every launcher enqueues on `stream` and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pqb {

// Partial-maximum workspace for the two-pass (per-tensor) formats: P floats per
// (tensor, batch slice).  P depends only on the shape, so the size query and
// the launch agree.
int amax_partials_per_slice(int64_t batch, int64_t per_slice, int ntensors);

// Pass 1 of the two-pass formats: partials[(t * batch + b) * P + i] = amax of
// share i of slice b of tensor t.
hipError_t launch_amax_partials(const void* const* x, bool bf16, int ntensors, int64_t batch,
                                int64_t per_slice, float* partials, int P, hipStream_t st);

// ---- FP8 E4M3 -------------------------------------------------------------
// `elem`: 0 E4M3, 1 E5M2, 2 INT8 (the Elem kinds of quant.h).
hipError_t launch_fp8_1x128(const void* x, bool bf16, int64_t n, uint8_t* codes, float* scales,
                            hipStream_t st, int elem = 0);
hipError_t launch_fp8_128x128(const void* x, bool bf16, int64_t batch, int64_t rows,
                              int64_t cols, uint8_t* codes, float* scales, hipStream_t st,
                              int elem = 0);
hipError_t launch_fp8_row(const void* x, bool bf16, int64_t nrows, int64_t cols, uint8_t* codes,
                          float* scales, hipStream_t st, int elem = 0);
// Per-tensor over `ntensors` tensors (1, or 2 for K and V) of `batch` slices.
hipError_t launch_fp8_tensor(const void* const* x, bool bf16, int ntensors, int64_t batch,
                             int64_t per_slice, uint8_t* const* codes, float* const* scales,
                             float* partials, hipStream_t st, int elem = 0);
hipError_t launch_fp8_1x128_dequant(const uint8_t* codes, const float* scales, int64_t n,
                                    bool out_bf16, void* out, hipStream_t st, int elem = 0);
hipError_t launch_fp8_dequant(const uint8_t* codes, const float* scales, int gran, int64_t batch,
                              int64_t rows, int64_t cols, bool out_bf16, void* out,
                              hipStream_t st, int elem = 0);

// ---- MXFP4 / NVFP4 ----------------------------------------------------------
hipError_t launch_mxfp4(const void* x, bool bf16, int64_t n, uint8_t* codes, uint8_t* scales,
                        hipStream_t st);
hipError_t launch_mxfp8(const void* x, bool bf16, int64_t n, uint8_t* codes, uint8_t* scales,
                        hipStream_t st);
hipError_t launch_mxfp8_dequant(const uint8_t* codes, const uint8_t* scales, int64_t n,
                                bool out_bf16, void* out, hipStream_t st);
hipError_t launch_mxfp4_dequant(const uint8_t* codes, const uint8_t* scales, int64_t n,
                                bool out_bf16, void* out, hipStream_t st);
hipError_t launch_nvfp4(const void* x, bool bf16, int64_t batch, int64_t per_slice,
                        uint8_t* codes, uint8_t* scales, float* gs, float* ws, hipStream_t st);
hipError_t launch_nvfp4_dequant(const uint8_t* codes, const uint8_t* scales, const float* gs,
                                int64_t batch, int64_t per_slice, bool out_bf16, void* out,
                                hipStream_t st);

// ---- INT4 group-128 asymmetric --------------------------------------------
hipError_t launch_int4(const void* x, bool bf16, int64_t n, uint8_t* codes, uint16_t* scales,
                       uint8_t* zeros, hipStream_t st);
hipError_t launch_int4_dequant(const uint8_t* codes, const uint16_t* scales, const uint8_t* zeros,
                               int64_t n, bool out_bf16, void* out, hipStream_t st);

// ---- fused multi-tensor launch ----------------------------------------------
// Jobs of the one-pass formats, fused into launches of up to kMaxBatchJobs
// (one family per launch; a family's jobs are split as evenly as possible).
constexpr int kMaxBatchJobs = 72;
enum MultiKind { kMultiFp8Blk = 0, kMultiFp8Tile = 1, kMultiMx = 2, kMultiInt4 = 3, kMultiMx8 = 4 };
struct MultiJob {
  const void* x;
  uint8_t* codes;
  void* scales;
  uint8_t* aux;
  int64_t batch, rows, cols;
  int kind;
  bool bf16;
  int elem;  // FP8 kinds: kE4M3 or kE5M2
};
// Launches the fused jobs take, or -1 if one of them would exceed the grid
// limit of 2^32 - 1 threads (launch_multi then enqueues nothing and returns
// hipErrorInvalidConfiguration).
int64_t multi_launches(const MultiJob* jobs, int njobs);
hipError_t launch_multi(const MultiJob* jobs, int njobs, hipStream_t st);

// ---- fused multi-tensor dequantization (k_dequant.hip) ---------------------
// Flat formats only: FP8 E4M3 / E5M2 1x128, MXFP4, MXFP8, one NVFP4 slice
// (aux = its tensor scale), INT4 (aux = zero-points); n = elements / 8.
enum DqKind { kDqFp8 = 0, kDqE5m2 = 1, kDqMx4 = 2, kDqMx8 = 3, kDqNv = 4, kDqInt4 = 5 };
struct DqMultiJob {
  const uint8_t* codes;
  const void* scales;
  const void* aux;
  void* out;
  int64_t nunits;
  int kind;
  bool bf16_out;
};
// Launches the jobs take, or -1 if one would exceed 2^32 - 1 threads
// (launch_dq_multi then enqueues nothing and returns hipErrorInvalidConfiguration).
int64_t dq_multi_launches(const DqMultiJob* jobs, int njobs);
hipError_t launch_dq_multi(const DqMultiJob* jobs, int njobs, hipStream_t st);

// ---- two-pass formats (k_twopass.hip) -------------------------------------
// Chunked pass 1 -> finalize -> pass 2 for slices whose length is a multiple
// of 8.  Workspace: twopass_workspace_bytes(); contents on entry do not matter.
size_t twopass_workspace_bytes(int ntensors, int64_t slices, int64_t per_slice, int64_t groups,
                               bool nv);
hipError_t launch_tensor_fp8(const void* const* x, bool bf16, int ntensors, int64_t slices,
                             int64_t per_slice, uint8_t* const* codes, float* const* scales,
                             float* ws, hipStream_t st, int elem = 0);

// FP8 KV-cache write with a scale mode per tensor: x is [layers, tokens, heads,
// head_dim]; scales [layers] (LAYER; STATIC: read) or [layers, heads] (HEAD).
enum KvMode { kKvLayer = 0, kKvHead = 1, kKvStatic = 2 };
constexpr int kMaxKvHeads = 256;
struct KvTensor {
  const void* x;
  uint8_t* codes;
  float* scales;
  int mode;
};
size_t kv_workspace_bytes(int64_t layers, int64_t tokens, int64_t heads, int64_t head_dim);
hipError_t launch_kv_fp8(const KvTensor* t, int ntensors, bool bf16, int64_t layers,
                         int64_t tokens, int64_t heads, int64_t head_dim, float* ws,
                         hipStream_t st);

// KIVI-style 2- or 4-bit KV quantization: x is [layers, tokens, heads,
// head_dim]; K groups are 32 tokens of one channel (tokens % 32 == 0), V
// groups 32 channels of one token (head_dim % 32 == 0).  Codes pack element i
// at bits b * (i % (8 / b)); scales and mins are float32, K [layers, tokens /
// 32, heads, head_dim], V [n / 32].
hipError_t launch_kivi_k(const void* x, bool bf16, int64_t layers, int64_t tokens, int64_t heads,
                         int64_t head_dim, int bits, uint8_t* codes, float* scales, float* mins,
                         hipStream_t st);
hipError_t launch_kivi_v(const void* x, bool bf16, int64_t n, int bits, uint8_t* codes,
                         float* scales, float* mins, hipStream_t st);
hipError_t launch_kivi_k_dequant(const uint8_t* codes, const float* scales, const float* mins,
                                 int64_t layers, int64_t tokens, int64_t heads, int64_t head_dim,
                                 int bits, bool out_bf16, void* out, hipStream_t st);
hipError_t launch_kivi_v_dequant(const uint8_t* codes, const float* scales, const float* mins,
                                 int64_t n, int bits, bool out_bf16, void* out, hipStream_t st);

// Block-scaled FP8 GEMM: C [M, N] = A [M, K] x B [N, K]^T with 1x128 scales on A
// and 128x128 scales on B, promoted per 128-deep K block; K % 128 == 0,
// N % 128 == 0.  out: 0 float32, 1 bf16, 2 FP8 E4M3 codes [M, N] with 1x128
// scales c_scales [M, N / 128] (c_scales unused otherwise).
hipError_t launch_gemm_fp8_bs(const uint8_t* a, const float* a_scales, const uint8_t* b,
                              const float* b_scales, int64_t M, int64_t N, int64_t K, int out,
                              void* c, float* c_scales, hipStream_t st);

// MXFP4 x MXFP4 product C [M, N] = dequant(A [M, K]) x dequant(B [N, K])^T on the
// block-scaled matrix cores; MXFP4 layout (codes [rows, K/2], E8M0 scales
// [rows, K/32]); K % 128 == 0, N % 128 == 0.
hipError_t launch_gemm_mxfp4(const uint8_t* a, const uint8_t* a_scales, const uint8_t* b,
                             const uint8_t* b_scales, int64_t M, int64_t N, int64_t K,
                             bool out_bf16, void* c, hipStream_t st);
// Streaming reference: reads read_bytes, writes read_bytes / reads_per_write.
hipError_t launch_stream_ref(const void* src, int64_t read_bytes, int reads_per_write,
                             int tiles_per_wave, void* dst, hipStream_t st);
hipError_t launch_gemm_nvfp4(const uint8_t* a, const uint8_t* a_scales, const float* a_gs,
                             const uint8_t* b, const uint8_t* b_scales, const float* b_gs, int64_t M,
                             int64_t N, int64_t K, bool out_bf16, void* c, hipStream_t st);

// W4A16 products y [M, N] = x [M, K] (bf16) x dequant(W)^T for INT4 group-128
// asymmetric weights W [N, K] (codes, bf16 scales, zero-point nibbles); all
// jobs of a call share M (1 <= M <= 8); K % 128 == 0; N * K / 128 < 2^31.
struct W4Job {
  const uint16_t* x;
  const uint8_t* codes;
  const uint16_t* scales;
  const uint8_t* zeros;
  void* y;
  int32_t N, K;
};
constexpr int kW4MaxJobs = 32;
struct W4Args {
  int32_t njobs;
  int32_t wg_begin[kW4MaxJobs + 1];
  W4Job job[kW4MaxJobs];
};
hipError_t launch_w4a16(const W4Job* jobs, int njobs, int M, bool out_bf16, hipStream_t st);
// The same products on the matrix cores for any M >= 1 (launched in slices of
// 32 activation rows).
hipError_t launch_w4a16_mfma(const W4Job* jobs, int njobs, int64_t M, bool out_bf16,
                             hipStream_t st);

// ---- division checks (k_check.hip) -----------------------------------------
hipError_t launch_check_recip(uint32_t first, int64_t n, float* out, hipStream_t st);
hipError_t launch_check_div(const float* s, int64_t ns, uint32_t x_first, int64_t nx, float* out,
                            hipStream_t st);

// ---- element codecs ---------------------------------------------------------
hipError_t launch_encode_elem(const float* y, int64_t n, uint8_t* out, hipStream_t st, int elem);
hipError_t launch_encode_e2m1(const float* y, int64_t n, uint8_t* out, hipStream_t st);

}  // namespace pqb
