// MXFP4 and NVFP4 quantize / dequantize kernels (E2M1 elements).
//
// MXFP4 (page "量化部署实战", section 伪量化实现): a 32-element block shares
// 2^X with X = floor(log2 max(amax, 1e-12)) - 2, stored as the E8M0 byte X+127.
// floor(log2 a) of a normal float is its unbiased exponent field.
// NVFP4 (same section): gs = max(amax_tensor, 1e-12) / (448*6); each 16-element
// block stores bs = E4M3(RN(RN(amax_block / 6) / gs)); elements are rounded
// against s = RN(max(dec(bs), 1e-12) * gs).
#include "launch.h"
#include "quant.h"

namespace pqb {
namespace {

template <typename T, int kUnr>
__global__ __launch_bounds__(kBlockThreads) void k_mxfp4(const T* __restrict__ x, int64_t nunits,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  __shared__ __align__(16) uint8_t lut[kE2M1LutSize];
  e2m1_lut_fill(lut, 0);
  __syncthreads();
  const int64_t nwaves = (int64_t)gridDim.x * (kBlockThreads / kWave);
  for (int64_t t0 = (int64_t)wave_index() * kUnr; t0 * kWave < nunits; t0 += nwaves * kUnr) {
    const int64_t u0 = t0 * kWave;
    if (u0 + kUnr * kWave <= nunits)
      mx_chunk<T, kUnr, false>(x, u0, nunits, codes, scales, lut);
    else
      mx_chunk<T, kUnr, true>(x, u0, nunits, codes, scales, lut);
  }
}

// Signed E2M1 values, nibble -> float.
__device__ __forceinline__ float e2m1_value(uint32_t nib) {
  const uint32_t m = nib & 7u;
  // m >= 2: 2^(m/2 - 1) * (1 + (m & 1) / 2); m == 1: 0.5; m == 0: 0
  uint32_t b = m >= 2u ? ((((m >> 1) + 126u) << 23) | ((m & 1u) << 22)) : (m ? 0x3F000000u : 0u);
  return as_f(b | ((nib & 8u) << 28));
}

template <bool kBf16Out>
__global__ __launch_bounds__(kBlockThreads) void k_mxfp4_dequant(const uint8_t* __restrict__ codes,
                                                                  const uint8_t* __restrict__ scales,
                                                                  int64_t nunits,
                                                                  void* __restrict__ out) {
  for (int64_t u = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x; u < nunits;
       u += (int64_t)gridDim.x * kBlockThreads) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(codes)[u];
    const float sc = as_f((uint32_t)scales[u >> 2] << 23);  // 2^(e - 127), e in [85, 252]
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = e2m1_value(w >> (4 * i)) * sc;
    store_out8<kBf16Out>(out, u, o);
  }
}

template <bool kBf16Out>
__global__ __launch_bounds__(kBlockThreads) void k_nvfp4_dequant(const uint8_t* __restrict__ codes,
                                                                  const uint8_t* __restrict__ scales,
                                                                  const float* __restrict__ gs,
                                                                  int64_t per_slice,
                                                                  void* __restrict__ out) {
  const int64_t b = blockIdx.y;
  const float g = gs[b];
  const int64_t nunits = per_slice / 8, u0 = b * nunits;
  for (int64_t u = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x; u < nunits;
       u += (int64_t)gridDim.x * kBlockThreads) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(codes)[u0 + u];
    const float s = fmaxf(e4m3_decode(scales[(u0 + u) >> 1]), 1e-12f) * g;
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = e2m1_value(w >> (4 * i)) * s;
    store_out8<kBf16Out>(out, u0 + u, o);
  }
}

// E2M1 nibble of each float (one byte per element).
__global__ __launch_bounds__(kBlockThreads) void k_encode_e2m1(const float* __restrict__ y,
                                                               int64_t n,
                                                               uint8_t* __restrict__ out) {
  __shared__ __align__(16) uint8_t lut[kE2M1LutSize];
  e2m1_lut_fill(lut, 0);
  __syncthreads();
  for (int64_t i = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kBlockThreads)
    out[i] = lut[e2m1_key(y[i])];
}

inline int grid_cap(int64_t work, int64_t per_block, int64_t cap) {
  int64_t g = (work + per_block - 1) / per_block;
  return (int)(g < 1 ? 1 : (g > cap ? cap : g));
}

}  // namespace

hipError_t launch_mxfp4(const void* x, bool bf16, int64_t n, uint8_t* codes, uint8_t* scales,
                        hipStream_t st) {
  // one chunk per wave (8 KiB of input: 8 tiles of bf16 or 4 of float32); the
  // table fill costs each workgroup two dword stores per thread and one barrier
  const int64_t nunits = n / 8, ntiles = (nunits + kWave - 1) / kWave;
  const int64_t waves = kBlockThreads / kWave;
  if (bf16)
    hipLaunchKernelGGL((k_mxfp4<uint16_t, 8>), dim3(grid_cap(ntiles, 8 * waves, 1 << 30)),
                       dim3(kBlockThreads), 0, st, (const uint16_t*)x, nunits, codes, scales);
  else
    hipLaunchKernelGGL((k_mxfp4<float, 4>), dim3(grid_cap(ntiles, 4 * waves, 1 << 30)),
                       dim3(kBlockThreads), 0, st, (const float*)x, nunits, codes, scales);
  return hipGetLastError();
}

hipError_t launch_mxfp4_dequant(const uint8_t* codes, const uint8_t* scales, int64_t n,
                                bool out_bf16, void* out, hipStream_t st) {
  const int64_t nunits = n / 8;
  const int grid = grid_cap(nunits, (int64_t)kBlockThreads * 4, 1 << 20);
  if (out_bf16)
    hipLaunchKernelGGL(k_mxfp4_dequant<true>, dim3(grid), dim3(kBlockThreads), 0, st, codes,
                       scales, nunits, out);
  else
    hipLaunchKernelGGL(k_mxfp4_dequant<false>, dim3(grid), dim3(kBlockThreads), 0, st, codes,
                       scales, nunits, out);
  return hipGetLastError();
}

hipError_t launch_nvfp4_dequant(const uint8_t* codes, const uint8_t* scales, const float* gs,
                                int64_t batch, int64_t per_slice, bool out_bf16, void* out,
                                hipStream_t st) {
  const int64_t nunits = per_slice / 8;
  const dim3 grid(grid_cap(nunits, (int64_t)kBlockThreads * 4, 8192), (unsigned)batch);
  if (out_bf16)
    hipLaunchKernelGGL(k_nvfp4_dequant<true>, grid, dim3(kBlockThreads), 0, st, codes, scales, gs,
                       per_slice, out);
  else
    hipLaunchKernelGGL(k_nvfp4_dequant<false>, grid, dim3(kBlockThreads), 0, st, codes, scales,
                       gs, per_slice, out);
  return hipGetLastError();
}

hipError_t launch_encode_e2m1(const float* y, int64_t n, uint8_t* out, hipStream_t st) {
  hipLaunchKernelGGL(k_encode_e2m1, dim3(grid_cap(n, kBlockThreads, 4096)), dim3(kBlockThreads),
                     0, st, y, n, out);
  return hipGetLastError();
}

}  // namespace pqb
