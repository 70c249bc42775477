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
  const int64_t nwaves = (int64_t)gridDim.x * (kBlockThreads / kWave);
  int64_t t0 = (int64_t)wave_index() * kUnr;
  // The first chunk's loads go out before the table fill and its barrier
  // (a small tensor is one chunk per wave: 5.7 -> 5.2 us for 12.6 MB).
  const int64_t u0 = t0 * kWave;
  const bool have = u0 < nunits, full = u0 + kUnr * kWave <= nunits;
  Raw8 raw[kUnr];
  if (have) {
    if (full)
      load_chunk<T, kUnr, false>(x, u0, nunits, raw);
    else
      load_chunk<T, kUnr, true>(x, u0, nunits, raw);
  }
  e2m1_lut_fill(lut, 0);
  __syncthreads();
  if (have) {
    if (full)
      mx_pack<T, kUnr, false>(x, raw, u0, nunits, codes, scales, lut);
    else
      mx_pack<T, kUnr, true>(x, raw, u0, nunits, codes, scales, lut);
  }
  for (t0 += nwaves * kUnr; t0 * kWave < nunits; t0 += nwaves * kUnr) {
    const int64_t u1 = t0 * kWave;
    if (u1 + kUnr * kWave <= nunits)
      mx_chunk<T, kUnr, false>(x, u1, nunits, codes, scales, lut);
    else
      mx_chunk<T, kUnr, true>(x, u1, nunits, codes, scales, lut);
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

// MXFP8: one chunk of 8 bf16 (4 float32) tiles per wave.
template <typename T, int kUnr>
__global__ __launch_bounds__(kBlockThreads) void k_mxfp8(const T* __restrict__ x, int64_t nunits,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int64_t u0 = ((int64_t)blockIdx.x * (kBlockThreads / kWave) + wave) * kUnr * kWave;
  if (u0 >= nunits) return;
  if (u0 + kUnr * kWave <= nunits)
    mx8_chunk<T, kUnr, false>(x, u0, nunits, codes, scales);
  else
    mx8_chunk<T, kUnr, true>(x, u0, nunits, codes, scales);
}

}  // namespace

hipError_t launch_mxfp4(const void* x, bool bf16, int64_t n, uint8_t* codes, uint8_t* scales,
                        hipStream_t st) {
  // one chunk of 4 tiles per wave (4 KiB of bf16 or 8 KiB of float32 input;
  // with the first chunk's loads ahead of the table fill, 4 bf16 tiles beat 8
  // by 4-5% from 117 MB to 1 GiB in a same-process A/B); one tile per wave
  // when 4-tile chunks would give fewer than 4096 waves, so that a small
  // tensor spreads over more waves (float32 [3072, 1024]: 5.5 -> 5.0 us;
  // 16M elements and up: equal)
  const int64_t nunits = n / 8, ntiles = (nunits + kWave - 1) / kWave;
  const int64_t waves = kBlockThreads / kWave;
  const bool small = (ntiles + 3) / 4 < 4096;
  if (bf16) {
    if (small)
      hipLaunchKernelGGL((k_mxfp4<uint16_t, 1>), dim3(grid_cap(ntiles, waves, 1 << 30)),
                         dim3(kBlockThreads), 0, st, (const uint16_t*)x, nunits, codes, scales);
    else
      hipLaunchKernelGGL((k_mxfp4<uint16_t, 4>), dim3(grid_cap(ntiles, 4 * waves, 1 << 30)),
                         dim3(kBlockThreads), 0, st, (const uint16_t*)x, nunits, codes, scales);
  } else {
    if (small)
      hipLaunchKernelGGL((k_mxfp4<float, 1>), dim3(grid_cap(ntiles, waves, 1 << 30)),
                         dim3(kBlockThreads), 0, st, (const float*)x, nunits, codes, scales);
    else
      hipLaunchKernelGGL((k_mxfp4<float, 4>), dim3(grid_cap(ntiles, 4 * waves, 1 << 30)),
                         dim3(kBlockThreads), 0, st, (const float*)x, nunits, codes, scales);
  }
  return hipGetLastError();
}

hipError_t launch_mxfp8(const void* x, bool bf16, int64_t n, uint8_t* codes, uint8_t* scales,
                        hipStream_t st) {
  const int64_t nunits = n / 8, ntiles = (nunits + kWave - 1) / kWave;
  const int64_t waves = kBlockThreads / kWave;
  if (bf16)
    hipLaunchKernelGGL((k_mxfp8<uint16_t, 8>), dim3(grid_cap(ntiles, 8 * waves, 1 << 30)),
                       dim3(kBlockThreads), 0, st, (const uint16_t*)x, nunits, codes, scales);
  else
    hipLaunchKernelGGL((k_mxfp8<float, 4>), dim3(grid_cap(ntiles, 4 * waves, 1 << 30)),
                       dim3(kBlockThreads), 0, st, (const float*)x, nunits, codes, scales);
  return hipGetLastError();
}

hipError_t launch_encode_e2m1(const float* y, int64_t n, uint8_t* out, hipStream_t st) {
  hipLaunchKernelGGL(k_encode_e2m1, dim3(grid_cap(n, kBlockThreads, 4096)), dim3(kBlockThreads),
                     0, st, y, n, out);
  return hipGetLastError();
}

}  // namespace pqb
