// INT4 group-128 asymmetric quantize / dequantize kernels.
//
// Integers -8..7 with one scale and zero-point per 128 elements (page
// "量化部署实战", 格式速查); q = clamp(round(x / s) + z, qmin, qmax) ("LLM 推理
// 优化 · 量化 学习笔记" §5.1); the 2-byte scale per 128 ("14. 量化：让每一步搬
// 更少的字节", 量化在做什么).  The group range [lo, hi] is widened to hold 0, its
// 15 steps give s = bf16(max(hi - lo, 1e-12) / 15) (the rounded s is the one
// used), and z = -8 - rint(lo / s) puts lo on -8.
#include "launch.h"
#include "quant.h"

namespace pqb {
namespace {

template <typename T, int kUnr>
__global__ __launch_bounds__(kBlockThreads) void k_int4(const T* __restrict__ x, int64_t nunits,
                                                         uint8_t* __restrict__ codes,
                                                         uint16_t* __restrict__ scales,
                                                         uint8_t* __restrict__ zeros) {
  const int64_t nwaves = (int64_t)gridDim.x * (kBlockThreads / kWave);
  for (int64_t t0 = (int64_t)wave_index() * kUnr; t0 * kWave < nunits; t0 += nwaves * kUnr) {
    const int64_t u0 = t0 * kWave;
    if (u0 + kUnr * kWave <= nunits)
      int4_chunk<T, kUnr, false>(x, u0, nunits, codes, scales, zeros);
    else
      int4_chunk<T, kUnr, true>(x, u0, nunits, codes, scales, zeros);
  }
}

inline int grid_for(int64_t work, int64_t per_block, int64_t cap) {
  int64_t g = (work + per_block - 1) / per_block;
  return (int)(g < 1 ? 1 : (g > cap ? cap : g));
}

}  // namespace

hipError_t launch_int4(const void* x, bool bf16, int64_t n, uint8_t* codes, uint16_t* scales,
                       uint8_t* zeros, hipStream_t st) {
  // one chunk per wave: 8 tiles of bf16 or 4 of float32 (8 KiB of input)
  const int64_t nunits = n / 8, ntiles = (nunits + kWave - 1) / kWave;
  const int64_t waves = kBlockThreads / kWave;
  if (bf16)
    hipLaunchKernelGGL((k_int4<uint16_t, 8>), dim3(grid_for(ntiles, 8 * waves, 1 << 30)),
                       dim3(kBlockThreads), 0, st, (const uint16_t*)x, nunits, codes, scales, zeros);
  else
    hipLaunchKernelGGL((k_int4<float, 4>), dim3(grid_for(ntiles, 4 * waves, 1 << 30)),
                       dim3(kBlockThreads), 0, st, (const float*)x, nunits, codes, scales, zeros);
  return hipGetLastError();
}

}  // namespace pqb
