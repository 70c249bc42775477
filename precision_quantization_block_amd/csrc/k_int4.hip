// INT4 group-128 asymmetric quantize / dequantize kernels.
//
// Integers -8..7 with one scale and zero-point per 128 elements (page
// "量化部署实战", 格式速查); q = clamp(round(x / s) + z, qmin, qmax) ("LLM 推理
// 优化 · 量化 学习笔记" §5.1); the 2-byte scale per 128 ("14. 量化：让每一步搬
// 更少的字节", 量化在做什么).  The group range [lo, hi] is widened to hold 0, its
// 15 steps give s = bf16(max(hi - lo, 1e-12) / 15) (the rounded s is the one
// used), and z = -8 - rint(lo / s) puts lo on -8.
#include "device.h"
#include "launch.h"

namespace pqb {
namespace {

constexpr float kInv15 = 1.0f / 15.0f;

// A group of 128 is 16 lanes x 8 elements (one DPP row).  Zero-points are two
// per byte over the flat group index; group 2j (lanes 0-15 of a 32-lane half)
// and group 2j+1 (lanes 16-31) share byte j.
template <typename T, int kUnr>
__global__ __launch_bounds__(kBlockThreads) void k_int4(const T* __restrict__ x, int64_t nunits,
                                                         uint8_t* __restrict__ codes,
                                                         uint16_t* __restrict__ scales,
                                                         uint8_t* __restrict__ zeros) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = ((int64_t)blockIdx.x * kBlockThreads + threadIdx.x) / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * (kBlockThreads / kWave);
  const int64_t ntiles = (nunits + kWave - 1) / kWave;
  for (int64_t t0 = wave * kUnr; t0 < ntiles; t0 += nwaves * kUnr) {
    Raw8 raw[kUnr];
#pragma unroll
    for (int k = 0; k < kUnr; ++k) {
      const int64_t u = (t0 + k) * kWave + lane;
      raw[k] = u < nunits ? load_raw8(x + u * 8) : Raw8{};
    }
#pragma unroll
    for (int k = 0; k < kUnr; ++k) {
      const int64_t u = (t0 + k) * kWave + lane;
      float v[8];
      widen8(raw[k], x, v);
      float lo = fminf(fminf(fminf(v[0], v[1]), fminf(v[2], v[3])),
                       fminf(fminf(v[4], v[5]), fminf(v[6], v[7])));
      float hi = fmaxf(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])),
                       fmaxf(fmaxf(v[4], v[5]), fmaxf(v[6], v[7])));
      lo = group_min<16>(fminf(lo, 0.0f));
      hi = group_max<16>(fmaxf(hi, 0.0f));
      const float t = div_const(fmaxf(hi - lo, 1e-12f), 15.0f, kInv15);
      const uint32_t sb = bf16_rne_bits(t);
      const float s = as_f(sb << 16);
      const float y = 1.0f / s;
      // div_mag is odd-symmetric (every step commutes with negation), so it
      // gives RN(lo / s) and RN(x / s) for negative operands too.
      const float z = fminf(fmaxf(-8.0f - rintf(div_mag(lo, s, y)), -8.0f), 7.0f);
      const int zb = (int)z + 8;  // q + 8 lies in [0, 15]
      uint32_t w = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int q = (int)rintf(div_mag(v[i], s, y)) + zb;
        q = min(max(q, 0), 15);
        w |= (uint32_t)q << (4 * i);
      }
      w ^= 0x88888888u;  // offset binary -> two's-complement nibbles
      const int zn = ((int)z) & 15;
      const int zn_odd = __shfl_down(zn, 16);
      if (u < nunits) {
        st_nt4(reinterpret_cast<uint32_t*>(codes) + u, w);
        if ((lane & 15) == 0) scales[u >> 4] = (uint16_t)sb;
        if ((lane & 31) == 0)
          zeros[u >> 5] = (uint8_t)(zn | ((u + 16 < nunits ? zn_odd : 0) << 4));
      }
    }
  }
}


// (q - z) * s is exact in float32: |q - z| <= 15 and s has 8 significant bits.
template <bool kBf16Out>
__global__ __launch_bounds__(kBlockThreads) void k_int4_dequant(const uint8_t* __restrict__ codes,
                                                                 const uint16_t* __restrict__ scales,
                                                                 const uint8_t* __restrict__ zeros,
                                                                 int64_t nunits,
                                                                 void* __restrict__ out) {
  for (int64_t u = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x; u < nunits;
       u += (int64_t)gridDim.x * kBlockThreads) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(codes)[u];
    const int64_t g = u >> 4;
    const float s = as_f((uint32_t)scales[g] << 16);
    const int z = ((int)(zeros[g >> 1] >> (4 * (g & 1))) << 28) >> 28;  // sign-extend
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = ((int)(w >> (4 * i)) << 28) >> 28;
      o[i] = (float)(q - z) * s;
    }
    store_out8<kBf16Out>(out, u, o);
  }
}

inline int grid_for(int64_t work, int64_t per_block, int64_t cap) {
  int64_t g = (work + per_block - 1) / per_block;
  return (int)(g < 1 ? 1 : (g > cap ? cap : g));
}

}  // namespace

hipError_t launch_int4(const void* x, bool bf16, int64_t n, uint8_t* codes, uint16_t* scales,
                       uint8_t* zeros, hipStream_t st) {
  constexpr int kUnr = 4;
  const int64_t nunits = n / 8, ntiles = (nunits + kWave - 1) / kWave;
  const int grid = grid_for(ntiles, (int64_t)kUnr * (kBlockThreads / kWave), 1 << 30);
  if (bf16)
    hipLaunchKernelGGL((k_int4<uint16_t, kUnr>), dim3(grid), dim3(kBlockThreads), 0, st,
                       (const uint16_t*)x, nunits, codes, scales, zeros);
  else
    hipLaunchKernelGGL((k_int4<float, kUnr>), dim3(grid), dim3(kBlockThreads), 0, st,
                       (const float*)x, nunits, codes, scales, zeros);
  return hipGetLastError();
}

hipError_t launch_int4_dequant(const uint8_t* codes, const uint16_t* scales, const uint8_t* zeros,
                               int64_t n, bool out_bf16, void* out, hipStream_t st) {
  const int64_t nunits = n / 8;
  const int grid = grid_for(nunits, kBlockThreads, 1 << 20);
  if (out_bf16)
    hipLaunchKernelGGL(k_int4_dequant<true>, dim3(grid), dim3(kBlockThreads), 0, st, codes, scales,
                       zeros, nunits, out);
  else
    hipLaunchKernelGGL(k_int4_dequant<false>, dim3(grid), dim3(kBlockThreads), 0, st, codes,
                       scales, zeros, nunits, out);
  return hipGetLastError();
}

}  // namespace pqb
