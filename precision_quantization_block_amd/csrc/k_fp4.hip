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

// ---------------------------------------------------------------------------
// NVFP4 pass 2 (pass 1 is the shared amax-partials kernel): 2 lanes x 8
// elements per block.  Each workgroup rebuilds gs, the E2M1 table and, for all
// 127 finite block-scale codes, the element scale s and RN(1/s) in LDS.
// ---------------------------------------------------------------------------
struct __align__(16) NvTables {
  uint8_t lut[kE2M1LutSize];
  float se[128], ye[128];
  uint32_t red[kBlockThreads / kWave];
};

template <typename T, int kUnr, bool kGuard>
__device__ __forceinline__ void nv_chunk(const T* __restrict__ xs, int64_t u0, int64_t nunits,
                                         uint8_t* __restrict__ cs, uint8_t* __restrict__ ss,
                                         float gs, float ygs, const NvTables& tb) {
  const int lane = threadIdx.x & (kWave - 1);
  const T* xb = xs + u0 * 8;
  Raw8 raw[kUnr];
#pragma unroll
  for (int k = 0; k < kUnr; ++k)
    raw[k] = (!kGuard || u0 + k * kWave + lane < nunits) ? load_raw8(xb + (k * kWave + lane) * 8)
                                                           : Raw8{};
#pragma unroll
  for (int k = 0; k < kUnr; ++k) {
    float v[8];
    widen8(raw[k], xs, v);
    const float ab = as_f(group_umax<2>(as_u(absmax8(v))));
    const float bq = div_rn(div_const(ab, 6.0f, kInv6), gs, ygs);  // <= 448 (1 + 2^-22)
    const uint32_t bs = cvt_e4m3x2<false>(bq, 0.0f, 0u) & 0x7Fu;     // bq >= 0
    const float s = tb.se[bs], ys = tb.ye[bs];
    uint32_t w = 0;
    if (s < 2.0f && s >= 0x1p-60f) {
      // Here every nonzero x has a nonzero RN(x / s) (|x / s| > 2^-150), so its
      // nibble carries the sign of x even when the magnitude is 0: with -0.0
      // mapped to +0 first, a quotient of -0 stands for "negative, rounds to
      // zero" and the table's key 1024 holds nibble 8.
#pragma unroll
      for (int i = 0; i < 8; ++i)
        w |= (uint32_t)tb.lut[e2m1_key(div_rn(v[i] + 0.0f, s, ys))] << (4 * i);
    } else {
      // IEEE division; a -0 quotient has sign(y) = 0, so it becomes +0 first.
#pragma unroll
      for (int i = 0; i < 8; ++i) w |= (uint32_t)tb.lut[e2m1_key(v[i] / s + 0.0f)] << (4 * i);
    }
    const int64_t u = u0 + k * kWave + lane;
    if (!kGuard || u < nunits) {
      st_nt4(cs + u * 4, w);
      if ((lane & 1) == 0) ss[u >> 1] = (uint8_t)bs;
    }
  }
}

template <typename T, int kUnr>
__global__ __launch_bounds__(kBlockThreads) void k_nvfp4_quant(const T* __restrict__ x,
                                                                int64_t per_slice,
                                                                uint8_t* __restrict__ codes,
                                                                uint8_t* __restrict__ scales,
                                                                float* __restrict__ gs_out,
                                                                const float* __restrict__ partials,
                                                                int P) {
  __shared__ NvTables tb;
  const int64_t b = blockIdx.y;
  uint32_t m = 0;
  for (int i = threadIdx.x; i < P; i += kBlockThreads) m = max(m, as_u(partials[b * P + i]));
  m = wave_umax(m);
  if ((threadIdx.x & (kWave - 1)) == 0) tb.red[threadIdx.x / kWave] = m;
  e2m1_lut_fill(tb.lut, 8);
  __syncthreads();
  m = max(max(tb.red[0], tb.red[1]), max(tb.red[2], tb.red[3]));
  const float gs = as_f(max(m, kAmaxFloorBits)) / 2688.0f;  // 448 * 6
  const float ygs = recip_rn(gs);
  for (int c = threadIdx.x; c < 127; c += kBlockThreads) {
    const float sc = fmaxf(e4m3_decode((uint32_t)c), 1e-12f) * gs;
    tb.se[c] = sc;
    tb.ye[c] = 1.0f / sc;
  }
  __syncthreads();
  if (blockIdx.x == 0 && threadIdx.x == 0) gs_out[b] = gs;

  const T* xs = x + b * per_slice;
  uint8_t* cs = codes + b * (per_slice / 2);
  uint8_t* ss = scales + b * (per_slice / 16);
  const int64_t nunits = per_slice / 8;
  const int64_t nwaves = (int64_t)gridDim.x * (kBlockThreads / kWave);
  for (int64_t t0 = (int64_t)wave_index() * kUnr; t0 * kWave < nunits; t0 += nwaves * kUnr) {
    const int64_t u0 = t0 * kWave;
    if (u0 + kUnr * kWave <= nunits)
      nv_chunk<T, kUnr, false>(xs, u0, nunits, cs, ss, gs, ygs, tb);
    else
      nv_chunk<T, kUnr, true>(xs, u0, nunits, cs, ss, gs, ygs, tb);
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

// Workgroups for the NVFP4 pass-2 kernel, which rebuilds gs, the E2M1 table
// and the 127-entry scale tables per workgroup: enough to fill the chip, few
// enough that each one amortizes its tables over many tiles.
constexpr int64_t kTableKernelCap = 256 * 8;

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

hipError_t launch_nvfp4(const void* x, bool bf16, int64_t batch, int64_t per_slice,
                        uint8_t* codes, uint8_t* scales, float* gs, float* partials,
                        hipStream_t st) {
  constexpr int kUnr = 2;
  const int P = amax_partials_per_slice(batch, per_slice, 1);
  const void* xs[1] = {x};
  hipError_t e = launch_amax_partials(xs, bf16, 1, batch, per_slice, partials, P, st);
  if (e != hipSuccess) return e;
  const int64_t nunits = per_slice / 8, ntiles = (nunits + kWave - 1) / kWave;
  int64_t cap = kTableKernelCap / (batch > 0 ? batch : 1);
  if (cap < 1) cap = 1;
  const int gx = grid_cap(ntiles, (int64_t)kUnr * (kBlockThreads / kWave), cap);
  const dim3 grid(gx, (unsigned)batch);
  if (bf16)
    hipLaunchKernelGGL((k_nvfp4_quant<uint16_t, kUnr>), grid, dim3(kBlockThreads), 0, st,
                       (const uint16_t*)x, per_slice, codes, scales, gs, partials, P);
  else
    hipLaunchKernelGGL((k_nvfp4_quant<float, kUnr>), grid, dim3(kBlockThreads), 0, st,
                       (const float*)x, per_slice, codes, scales, gs, partials, P);
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
