// FP8 E4M3 quantize kernels: 1x128 blocks, 128x128 tiles, rows, per tensor.
//
// Scale of a scope: s = RN(max(amax, 1e-12) / 448); codes are E4M3(RN(x / s))
// (the page "量化部署实战", section 伪量化实现).  The clamp to +-448 that the
// page applies before the cast never binds: |x| <= amax gives |x/s| <= 448 up
// to one rounding, which still rounds to 448.
#include "device.h"
#include "launch.h"

namespace pqb {
namespace {

constexpr float kInv448 = 1.0f / 448.0f;  // RN(1/448), folded at compile time

__device__ __forceinline__ float fp8_scale(float amax) {
  return div_const(fmaxf(amax, 1e-12f), 448.0f, kInv448);
}

// RN(x / s) with the sign of x (E4M3 keeps the sign of every quotient).
__device__ __forceinline__ float fp8_quot(float x, float s, float y) {
  return with_sign_of(div_mag(fabsf(x), s, y), x);
}

// Quantize eight values with scale s (and y = RN(1/s)); two code dwords.
__device__ __forceinline__ uint2 fp8_pack8(const float v[8], float s, float y) {
  uint32_t w0 = e4m3_bytes4(fp8_quot(v[0], s, y), fp8_quot(v[1], s, y), fp8_quot(v[2], s, y),
                            fp8_quot(v[3], s, y));
  uint32_t w1 = e4m3_bytes4(fp8_quot(v[4], s, y), fp8_quot(v[5], s, y), fp8_quot(v[6], s, y),
                            fp8_quot(v[7], s, y));
  return make_uint2(w0, w1);
}

__device__ __forceinline__ void store_codes8(uint8_t* p, uint2 w) { st_nt8(p, w.x, w.y); }

// ---------------------------------------------------------------------------
// 1x128: a 128-element block is 16 lanes x 8 elements, one DPP row.  Each wave
// walks kUnr consecutive tiles of 64 units (8 elements each) per iteration.
// ---------------------------------------------------------------------------
template <typename T, int kUnr>
__global__ __launch_bounds__(kBlockThreads) void k_fp8_1x128(const T* __restrict__ x,
                                                              int64_t nunits,
                                                              uint8_t* __restrict__ codes,
                                                              float* __restrict__ scales) {
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
      const float s = fp8_scale(group_max<16>(absmax8(v)));
      const float y = 1.0f / s;
      const uint2 w = fp8_pack8(v, s, y);
      if (u < nunits) {
        store_codes8(codes + u * 8, w);
        if ((lane & 15) == 0) scales[u >> 4] = s;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 128x128 (br x 128 with br = min(128, rows)): one workgroup per tile.  Lane l
// of wave w covers unit (l % 16) of tile rows w*4 + l/16 + 16k, k < 8; the
// tile's amax is reduced through DPP, a cross-row shuffle and LDS.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kBlockThreads) void k_fp8_128x128(const T* __restrict__ x,
                                                                int64_t rows, int64_t cols,
                                                                int br,
                                                                uint8_t* __restrict__ codes,
                                                                float* __restrict__ scales) {
  __shared__ float red[kBlockThreads / kWave];
  const int64_t tiles_c = cols / 128, tiles_r = rows / br;
  const int64_t t = blockIdx.x;
  const int64_t tc = t % tiles_c, trb = t / tiles_c;  // trb = b * tiles_r + tr
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int r0 = wave * 4 + (lane >> 4);
  const int64_t base = trb * br * cols + tc * 128 + (lane & 15) * 8;  // rows of a slice are
                                                                      // contiguous across b
  Raw8 raw[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int r = r0 + 16 * k;
    raw[k] = r < br ? load_raw8(x + base + (int64_t)r * cols) : Raw8{};
  }
  float v[8][8];
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    widen8(raw[k], x, v[k]);
    m = fmaxf(m, absmax8(v[k]));
  }
  m = wave_max(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = fp8_scale(m);
  const float y = 1.0f / s;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int r = r0 + 16 * k;
    const uint2 w = fp8_pack8(v[k], s, y);
    if (r < br) store_codes8(codes + base + (int64_t)r * cols, w);
  }
  if (threadIdx.x == 0) scales[t] = s;
}

// ---------------------------------------------------------------------------
// Per row, vector path (cols % 8 == 0, cols <= 512 * kMaxU): one wave per row,
// the row stays in registers between the reduction and the quantization.
// ---------------------------------------------------------------------------
template <typename T, int kMaxU>
__global__ __launch_bounds__(kBlockThreads) void k_fp8_row_vec(const T* __restrict__ x,
                                                                int64_t nrows, int64_t cols,
                                                                uint8_t* __restrict__ codes,
                                                                float* __restrict__ scales) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * (kBlockThreads / kWave) + threadIdx.x / kWave;
  if (row >= nrows) return;  // whole wave leaves together
  const int64_t upr = cols / 8;
  const T* xr = x + row * cols;
  Raw8 raw[kMaxU];
#pragma unroll
  for (int k = 0; k < kMaxU; ++k) {
    const int64_t u = (int64_t)k * kWave + lane;
    raw[k] = u < upr ? load_raw8(xr + u * 8) : Raw8{};
  }
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < kMaxU; ++k) {
    float v[8];
    widen8(raw[k], x, v);
    m = fmaxf(m, absmax8(v));
  }
  m = wave_max(m);
  const float s = fp8_scale(m);
  const float y = 1.0f / s;
#pragma unroll
  for (int k = 0; k < kMaxU; ++k) {
    const int64_t u = (int64_t)k * kWave + lane;
    float v[8];
    widen8(raw[k], x, v);
    const uint2 w = fp8_pack8(v, s, y);
    if (u < upr) store_codes8(codes + row * cols + u * 8, w);
  }
  if (lane == 0) scales[row] = s;
}

// Per row, any width: one wave per row, element-wise, reading the row twice
// (the second read is served by the caches).
template <typename T>
__device__ __forceinline__ float ld1(const T* p);
template <>
__device__ __forceinline__ float ld1<uint16_t>(const uint16_t* p) {
  return as_f((uint32_t)*p << 16);
}
template <>
__device__ __forceinline__ float ld1<float>(const float* p) {
  return *p;
}

__device__ __forceinline__ uint8_t e4m3_byte(float q) {
  return (uint8_t)(cvt_e4m3x2<false>(q, 0.0f, 0u) & 0xFFu);
}

template <typename T>
__global__ __launch_bounds__(kBlockThreads) void k_fp8_row_any(const T* __restrict__ x,
                                                                int64_t nrows, int64_t cols,
                                                                uint8_t* __restrict__ codes,
                                                                float* __restrict__ scales) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * (kBlockThreads / kWave) + threadIdx.x / kWave;
  if (row >= nrows) return;
  const T* xr = x + row * cols;
  float m = 0.0f;
  for (int64_t c = lane; c < cols; c += kWave) m = fmaxf(m, fabsf(ld1(xr + c)));
  m = wave_max(m);
  const float s = fp8_scale(m);
  const float y = 1.0f / s;
  for (int64_t c = lane; c < cols; c += kWave) codes[row * cols + c] = e4m3_byte(fp8_quot(ld1(xr + c), s, y));
  if (lane == 0) scales[row] = s;
}

// ---------------------------------------------------------------------------
// Per tensor (per batch slice), two passes.  Pass 1: each workgroup writes the
// amax of its share of a slice to partials[(tensor * batch + b) * P + blockIdx.x].
// Pass 2: each workgroup reduces the slice's P partials, forms s and quantizes
// its share.  blockIdx.y = slice, blockIdx.z = tensor (K or V for the KV write).
// ---------------------------------------------------------------------------
struct TensorArgs {
  const void* x[2];
  uint8_t* codes[2];
  float* scales[2];
};

__device__ __forceinline__ float block_max(float m, float* red) {
  m = wave_max(m);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return m;
}

template <typename T, bool kVec>
__global__ __launch_bounds__(kBlockThreads) void k_amax_partial(TensorArgs a, int64_t per_slice,
                                                                 float* __restrict__ partials) {
  __shared__ float red[kBlockThreads / kWave];
  const int64_t b = blockIdx.y, P = gridDim.x;
  const T* xs = reinterpret_cast<const T*>(a.x[blockIdx.z]) + b * per_slice;
  float m = 0.0f;
  if constexpr (kVec) {
    const int64_t nunits = per_slice / 8;
    const int64_t stride = P * kBlockThreads;
    int64_t u = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x;
    for (; u + 3 * stride < nunits; u += 4 * stride) {
      Raw8 r0 = load_raw8(xs + u * 8), r1 = load_raw8(xs + (u + stride) * 8);
      Raw8 r2 = load_raw8(xs + (u + 2 * stride) * 8), r3 = load_raw8(xs + (u + 3 * stride) * 8);
      float v[8];
      widen8(r0, xs, v); m = fmaxf(m, absmax8(v));
      widen8(r1, xs, v); m = fmaxf(m, absmax8(v));
      widen8(r2, xs, v); m = fmaxf(m, absmax8(v));
      widen8(r3, xs, v); m = fmaxf(m, absmax8(v));
    }
    for (; u < nunits; u += stride) {
      float v[8];
      widen8(load_raw8(xs + u * 8), xs, v);
      m = fmaxf(m, absmax8(v));
    }
  } else {
    for (int64_t i = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x; i < per_slice;
         i += P * kBlockThreads)
      m = fmaxf(m, fabsf(ld1(xs + i)));
  }
  m = block_max(m, red);
  if (threadIdx.x == 0) partials[((int64_t)blockIdx.z * gridDim.y + b) * P + blockIdx.x] = m;
}

// Reduce the P partials of one slice (all threads receive the maximum).
__device__ __forceinline__ float reduce_partials(const float* __restrict__ p, int P, float* red) {
  float m = 0.0f;
  for (int i = threadIdx.x; i < P; i += kBlockThreads) m = fmaxf(m, p[i]);
  return block_max(m, red);
}

template <typename T, bool kVec>
__global__ __launch_bounds__(kBlockThreads) void k_fp8_tensor_quant(TensorArgs a,
                                                                     int64_t per_slice,
                                                                     const float* __restrict__ partials,
                                                                     int P) {
  __shared__ float red[kBlockThreads / kWave];
  const int64_t b = blockIdx.y;
  const int tz = blockIdx.z;
  const float m = reduce_partials(partials + ((int64_t)tz * gridDim.y + b) * P, P, red);
  const float s = fp8_scale(m);
  const float y = 1.0f / s;
  const T* xs = reinterpret_cast<const T*>(a.x[tz]) + b * per_slice;
  uint8_t* cs = a.codes[tz] + b * per_slice;
  const int64_t stride = (int64_t)gridDim.x * kBlockThreads;
  if constexpr (kVec) {
    const int64_t nunits = per_slice / 8;
    int64_t u = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x;
    for (; u + stride < nunits; u += 2 * stride) {
      Raw8 r0 = load_raw8(xs + u * 8), r1 = load_raw8(xs + (u + stride) * 8);
      float v[8];
      widen8(r0, xs, v);
      store_codes8(cs + u * 8, fp8_pack8(v, s, y));
      widen8(r1, xs, v);
      store_codes8(cs + (u + stride) * 8, fp8_pack8(v, s, y));
    }
    for (; u < nunits; u += stride) {
      float v[8];
      widen8(load_raw8(xs + u * 8), xs, v);
      store_codes8(cs + u * 8, fp8_pack8(v, s, y));
    }
  } else {
    for (int64_t i = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x; i < per_slice; i += stride)
      cs[i] = e4m3_byte(fp8_quot(ld1(xs + i), s, y));
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) a.scales[tz][b] = s;
}

// ---------------------------------------------------------------------------
// Dequantization: out = dec(code) * s, float32 or RNE to bf16.  One workgroup
// row-chunk at a time: blockIdx.y strides over the rows of all slices.
// ---------------------------------------------------------------------------
template <bool kBf16Out>
__device__ __forceinline__ void store_out(void* out, int64_t i, float v) {
  if constexpr (kBf16Out)
    reinterpret_cast<uint16_t*>(out)[i] = (uint16_t)bf16_rne_bits(v);
  else
    reinterpret_cast<float*>(out)[i] = v;
}

template <bool kBf16Out>
__global__ __launch_bounds__(kBlockThreads) void k_fp8_dequant(const uint8_t* __restrict__ codes,
                                                                const float* __restrict__ scales,
                                                                int gran, int64_t nrows_total,
                                                                int64_t rows, int64_t cols, int br,
                                                                void* __restrict__ out) {
  for (int64_t gr = blockIdx.y; gr < nrows_total; gr += gridDim.y) {
    const int64_t b = gr / rows, r = gr - b * rows;
    for (int64_t c = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x; c < cols;
         c += (int64_t)gridDim.x * kBlockThreads) {
      int64_t si;
      switch (gran) {
        case 0: si = b; break;
        case 1: si = gr; break;
        case 2: si = gr * (cols / 128) + c / 128; break;
        default: si = (b * (rows / br) + r / br) * (cols / 128) + c / 128; break;
      }
      const int64_t i = gr * cols + c;
      store_out<kBf16Out>(out, i, e4m3_decode(codes[i]) * scales[si]);
    }
  }
}

inline int blocks_for(int64_t work, int64_t per_block, int64_t cap) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (int)g;
}

}  // namespace

int amax_partials_per_slice(int64_t batch, int64_t per_slice, int ntensors) {
  int64_t slices = batch * ntensors;
  if (slices < 1) slices = 1;
  int64_t p = (2048 + slices - 1) / slices;  // about 2048 workgroups in all
  int64_t by_size = (per_slice + 8 * kBlockThreads * 4 - 1) / (8 * kBlockThreads * 4);
  if (p > by_size) p = by_size;
  if (p > 1024) p = 1024;
  if (p < 1) p = 1;
  return (int)p;
}

hipError_t launch_fp8_1x128(const void* x, bool bf16, int64_t n, uint8_t* codes, float* scales,
                            hipStream_t st) {
  constexpr int kUnr = 4;
  const int64_t nunits = n / 8;
  const int64_t ntiles = (nunits + kWave - 1) / kWave;
  const int grid = blocks_for(ntiles, (int64_t)kUnr * (kBlockThreads / kWave), 1 << 30);
  if (bf16)
    hipLaunchKernelGGL((k_fp8_1x128<uint16_t, kUnr>), dim3(grid), dim3(kBlockThreads), 0, st,
                       (const uint16_t*)x, nunits, codes, scales);
  else
    hipLaunchKernelGGL((k_fp8_1x128<float, kUnr>), dim3(grid), dim3(kBlockThreads), 0, st,
                       (const float*)x, nunits, codes, scales);
  return hipGetLastError();
}

hipError_t launch_fp8_128x128(const void* x, bool bf16, int64_t batch, int64_t rows,
                              int64_t cols, uint8_t* codes, float* scales, hipStream_t st) {
  const int br = (int)(rows < 128 ? rows : 128);
  const int64_t tiles = batch * (rows / br) * (cols / 128);
  if (bf16)
    hipLaunchKernelGGL(k_fp8_128x128<uint16_t>, dim3((unsigned)tiles), dim3(kBlockThreads), 0, st,
                       (const uint16_t*)x, rows, cols, br, codes, scales);
  else
    hipLaunchKernelGGL(k_fp8_128x128<float>, dim3((unsigned)tiles), dim3(kBlockThreads), 0, st,
                       (const float*)x, rows, cols, br, codes, scales);
  return hipGetLastError();
}

hipError_t launch_fp8_row(const void* x, bool bf16, int64_t nrows, int64_t cols, uint8_t* codes,
                          float* scales, hipStream_t st) {
  constexpr int kMaxU = 16;  // up to 8192 columns in registers
  const int grid = (int)((nrows + 3) / 4);
  const bool vec = cols % 8 == 0 && cols <= (int64_t)kWave * 8 * kMaxU;
  if (bf16) {
    if (vec)
      hipLaunchKernelGGL((k_fp8_row_vec<uint16_t, kMaxU>), dim3(grid), dim3(kBlockThreads), 0, st,
                         (const uint16_t*)x, nrows, cols, codes, scales);
    else
      hipLaunchKernelGGL(k_fp8_row_any<uint16_t>, dim3(grid), dim3(kBlockThreads), 0, st,
                         (const uint16_t*)x, nrows, cols, codes, scales);
  } else {
    if (vec)
      hipLaunchKernelGGL((k_fp8_row_vec<float, kMaxU>), dim3(grid), dim3(kBlockThreads), 0, st,
                         (const float*)x, nrows, cols, codes, scales);
    else
      hipLaunchKernelGGL(k_fp8_row_any<float>, dim3(grid), dim3(kBlockThreads), 0, st,
                         (const float*)x, nrows, cols, codes, scales);
  }
  return hipGetLastError();
}

hipError_t launch_amax_partials(const void* const* x, bool bf16, int ntensors, int64_t batch,
                                int64_t per_slice, float* partials, int P, hipStream_t st) {
  TensorArgs a{};
  for (int i = 0; i < ntensors; ++i) a.x[i] = x[i];
  const dim3 g1(P, (unsigned)batch, ntensors);
  const bool vec = per_slice % 8 == 0;
  if (bf16) {
    if (vec)
      hipLaunchKernelGGL((k_amax_partial<uint16_t, true>), g1, dim3(kBlockThreads), 0, st, a,
                         per_slice, partials);
    else
      hipLaunchKernelGGL((k_amax_partial<uint16_t, false>), g1, dim3(kBlockThreads), 0, st, a,
                         per_slice, partials);
  } else {
    if (vec)
      hipLaunchKernelGGL((k_amax_partial<float, true>), g1, dim3(kBlockThreads), 0, st, a,
                         per_slice, partials);
    else
      hipLaunchKernelGGL((k_amax_partial<float, false>), g1, dim3(kBlockThreads), 0, st, a,
                         per_slice, partials);
  }
  return hipGetLastError();
}

hipError_t launch_fp8_tensor(const void* const* x, bool bf16, int ntensors, int64_t batch,
                             int64_t per_slice, uint8_t* const* codes, float* const* scales,
                             float* partials, hipStream_t st) {
  TensorArgs a{};
  for (int i = 0; i < ntensors; ++i) {
    a.x[i] = x[i];
    a.codes[i] = codes[i];
    a.scales[i] = scales[i];
  }
  const int P = amax_partials_per_slice(batch, per_slice, ntensors);
  hipError_t e = launch_amax_partials(x, bf16, ntensors, batch, per_slice, partials, P, st);
  if (e != hipSuccess) return e;
  const bool vec = per_slice % 8 == 0;
  // pass 2: about 8 units per thread, at most 1024 workgroups per slice
  const int q = blocks_for(per_slice / 8, (int64_t)kBlockThreads * 8, 1024);
  const dim3 g2(q, (unsigned)batch, ntensors);
  if (bf16) {
    if (vec)
      hipLaunchKernelGGL((k_fp8_tensor_quant<uint16_t, true>), g2, dim3(kBlockThreads), 0, st, a,
                         per_slice, partials, P);
    else
      hipLaunchKernelGGL((k_fp8_tensor_quant<uint16_t, false>), g2, dim3(kBlockThreads), 0, st,
                         a, per_slice, partials, P);
  } else {
    if (vec)
      hipLaunchKernelGGL((k_fp8_tensor_quant<float, true>), g2, dim3(kBlockThreads), 0, st, a,
                         per_slice, partials, P);
    else
      hipLaunchKernelGGL((k_fp8_tensor_quant<float, false>), g2, dim3(kBlockThreads), 0, st, a,
                         per_slice, partials, P);
  }
  return hipGetLastError();
}

hipError_t launch_fp8_dequant(const uint8_t* codes, const float* scales, int gran, int64_t batch,
                              int64_t rows, int64_t cols, bool out_bf16, void* out,
                              hipStream_t st) {
  const int br = (int)(rows < 128 ? rows : 128);
  const int64_t nrows = batch * rows;
  const dim3 grid(blocks_for(cols, kBlockThreads, 64), (unsigned)(nrows < 65535 ? nrows : 65535));
  if (out_bf16)
    hipLaunchKernelGGL(k_fp8_dequant<true>, grid, dim3(kBlockThreads), 0, st, codes, scales, gran,
                       nrows, rows, cols, br, out);
  else
    hipLaunchKernelGGL(k_fp8_dequant<false>, grid, dim3(kBlockThreads), 0, st, codes, scales,
                       gran, nrows, rows, cols, br, out);
  return hipGetLastError();
}

namespace {
__global__ __launch_bounds__(kBlockThreads) void k_encode_e4m3(const float* __restrict__ y,
                                                               int64_t n,
                                                               uint8_t* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kBlockThreads)
    out[i] = e4m3_byte(y[i]);
}
}  // namespace

hipError_t launch_encode_e4m3(const float* y, int64_t n, uint8_t* out, hipStream_t st) {
  hipLaunchKernelGGL(k_encode_e4m3, dim3(blocks_for(n, kBlockThreads, 4096)), dim3(kBlockThreads),
                     0, st, y, n, out);
  return hipGetLastError();
}

}  // namespace pqb
