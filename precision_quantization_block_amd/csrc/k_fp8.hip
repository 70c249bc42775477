// Scaled one-byte codes: FP8 E4M3, FP8 E5M2 and symmetric INT8 with 1x128
// blocks, 128x128 tiles, rows and (for slices whose length is not a multiple
// of 8) per tensor; the per-chunk bodies are in quant.h, the chunked per-tensor
// path in k_twopass.hip.
//
// Scale of a scope: s = RN(max(amax, 1e-12) / M) with M = 448 (E4M3), 57344
// (E5M2) or 127 (INT8); codes are the element code of RN(x / s) (page "量化部署
// 实战", section 伪量化实现; the E5M2 row of the low-precision float table and
// the symmetric INT8 scale on "14. 量化：让每一步搬更少的字节").  The page's
// clamp to +-M never binds: |x| <= amax gives |x/s| <= M up to one rounding,
// which still rounds to M.
#include "launch.h"
#include "quant.h"

namespace pqb {
namespace {

template <typename T, int kUnr, int kElem>
__global__ __launch_bounds__(kBlockThreads) void k_fp8_1x128(const T* __restrict__ x,
                                                              int64_t nunits,
                                                              uint8_t* __restrict__ codes,
                                                              float* __restrict__ scales) {
  const int64_t nwaves = (int64_t)gridDim.x * (kBlockThreads / kWave);
  for (int64_t t0 = (int64_t)wave_index() * kUnr; t0 * kWave < nunits; t0 += nwaves * kUnr) {
    const int64_t u0 = t0 * kWave;
    if (u0 + kUnr * kWave <= nunits)
      fp8_1x128_chunk<T, kUnr, false, kElem>(x, u0, nunits, codes, scales);
    else
      fp8_1x128_chunk<T, kUnr, true, kElem>(x, u0, nunits, codes, scales);
  }
}

constexpr int kTileWaves = 8;  // 512 threads per 128x128 tile: 4 rows of it per lane

// Large launches take two adjacent tiles per workgroup: twice the loads in
// flight per lane and half the barriers per byte (1 GiB bf16: 272 -> 255 us).
// With few tiles the halved workgroup count costs more than that gains
// (896 tiles: 9.8 -> 10.6 us), hence the threshold.
constexpr int64_t kPairTilesFrom = 4096;

template <typename T, int kElem, int kTiles>
__global__ __launch_bounds__(kTileWaves * kWave) void k_fp8_128x128(const T* __restrict__ x,
                                                                     int64_t rows, int64_t cols,
                                                                     int br,
                                                                     uint8_t* __restrict__ codes,
                                                                     float* __restrict__ scales) {
  __shared__ uint32_t red[kTiles * kTileWaves];
  fp8_tile_128x128<T, kTileWaves, kElem, kTiles>(x, rows, cols, br, (int64_t)blockIdx.x * kTiles,
                                                 codes, scales, red);
}

template <typename T, int kMaxU, int kElem>
__global__ __launch_bounds__(kBlockThreads) void k_fp8_row_vec(const T* __restrict__ x,
                                                                int64_t nrows, int64_t cols,
                                                                uint8_t* __restrict__ codes,
                                                                float* __restrict__ scales) {
  const int64_t row = wave_index();
  if (row < nrows) fp8_row_vec<T, kMaxU, kElem>(x, row, cols, codes, scales);  // whole waves
}

template <typename T, int kElem>
__global__ __launch_bounds__(kBlockThreads) void k_fp8_row_any(const T* __restrict__ x,
                                                                int64_t nrows, int64_t cols,
                                                                uint8_t* __restrict__ codes,
                                                                float* __restrict__ scales) {
  const int64_t row = wave_index();
  if (row < nrows) fp8_row_any<T, kElem>(x, row, cols, codes, scales);
}

// ---------------------------------------------------------------------------
// Per tensor for slices whose length is not a multiple of 8 (element-wise).
// Pass 1: each workgroup writes the amax of its share of a slice to
// partials[(tensor * batch + b) * P + blockIdx.x].  Pass 2: each workgroup
// reduces the slice's P partials, forms s and quantizes its share.
// blockIdx.y = slice, blockIdx.z = tensor (K or V for the KV write).
// ---------------------------------------------------------------------------
struct TensorArgs {
  const void* x[2];
  uint8_t* codes[2];
  float* scales[2];
};

// Max of non-negative float bit patterns over the workgroup (all threads get it).
__device__ __forceinline__ uint32_t block_umax(uint32_t m, uint32_t* red) {
  m = wave_umax(m);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = max(max(red[0], red[1]), max(red[2], red[3]));
  __syncthreads();
  return m;
}

template <typename T>
__global__ __launch_bounds__(kBlockThreads) void k_amax_partial(TensorArgs a, int64_t per_slice,
                                                                 float* __restrict__ partials) {
  __shared__ uint32_t red[kBlockThreads / kWave];
  const int64_t b = blockIdx.y, P = gridDim.x;
  const T* xs = reinterpret_cast<const T*>(a.x[blockIdx.z]) + b * per_slice;
  uint32_t m = 0;
  for (int64_t i = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x; i < per_slice;
       i += P * kBlockThreads)
    m = max(m, as_u(fabsf(ld1(xs + i))));
  m = block_umax(m, red);
  if (threadIdx.x == 0) partials[((int64_t)blockIdx.z * gridDim.y + b) * P + blockIdx.x] = as_f(m);
}

// Reduce the P partials of one slice (all threads receive the maximum).
__device__ __forceinline__ uint32_t reduce_partials(const float* __restrict__ p, int P,
                                                    uint32_t* red) {
  uint32_t m = 0;
  for (int i = threadIdx.x; i < P; i += kBlockThreads) m = max(m, as_u(p[i]));
  return block_umax(m, red);
}

template <typename T, int kElem>
__global__ __launch_bounds__(kBlockThreads) void k_fp8_tensor_quant(TensorArgs a,
                                                                     int64_t per_slice,
                                                                     const float* __restrict__ partials,
                                                                     int P) {
  __shared__ uint32_t red[kBlockThreads / kWave];
  const int64_t b = blockIdx.y;
  const int tz = blockIdx.z;
  const float s =
      fp8_scale_bits<kElem>(reduce_partials(partials + ((int64_t)tz * gridDim.y + b) * P, P, red));
  const float y = recip_rn(s);
  const T* xs = reinterpret_cast<const T*>(a.x[tz]) + b * per_slice;
  uint8_t* cs = a.codes[tz] + b * per_slice;
  const int64_t stride = (int64_t)gridDim.x * kBlockThreads;
  for (int64_t i = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x; i < per_slice; i += stride)
    cs[i] = elem_byte<kElem>(div_rn(ld1(xs + i), s, y));
  if (blockIdx.x == 0 && threadIdx.x == 0) a.scales[tz][b] = s;
}

// ---------------------------------------------------------------------------
// Dequantization of the per-tensor, per-row and 128x128 scopes: out =
// dec(code) * s, float32 or RNE bf16.  When cols % 8 == 0 a wave expands one
// segment of a row, kDqSegUnits units of 8 elements (2 per lane, all loaded
// before the first store), and the segment's scale index is formed once; the
// segments of all rows of all slices are numbered in sequence.  Otherwise a
// wave expands one row element by element.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint2 ld_codes8(const uint8_t* p) {
  return *reinterpret_cast<const uint2*>(p);
}

constexpr int kDqSegLane = 2;                       // units per lane of a segment
// (1 GiB bf16, same-process A/B: per row 272.9 / 264.3 / 285.3 us with 4 / 2 / 8)
constexpr int kDqSegUnits = kDqSegLane * kWave;     // units per segment

// Scale index of column c of global row gr: si0 + (c / 128) * tile_stride.
// I is the index type of the divisions: uint32_t when every count fits, which
// spares a 64-bit division routine per segment.
template <typename I>
__device__ __forceinline__ void row_scale_index(int gran, I gr, I rows, I cols, int br,
                                                int64_t& si0, int64_t& tile_stride) {
  tile_stride = 0;
  switch (gran) {
    case 0: si0 = (int64_t)(gr / rows); break;
    case 1: si0 = (int64_t)gr; break;
    default: {
      const I b = gr / rows, r = gr - b * rows;
      si0 = ((int64_t)b * (int64_t)(rows / (I)br) + (int64_t)(r / (I)br)) * (int64_t)(cols / 128);
      tile_stride = 1;
      break;
    }
  }
}

template <bool kBf16Out, int kElem, typename I>
__global__ __launch_bounds__(kBlockThreads) void k_fp8_dequant_segs(const uint8_t* __restrict__ codes,
                                                                     const float* __restrict__ scales,
                                                                     int gran, int64_t nsegs,
                                                                     int64_t rows, int64_t cols,
                                                                     int br,
                                                                     void* __restrict__ out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int64_t upr = cols / 8;
  const I spr = (I)((upr + kDqSegUnits - 1) / kDqSegUnits);
  const int64_t nw = (int64_t)gridDim.x * (kBlockThreads / kWave);
  for (int64_t w = (int64_t)blockIdx.x * (kBlockThreads / kWave) + wave; w < nsegs; w += nw) {
    const I gri = (I)w / spr;
    const int64_t gr = (int64_t)gri, u0 = (int64_t)((I)w - gri * spr) * kDqSegUnits;
    int64_t si0, tile_stride;
    row_scale_index<I>(gran, gri, (I)rows, (I)cols, br, si0, tile_stride);
    uint2 c[kDqSegLane];
    float sc[kDqSegLane];
    if (kBf16Out && u0 + kDqSegUnits <= upr) {
      // A whole segment with bf16 output: no per-lane bound, so no branch lets
      // the compiler sink a load next to its use.  It spans kDqSegUnits / 16
      // = 8 scale groups of 128 columns; lane l loads the scale of group l % 8
      // once and each tile takes its lanes' scales by lane permute (unit
      // 64 k + l lies in group 4 k + l / 16), one scale load per segment
      // instead of one per tile.  On 1 GiB, 128x128 dequant took 250 us
      // against 263 us, with the same bytes; float32 output, whose two
      // 16-byte stores per unit each leave gaps, went from 719 to 884 us this
      // way, so it keeps the form below.
      static_assert(kDqSegUnits / 16 == 8 && kDqSegLane == 2, "8 groups per segment");
      const float sl = scales[si0 + ((u0 >> 4) + (lane & 7)) * tile_stride];
#pragma unroll
      for (int k = 0; k < kDqSegLane; ++k)
        c[k] = ld_codes8(codes + gr * cols + (u0 + k * kWave + lane) * 8);
#pragma unroll
      for (int k = 0; k < kDqSegLane; ++k)
        sc[k] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
                                              4 * (4 * k + (lane >> 4)), __builtin_bit_cast(int, sl)));
#pragma unroll
      for (int k = 0; k < kDqSegLane; ++k) {
        float o[8];
        fp8_decode8<kElem>(c[k], sc[k], o);
        store_out8<kBf16Out>(out, gr * upr + u0 + k * kWave + lane, o);
      }
      continue;
    }
#pragma unroll
    for (int k = 0; k < kDqSegLane; ++k) {
      const int64_t u = u0 + k * kWave + lane;
      if (u < upr) {
        c[k] = ld_codes8(codes + gr * cols + u * 8);
        sc[k] = scales[si0 + (u >> 4) * tile_stride];
      }
    }
#pragma unroll
    for (int k = 0; k < kDqSegLane; ++k) {
      const int64_t u = u0 + k * kWave + lane;
      if (u < upr) {
        float o[8];
        fp8_decode8<kElem>(c[k], sc[k], o);
        store_out8<kBf16Out>(out, gr * upr + u, o);
      }
    }
  }
}

template <bool kBf16Out, int kElem>
__global__ __launch_bounds__(kBlockThreads) void k_fp8_dequant_rows(const uint8_t* __restrict__ codes,
                                                                     const float* __restrict__ scales,
                                                                     int gran, int64_t nrows_total,
                                                                     int64_t rows, int64_t cols,
                                                                     int br,
                                                                     void* __restrict__ out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t nw = (int64_t)gridDim.x * (kBlockThreads / kWave);
  for (int64_t gr = wave_index(); gr < nrows_total; gr += nw) {
    int64_t si0, tile_stride;
    row_scale_index<int64_t>(gran, gr, rows, cols, br, si0, tile_stride);
    for (int64_t c = lane; c < cols; c += kWave) {
      const float v = elem_decode2<kElem, false>(codes[gr * cols + c]).x *
                      scales[si0 + (c >> 7) * tile_stride];
      if constexpr (kBf16Out)
        reinterpret_cast<uint16_t*>(out)[gr * cols + c] = (uint16_t)bf16x2_rne(v, 0.0f);
      else
        reinterpret_cast<float*>(out)[gr * cols + c] = v;
    }
  }
}

template <int kElem>
__global__ __launch_bounds__(kBlockThreads) void k_encode_elem(const float* __restrict__ y,
                                                               int64_t n,
                                                               uint8_t* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kBlockThreads)
    out[i] = elem_byte<kElem>(y[i]);
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
                            hipStream_t st, int elem) {
  // chunks of 4 tiles per wave; from 2^28 elements 2 tiles (same-process
  // A/B on bf16: [8192 x 7168] 29.5 us with 4 against 30.5 with 2; 1 GiB
  // 256.6 us with 4 against 249.3 with 2)
  const int64_t nunits = n / 8;
  const int64_t ntiles = (nunits + kWave - 1) / kWave;
  const bool big = n >= ((int64_t)1 << 28);
  return with_elem(elem, [&](auto e) {
    constexpr int E = decltype(e)::value;
    auto go = [&](auto unr) {
      constexpr int kUnr = decltype(unr)::value;
      const int grid = blocks_for(ntiles, (int64_t)kUnr * (kBlockThreads / kWave), 1 << 29);
      if (bf16)
        hipLaunchKernelGGL((k_fp8_1x128<uint16_t, kUnr, E>), dim3(grid), dim3(kBlockThreads), 0,
                           st, (const uint16_t*)x, nunits, codes, scales);
      else
        hipLaunchKernelGGL((k_fp8_1x128<float, kUnr, E>), dim3(grid), dim3(kBlockThreads), 0, st,
                           (const float*)x, nunits, codes, scales);
    };
    if (big)
      go(std::integral_constant<int, 2>{});
    else
      go(std::integral_constant<int, 4>{});
  });
}

hipError_t launch_fp8_128x128(const void* x, bool bf16, int64_t batch, int64_t rows,
                              int64_t cols, uint8_t* codes, float* scales, hipStream_t st,
                              int elem) {
  const int br = (int)(rows < 128 ? rows : 128);
  const int64_t tiles = batch * (rows / br) * (cols / 128);
  const bool pair = (cols / 128) % 2 == 0 && tiles >= kPairTilesFrom;
  return with_elem(elem, [&](auto e) {
    constexpr int E = decltype(e)::value;
    auto go = [&](auto kernel, const auto* xp, int64_t wgs) {
      hipLaunchKernelGGL(kernel, dim3((unsigned)wgs), dim3(kTileWaves * kWave), 0, st, xp, rows,
                         cols, br, codes, scales);
    };
    if (bf16) {
      if (pair)
        go(k_fp8_128x128<uint16_t, E, 2>, (const uint16_t*)x, tiles / 2);
      else
        go(k_fp8_128x128<uint16_t, E, 1>, (const uint16_t*)x, tiles);
    } else {
      if (pair)
        go(k_fp8_128x128<float, E, 2>, (const float*)x, tiles / 2);
      else
        go(k_fp8_128x128<float, E, 1>, (const float*)x, tiles);
    }
  });
}

hipError_t launch_fp8_row(const void* x, bool bf16, int64_t nrows, int64_t cols, uint8_t* codes,
                          float* scales, hipStream_t st, int elem) {
  constexpr int kMaxU = 16;  // up to 8192 columns in registers
  const int grid = (int)((nrows + 3) / 4);
  const bool vec = cols % 8 == 0 && cols <= (int64_t)kWave * 8 * kMaxU;
  return with_elem(elem, [&](auto e) {
    constexpr int E = decltype(e)::value;
    if (bf16) {
      if (vec)
        hipLaunchKernelGGL((k_fp8_row_vec<uint16_t, kMaxU, E>), dim3(grid), dim3(kBlockThreads), 0,
                           st, (const uint16_t*)x, nrows, cols, codes, scales);
      else
        hipLaunchKernelGGL((k_fp8_row_any<uint16_t, E>), dim3(grid), dim3(kBlockThreads), 0, st,
                           (const uint16_t*)x, nrows, cols, codes, scales);
    } else {
      if (vec)
        hipLaunchKernelGGL((k_fp8_row_vec<float, kMaxU, E>), dim3(grid), dim3(kBlockThreads), 0,
                           st, (const float*)x, nrows, cols, codes, scales);
      else
        hipLaunchKernelGGL((k_fp8_row_any<float, E>), dim3(grid), dim3(kBlockThreads), 0, st,
                           (const float*)x, nrows, cols, codes, scales);
    }
  });
}

hipError_t launch_fp8_tensor(const void* const* x, bool bf16, int ntensors, int64_t batch,
                             int64_t per_slice, uint8_t* const* codes, float* const* scales,
                             float* partials, hipStream_t st, int elem) {
  if (per_slice % 8 == 0)
    return launch_tensor_fp8(x, bf16, ntensors, batch, per_slice, codes, scales, partials, st,
                             elem);
  // slices whose length is not a multiple of 8: element-wise grid-stride passes
  TensorArgs a{};
  for (int i = 0; i < ntensors; ++i) {
    a.x[i] = x[i];
    a.codes[i] = codes[i];
    a.scales[i] = scales[i];
  }
  const int P = amax_partials_per_slice(batch, per_slice, ntensors);
  const dim3 g1(P, (unsigned)batch, ntensors);
  if (bf16)
    hipLaunchKernelGGL(k_amax_partial<uint16_t>, g1, dim3(kBlockThreads), 0, st, a, per_slice,
                       partials);
  else
    hipLaunchKernelGGL(k_amax_partial<float>, g1, dim3(kBlockThreads), 0, st, a, per_slice,
                       partials);
  const hipError_t e1 = hipGetLastError();
  if (e1 != hipSuccess) return e1;
  // pass 2: about 8 elements per thread, at most 1024 workgroups per slice
  const int q = blocks_for(per_slice, (int64_t)kBlockThreads * 8, 1024);
  const dim3 g2(q, (unsigned)batch, ntensors);
  return with_elem(elem, [&](auto e) {
    constexpr int E = decltype(e)::value;
    if (bf16)
      hipLaunchKernelGGL((k_fp8_tensor_quant<uint16_t, E>), g2, dim3(kBlockThreads), 0, st, a,
                         per_slice, partials, P);
    else
      hipLaunchKernelGGL((k_fp8_tensor_quant<float, E>), g2, dim3(kBlockThreads), 0, st, a,
                         per_slice, partials, P);
  });
}

hipError_t launch_fp8_dequant(const uint8_t* codes, const float* scales, int gran, int64_t batch,
                              int64_t rows, int64_t cols, bool out_bf16, void* out,
                              hipStream_t st, int elem) {
  const int64_t n = batch * rows * cols;
  if (gran == 2)  // 1x128: cols % 128 == 0, flat
    return launch_fp8_1x128_dequant(codes, scales, n, out_bf16, out, st, elem);
  const int br = (int)(rows < 128 ? rows : 128);
  const int64_t nrows = batch * rows;
  return with_elem(elem, [&](auto e) {
    constexpr int E = decltype(e)::value;
    if (cols % 8 == 0) {
      const int64_t nsegs = nrows * ((cols / 8 + kDqSegUnits - 1) / kDqSegUnits);
      const int grid = blocks_for(nsegs, kBlockThreads / kWave, 1 << 20);
      // 32-bit divisions while segment, row and column counts fit
      const bool narrow = nsegs <= UINT32_MAX && cols <= UINT32_MAX;
      auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3(grid), dim3(kBlockThreads), 0, st, codes, scales, gran,
                           nsegs, rows, cols, br, out);
      };
      if (out_bf16)
        narrow ? go(k_fp8_dequant_segs<true, E, uint32_t>) : go(k_fp8_dequant_segs<true, E, int64_t>);
      else
        narrow ? go(k_fp8_dequant_segs<false, E, uint32_t>) : go(k_fp8_dequant_segs<false, E, int64_t>);
    } else {
      const int grid = blocks_for(nrows, kBlockThreads / kWave, 1 << 16);
      if (out_bf16)
        hipLaunchKernelGGL((k_fp8_dequant_rows<true, E>), dim3(grid), dim3(kBlockThreads), 0, st,
                           codes, scales, gran, nrows, rows, cols, br, out);
      else
        hipLaunchKernelGGL((k_fp8_dequant_rows<false, E>), dim3(grid), dim3(kBlockThreads), 0, st,
                           codes, scales, gran, nrows, rows, cols, br, out);
    }
  });
}

hipError_t launch_encode_elem(const float* y, int64_t n, uint8_t* out, hipStream_t st, int elem) {
  return with_elem(elem, [&](auto e) {
    constexpr int E = decltype(e)::value;
    hipLaunchKernelGGL(k_encode_elem<E>, dim3(blocks_for(n, kBlockThreads, 4096)),
                       dim3(kBlockThreads), 0, st, y, n, out);
  });
}

}  // namespace pqb
