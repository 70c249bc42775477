// Per-chunk quantization bodies shared by the single-tensor kernels
// (k_fp8.hip, k_fp4.hip, k_int4.hip) and the fused multi-tensor kernel
// (k_multi.hip).  A "unit" is 8 consecutive elements (one lane's load); a
// "tile" is 64 units (one wave-wide load); a chunk is kUnr consecutive tiles
// streamed by one wave.  kGuard selects the bounds-checked variant used only
// for the last, partial chunk of a tensor.
#pragma once

#include "device.h"

namespace pqb {

constexpr float kInv448 = 1.0f / 448.0f;  // RN(1/448), folded at compile time
constexpr float kInv6 = 1.0f / 6.0f;
constexpr float kInv15 = 1.0f / 15.0f;
constexpr float kRound = 12582912.0f;  // 1.5 * 2^23: adding it rounds |q| < 2^22 to an
                                       // integer, ties to even (the constant is even)

// ---------------------------------------------------------------------------
// FP8 E4M3 (page "量化部署实战", section 伪量化实现): s = RN(max(amax, 1e-12) /
// 448), codes E4M3(RN(x / s)).  The page's clamp to +-448 never binds: |x| <=
// amax gives |x/s| <= 448 up to one rounding, which still rounds to 448.
// ---------------------------------------------------------------------------

// ---------------------------------------------------------------------------
// Element formats of the scaled one-byte codes.  All share the scopes (per
// tensor, row, 1x128, 128x128 tile) and s = RN(max(amax, 1e-12) / M):
//   kE4M3  M = 448    code E4M3(RN(x / s))               (page "量化部署实战")
//   kE5M2  M = 57344  code E5M2(RN(x / s))               (E5M2 row of the
//          low-precision float table, "14. 量化：让每一步搬更少的字节")
//   kI8    M = 127    code rint(RN(x / s)) as int8       (symmetric INT8,
//          "14. 量化：让每一步搬更少的字节", 量化在做什么)
// |x| <= amax keeps |x / s| <= M up to one rounding, which still rounds to M,
// so no clamp is needed.  RN(a / M) uses one correction with RN(1/M); a CPU
// check found it equal to IEEE division for every significand in three
// binades for each M.
// ---------------------------------------------------------------------------
enum Elem : int { kE4M3 = 0, kE5M2 = 1, kI8 = 2 };

template <int kElem>
struct ElemMax;
template <>
struct ElemMax<kE4M3> {
  static constexpr float m = 448.0f, inv = 1.0f / 448.0f;
};
template <>
struct ElemMax<kE5M2> {
  static constexpr float m = 57344.0f, inv = 1.0f / 57344.0f;
};
template <>
struct ElemMax<kI8> {
  static constexpr float m = 127.0f, inv = 1.0f / 127.0f;
};

// Host side: calls f(std::integral_constant<int, kElem>) for a runtime element
// kind and returns the launch status.
template <typename F>
inline hipError_t with_elem(int elem, F f) {
  switch (elem) {
    case kE4M3: f(std::integral_constant<int, kE4M3>{}); break;
    case kE5M2: f(std::integral_constant<int, kE5M2>{}); break;
    case kI8: f(std::integral_constant<int, kI8>{}); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int kElem>
__device__ __forceinline__ uint32_t elem_bytes4(float a, float b, float c, float d) {
  if constexpr (kElem == kE5M2)
    return e5m2_bytes4(a, b, c, d);
  else if constexpr (kElem == kI8)
    return int8_bytes4(a, b, c, d);
  else
    return e4m3_bytes4(a, b, c, d);
}

// s from the bit pattern of a scope's amax (a non-negative float).
template <int kElem = kE4M3>
__device__ __forceinline__ float fp8_scale_bits(uint32_t amax_bits) {
  return div_const(as_f(max(amax_bits, kAmaxFloorBits)), ElemMax<kElem>::m, ElemMax<kElem>::inv);
}

// Eight values -> eight codes (two dwords) with scale s and y = RN(1/s).
template <int kElem = kE4M3>
__device__ __forceinline__ uint2 fp8_pack8(const float v[8], float s, float y) {
  const uint32_t w0 = elem_bytes4<kElem>(div_rn(v[0], s, y), div_rn(v[1], s, y),
                                         div_rn(v[2], s, y), div_rn(v[3], s, y));
  const uint32_t w1 = elem_bytes4<kElem>(div_rn(v[4], s, y), div_rn(v[5], s, y),
                                         div_rn(v[6], s, y), div_rn(v[7], s, y));
  return make_uint2(w0, w1);
}

__device__ __forceinline__ void store_codes8(uint8_t* p, uint2 w) { st_nt8(p, w.x, w.y); }

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

template <int kElem = kE4M3>
__device__ __forceinline__ uint8_t elem_byte(float q) {
  return (uint8_t)(elem_bytes4<kElem>(q, 0.0f, 0.0f, 0.0f) & 0xFFu);
}

template <typename T, int kUnr, bool kGuard>
__device__ __forceinline__ void load_chunk(const T* __restrict__ x, int64_t u0, int64_t nunits,
                                           Raw8 raw[kUnr]) {
  const int lane = threadIdx.x & (kWave - 1);
  const T* xb = x + u0 * 8;
#pragma unroll
  for (int k = 0; k < kUnr; ++k)
    raw[k] = (!kGuard || u0 + k * kWave + lane < nunits) ? load_raw8(xb + (k * kWave + lane) * 8)
                                                           : Raw8{};
}

// Grid-stride walk over units u, u + stride, ... < nunits with kLoads loads in
// flight per thread: body(raw, unit) runs once per unit, in order.
constexpr int kStreamLoads = 2;
template <typename T, int kLoads, typename Body>
__device__ __forceinline__ void stream_units(const T* __restrict__ xs, int64_t u, int64_t nunits,
                                             int64_t stride, Body body) {
  for (; u + (kLoads - 1) * stride < nunits; u += kLoads * stride) {
    Raw8 r[kLoads];
#pragma unroll
    for (int k = 0; k < kLoads; ++k) r[k] = load_raw8(xs + (u + k * stride) * 8);
#pragma unroll
    for (int k = 0; k < kLoads; ++k) body(r[k], u + k * stride);
  }
  for (; u < nunits; u += stride) body(load_raw8(xs + u * 8), u);
}

// 1x128 blocks: a block is 16 lanes x 8 elements, one DPP row.
template <typename T, int kUnr, bool kGuard, int kElem = kE4M3>
__device__ __forceinline__ void fp8_1x128_chunk(const T* __restrict__ x, int64_t u0, int64_t nunits,
                                                uint8_t* __restrict__ codes,
                                                float* __restrict__ scales) {
  const int lane = threadIdx.x & (kWave - 1);
  Raw8 raw[kUnr];
  load_chunk<T, kUnr, kGuard>(x, u0, nunits, raw);
#pragma unroll
  for (int k = 0; k < kUnr; ++k) {
    float v[8];
    widen8(raw[k], x, v);
    const float s = fp8_scale_bits<kElem>(group_umax<16>(as_u(absmax8(v))));
    const float y = recip_rn(s);
    const uint2 w = fp8_pack8<kElem>(v, s, y);
    const int64_t u = u0 + k * kWave + lane;
    if (!kGuard || u < nunits) {
      store_codes8(codes + u * 8, w);
      if ((lane & 15) == 0) scales[u >> 4] = s;
    }
  }
}

// kTiles horizontally adjacent br x 128 tiles (br = min(128, rows)), the
// first being tile t, per workgroup of kWaves waves (4 or 8).  Lane l of wave
// w covers unit (l % 16) of tile rows w*4 + l/16 + 4*kWaves*k, k < 32 /
// kWaves, of every tile; all loads are issued before the first reduction.
// Each tile's amax is reduced through DPP, a cross-row shuffle and LDS
// (`red`, kTiles * kWaves words), with one barrier for all.  All threads of
// the workgroup must call it; with kTiles = 2, t is even and the tile row
// holds an even number of tiles.
template <typename T, int kWaves, int kElem = kE4M3, int kTiles = 1>
__device__ __forceinline__ void fp8_tile_128x128(const T* __restrict__ x, int64_t rows,
                                                 int64_t cols, int br, int64_t t,
                                                 uint8_t* __restrict__ codes,
                                                 float* __restrict__ scales, uint32_t* red) {
  constexpr int kRowStep = 4 * kWaves, kRowsPerLane = 128 / kRowStep;
  const int64_t tiles_c = cols / 128;
  const int64_t tc = t % tiles_c, trb = t / tiles_c;  // trb = b * (rows / br) + tile row
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int r0 = wave * 4 + (lane >> 4);
  // rows of consecutive batch slices are contiguous, so tile row trb starts at row trb*br
  const int64_t base = trb * br * cols + tc * 128 + (lane & 15) * 8;
  Raw8 raw[kTiles][kRowsPerLane];
#pragma unroll
  for (int h = 0; h < kTiles; ++h)
#pragma unroll
    for (int k = 0; k < kRowsPerLane; ++k) {
      const int r = r0 + kRowStep * k;
      raw[h][k] = r < br ? load_raw8(x + base + 128 * h + (int64_t)r * cols) : Raw8{};
    }
  uint32_t m[kTiles];
#pragma unroll
  for (int h = 0; h < kTiles; ++h) {
    m[h] = 0;
#pragma unroll
    for (int k = 0; k < kRowsPerLane; ++k) {
      float v[8];
      widen8(raw[h][k], x, v);
      m[h] = max(m[h], as_u(absmax8(v)));
    }
    m[h] = wave_umax(m[h]);
    if (lane == 0) red[h * kWaves + wave] = m[h];
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < kTiles; ++h) {
#pragma unroll
    for (int i = 0; i < kWaves; ++i) m[h] = max(m[h], red[h * kWaves + i]);
    const float s = fp8_scale_bits<kElem>(m[h]);
    const float y = recip_rn(s);
#pragma unroll
    for (int k = 0; k < kRowsPerLane; ++k) {
      const int r = r0 + kRowStep * k;
      float v[8];
      widen8(raw[h][k], x, v);
      const uint2 w = fp8_pack8<kElem>(v, s, y);
      if (r < br) store_codes8(codes + base + 128 * h + (int64_t)r * cols, w);
    }
    if (threadIdx.x == 0) scales[t + h] = s;
  }
}

// One row per wave, held in registers (cols % 8 == 0, cols <= 512 * kMaxU).
template <typename T, int kMaxU, int kElem = kE4M3>
__device__ __forceinline__ void fp8_row_vec(const T* __restrict__ x, int64_t row, int64_t cols,
                                            uint8_t* __restrict__ codes,
                                            float* __restrict__ scales) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t upr = cols / 8;
  const T* xr = x + row * cols;
  Raw8 raw[kMaxU];
#pragma unroll
  for (int k = 0; k < kMaxU; ++k) {
    const int64_t u = (int64_t)k * kWave + lane;
    raw[k] = u < upr ? load_raw8(xr + u * 8) : Raw8{};
  }
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < kMaxU; ++k) {
    float v[8];
    widen8(raw[k], x, v);
    m = max(m, as_u(absmax8(v)));
  }
  const float s = fp8_scale_bits<kElem>(wave_umax(m));
  const float y = recip_rn(s);
#pragma unroll
  for (int k = 0; k < kMaxU; ++k) {
    const int64_t u = (int64_t)k * kWave + lane;
    float v[8];
    widen8(raw[k], x, v);
    const uint2 w = fp8_pack8<kElem>(v, s, y);
    if (u < upr) store_codes8(codes + row * cols + u * 8, w);
  }
  if (lane == 0) scales[row] = s;
}

// One row per wave, any width, element-wise (the second read hits the caches).
template <typename T, int kElem = kE4M3>
__device__ __forceinline__ void fp8_row_any(const T* __restrict__ x, int64_t row, int64_t cols,
                                            uint8_t* __restrict__ codes,
                                            float* __restrict__ scales) {
  const int lane = threadIdx.x & (kWave - 1);
  const T* xr = x + row * cols;
  uint32_t m = 0;
  for (int64_t c = lane; c < cols; c += kWave) m = max(m, as_u(fabsf(ld1(xr + c))));
  const float s = fp8_scale_bits<kElem>(wave_umax(m));
  const float y = recip_rn(s);
  for (int64_t c = lane; c < cols; c += kWave)
    codes[row * cols + c] = elem_byte<kElem>(div_rn(ld1(xr + c), s, y));
  if (lane == 0) scales[row] = s;
}

// ---------------------------------------------------------------------------
// MXFP4 (same section): a 32-element block shares 2^X, X = floor(log2 max(amax,
// 1e-12)) - 2 (the unbiased exponent of a normal float minus 2), stored as
// the E8M0 byte X + 127.  A block is 4 lanes x 8 elements.  y = x * 2^-X is
// exactly RN(x / 2^X), so the E2M1 table (built with neg_zero_nibble 0) sees
// the page's quotient, signed zeros included.
// ---------------------------------------------------------------------------
template <typename T, int kUnr, bool kGuard>
__device__ __forceinline__ void mx_pack(const T* __restrict__ x, const Raw8 (&raw)[kUnr], int64_t u0,
                                        int64_t nunits, uint8_t* __restrict__ codes,
                                        uint8_t* __restrict__ scales, const uint8_t* lut) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int k = 0; k < kUnr; ++k) {
    float v[8];
    widen8(raw[k], x, v);
    const uint32_t a = max(group_umax<4>(as_u(absmax8(v))), kAmaxFloorBits);
    const uint32_t ef = a >> 23;                // biased exponent of a normal a
    const float mul = as_f((256u - ef) << 23);  // 2^-X with X = ef - 129
    uint32_t w = lut[e2m1_key(v[0] * mul)];
#pragma unroll
    for (int i = 1; i < 8; ++i) w |= (uint32_t)lut[e2m1_key(v[i] * mul)] << (4 * i);
    const int64_t u = u0 + k * kWave + lane;
    if (!kGuard || u < nunits) {
      st_nt4(codes + u * 4, w);
      if ((lane & 3) == 0) scales[u >> 2] = (uint8_t)(ef - 2u);
    }
  }
}

// Load and pack one chunk (the loads may instead be issued earlier, then
// mx_pack called on the raw tiles).
template <typename T, int kUnr, bool kGuard>
__device__ __forceinline__ void mx_chunk(const T* __restrict__ x, int64_t u0, int64_t nunits,
                                         uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                         const uint8_t* lut) {
  Raw8 raw[kUnr];
  load_chunk<T, kUnr, kGuard>(x, u0, nunits, raw);
  mx_pack<T, kUnr, kGuard>(x, raw, u0, nunits, codes, scales, lut);
}

// ---------------------------------------------------------------------------
// NVFP4 (page "量化部署实战", section 伪量化实现), pass 2: 2 lanes x 8 elements
// per 16-element block.  The block scale code is E4M3((amax_b / 6) / gs); the
// element scale of every finite code, s = max(dec(code), 1e-12) * gs, and
// RN(1/s) come from a table in LDS, as does the E2M1 rule.
// ---------------------------------------------------------------------------
struct __align__(16) NvTables {
  uint8_t lut[kE2M1LutSize];
  float se[128], ye[128];
};

template <typename T, int kUnr, bool kGuard>
__device__ __forceinline__ void nv_pack(const T* __restrict__ xs, const Raw8 (&raw)[kUnr], int64_t u0,
                                        int64_t nunits, uint8_t* __restrict__ cs,
                                        uint8_t* __restrict__ ss, float gs, float ygs,
                                        const NvTables& tb) {
  const int lane = threadIdx.x & (kWave - 1);
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

// ---------------------------------------------------------------------------
// Decoders shared by the dequantization kernels.
// ---------------------------------------------------------------------------
// Eight codes (two dwords) -> eight values times s.
template <int kElem, bool kHi>
__device__ __forceinline__ f32x2 elem_decode2(uint32_t w) {
  if constexpr (kElem == kE5M2)
    return e5m2x2_decode<kHi>(w);
  else if constexpr (kElem == kI8)
    return int8x2_decode<kHi>(w);
  else
    return e4m3x2_decode<kHi>(w);
}

template <int kElem = kE4M3>
__device__ __forceinline__ void fp8_decode8(uint2 w, float s, float o[8]) {
  const f32x2 a = elem_decode2<kElem, false>(w.x), b = elem_decode2<kElem, true>(w.x);
  const f32x2 c = elem_decode2<kElem, false>(w.y), d = elem_decode2<kElem, true>(w.y);
  o[0] = a.x * s; o[1] = a.y * s; o[2] = b.x * s; o[3] = b.y * s;
  o[4] = c.x * s; o[5] = c.y * s; o[6] = d.x * s; o[7] = d.y * s;
}


// ---------------------------------------------------------------------------
// MXFP8 (32-element blocks, E8M0 scale, E4M3 elements; pages "LLM 推理优化 ·
// 量化学习笔记" §4.2 / §4.5): 2^X with X = floor(log2 max(amax, 1e-12)) - 8
// (E4M3's largest exponent is 8, as 2 is E2M1's for MXFP4); codes
// E4M3(clamp(x * 2^-X, +-448)), where x * 2^-X is exact and the block maximum
// lands in [256, 512), so the clamp binds for large significands.  A block is 4
// lanes x 8 elements; the scale byte is X + 127.
// ---------------------------------------------------------------------------
template <typename T, int kUnr, bool kGuard>
__device__ __forceinline__ void mx8_chunk(const T* __restrict__ x, int64_t u0, int64_t nunits,
                                          uint8_t* __restrict__ codes,
                                          uint8_t* __restrict__ scales) {
  const int lane = threadIdx.x & (kWave - 1);
  Raw8 raw[kUnr];
  load_chunk<T, kUnr, kGuard>(x, u0, nunits, raw);
#pragma unroll
  for (int k = 0; k < kUnr; ++k) {
    float v[8];
    widen8(raw[k], x, v);
    const uint32_t a = max(group_umax<4>(as_u(absmax8(v))), kAmaxFloorBits);
    const uint32_t ef = a >> 23;                // biased exponent of a normal a
    const float mul = as_f((262u - ef) << 23);  // 2^-X with X = ef - 135
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = __builtin_amdgcn_fmed3f(v[i] * mul, -448.0f, 448.0f);
    const uint2 w = make_uint2(e4m3_bytes4(q[0], q[1], q[2], q[3]),
                               e4m3_bytes4(q[4], q[5], q[6], q[7]));
    const int64_t u = u0 + k * kWave + lane;
    if (!kGuard || u < nunits) {
      store_codes8(codes + u * 8, w);
      if ((lane & 3) == 0) scales[u >> 2] = (uint8_t)(ef - 8u);
    }
  }
}

// ---------------------------------------------------------------------------
// INT4 group-128 asymmetric: integers -8..7 with one scale and zero-point per
// 128 elements (page "量化部署实战", 格式速查); q = clamp(round(x / s) + z, qmin,
// qmax) ("LLM 推理优化 · 量化 学习笔记" §5.1); 2-byte scale per 128 ("14. 量化：
// 让每一步搬更少的字节", 量化在做什么).  The group range [lo, hi] is widened to
// hold 0, its 15 steps give s = bf16(max(hi - lo, 1e-12) / 15) (the rounded s
// is the one used), and z = -8 - rint(lo / s) puts lo on -8.  A group is 16
// lanes x 8 elements; zero-points are two per byte over the flat group index
// (group 2j in lanes 0-15 of a 32-lane half, group 2j+1 in lanes 16-31).
// ---------------------------------------------------------------------------
template <typename T, int kUnr, bool kGuard>
__device__ __forceinline__ void int4_chunk(const T* __restrict__ x, int64_t u0, int64_t nunits,
                                           uint8_t* __restrict__ codes,
                                           uint16_t* __restrict__ scales,
                                           uint8_t* __restrict__ zeros) {
  const int lane = threadIdx.x & (kWave - 1);
  Raw8 raw[kUnr];
  load_chunk<T, kUnr, kGuard>(x, u0, nunits, raw);
#pragma unroll
  for (int k = 0; k < kUnr; ++k) {
    float v[8];
    widen8(raw[k], x, v);
    // hi = max(0, max x) >= 0 and -lo = -min(0, min x) >= 0, reduced as bit
    // patterns.  A lane whose values are all on one side yields a zero that may
    // be -0.0; taking |.| first keeps its pattern 0 so it cannot win the max.
    const float h = max3f(max3f(v[0], v[1], v[2]), max3f(v[3], v[4], v[5]), max3f(v[6], v[7], 0.0f));
    const float l = min3f(min3f(v[0], v[1], v[2]), min3f(v[3], v[4], v[5]), min3f(v[6], v[7], 0.0f));
    const float hi = as_f(group_umax<16>(as_u(fabsf(h))));
    const float lo = -as_f(group_umax<16>(as_u(fabsf(l))));
    const float t = div_const(as_f(max(as_u(hi - lo), kAmaxFloorBits)), 15.0f, kInv15);
    const uint32_t sb = bf16_rne_bits(t);
    const float s = as_f(sb << 16);
    const float y = recip_rn(s);
    // div_rn commutes with negation, so it also gives RN(lo / s) for lo <= 0
    const float z = fminf(fmaxf(-8.0f - rintf(div_rn(lo, s, y)), -8.0f), 7.0f);
    // q + 8 = rint(x / s) + z + 8, clamped to [0, 15]: the integer sits in the low
    // bits of x/s + 1.5 * 2^23
    const int zofs = (int)z + 8 - (int)0x4B400000;
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = (int)as_u(div_rn(v[i], s, y) + kRound) + zofs;
      w |= (uint32_t)min(max(q, 0), 15) << (4 * i);
    }
    w ^= 0x88888888u;  // offset binary -> two's-complement nibbles
    const int zn = ((int)z) & 15;
    const int zn_odd = __shfl_down(zn, 16);
    const int64_t u = u0 + k * kWave + lane;
    if (!kGuard || u < nunits) {
      st_nt4(reinterpret_cast<uint32_t*>(codes) + u, w);
      if ((lane & 15) == 0) scales[u >> 4] = (uint16_t)sb;
      if ((lane & 31) == 0) zeros[u >> 5] = (uint8_t)(zn | ((u + 16 < nunits ? zn_odd : 0) << 4));
    }
  }
}

}  // namespace pqb
