// Device building blocks shared by the pqb kernels (gfx950, wave64).
//
// Arithmetic contract: IEEE binary32, round-to-nearest-even, subnormals kept.
// The library is compiled with -ffp-contract=off, so every fused multiply-add
// below is written out explicitly and nothing else is fused.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pqb {

constexpr int kWave = 64;
constexpr int kBlockThreads = 256;

__device__ __forceinline__ float as_f(uint32_t b) { return __uint_as_float(b); }
__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }

// ---------------------------------------------------------------------------
// Loads: eight consecutive elements per lane, widened exactly to float.
// ---------------------------------------------------------------------------

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) 16-byte load and 4/8/16-byte stores.
__device__ __forceinline__ uint4 ld_nt16(const void* p) {
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_nt4(void* p, uint32_t w) {
  __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(p));
}
__device__ __forceinline__ void st_nt8(void* p, uint32_t a, uint32_t b) {
  u32x2 v = {a, b};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ void st_nt16(void* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 v = {a, b, c, d};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

struct Raw8 {  // the 16 or 32 bytes one lane loads
  uint4 a, b;
};

__device__ __forceinline__ Raw8 load_raw8(const uint16_t* p) {
  Raw8 r;
  r.a = ld_nt16(p);
  r.b = make_uint4(0, 0, 0, 0);
  return r;
}

__device__ __forceinline__ Raw8 load_raw8(const float* p) {
  Raw8 r;
  r.a = ld_nt16(p);
  r.b = ld_nt16(p + 4);
  return r;
}

// Eight float32 results stored as float32 (32 bytes) or RNE bf16 (16 bytes) at
// unit u of `out` (element 8u).
__device__ __forceinline__ uint32_t bf16_rne_bits(float v);
template <bool kBf16Out>
__device__ __forceinline__ void store_out8(void* out, int64_t u, const float o[8]) {
  if constexpr (kBf16Out) {
    st_nt16(reinterpret_cast<uint16_t*>(out) + 8 * u,
            bf16_rne_bits(o[0]) | (bf16_rne_bits(o[1]) << 16),
            bf16_rne_bits(o[2]) | (bf16_rne_bits(o[3]) << 16),
            bf16_rne_bits(o[4]) | (bf16_rne_bits(o[5]) << 16),
            bf16_rne_bits(o[6]) | (bf16_rne_bits(o[7]) << 16));
  } else {
    float* p = reinterpret_cast<float*>(out) + 8 * u;
    st_nt16(p, __float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
            __float_as_uint(o[3]));
    st_nt16(p + 4, __float_as_uint(o[4]), __float_as_uint(o[5]), __float_as_uint(o[6]),
            __float_as_uint(o[7]));
  }
}

// bf16 -> f32 is a 16-bit shift of the bit pattern (exact).
__device__ __forceinline__ void widen8(const Raw8& r, const uint16_t*, float v[8]) {
  v[0] = as_f(r.a.x << 16); v[1] = as_f(r.a.x & 0xFFFF0000u);
  v[2] = as_f(r.a.y << 16); v[3] = as_f(r.a.y & 0xFFFF0000u);
  v[4] = as_f(r.a.z << 16); v[5] = as_f(r.a.z & 0xFFFF0000u);
  v[6] = as_f(r.a.w << 16); v[7] = as_f(r.a.w & 0xFFFF0000u);
}

__device__ __forceinline__ void widen8(const Raw8& r, const float*, float v[8]) {
  v[0] = as_f(r.a.x); v[1] = as_f(r.a.y); v[2] = as_f(r.a.z); v[3] = as_f(r.a.w);
  v[4] = as_f(r.b.x); v[5] = as_f(r.b.y); v[6] = as_f(r.b.z); v[7] = as_f(r.b.w);
}

// Largest |v| of eight values (|v| >= 0, inputs finite).
__device__ __forceinline__ float absmax8(const float v[8]) {
  float m0 = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fabsf(v[2]));
  float m1 = fmaxf(fmaxf(fabsf(v[3]), fabsf(v[4])), fabsf(v[5]));
  return fmaxf(fmaxf(m0, m1), fmaxf(fabsf(v[6]), fabsf(v[7])));
}

// ---------------------------------------------------------------------------
// Cross-lane reductions with DPP inside a row of 16 lanes.
// ---------------------------------------------------------------------------

template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return as_f(__builtin_amdgcn_update_dpp(0, (int)as_u(v), kCtrl, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

// Max (or min) over aligned groups of kLanes lanes (2, 4, 8 or 16); every
// lane of the group receives the result.
template <int kLanes>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (kLanes >= 2) v = fmaxf(v, dpp<kDppXor1>(v));
  if constexpr (kLanes >= 4) v = fmaxf(v, dpp<kDppXor2>(v));
  if constexpr (kLanes >= 8) v = fmaxf(v, dpp<kDppHalfMirror>(v));
  if constexpr (kLanes >= 16) v = fmaxf(v, dpp<kDppMirror>(v));
  return v;
}

template <int kLanes>
__device__ __forceinline__ float group_min(float v) {
  if constexpr (kLanes >= 2) v = fminf(v, dpp<kDppXor1>(v));
  if constexpr (kLanes >= 4) v = fminf(v, dpp<kDppXor2>(v));
  if constexpr (kLanes >= 8) v = fminf(v, dpp<kDppHalfMirror>(v));
  if constexpr (kLanes >= 16) v = fminf(v, dpp<kDppMirror>(v));
  return v;
}

// Max over the whole wave (every lane receives it).
__device__ __forceinline__ float wave_max(float v) {
  v = group_max<16>(v);
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// ---------------------------------------------------------------------------
// Correctly rounded division.
// ---------------------------------------------------------------------------

// RN(a / s) for a >= 0 from y = RN(1/s).  Markstein's correction (P.
// Markstein, IBM J. Res. Dev. 34(1), 1990; Muller et al., Handbook of
// Floating-Point Arithmetic, division with an FMA): when y is within half an
// ulp of 1/s and q is within one ulp of a/s, the residual r = a - s*q is exact
// and RN(q + r*y) = RN(a/s).  q0 = RN(a*y) can be up to 1.5 ulp off, so a first
// correction brings it within one ulp and the second one is exact.  (The
// residual is carried negated, s*q - a, which changes no value or rounding.)
// Exactness needs normal residuals: with s >= 2^-60 (every caller guarantees
// it or takes a true division instead) every quotient at or above 2^-20 is
// exact.  Smaller quotients come out within a few ulps and non-negative; every
// code this library derives from such a quotient is the code of zero.
__device__ __forceinline__ float div_mag(float a, float s, float y) {
  float q = a * y;
  float r = __builtin_fmaf(q, s, -a);
  q = __builtin_fmaf(-r, y, q);
  r = __builtin_fmaf(q, s, -a);
  return __builtin_fmaf(-r, y, q);
}

// |q| with the sign bit of x: RN(x / s) from the magnitude quotient (IEEE
// division gives its result the sign of x, zero included, since s > 0).
__device__ __forceinline__ float with_sign_of(float mag, float x) {
  return as_f((as_u(mag) & 0x7FFFFFFFu) | (as_u(x) & 0x80000000u));
}

// RN(a / d) for a constant d with c = RN(1/d): one Markstein correction.  For
// d in {3, 7, 15, 448, 6, 2688} this was checked against IEEE division for
// every significand in three consecutive binades (so for every normal a whose
// quotient is normal).
__device__ __forceinline__ float div_const(float a, float d, float c) {
  float q = a * c;
  float r = __builtin_fmaf(q, d, -a);
  return __builtin_fmaf(-r, c, q);
}

// ---------------------------------------------------------------------------
// Rounding to the target grids.
// ---------------------------------------------------------------------------

// Two float32 values -> two E4M3 bytes (round-to-nearest-even, subnormals kept,
// sign kept), written into the low (kHi = false) or high 16 bits of `old`.
template <bool kHi>
__device__ __forceinline__ uint32_t cvt_e4m3x2(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, kHi);
}

__device__ __forceinline__ uint32_t e4m3_bytes4(float a, float b, float c, float d) {
  uint32_t w = cvt_e4m3x2<false>(a, b, 0u);
  return cvt_e4m3x2<true>(c, d, w);
}

// E2M1 nibble of y (nearest value, ties to the smaller magnitude, sign bit for
// y < 0, saturating at 6) by table lookup.  The seven decision points 0.25,
// 0.75, 1.25, 1.75, 2.5, 3.5 and 5 are float32 values whose bit patterns are
// multiples of 2^21, so |y| > t exactly when ceil(bits(|y|) / 2^21) exceeds
// t's pattern / 2^21.  The key ceil(bits(y) / 2^21) therefore decides the
// nibble; a set sign bit adds 1024.  Key 1024 alone is -0.0: `neg_zero_nibble`
// says what it stands for (0 when it is a true -0.0 quotient, whose sign the
// rule drops; 8 when the caller has folded the sign of a nonzero negative x
// onto a magnitude quotient that is zero).
constexpr int kE2M1LutSize = 2048;

__device__ __forceinline__ uint32_t e2m1_key(float y) { return (as_u(y) + 0x1FFFFFu) >> 21; }

// Fill the table (call with all threads of the block, then __syncthreads()).
__device__ __forceinline__ void e2m1_lut_fill(uint8_t* lut, int neg_zero_nibble) {
  constexpr int kT[7] = {500, 506, 509, 511, 513, 515, 517};  // bits(t) >> 21
  for (int k = threadIdx.x; k < kE2M1LutSize; k += blockDim.x) {
    int mag = k & 1023, neg = k >> 10;
    int m = 0;
#pragma unroll
    for (int j = 0; j < 7; ++j) m += mag > kT[j];
    lut[k] = (uint8_t)(neg ? (mag > 0 ? 8 | m : neg_zero_nibble) : m);
  }
}

// Round-to-nearest-even of a float32 to bf16 bits.
__device__ __forceinline__ uint32_t bf16_rne_bits(float v) {
  uint32_t b = as_u(v);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------------
// E4M3 decode (for dequantization): code -> float (NaN codes never occur).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  // normal: 2^(e-7) * (1 + m/8); subnormal: m * 2^-9
  uint32_t nb = ((e + 120u) << 23) | (m << 20);
  float v = e ? as_f(nb) : (float)m * 0x1p-9f;
  return (c & 0x80u) ? -v : v;
}

}  // namespace pqb
