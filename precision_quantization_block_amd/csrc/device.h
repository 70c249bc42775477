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
__device__ __forceinline__ uint2 ld_nt8(const void* p) {
  u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ void st_nt1(void* p, uint32_t w) {
  __builtin_nontemporal_store((uint8_t)w, reinterpret_cast<uint8_t*>(p));
}
__device__ __forceinline__ void st_nt2(void* p, uint32_t w) {
  __builtin_nontemporal_store((uint16_t)w, reinterpret_cast<uint16_t*>(p));
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

// Largest |v| of eight values (|v| >= 0, inputs finite): four 3-input maxes
// (the third input of the last one is 0, which changes nothing for |v| >= 0).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
}
__device__ __forceinline__ float min3f(float a, float b, float c) {
  return __builtin_fminf(__builtin_fminf(a, b), c);
}
__device__ __forceinline__ float absmax8(const float v[8]) {
  const float m1 = max3f(fabsf(v[0]), fabsf(v[1]), fabsf(v[2]));
  const float m2 = max3f(fabsf(v[3]), fabsf(v[4]), fabsf(v[5]));
  const float m3 = max3f(fabsf(v[6]), fabsf(v[7]), 0.0f);
  return max3f(m1, m2, m3);
}

// ---------------------------------------------------------------------------
// Cross-lane reductions with DPP inside a row of 16 lanes.
// ---------------------------------------------------------------------------

template <int kCtrl>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

// Max over aligned groups of kLanes lanes (2, 4, 8 or 16) of non-negative
// floats given as bit patterns (for those the unsigned order is the float
// order, and no NaN handling is needed); every lane of the group receives it.
template <int kLanes>
__device__ __forceinline__ uint32_t group_umax(uint32_t v) {
  if constexpr (kLanes >= 2) v = max(v, dpp<kDppXor1>(v));
  if constexpr (kLanes >= 4) v = max(v, dpp<kDppXor2>(v));
  if constexpr (kLanes >= 8) v = max(v, dpp<kDppHalfMirror>(v));
  if constexpr (kLanes >= 16) v = max(v, dpp<kDppMirror>(v));
  return v;
}

// Max of non-negative float bit patterns over the whole wave.
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  v = group_umax<16>(v);
  v = max(v, (uint32_t)__shfl_xor((int)v, 16));
  v = max(v, (uint32_t)__shfl_xor((int)v, 32));
  return v;
}

__device__ __forceinline__ float wave_max(float v) { return as_f(wave_umax(as_u(v))); }

// ---------------------------------------------------------------------------
// Correctly rounded division.
// ---------------------------------------------------------------------------

// RN(1/s) for every float s in [2^-64, 2^126): the hardware reciprocal and one
// Newton step, e = 1 - s*r and y = r + e*r, each rounded once.  This equals IEEE
// division for every float in that range (checked exhaustively on gfx950, all
// 1.6e9 values); every scale this library forms lies inside it.
__device__ __forceinline__ float recip_rn(float s) {
  const float r = __builtin_amdgcn_rcpf(s);
  return __builtin_fmaf(__builtin_fmaf(-s, r, 1.0f), r, r);
}

// RN(x / s) from y = RN(1/s): q = RN(x*y), then one Markstein correction with
// the residual r = s*q - x (P. Markstein, IBM J. Res. Dev. 34(1), 1990; Muller
// et al., Handbook of Floating-Point Arithmetic, division with an FMA).  For
// x, s with significands in [1, 2) the result equals IEEE division for all
// 2^46 pairs (checked exhaustively on gfx950); scaling by powers of two carries
// this to every x, s whose quotient and residual are normal.  Every step
// commutes with negating x, and the signed zeros come out as IEEE division
// gives them (x = -0 gives -0; a negative x never gives +0).  Where the
// quotient is below about 2^-100 it is only close to RN(x/s); every code this
// library derives from such a quotient is a code of zero.
__device__ __forceinline__ float div_rn(float x, float s, float y) {
  const float q = x * y;
  const float r = __builtin_fmaf(q, s, -x);
  return __builtin_fmaf(-r, y, q);
}

// RN(a / d) for a constant d with c = RN(1/d): the same correction.  For d in
// {6, 15, 448, 2688} this was checked against IEEE division for every
// significand in three consecutive binades (so for every normal a whose
// quotient is normal).
__device__ __forceinline__ float div_const(float a, float d, float c) { return div_rn(a, d, c); }

// ---------------------------------------------------------------------------
// Rounding to the target grids.
// ---------------------------------------------------------------------------

// Two float32 values -> two E4M3 bytes (round-to-nearest-even, subnormals kept,
// sign kept), written into the low (kHi = false) or high 16 bits of `old`.
template <bool kHi>
__device__ __forceinline__ uint32_t cvt_e4m3x2(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, kHi);
}

// Four values -> four E4M3 bytes.  The first conversion's untouched high half
// is overwritten by the second, so its starting value does not matter.
__device__ __forceinline__ uint32_t e4m3_bytes4(float a, float b, float c, float d) {
  uint32_t w = cvt_e4m3x2<false>(a, b, as_u(a));
  return cvt_e4m3x2<true>(c, d, w);
}

// Two values -> two E5M2 bytes (round-to-nearest-even, subnormals kept, sign
// kept), written into the low (kHi = false) or high 16 bits of `old`.
template <bool kHi>
__device__ __forceinline__ uint32_t cvt_e5m2x2(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, (int)old, kHi);
}

__device__ __forceinline__ uint32_t e5m2_bytes4(float a, float b, float c, float d) {
  uint32_t w = cvt_e5m2x2<false>(a, b, as_u(a));
  return cvt_e5m2x2<true>(c, d, w);
}

// Four integer-valued floats in [-128, 127] -> four two's-complement bytes:
// adding 1.5 * 2^23 rounds to an integer (ties to even) and leaves it in the
// low bits of the sum's pattern.
constexpr float kRoundInt = 12582912.0f;
__device__ __forceinline__ uint32_t int8_bytes4(float a, float b, float c, float d) {
  const uint32_t qa = as_u(a + kRoundInt), qb = as_u(b + kRoundInt);
  const uint32_t qc = as_u(c + kRoundInt), qd = as_u(d + kRoundInt);
  return (qa & 0xFFu) | ((qb & 0xFFu) << 8) | ((qc & 0xFFu) << 16) | (qd << 24);
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
// Keys below 501 have magnitude 0 and keys above 517 magnitude 7, so most
// 4-key dwords are constants; only the few around the decision points are
// computed key by key.
__device__ __forceinline__ uint32_t e2m1_entry(int k, int neg_zero_nibble) {
  constexpr int kT[7] = {500, 506, 509, 511, 513, 515, 517};  // bits(t) >> 21
  const int mag = k & 1023, neg = k >> 10;
  int m = 0;
#pragma unroll
  for (int j = 0; j < 7; ++j) m += mag > kT[j];
  return (uint32_t)(neg ? (mag > 0 ? 8 | m : neg_zero_nibble) : m);
}

__device__ __forceinline__ void e2m1_lut_fill(uint8_t* lut, int neg_zero_nibble) {
  uint32_t* w = reinterpret_cast<uint32_t*>(lut);
  for (int d = threadIdx.x; d < kE2M1LutSize / 4; d += blockDim.x) {
    const int k0 = 4 * d, mag0 = k0 & 1023;
    const uint32_t sign = (k0 >> 10) ? 0x08080808u : 0u;
    uint32_t word;
    if (mag0 >= 4 && mag0 + 3 <= 500) {
      word = sign;                 // magnitude 0
    } else if (mag0 >= 518) {
      word = sign | 0x07070707u;   // magnitude 7 (saturated at 6)
    } else {
      word = e2m1_entry(k0, neg_zero_nibble) | (e2m1_entry(k0 + 1, neg_zero_nibble) << 8) |
             (e2m1_entry(k0 + 2, neg_zero_nibble) << 16) |
             (e2m1_entry(k0 + 3, neg_zero_nibble) << 24);
    }
    w[d] = word;
  }
}

// Round-to-nearest-even of a float32 to bf16 bits (integer form).
__device__ __forceinline__ uint32_t bf16_rne_bits(float v) {
  uint32_t b = as_u(v);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Two float32 -> two bf16 (round-to-nearest-even) packed in one dword, low
// half first; the hardware conversion.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// ---------------------------------------------------------------------------
// E4M3 decode (for dequantization).  Every E4M3 value is a float32, so the
// hardware conversion is exact; NaN codes never occur in quantizer output.
// ---------------------------------------------------------------------------
template <bool kHi>
__device__ __forceinline__ f32x2 e4m3x2_decode(uint32_t w) {
  const auto v = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, kHi);
  return f32x2{v[0], v[1]};
}

__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)(c & 0xFFu), false)[0];
}

template <bool kHi>
__device__ __forceinline__ f32x2 e5m2x2_decode(uint32_t w) {
  const auto v = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, kHi);
  return f32x2{v[0], v[1]};
}

template <bool kHi>
__device__ __forceinline__ f32x2 int8x2_decode(uint32_t w) {
  const int sh = kHi ? 16 : 0;
  return f32x2{(float)((int)(w << (24 - sh)) >> 24), (float)((int)(w << (16 - sh)) >> 24)};
}

// Eight float32 results stored as float32 or as RNE bf16 at unit u (element 8u).
template <bool kBf16Out>
__device__ __forceinline__ void store_out8(void* out, int64_t u, const float o[8]) {
  if constexpr (kBf16Out) {
    st_nt16(reinterpret_cast<uint16_t*>(out) + 8 * u, bf16x2_rne(o[0], o[1]),
            bf16x2_rne(o[2], o[3]), bf16x2_rne(o[4], o[5]), bf16x2_rne(o[6], o[7]));
  } else {
    float* p = reinterpret_cast<float*>(out) + 8 * u;
    st_nt16(p, as_u(o[0]), as_u(o[1]), as_u(o[2]), as_u(o[3]));
    st_nt16(p + 4, as_u(o[4]), as_u(o[5]), as_u(o[6]), as_u(o[7]));
  }
}

// Bit pattern of max(amax, 1e-12f), the floor every scale formula applies.
constexpr uint32_t kAmaxFloorBits = __builtin_bit_cast(uint32_t, 1e-12f);

// Wave index that the compiler knows to be uniform across the wave.
__device__ __forceinline__ int wave_index() {
  return __builtin_amdgcn_readfirstlane((int)(blockIdx.x * (kBlockThreads / kWave) +
                                              threadIdx.x / kWave));
}

}  // namespace pqb
