// KIVI-style 2- or 4-bit KV quantization (page "量化部署实战", KV Cache 量化
// section: K per channel with a zero-point absorbs the constant bias; "14. 量化：
// 让每一步搬更少的字节", 路线三: KIVI quantizes K per channel and V per token):
// for a group with minimum m (a zero minimum taken as +0) and maximum M,
// s = RN(max(M - m, 1e-12) / (2^b - 1)), q = clamp(rint(RN((x - m) / s)), 0,
// 2^b - 1), dequant RN(RN(q * s) + m).
// K groups are 32 tokens of one channel, V groups 32 channels of one token.
// Layout [layers, tokens, heads, head_dim]; codes packed along the flat index
// (element i at bits b * (i % (8 / b)) of byte i * b / 8); float32 scales and
// minimums, K [layers, tokens / 32, heads, head_dim], V [layers, tokens, heads,
// head_dim / 32].
//
// K: a lane owns 4 channels of one 32-token group: it issues all 32 row loads
// (8 bytes of bf16, 16 of float32 each; consecutive lanes read consecutive
// channels), takes min and max per channel in registers, then writes the 4
// codes of each row (1 or 2 bytes, contiguous across the wave) and the 4
// scales and minimums as one 16-byte store each.  V: a lane owns one unit of 8
// channels, a group is 4 lanes (DPP min / max), one chunk of tiles per wave.
// Store kinds were chosen by measurement on the full 28 x 32768 x 8 x 128 cache:
// nontemporal for the 2-byte code stores (K 4-bit, V 2-bit) and the 4-byte V
// 4-bit codes; ordinary stores for single code bytes and for the V scales and
// minimums, where nontemporal stores ran up to 9% slower.
#include "launch.h"
#include "quant.h"

namespace pqb {
namespace {

// Float min / max over aligned groups of kLanes lanes (DPP on the bit patterns).
template <int kLanes>
__device__ __forceinline__ float group_fmax(float v) {
  if constexpr (kLanes >= 2) v = fmaxf(v, as_f(dpp<kDppXor1>(as_u(v))));
  if constexpr (kLanes >= 4) v = fmaxf(v, as_f(dpp<kDppXor2>(as_u(v))));
  return v;
}
template <int kLanes>
__device__ __forceinline__ float group_fmin(float v) {
  if constexpr (kLanes >= 2) v = fminf(v, as_f(dpp<kDppXor1>(as_u(v))));
  if constexpr (kLanes >= 4) v = fminf(v, as_f(dpp<kDppXor2>(as_u(v))));
  return v;
}

template <int kBits>
struct KiviLevels {
  static constexpr float qmax = (float)((1 << kBits) - 1), inv = 1.0f / qmax;
};

// Division parameters of a group with scale s: RN(a / s) is taken as RN((a f)
// / (s f)) with f = 2^-4 when s >= 2^126, so that the reciprocal y = RN(1 /
// (s f)) stays normal (recip_rn is exact below 2^126); f = 1 otherwise.  a f is
// exact unless a < 2^-122, where the quotient is below 2^-248 and the code is 0
// either way.
struct KiviDiv {
  float f, sf, y;
};

__device__ __forceinline__ KiviDiv kivi_div(float s) {
  const float f = s >= 0x1p126f ? 0x1p-4f : 1.0f;
  const float sf = s * f;
  return KiviDiv{f, sf, recip_rn(sf)};
}

// Code of x in a group with minimum m: clamp(rint(RN(RN(x - m) / s)), 0, 2^b - 1).
// x - m >= 0, and the quotient is at most 2^b - 1 up to one rounding.
template <int kBits>
__device__ __forceinline__ uint32_t kivi_code(float x, float m, const KiviDiv& d) {
  const float q = __builtin_amdgcn_fmed3f(rintf(div_rn((x - m) * d.f, d.sf, d.y)), 0.0f,
                                          KiviLevels<kBits>::qmax);
  return (uint32_t)q;
}

template <int kBits>
__device__ __forceinline__ float kivi_scale(float mn, float mx) {
  return div_const(fmaxf(mx - mn, 1e-12f), KiviLevels<kBits>::qmax, KiviLevels<kBits>::inv);
}

// Four channels of one row: raw bf16 (two dwords) or float32 (four dwords).
template <typename T>
struct Raw4 {
  uint32_t w[sizeof(T) == 2 ? 2 : 4];
};

template <typename T>
__device__ __forceinline__ Raw4<T> load4(const T* p) {
  Raw4<T> r;
  if constexpr (sizeof(T) == 2) {
    const uint2 v = ld_nt8(p);
    r.w[0] = v.x;
    r.w[1] = v.y;
  } else {
    const uint4 v = ld_nt16(p);
    r.w[0] = v.x;
    r.w[1] = v.y;
    r.w[2] = v.z;
    r.w[3] = v.w;
  }
  return r;
}

template <typename T>
__device__ __forceinline__ void widen4(const Raw4<T>& r, float v[4]) {
  if constexpr (sizeof(T) == 2) {
    v[0] = as_f(r.w[0] << 16);
    v[1] = as_f(r.w[0] & 0xFFFF0000u);
    v[2] = as_f(r.w[1] << 16);
    v[3] = as_f(r.w[1] & 0xFFFF0000u);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = as_f(r.w[i]);
  }
}

// K: thread t owns channels [4c, 4c + 4) of token group `slab` (= layer * (T /
// 32) + token group), with c = t % R4, R4 = heads * head_dim / 4.
// slab = t / R4 and c = t % R4, in 32 bits while the thread count fits (a
// 64-bit division is a routine of its own in every thread).
__device__ __forceinline__ void slab_of(int64_t t, int64_t nthreads, int64_t R4, int64_t& slab,
                                        int64_t& c) {
  if (nthreads <= (int64_t)UINT32_MAX) {
    const uint32_t s32 = (uint32_t)t / (uint32_t)R4;
    slab = s32;
    c = (int64_t)((uint32_t)t - s32 * (uint32_t)R4);
  } else {
    slab = t / R4;
    c = t - slab * R4;
  }
}

template <typename T, int kBits>
__global__ __launch_bounds__(kBlockThreads) void k_kivi_k(const T* __restrict__ x, int64_t nslabs,
                                                          int64_t R4, uint8_t* __restrict__ codes,
                                                          float* __restrict__ scales,
                                                          float* __restrict__ mins) {
  const int64_t t = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x;
  if (t >= nslabs * R4) return;
  int64_t slab, c;
  slab_of(t, nslabs * R4, R4, slab, c);
  const int64_t row = 4 * R4;  // row length in elements
  const T* base = x + slab * 32 * row + 4 * c;
  Raw4<T> r[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) r[i] = load4(base + i * row);
  float mn[4], mx[4];
  {
    float v[4];
    widen4(r[0], v);
#pragma unroll
    for (int j = 0; j < 4; ++j) mn[j] = mx[j] = v[j];
  }
#pragma unroll
  for (int i = 1; i < 32; ++i) {
    float v[4];
    widen4(r[i], v);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      mn[j] = fminf(mn[j], v[j]);
      mx[j] = fmaxf(mx[j], v[j]);
    }
  }
  float s[4];
  KiviDiv d[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    mn[j] += 0.0f;  // a zero minimum is +0 whatever the signs of the zeros
    s[j] = kivi_scale<kBits>(mn[j], mx[j]);
    d[j] = kivi_div(s[j]);
  }
  const int64_t g0 = slab * row + 4 * c;  // group index of channel 0 of this lane
  st_nt16(scales + g0, as_u(s[0]), as_u(s[1]), as_u(s[2]), as_u(s[3]));
  st_nt16(mins + g0, as_u(mn[0]), as_u(mn[1]), as_u(mn[2]), as_u(mn[3]));
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float v[4];
    widen4(r[i], v);
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) w |= kivi_code<kBits>(v[j], mn[j], d[j]) << (kBits * j);
    const int64_t e0 = (slab * 32 + i) * row + 4 * c;  // flat index of channel 0
    if constexpr (kBits == 4)
      st_nt2(codes + e0 / 2, w);
    else
      codes[e0 / 4] = (uint8_t)w;
  }
}

// V: unit u (8 channels) belongs to group u / 4; one chunk of kUnr tiles per wave.
template <typename T, int kUnr, int kBits, bool kGuard>
__device__ __forceinline__ void kivi_v_chunk(const T* __restrict__ x, int64_t u0, int64_t nunits,
                                             uint8_t* __restrict__ codes,
                                             float* __restrict__ scales,
                                             float* __restrict__ mins) {
  const int lane = threadIdx.x & (kWave - 1);
  Raw8 raw[kUnr];
  load_chunk<T, kUnr, kGuard>(x, u0, nunits, raw);
#pragma unroll
  for (int k = 0; k < kUnr; ++k) {
    float v[8];
    widen8(raw[k], x, v);
    const float mn = group_fmin<4>(min3f(min3f(v[0], v[1], v[2]), min3f(v[3], v[4], v[5]),
                                         fminf(v[6], v[7]))) + 0.0f;  // -0 becomes +0
    const float mx = group_fmax<4>(max3f(max3f(v[0], v[1], v[2]), max3f(v[3], v[4], v[5]),
                                         fmaxf(v[6], v[7])));
    const float s = kivi_scale<kBits>(mn, mx);
    const KiviDiv d = kivi_div(s);
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= kivi_code<kBits>(v[i], mn, d) << (kBits * i);
    const int64_t u = u0 + k * kWave + lane;
    if (!kGuard || u < nunits) {
      if constexpr (kBits == 4)
        st_nt4(codes + 4 * u, w);
      else
        st_nt2(codes + 2 * u, w);
      if ((lane & 3) == 0) {
        scales[u >> 2] = s;
        mins[u >> 2] = mn;
      }
    }
  }
}

template <typename T, int kUnr, int kBits>
__global__ __launch_bounds__(kBlockThreads) void k_kivi_v(const T* __restrict__ x, int64_t nunits,
                                                          uint8_t* __restrict__ codes,
                                                          float* __restrict__ scales,
                                                          float* __restrict__ mins) {
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int64_t u0 = ((int64_t)blockIdx.x * (kBlockThreads / kWave) + wave) * kUnr * kWave;
  if (u0 >= nunits) return;
  if (u0 + kUnr * kWave <= nunits)
    kivi_v_chunk<T, kUnr, kBits, false>(x, u0, nunits, codes, scales, mins);
  else
    kivi_v_chunk<T, kUnr, kBits, true>(x, u0, nunits, codes, scales, mins);
}

// q * s + m with two roundings, as the dequantization formula is written (the
// library is built with -ffp-contract=off, so no fused multiply-add forms).
__device__ __forceinline__ float kivi_value(uint32_t q, float s, float m) {
  const float p = (float)q * s;
  return p + m;
}

template <bool kBf16Out, int kBits>
__global__ __launch_bounds__(kBlockThreads) void k_kivi_k_dequant(const uint8_t* __restrict__ codes,
                                                                  const float* __restrict__ scales,
                                                                  const float* __restrict__ mins,
                                                                  int64_t nslabs, int64_t R4,
                                                                  void* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x;
  if (t >= nslabs * R4) return;
  int64_t slab, c;
  slab_of(t, nslabs * R4, R4, slab, c);
  const int64_t row = 4 * R4;
  const int64_t g0 = slab * row + 4 * c;
  const uint4 sv = *reinterpret_cast<const uint4*>(scales + g0);
  const uint4 mv = *reinterpret_cast<const uint4*>(mins + g0);
  const float s[4] = {as_f(sv.x), as_f(sv.y), as_f(sv.z), as_f(sv.w)};
  const float m[4] = {as_f(mv.x), as_f(mv.y), as_f(mv.z), as_f(mv.w)};
  // The codes of all 32 rows are loaded before the first store (4-bit codes
  // as nontemporal loads).
  uint32_t ws[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    if constexpr (kBits == 4)
      ws[i] = __builtin_nontemporal_load(
          reinterpret_cast<const uint16_t*>(codes + ((slab * 32 + i) * row + 4 * c) / 2));
    else
      ws[i] = codes[((slab * 32 + i) * row + 4 * c) / 4];
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int64_t e0 = (slab * 32 + i) * row + 4 * c;
    const uint32_t w = ws[i];
    float o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = kivi_value((w >> (kBits * j)) & ((1u << kBits) - 1), s[j], m[j]);
    if constexpr (kBf16Out) {
      uint16_t* p = reinterpret_cast<uint16_t*>(out) + e0;
      st_nt8(p, bf16x2_rne(o[0], o[1]), bf16x2_rne(o[2], o[3]));
    } else {
      st_nt16(reinterpret_cast<float*>(out) + e0, as_u(o[0]), as_u(o[1]), as_u(o[2]), as_u(o[3]));
    }
  }
}

// V dequantize: each wave owns kVdTiles wave-wide tiles of units (lane unit
// u0 + 64 k + lane); all code and parameter loads are issued before the stores.
constexpr int kVdTiles = 4;

template <bool kBf16Out, int kBits>
__global__ __launch_bounds__(kBlockThreads) void k_kivi_v_dequant(const uint8_t* __restrict__ codes,
                                                                  const float* __restrict__ scales,
                                                                  const float* __restrict__ mins,
                                                                  int64_t nunits,
                                                                  void* __restrict__ out) {
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int64_t u0 = ((int64_t)blockIdx.x * (kBlockThreads / kWave) + wave) * kVdTiles * kWave +
                     (threadIdx.x & (kWave - 1));
  uint32_t w[kVdTiles];
  float s[kVdTiles], m[kVdTiles];
#pragma unroll
  for (int k = 0; k < kVdTiles; ++k) {
    const int64_t u = u0 + k * kWave;
    if (u < nunits) {
      w[k] = kBits == 4 ? reinterpret_cast<const uint32_t*>(codes)[u]
                        : reinterpret_cast<const uint16_t*>(codes)[u];
      s[k] = scales[u >> 2];
      m[k] = mins[u >> 2];
    }
  }
#pragma unroll
  for (int k = 0; k < kVdTiles; ++k) {
    const int64_t u = u0 + k * kWave;
    if (u < nunits) {
      float o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        o[i] = kivi_value((w[k] >> (kBits * i)) & ((1u << kBits) - 1), s[k], m[k]);
      store_out8<kBf16Out>(out, u, o);
    }
  }
}

template <typename F>
hipError_t with_bits(int bits, F f) {
  if (bits == 2)
    f(std::integral_constant<int, 2>{});
  else if (bits == 4)
    f(std::integral_constant<int, 4>{});
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

int grid_of(int64_t threads) { return (int)((threads + kBlockThreads - 1) / kBlockThreads); }

}  // namespace

hipError_t launch_kivi_k(const void* x, bool bf16, int64_t layers, int64_t tokens, int64_t heads,
                         int64_t head_dim, int bits, uint8_t* codes, float* scales, float* mins,
                         hipStream_t st) {
  const int64_t nslabs = layers * (tokens / 32), R4 = heads * head_dim / 4;
  return with_bits(bits, [&](auto b) {
    constexpr int B = decltype(b)::value;
    if (bf16)
      hipLaunchKernelGGL((k_kivi_k<uint16_t, B>), dim3(grid_of(nslabs * R4)), dim3(kBlockThreads),
                         0, st, (const uint16_t*)x, nslabs, R4, codes, scales, mins);
    else
      hipLaunchKernelGGL((k_kivi_k<float, B>), dim3(grid_of(nslabs * R4)), dim3(kBlockThreads), 0,
                         st, (const float*)x, nslabs, R4, codes, scales, mins);
  });
}

hipError_t launch_kivi_v(const void* x, bool bf16, int64_t n, int bits, uint8_t* codes,
                         float* scales, float* mins, hipStream_t st) {
  const int64_t nunits = n / 8, waves = kBlockThreads / kWave;
  return with_bits(bits, [&](auto b) {
    constexpr int B = decltype(b)::value;
    if (bf16) {
      const int64_t per_wg = 8 * kWave * waves;
      hipLaunchKernelGGL((k_kivi_v<uint16_t, 8, B>), dim3((unsigned)((nunits + per_wg - 1) / per_wg)),
                         dim3(kBlockThreads), 0, st, (const uint16_t*)x, nunits, codes, scales,
                         mins);
    } else {
      const int64_t per_wg = 4 * kWave * waves;
      hipLaunchKernelGGL((k_kivi_v<float, 4, B>), dim3((unsigned)((nunits + per_wg - 1) / per_wg)),
                         dim3(kBlockThreads), 0, st, (const float*)x, nunits, codes, scales, mins);
    }
  });
}

hipError_t launch_kivi_k_dequant(const uint8_t* codes, const float* scales, const float* mins,
                                 int64_t layers, int64_t tokens, int64_t heads, int64_t head_dim,
                                 int bits, bool out_bf16, void* out, hipStream_t st) {
  const int64_t nslabs = layers * (tokens / 32), R4 = heads * head_dim / 4;
  return with_bits(bits, [&](auto b) {
    constexpr int B = decltype(b)::value;
    if (out_bf16)
      hipLaunchKernelGGL((k_kivi_k_dequant<true, B>), dim3(grid_of(nslabs * R4)),
                         dim3(kBlockThreads), 0, st, codes, scales, mins, nslabs, R4, out);
    else
      hipLaunchKernelGGL((k_kivi_k_dequant<false, B>), dim3(grid_of(nslabs * R4)),
                         dim3(kBlockThreads), 0, st, codes, scales, mins, nslabs, R4, out);
  });
}

hipError_t launch_kivi_v_dequant(const uint8_t* codes, const float* scales, const float* mins,
                                 int64_t n, int bits, bool out_bf16, void* out, hipStream_t st) {
  const int64_t nunits = n / 8;
  const int grid = grid_of((nunits + kVdTiles - 1) / kVdTiles);
  return with_bits(bits, [&](auto b) {
    constexpr int B = decltype(b)::value;
    if (out_bf16)
      hipLaunchKernelGGL((k_kivi_v_dequant<true, B>), dim3(grid), dim3(kBlockThreads), 0, st, codes,
                         scales, mins, nunits, out);
    else
      hipLaunchKernelGGL((k_kivi_v_dequant<false, B>), dim3(grid), dim3(kBlockThreads), 0, st,
                         codes, scales, mins, nunits, out);
  });
}

}  // namespace pqb
