// Dequantization of the flat formats (page "量化部署实战", section 伪量化实现:
// the fake-quant functions return decoded code times scale, as float32).
//
// Lane l of a wave expands unit u = u0 + 64 k + l (8 elements) of each of the
// kDqTiles wave-wide tiles of its chunk: the wave's code loads (4 bytes of
// nibbles or 8 FP8 bytes per lane) and its 16-byte output stores (bf16; two
// for float32) each cover one contiguous range, so every store instruction
// writes whole 1 KiB (2 KiB) spans.  All loads of the chunk are issued before
// the first store.  Outputs are float32 or RNE bf16.
#include <vector>

#include "launch.h"
#include "quant.h"

namespace pqb {
namespace {

constexpr int kDqTiles = 4;
constexpr int kDqWaves = kBlockThreads / kWave;

// Unit of this lane in tile 0 of its wave's chunk, for workgroup `blk` of a
// job (blockIdx.x in the single-tensor kernels, the job-local index in the
// batch kernel).
__device__ __forceinline__ int64_t dq_unit0(int64_t blk) {
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  return (blk * kDqWaves + wave) * kDqTiles * kWave + (threadIdx.x & (kWave - 1));
}

int dq_grid(int64_t nunits) {
  const int64_t per_wg = (int64_t)kDqTiles * kWave * kDqWaves;
  const int64_t g = (nunits + per_wg - 1) / per_wg;
  return (int)(g < 1 ? 1 : g);
}

// FP8 1x128: unit u's scale is u / 16.
template <bool kBf16Out, int kElem>
__device__ __forceinline__ void dq_fp8_1x128_body(int64_t blk, const uint8_t* __restrict__ codes,
                                                  const float* __restrict__ scales, int64_t nunits,
                                                  void* __restrict__ out) {
  const int64_t u0 = dq_unit0(blk);
  uint2 c[kDqTiles];
  float s[kDqTiles];
#pragma unroll
  for (int k = 0; k < kDqTiles; ++k) {
    const int64_t u = u0 + k * kWave;
    if (u < nunits) {
      c[k] = ld_nt8(codes + u * 8);
      s[k] = scales[u >> 4];
    }
  }
#pragma unroll
  for (int k = 0; k < kDqTiles; ++k) {
    const int64_t u = u0 + k * kWave;
    if (u < nunits) {
      float o[8];
      fp8_decode8<kElem>(c[k], s[k], o);
      store_out8<kBf16Out>(out, u, o);
    }
  }
}

// MXFP4 with the gfx950 scaled FP4 conversion, two nibbles per instruction
// (byte j of w gives elements 2j and 2j + 1, low nibble first).  With a scale
// 2^k it returns +-V * 2^k exactly, signed zeros included, in float32 or bf16:
// a GPU check over every code byte, byte position and E8M0 scale found it
// equal, bit for bit, to the decoded value times the scale.  (It uses only the
// scale's exponent, so NVFP4's arbitrary scales cannot go through it.)
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

template <bool kBf16Out>
__device__ __forceinline__ void mx_expand8(uint32_t w, float s, void* out, int64_t u) {
  if constexpr (kBf16Out) {
    const uint32_t p0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0));
    const uint32_t p1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1));
    const uint32_t p2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2));
    const uint32_t p3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3));
    st_nt16(reinterpret_cast<uint16_t*>(out) + 8 * u, p0, p1, p2, p3);
  } else {
    const f32x2v a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 0);
    const f32x2v b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 1);
    const f32x2v c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 2);
    const f32x2v d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 3);
    float* p = reinterpret_cast<float*>(out) + 8 * u;
    st_nt16(p, as_u(a[0]), as_u(a[1]), as_u(b[0]), as_u(b[1]));
    st_nt16(p + 4, as_u(c[0]), as_u(c[1]), as_u(d[0]), as_u(d[1]));
  }
}

// MXFP4: unit u is a quarter of block u / 4; +-V * 2^(e - 127) is exact.
template <bool kBf16Out>
__device__ __forceinline__ void dq_mxfp4_body(int64_t blk, const uint8_t* __restrict__ codes,
                                              const uint8_t* __restrict__ scales, int64_t nunits,
                                              void* __restrict__ out) {
  const int64_t u0 = dq_unit0(blk);
  uint32_t c[kDqTiles], e[kDqTiles];
#pragma unroll
  for (int k = 0; k < kDqTiles; ++k) {
    const int64_t u = u0 + k * kWave;
    if (u < nunits) {
      c[k] = reinterpret_cast<const uint32_t*>(codes)[u];
      e[k] = scales[u >> 2];
    }
  }
#pragma unroll
  for (int k = 0; k < kDqTiles; ++k) {
    const int64_t u = u0 + k * kWave;
    if (u < nunits) {
      mx_expand8<kBf16Out>(c[k], as_f(e[k] << 23), out, u);  // 2^(e - 127), e in [85, 252]
    }
  }
}

// MXFP8: unit u is a quarter of block u / 4; dec(code) * 2^(e - 127) is exact.
template <bool kBf16Out>
__device__ __forceinline__ void dq_mxfp8_body(int64_t blk, const uint8_t* __restrict__ codes,
                                              const uint8_t* __restrict__ scales, int64_t nunits,
                                              void* __restrict__ out) {
  const int64_t u0 = dq_unit0(blk);
  uint2 c[kDqTiles];
  uint32_t e[kDqTiles];
#pragma unroll
  for (int k = 0; k < kDqTiles; ++k) {
    const int64_t u = u0 + k * kWave;
    if (u < nunits) {
      c[k] = ld_nt8(codes + u * 8);
      e[k] = scales[u >> 2];
    }
  }
#pragma unroll
  for (int k = 0; k < kDqTiles; ++k) {
    const int64_t u = u0 + k * kWave;
    if (u < nunits) {
      float o[8];
      fp8_decode8<kE4M3>(c[k], as_f(e[k] << 23), o);  // 2^(e - 127), e in [79, 246]
      store_out8<kBf16Out>(out, u, o);
    }
  }
}

// NVFP4, slice b = blockIdx.y: unit u is half of block u / 2; element scale
// max(dec(block scale), 1e-12) * gs.  The nibbles are expanded by the scaled
// FP4 conversion at scale 1, which returns +-V exactly (signed zeros
// included), and each value is then multiplied by the element scale: one
// rounding, as V * s.
// (base: the slice's first unit; g its tensor scale)
template <bool kBf16Out>
__device__ __forceinline__ void dq_nvfp4_body(int64_t blk, const uint8_t* __restrict__ codes,
                                              const uint8_t* __restrict__ scales, float g,
                                              int64_t nunits, int64_t base,
                                              void* __restrict__ out) {
  const int64_t u0 = dq_unit0(blk);
  uint32_t c[kDqTiles], bs[kDqTiles];
#pragma unroll
  for (int k = 0; k < kDqTiles; ++k) {
    const int64_t u = u0 + k * kWave;
    if (u < nunits) {
      c[k] = reinterpret_cast<const uint32_t*>(codes)[base + u];
      bs[k] = scales[(base + u) >> 1];
    }
  }
#pragma unroll
  for (int k = 0; k < kDqTiles; ++k) {
    const int64_t u = u0 + k * kWave;
    if (u < nunits) {
      const float s = fmaxf(e4m3_decode(bs[k]), 1e-12f) * g;
      float o[8];
      const f32x2v v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[k], 1.0f, 0);
      const f32x2v v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[k], 1.0f, 1);
      const f32x2v v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[k], 1.0f, 2);
      const f32x2v v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[k], 1.0f, 3);
      o[0] = v0[0] * s; o[1] = v0[1] * s; o[2] = v1[0] * s; o[3] = v1[1] * s;
      o[4] = v2[0] * s; o[5] = v2[1] * s; o[6] = v3[0] * s; o[7] = v3[1] * s;
      store_out8<kBf16Out>(out, base + u, o);
    }
  }
}

// INT4: unit u lies in group u / 16; (q - z) * s is exact in float32
// (|q - z| <= 15 and s has 8 significant bits).
template <bool kGuard>
__device__ __forceinline__ void dq_int4_chunk(const uint8_t* __restrict__ codes,
                                              const uint16_t* __restrict__ scales,
                                              const uint8_t* __restrict__ zeros, int64_t nunits,
                                              int64_t u0, void* __restrict__ out) {
  // A wave's chunk spans kDqTiles * 64 units = 16 groups (cols is a multiple
  // of 128, so groups never straddle chunks or rows).  Lane l fetches the
  // scale and zero-point nibble of group l % 16 of the chunk, two loads per
  // chunk, and each tile takes its lanes' groups from those lanes with a lane
  // permute: unit k 64 + l lies in group 4 k + l / 16.  Gathering them per
  // unit instead took two loads per tile; on 1 GiB with bf16 output this
  // form takes 216 us against 225 us for that one, with the same bytes.
  static_assert(kDqTiles * kWave / 16 == 16, "one lane per group of the chunk");
  const int lane = (int)threadIdx.x & (kWave - 1);
  // Every load is unconditional, its index clamped into the tensor (values of
  // lanes past the end are never stored), so that no branch makes the
  // compiler wait for a load before the next is issued.
  const int64_t ngroups = nunits >> 4;
  const int64_t g = min(((u0 - lane) >> 4) + (lane & 15), ngroups - 1);
  const uint32_t sraw = scales[g], zraw = zeros[g >> 1];
  uint32_t c[kDqTiles];
#pragma unroll
  for (int k = 0; k < kDqTiles; ++k)
    c[k] = reinterpret_cast<const uint32_t*>(codes)[min(u0 + k * kWave, nunits - 1)];
  const uint32_t meta = sraw | ((zraw >> (4 * (g & 1)) & 0xFu) << 16);  // scale | zero << 16
#pragma unroll
  for (int k = 0; k < kDqTiles; ++k) {
    const uint32_t m = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (4 * k + (lane >> 4)), (int)meta);
    const int64_t u = u0 + k * kWave;
    if (!kGuard || u < nunits) {
      const float s = as_f(m << 16);
      const int z = ((int)(m >> 16) << 28) >> 28;  // sign-extend
      float o[8];
      // q - z as (q + 8) - (z + 8), a difference of small integers in float32
      // (exact), times s: one rounding, as the oracle, a zero difference
      // giving +0.  q + 8 of a nibble is the nibble with its top bit flipped,
      // converted from a byte.  (Forming (q + 8) s - (z + 8) s in one fused
      // multiply-add instead would overflow at (z + 8) s for groups whose
      // range is near the float32 maximum.)
      const float zf = (float)(z + 8);
      const uint32_t lo = (c[k] & 0x0F0F0F0Fu) ^ 0x08080808u;          // elements 0, 2, 4, 6
      const uint32_t hi = ((c[k] >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u;   // elements 1, 3, 5, 7
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[2 * j] = ((float)((lo >> (8 * j)) & 0xFFu) - zf) * s;
        o[2 * j + 1] = ((float)((hi >> (8 * j)) & 0xFFu) - zf) * s;
      }
      store_out8<true>(out, u, o);
    }
  }
}

// A full chunk has no per-lane bound, so no branch lets the compiler sink a
// load next to its use; only the chunk holding the end takes the guarded form.
template <bool kBf16Out>
__device__ __forceinline__ void dq_int4_body(int64_t blk, const uint8_t* __restrict__ codes,
                                             const uint16_t* __restrict__ scales,
                                             const uint8_t* __restrict__ zeros, int64_t nunits,
                                             void* __restrict__ out) {
  if (nunits <= 0) return;
  if constexpr (!kBf16Out) {
    // float32 output: each unit's scale and zero-point gathered per tile.  The
    // chunked form above gave the same bytes but took this output on 1 GiB
    // from 610 to 901 us, so it serves bf16 output only.
    const int64_t v0 = dq_unit0(blk);
    uint32_t c[kDqTiles], sb[kDqTiles], zb[kDqTiles];
#pragma unroll
    for (int k = 0; k < kDqTiles; ++k) {
      const int64_t u = v0 + k * kWave;
      if (u < nunits) {
        c[k] = reinterpret_cast<const uint32_t*>(codes)[u];
        sb[k] = scales[u >> 4];
        zb[k] = zeros[u >> 5];
      }
    }
#pragma unroll
    for (int k = 0; k < kDqTiles; ++k) {
      const int64_t u = v0 + k * kWave;
      if (u < nunits) {
        const float s = as_f(sb[k] << 16);
        const int z = ((int)(zb[k] >> (4 * ((u >> 4) & 1))) << 28) >> 28;  // sign-extend
        float o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int q = ((int)(c[k] >> (4 * i)) << 28) >> 28;
          o[i] = (float)(q - z) * s;
        }
        store_out8<false>(out, u, o);
      }
    }
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int64_t wave_u0 = (blk * kDqWaves + wave) * kDqTiles * kWave;  // uniform
  const int64_t u0 = wave_u0 + (threadIdx.x & (kWave - 1));
  if (wave_u0 + kDqTiles * kWave <= nunits)
    dq_int4_chunk<false>(codes, scales, zeros, nunits, u0, out);
  else
    dq_int4_chunk<true>(codes, scales, zeros, nunits, u0, out);
}

// Single-tensor kernels: one body call per workgroup.
template <bool kBf16Out, int kElem>
__global__ __launch_bounds__(kBlockThreads) void k_dq_fp8_1x128(const uint8_t* __restrict__ codes,
                                                                const float* __restrict__ scales,
                                                                int64_t nunits,
                                                                void* __restrict__ out) {
  dq_fp8_1x128_body<kBf16Out, kElem>(blockIdx.x, codes, scales, nunits, out);
}

template <bool kBf16Out>
__global__ __launch_bounds__(kBlockThreads) void k_dq_mxfp4(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales,
                                                            int64_t nunits,
                                                            void* __restrict__ out) {
  dq_mxfp4_body<kBf16Out>(blockIdx.x, codes, scales, nunits, out);
}

template <bool kBf16Out>
__global__ __launch_bounds__(kBlockThreads) void k_dq_mxfp8(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales,
                                                            int64_t nunits,
                                                            void* __restrict__ out) {
  dq_mxfp8_body<kBf16Out>(blockIdx.x, codes, scales, nunits, out);
}

// NVFP4, slice b = blockIdx.y.
template <bool kBf16Out>
__global__ __launch_bounds__(kBlockThreads) void k_dq_nvfp4(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales,
                                                            const float* __restrict__ gs,
                                                            int64_t per_slice,
                                                            void* __restrict__ out) {
  const int64_t b = blockIdx.y, nunits = per_slice / 8;
  dq_nvfp4_body<kBf16Out>(blockIdx.x, codes, scales, gs[b], nunits, b * nunits, out);
}

template <bool kBf16Out>
__global__ __launch_bounds__(kBlockThreads) void k_dq_int4(const uint8_t* __restrict__ codes,
                                                           const uint16_t* __restrict__ scales,
                                                           const uint8_t* __restrict__ zeros,
                                                           int64_t nunits,
                                                           void* __restrict__ out) {
  dq_int4_body<kBf16Out>(blockIdx.x, codes, scales, zeros, nunits, out);
}

// Fused dequantization of several tensors (pqb_dequantize_batch), one launch
// per output type and up to kMaxBatchJobs jobs: every job gets a contiguous
// range of workgroups, a workgroup finds its job by binary search over the
// prefix table (uniform) and runs that job's body with its local index.  An
// NVFP4 job is one slice (the host splits a batch of slices), its tensor scale
// read through `aux`.
struct DqJob {
  const uint8_t* codes;
  const void* scales;
  const void* aux;   // INT4 zero-points; NVFP4: the slice's tensor scale
  void* out;
  int64_t nunits;
  uint32_t kind;
  uint32_t pad;
};
struct DqArgs {
  int32_t njobs;
  int32_t pad;
  int64_t wg_begin[kMaxBatchJobs + 1];
  DqJob job[kMaxBatchJobs];
};
static_assert(sizeof(DqArgs) <= 4096, "kernel arguments must stay within 4 KiB");

template <bool kBf16Out>
__global__ __launch_bounds__(kBlockThreads) void k_dq_multi(DqArgs a) {
  const int64_t wg = blockIdx.x;
  int lo = 0, hi = a.njobs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.wg_begin[mid] <= wg)
      lo = mid;
    else
      hi = mid - 1;
  }
  const DqJob& jb = a.job[lo];
  const int64_t local = wg - a.wg_begin[lo];
  switch (jb.kind) {
    case kDqFp8:
      dq_fp8_1x128_body<kBf16Out, kE4M3>(local, jb.codes, (const float*)jb.scales, jb.nunits,
                                          jb.out);
      break;
    case kDqE5m2:
      dq_fp8_1x128_body<kBf16Out, kE5M2>(local, jb.codes, (const float*)jb.scales, jb.nunits,
                                          jb.out);
      break;
    case kDqMx4:
      dq_mxfp4_body<kBf16Out>(local, jb.codes, (const uint8_t*)jb.scales, jb.nunits, jb.out);
      break;
    case kDqMx8:
      dq_mxfp8_body<kBf16Out>(local, jb.codes, (const uint8_t*)jb.scales, jb.nunits, jb.out);
      break;
    case kDqNv:
      dq_nvfp4_body<kBf16Out>(local, jb.codes, (const uint8_t*)jb.scales,
                              *(const float*)jb.aux, jb.nunits, 0, jb.out);
      break;
    default:
      dq_int4_body<kBf16Out>(local, jb.codes, (const uint16_t*)jb.scales,
                             (const uint8_t*)jb.aux, jb.nunits, jb.out);
  }
}

struct DqLaunch {
  bool bf16;
  int64_t wgs;
  DqArgs args;
};

// Jobs of one output type into launches of at most kMaxBatchJobs, as even in
// job count as possible; false if a launch would exceed 2^32 - 1 threads.
bool plan_dq(const std::vector<const DqMultiJob*>& jobs, bool bf16, std::vector<DqLaunch>& out) {
  const size_t n = jobs.size();
  if (n == 0) return true;
  const size_t nl = (n + kMaxBatchJobs - 1) / kMaxBatchJobs, per = (n + nl - 1) / nl;
  const int64_t per_wg = (int64_t)kDqTiles * kWave * kDqWaves;
  for (size_t base = 0; base < n; base += per) {
    const int cnt = (int)(n - base < per ? n - base : per);
    DqLaunch L;
    L.bf16 = bf16;
    L.args = DqArgs{};
    L.args.njobs = cnt;
    int64_t wg = 0;
    for (int i = 0; i < cnt; ++i) {
      const DqMultiJob& m = *jobs[base + i];
      DqJob& j = L.args.job[i];
      j.codes = m.codes;
      j.scales = m.scales;
      j.aux = m.aux;
      j.out = m.out;
      j.nunits = m.nunits;
      j.kind = (uint32_t)m.kind;
      L.args.wg_begin[i] = wg;
      wg += (m.nunits + per_wg - 1) / per_wg;
    }
    L.args.wg_begin[cnt] = wg;
    L.wgs = wg;
    if (wg > (int64_t)(0xFFFFFFFFu / (uint32_t)kBlockThreads)) return false;
    if (wg > 0) out.push_back(L);
  }
  return true;
}

bool plan_dq_all(const DqMultiJob* jobs, int njobs, std::vector<DqLaunch>& out) {
  std::vector<const DqMultiJob*> by[2];
  for (int i = 0; i < njobs; ++i) by[jobs[i].bf16_out ? 1 : 0].push_back(&jobs[i]);
  return plan_dq(by[0], false, out) && plan_dq(by[1], true, out);
}

}  // namespace

hipError_t launch_fp8_1x128_dequant(const uint8_t* codes, const float* scales, int64_t n,
                                    bool out_bf16, void* out, hipStream_t st, int elem) {
  const int64_t nl = n / 8;
  return with_elem(elem, [&](auto e) {
    constexpr int E = decltype(e)::value;
    if (out_bf16)
      hipLaunchKernelGGL((k_dq_fp8_1x128<true, E>), dim3(dq_grid(nl)), dim3(kBlockThreads), 0, st,
                         codes, scales, nl, out);
    else
      hipLaunchKernelGGL((k_dq_fp8_1x128<false, E>), dim3(dq_grid(nl)), dim3(kBlockThreads), 0,
                         st, codes, scales, nl, out);
  });
}

hipError_t launch_mxfp4_dequant(const uint8_t* codes, const uint8_t* scales, int64_t n,
                                bool out_bf16, void* out, hipStream_t st) {
  const int64_t nl = n / 8;
  if (out_bf16)
    hipLaunchKernelGGL(k_dq_mxfp4<true>, dim3(dq_grid(nl)), dim3(kBlockThreads), 0, st, codes,
                       scales, nl, out);
  else
    hipLaunchKernelGGL(k_dq_mxfp4<false>, dim3(dq_grid(nl)), dim3(kBlockThreads), 0, st, codes,
                       scales, nl, out);
  return hipGetLastError();
}

hipError_t launch_mxfp8_dequant(const uint8_t* codes, const uint8_t* scales, int64_t n,
                                bool out_bf16, void* out, hipStream_t st) {
  const int64_t nl = n / 8;
  if (out_bf16)
    hipLaunchKernelGGL(k_dq_mxfp8<true>, dim3(dq_grid(nl)), dim3(kBlockThreads), 0, st, codes,
                       scales, nl, out);
  else
    hipLaunchKernelGGL(k_dq_mxfp8<false>, dim3(dq_grid(nl)), dim3(kBlockThreads), 0, st, codes,
                       scales, nl, out);
  return hipGetLastError();
}

hipError_t launch_nvfp4_dequant(const uint8_t* codes, const uint8_t* scales, const float* gs,
                                int64_t batch, int64_t per_slice, bool out_bf16, void* out,
                                hipStream_t st) {
  const dim3 grid(dq_grid(per_slice / 8), (unsigned)batch);
  if (out_bf16)
    hipLaunchKernelGGL(k_dq_nvfp4<true>, grid, dim3(kBlockThreads), 0, st, codes, scales, gs,
                       per_slice, out);
  else
    hipLaunchKernelGGL(k_dq_nvfp4<false>, grid, dim3(kBlockThreads), 0, st, codes, scales, gs,
                       per_slice, out);
  return hipGetLastError();
}

hipError_t launch_int4_dequant(const uint8_t* codes, const uint16_t* scales, const uint8_t* zeros,
                               int64_t n, bool out_bf16, void* out, hipStream_t st) {
  const int64_t nl = n / 8;
  if (out_bf16)
    hipLaunchKernelGGL(k_dq_int4<true>, dim3(dq_grid(nl)), dim3(kBlockThreads), 0, st, codes,
                       scales, zeros, nl, out);
  else
    hipLaunchKernelGGL(k_dq_int4<false>, dim3(dq_grid(nl)), dim3(kBlockThreads), 0, st, codes,
                       scales, zeros, nl, out);
  return hipGetLastError();
}

}  // namespace pqb

namespace pqb {

int64_t dq_multi_launches(const DqMultiJob* jobs, int njobs) {
  std::vector<DqLaunch> plan;
  if (!plan_dq_all(jobs, njobs, plan)) return -1;
  return (int64_t)plan.size();
}

hipError_t launch_dq_multi(const DqMultiJob* jobs, int njobs, hipStream_t st) {
  std::vector<DqLaunch> plan;
  if (!plan_dq_all(jobs, njobs, plan)) return hipErrorInvalidConfiguration;
  for (const DqLaunch& L : plan) {
    if (L.bf16)
      hipLaunchKernelGGL(k_dq_multi<true>, dim3((unsigned)L.wgs), dim3(kBlockThreads), 0, st,
                         L.args);
    else
      hipLaunchKernelGGL(k_dq_multi<false>, dim3((unsigned)L.wgs), dim3(kBlockThreads), 0, st,
                         L.args);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pqb
