// Formats whose scale depends on a whole tensor: FP8 per tensor, the FP8 KV
// write (per layer, per head or static; page "量化部署实战", sections 伪量化实现
// and KV Cache 量化：误差要和信号比) and NVFP4's tensor scale (same page).
//
// Three launches, each streaming one 8 KiB chunk of input per wave (8 bf16 or
// 4 float32 tiles), the access pattern that sustains the highest bandwidth:
//   pass 1    every workgroup writes the amax of its share, per group (the
//             slice, or each head), into group-major partials;
//   finalize  one workgroup per slice reduces them, writes the output scales
//             and a small table for pass 2 (s per group; for NVFP4 gs, RN(1/gs)
//             and s, RN(1/s) of all 127 block-scale codes);
//   pass 2    quantizes with the finished table.
// When every slice has few partials (at most kFoldMaxPartials, no per-head
// groups) the finalize launch is left out: each pass-2 workgroup reduces its
// slice's partials itself (from L2) and forms the same scale or table with the
// same arithmetic, so a small tensor takes two launches instead of three.
// On that path pass 1 also reads through the caches (the input loads are
// otherwise non-temporal): both passes launch the same grid, so a workgroup
// reads the same units on the same XCD twice, and a share of at most a few
// MiB per XCD is still in that XCD's L2 when pass 2 reads it (float32
// [3072, 1024]: NVFP4 10.8 -> 9.5 us, FP8 per tensor 10.1 -> 8.6 us per
// call).  Large slices keep non-temporal loads in both passes: there the
// first read evicts itself before the second, and allocating it only slows
// the stream.
// A slice is one batch slice (per-tensor FP8, NVFP4) or one layer of K or V.
// Per head, a lane follows its unit's column through the chunk: one 64-bit
// remainder per chunk, then +64 units per tile with one wrap, and the head is
// a multiply-high by ceil(2^32 / head_units) (exact for the bounded sizes;
// the column itself when head_units is 1).
#include "launch.h"
#include "quant.h"

namespace pqb {
namespace {

constexpr int kWgWaves = kBlockThreads / kWave;

// Tiles per wave chunk (U): 8 bf16 or 4 float32 tiles (8 KiB of input), or
// half that when a slice would give fewer than 2048 waves at the full size, so
// that a small tensor spreads over more waves (NVFP4 on bf16 [4096, 1024]:
// 10.9 -> 9.3 us; on float32 [3072, 1024]: 11.9 -> 11.0 us; a 16M-element
// slice is 4% faster at the full size).  Every kernel of a call uses the same U.
int chunk_tiles(int64_t per_slice, bool bf16) {
  const int full = bf16 ? 8 : 4;
  const int64_t waves = (per_slice / 8 + (int64_t)full * kWave - 1) / ((int64_t)full * kWave);
  return waves < 2048 ? full / 2 : full;
}

struct TpArgs {
  const void* x[2];
  uint8_t* codes[2];
  void* scales[2];  // FP8 / KV: float scales (STATIC: read); NVFP4: u8 block scales
  float* gs[2];     // NVFP4 tensor scales
  int32_t mode[2];  // kKvLayer (also per-tensor FP8 and NVFP4), kKvHead, kKvStatic
};

struct TpGeo {
  int64_t per_slice;  // elements per slice (multiple of 8)
  int64_t slices;     // per tensor
  int32_t W;          // pass-1 workgroups per slice
  int32_t G;          // group stride of partials and of the FP8 final table (1 or heads)
  int32_t row_units;  // per head: units per token row (heads * head_dim / 8)
  uint32_t head_magic;  // per head: ceil(2^32 / (head_dim / 8))
};

// NVFP4 final table per slice: [0] gs, [1] RN(1/gs), [2 + c] s of block-scale
// code c, [2 + 128 + c] RN(1/s), c < 127; 258 floats, padded to 264.
constexpr int kNvSe = 2, kNvYe = 2 + 128, kNvFinal = 264;

__device__ __forceinline__ int groups_of(const TpArgs& a, const TpGeo& g, int tz) {
  return a.mode[tz] == kKvHead ? g.G : 1;
}

// Column (unit index within a token row) of this lane's first unit of a chunk,
// and the per-tile step, for the per-head scope.
struct ColWalk {
  uint32_t c, step, R, magic;
  // 32-bit remainder while a slice's unit indices fit (a 64-bit one costs a
  // division routine per lane and chunk)
  __device__ __forceinline__ ColWalk(int64_t u0, const TpGeo& g)
      : c(g.per_slice / 8 + kWave <= (int64_t)UINT32_MAX
              ? ((uint32_t)u0 + (uint32_t)(threadIdx.x & (kWave - 1))) % (uint32_t)g.row_units
              : (uint32_t)((u0 + (threadIdx.x & (kWave - 1))) % g.row_units)),
        step((uint32_t)(kWave % g.row_units)),
        R((uint32_t)g.row_units),
        magic(g.head_magic) {}
  // magic == 0 stands for head_units == 1 (ceil(2^32 / 1) does not fit 32 bits)
  __device__ __forceinline__ int head() const { return (int)(magic ? __umulhi(c, magic) : c); }
  __device__ __forceinline__ void next() {
    c += step;
    if (c >= R) c -= R;
  }
};

// ---------------------------------------------------------------------------
// pass 1
// ---------------------------------------------------------------------------
// Plain (allocating) loads of one chunk, for the folded pass 1; missing units
// read as zeros.
template <typename T, int U>
__device__ __forceinline__ void load_chunk_cached(const T* __restrict__ x, int64_t u0,
                                                  int64_t nunits, Raw8 raw[U]) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int64_t u = u0 + k * kWave + lane;
    raw[k] = Raw8{};
    if (u < nunits) {
      const uint4* p = reinterpret_cast<const uint4*>(x + u * 8);
      raw[k].a = p[0];
      if constexpr (sizeof(T) == 4) raw[k].b = p[1];
    }
  }
}

template <typename T, int U, bool kCached>
__global__ __launch_bounds__(kBlockThreads) void k_tp_amax(TpArgs a, TpGeo g,
                                                           float* __restrict__ partials) {
  __shared__ uint32_t red[kMaxKvHeads > kWgWaves ? kMaxKvHeads : kWgWaves];
  const int tz = blockIdx.z;
  if (a.mode[tz] == kKvStatic) return;  // uniform over the workgroup
  const int64_t b = blockIdx.y;
  const int G = groups_of(a, g, tz);
  const T* xs = reinterpret_cast<const T*>(a.x[tz]) + b * g.per_slice;
  const int64_t nunits = g.per_slice / 8;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int64_t u0 = ((int64_t)blockIdx.x * kWgWaves + wave) * U * kWave;
  float* out = partials + ((int64_t)tz * g.slices + b) * g.G * g.W + blockIdx.x;
  Raw8 raw[U];
  const bool any = u0 < nunits;
  if (any) {
    if constexpr (kCached)
      load_chunk_cached<T, U>(xs, u0, nunits, raw);
    else if (u0 + U * kWave <= nunits)
      load_chunk<T, U, false>(xs, u0, nunits, raw);
    else
      load_chunk<T, U, true>(xs, u0, nunits, raw);  // missing units read as zeros
  }
  if (G == 1) {
    uint32_t m = 0;
    if (any) {
#pragma unroll
      for (int k = 0; k < U; ++k) {
        float v[8];
        widen8(raw[k], xs, v);
        m = max(m, as_u(absmax8(v)));
      }
    }
    m = wave_umax(m);
    if ((threadIdx.x & (kWave - 1)) == 0) red[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t r = red[0];
      for (int i = 1; i < kWgWaves; ++i) r = max(r, red[i]);
      out[0] = as_f(r);
    }
    return;
  }
  for (int i = threadIdx.x; i < G; i += kBlockThreads) red[i] = 0;
  __syncthreads();
  if (any) {
    ColWalk col(u0, g);
#pragma unroll
    for (int k = 0; k < U; ++k) {
      float v[8];
      widen8(raw[k], xs, v);
      atomicMax(&red[col.head()], as_u(absmax8(v)));  // zeros for missing units
      col.next();
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G; i += kBlockThreads) out[(int64_t)i * g.W] = as_f(red[i]);
}

// ---------------------------------------------------------------------------
// finalize: grid (slices, tensors)
// ---------------------------------------------------------------------------
// Finalize workgroups are 1024 threads with 8 loads in flight each: a slice
// of 1 GiB of bf16 has 32768 partials, and the reduction is latency-bound.
constexpr int kFinThreads = 1024, kFinWaves = kFinThreads / kWave, kFinLoads = 8;

__device__ __forceinline__ uint32_t reduce_row(const float* __restrict__ p, int W, uint32_t* red) {
  uint32_t m = 0;
  int i = threadIdx.x;
  for (; i + (kFinLoads - 1) * kFinThreads < W; i += kFinLoads * kFinThreads) {
    uint32_t v[kFinLoads];
#pragma unroll
    for (int k = 0; k < kFinLoads; ++k) v[k] = as_u(p[i + k * kFinThreads]);
#pragma unroll
    for (int k = 0; k < kFinLoads; ++k) m = max(m, v[k]);
  }
  for (; i < W; i += kFinThreads) m = max(m, as_u(p[i]));
  m = wave_umax(m);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = m;
  __syncthreads();
  m = red[0];
  for (int w = 1; w < kFinWaves; ++w) m = max(m, red[w]);
  __syncthreads();
  return m;
}

// Max of a slice's W partials over one 256-thread workgroup (every thread
// gets it); `red` holds kWgWaves words.  All threads must call it.
constexpr int kFoldMaxPartials = 1024;
__device__ __forceinline__ uint32_t fold_partials(const float* __restrict__ p, int W, uint32_t* red) {
  uint32_t m = 0;
  for (int i = threadIdx.x; i < W; i += kBlockThreads) m = max(m, as_u(p[i]));
  m = wave_umax(m);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int w = 1; w < kWgWaves; ++w) m = max(m, red[w]);
  return m;
}

template <int kElem>
__global__ __launch_bounds__(kFinThreads) void k_tp_finalize_fp8(TpArgs a, TpGeo g,
                                                                 const float* __restrict__ partials,
                                                                 float* __restrict__ fin) {
  __shared__ uint32_t red[kFinWaves];
  const int tz = blockIdx.y;
  if (a.mode[tz] == kKvStatic) return;
  const int64_t b = blockIdx.x, slot = (int64_t)tz * g.slices + b;
  const int G = groups_of(a, g, tz);
  float* sc = reinterpret_cast<float*>(a.scales[tz]);
  for (int grp = 0; grp < G; ++grp) {
    const float s =
        fp8_scale_bits<kElem>(reduce_row(partials + (slot * g.G + grp) * g.W, g.W, red));
    if (threadIdx.x == 0) {
      fin[slot * g.G + grp] = s;
      sc[b * G + grp] = s;
    }
  }
}

__global__ __launch_bounds__(kFinThreads) void k_tp_finalize_nv(TpArgs a, TpGeo g,
                                                                const float* __restrict__ partials,
                                                                float* __restrict__ fin) {
  __shared__ uint32_t red[kFinWaves];
  const int64_t b = blockIdx.x;
  const uint32_t m = reduce_row(partials + b * g.W, g.W, red);
  const float gs = as_f(max(m, kAmaxFloorBits)) / 2688.0f;  // 448 * 6, IEEE division
  float* f = fin + b * kNvFinal;
  if (threadIdx.x == 0) {
    f[0] = gs;
    f[1] = recip_rn(gs);
    a.gs[0][b] = gs;
  }
  // element scale of every finite block-scale code: max(dec(code), 1e-12) * gs
  for (int c = threadIdx.x; c < 127; c += kFinThreads) {
    const float sc = fmaxf(e4m3_decode((uint32_t)c), 1e-12f) * gs;
    f[kNvSe + c] = sc;
    f[kNvYe + c] = 1.0f / sc;  // IEEE division
  }
}

// ---------------------------------------------------------------------------
// pass 2
// ---------------------------------------------------------------------------
// Eight codes with the static-scale clamp: |x| is first limited to 512 s (so
// x * RN(1/s) cannot overflow; any |x/s| >= 512 saturates anyway), then the
// correctly rounded quotient is clamped to +-448.
__device__ __forceinline__ uint2 fp8_pack8_clamped(const float v[8], float s, float y, float lim) {
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    q[i] = __builtin_amdgcn_fmed3f(div_rn(__builtin_amdgcn_fmed3f(v[i], -lim, lim), s, y), -448.0f,
                                   448.0f);
  return make_uint2(e4m3_bytes4(q[0], q[1], q[2], q[3]), e4m3_bytes4(q[4], q[5], q[6], q[7]));
}

template <typename T, int U, int kMode, bool kGuard, int kElem>
__device__ __forceinline__ void fp8_tp_chunk(const T* __restrict__ xs, int64_t u0, int64_t nunits,
                                             uint8_t* __restrict__ cs, float s, float y,
                                             const float* ss, const float* ys, const TpGeo& g) {
  const int lane = threadIdx.x & (kWave - 1);
  Raw8 raw[U];
  load_chunk<T, U, kGuard>(xs, u0, nunits, raw);
  [[maybe_unused]] ColWalk col(kMode == kKvHead ? u0 : 0, g);
  const float lim = s * 512.0f;
#pragma unroll
  for (int k = 0; k < U; ++k) {
    float v[8];
    widen8(raw[k], xs, v);
    uint2 w;
    if constexpr (kMode == kKvHead) {
      const int h = col.head();
      w = fp8_pack8<kElem>(v, ss[h], ys[h]);
      col.next();
    } else if constexpr (kMode == kKvStatic) {
      w = fp8_pack8_clamped(v, s, y, lim);
    } else {
      w = fp8_pack8<kElem>(v, s, y);
    }
    const int64_t u = u0 + k * kWave + lane;
    if (!kGuard || u < nunits) store_codes8(cs + u * 8, w);
  }
}

// kFold: `fin` holds the partials (no per-head groups); each workgroup
// reduces its slice's own, and workgroup 0 of the slice writes the scale.
template <typename T, int kElem, bool kFold, int U>
__global__ __launch_bounds__(kBlockThreads) void k_tp_fp8(TpArgs a, TpGeo g,
                                                          const float* __restrict__ fin) {
  __shared__ float ss[kMaxKvHeads], ys[kMaxKvHeads];
  __shared__ uint32_t red[kWgWaves];
  const int tz = blockIdx.z, mode = a.mode[tz];
  const int64_t b = blockIdx.y, slot = (int64_t)tz * g.slices + b;
  float s = 0.0f, y = 0.0f;
  if constexpr (kFold) {
    if (mode == kKvStatic) {
      s = reinterpret_cast<const float*>(a.scales[tz])[b];
    } else {
      s = fp8_scale_bits<kElem>(fold_partials(fin + slot * g.W, g.W, red));
      if (blockIdx.x == 0 && threadIdx.x == 0) reinterpret_cast<float*>(a.scales[tz])[b] = s;
    }
    y = recip_rn(s);
  } else if (mode == kKvHead) {
    for (int i = threadIdx.x; i < g.G; i += kBlockThreads) {
      const float si = fin[slot * g.G + i];
      ss[i] = si;
      ys[i] = recip_rn(si);
    }
    __syncthreads();
  } else {
    s = mode == kKvStatic ? reinterpret_cast<const float*>(a.scales[tz])[b] : fin[slot * g.G];
    y = recip_rn(s);
  }
  const T* xs = reinterpret_cast<const T*>(a.x[tz]) + b * g.per_slice;
  uint8_t* cs = a.codes[tz] + b * g.per_slice;
  const int64_t nunits = g.per_slice / 8;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int64_t u0 = ((int64_t)blockIdx.x * kWgWaves + wave) * U * kWave;
  if (u0 >= nunits) return;
  const bool full = u0 + U * kWave <= nunits;
  switch (mode) {
    case kKvHead:
      if (full) fp8_tp_chunk<T, U, kKvHead, false, kElem>(xs, u0, nunits, cs, s, y, ss, ys, g);
      else fp8_tp_chunk<T, U, kKvHead, true, kElem>(xs, u0, nunits, cs, s, y, ss, ys, g);
      break;
    case kKvStatic:
      if (full) fp8_tp_chunk<T, U, kKvStatic, false, kElem>(xs, u0, nunits, cs, s, y, ss, ys, g);
      else fp8_tp_chunk<T, U, kKvStatic, true, kElem>(xs, u0, nunits, cs, s, y, ss, ys, g);
      break;
    default:
      if (full) fp8_tp_chunk<T, U, kKvLayer, false, kElem>(xs, u0, nunits, cs, s, y, ss, ys, g);
      else fp8_tp_chunk<T, U, kKvLayer, true, kElem>(xs, u0, nunits, cs, s, y, ss, ys, g);
  }
}

// kFold: `fin` holds the partials; each workgroup reduces its slice's own and
// forms gs and the block-scale table as k_tp_finalize_nv does, and workgroup 0
// of the slice writes gs.
template <typename T, bool kFold, int U>
__global__ __launch_bounds__(kBlockThreads) void k_tp_nv(TpArgs a, TpGeo g,
                                                         const float* __restrict__ fin) {
  __shared__ NvTables tb;
  __shared__ uint32_t red[kWgWaves];
  const int64_t b = blockIdx.y;
  float gs, ygs;
  e2m1_lut_fill(tb.lut, 8);
  if constexpr (kFold) {
    const uint32_t m = fold_partials(fin + b * g.W, g.W, red);
    gs = as_f(max(m, kAmaxFloorBits)) / 2688.0f;  // 448 * 6, IEEE division
    ygs = recip_rn(gs);
    if (blockIdx.x == 0 && threadIdx.x == 0) a.gs[0][b] = gs;
    for (int c = threadIdx.x; c < 127; c += kBlockThreads) {
      const float sc = fmaxf(e4m3_decode((uint32_t)c), 1e-12f) * gs;
      tb.se[c] = sc;
      tb.ye[c] = 1.0f / sc;  // IEEE division
    }
  } else {
    const float* f = fin + b * kNvFinal;
    for (int c = threadIdx.x; c < 127; c += kBlockThreads) {
      tb.se[c] = f[kNvSe + c];
      tb.ye[c] = f[kNvYe + c];
    }
    gs = f[0];
    ygs = f[1];
  }
  __syncthreads();
  const T* xs = reinterpret_cast<const T*>(a.x[0]) + b * g.per_slice;
  uint8_t* cs = a.codes[0] + b * (g.per_slice / 2);
  uint8_t* bs = reinterpret_cast<uint8_t*>(a.scales[0]) + b * (g.per_slice / 16);
  const int64_t nunits = g.per_slice / 8;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int64_t u0 = ((int64_t)blockIdx.x * kWgWaves + wave) * U * kWave;
  if (u0 >= nunits) return;
  Raw8 raw[U];
  if (u0 + U * kWave <= nunits) {
    load_chunk<T, U, false>(xs, u0, nunits, raw);
    nv_pack<T, U, false>(xs, raw, u0, nunits, cs, bs, gs, ygs, tb);
  } else {
    load_chunk<T, U, true>(xs, u0, nunits, raw);
    nv_pack<T, U, true>(xs, raw, u0, nunits, cs, bs, gs, ygs, tb);
  }
}

int64_t wgs_per_slice(int64_t per_slice, bool bf16) {
  const int64_t units_per_wg = (int64_t)chunk_tiles(per_slice, bf16) * kWave * kWgWaves;
  const int64_t w = (per_slice / 8 + units_per_wg - 1) / units_per_wg;
  return w < 1 ? 1 : w;
}

// ceil(2^32 / head_units) for head_units >= 2; 0 (identity) for head_units == 1.
uint32_t head_magic(int64_t head_units) {
  return head_units == 1 ? 0u : (uint32_t)((0xFFFFFFFFull / (uint64_t)head_units) + 1);
}

template <typename T, int U>
hipError_t launch_tp_t(const TpArgs& a, int nt, const TpGeo& g, bool nv, float* ws,
                       hipStream_t st, int elem) {
  float* partials = ws;
  float* fin = ws + (int64_t)nt * g.slices * g.G * g.W;
  bool dynamic = false;
  for (int i = 0; i < nt; ++i) dynamic |= a.mode[i] != kKvStatic;
  const dim3 grid((unsigned)g.W, (unsigned)g.slices, (unsigned)nt);
  // two launches (no finalize) when pass 2 can reduce the partials itself: no
  // per-head scope (even with one head, pass 2 then reads per-head tables)
  bool per_head = false;
  for (int i = 0; i < nt; ++i) per_head |= a.mode[i] == kKvHead;
  const bool fold = dynamic && !per_head && g.G == 1 && g.W <= kFoldMaxPartials;
  if (fold) {
    hipLaunchKernelGGL((k_tp_amax<T, U, true>), grid, dim3(kBlockThreads), 0, st, a, g, partials);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (nv) {
      hipLaunchKernelGGL((k_tp_nv<T, true, U>), grid, dim3(kBlockThreads), 0, st, a, g, partials);
      return hipGetLastError();
    }
    return with_elem(elem, [&](auto el) {
      constexpr int E = decltype(el)::value;
      hipLaunchKernelGGL((k_tp_fp8<T, E, true, U>), grid, dim3(kBlockThreads), 0, st, a, g, partials);
    });
  }
  if (dynamic) {
    hipLaunchKernelGGL((k_tp_amax<T, U, false>), grid, dim3(kBlockThreads), 0, st, a, g, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (nv)
      hipLaunchKernelGGL(k_tp_finalize_nv, dim3((unsigned)g.slices, 1), dim3(kFinThreads), 0,
                         st, a, g, partials, fin);
    else
      e = with_elem(elem, [&](auto el) {
        hipLaunchKernelGGL(k_tp_finalize_fp8<decltype(el)::value>,
                           dim3((unsigned)g.slices, (unsigned)nt), dim3(kFinThreads), 0, st, a, g,
                           partials, fin);
      });
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (nv) {
    hipLaunchKernelGGL((k_tp_nv<T, false, U>), grid, dim3(kBlockThreads), 0, st, a, g, fin);
  } else {
    return with_elem(elem, [&](auto el) {
      constexpr int E = decltype(el)::value;
      hipLaunchKernelGGL((k_tp_fp8<T, E, false, U>), grid, dim3(kBlockThreads), 0, st, a, g, fin);
    });
  }
  return hipGetLastError();
}

hipError_t launch_tp(const TpArgs& a, int nt, bool bf16, const TpGeo& g, bool nv, float* ws,
                     hipStream_t st, int elem = kE4M3) {
  const bool half = chunk_tiles(g.per_slice, bf16) < (bf16 ? 8 : 4);
  if (bf16)
    return half ? launch_tp_t<uint16_t, 4>(a, nt, g, nv, ws, st, elem)
                : launch_tp_t<uint16_t, 8>(a, nt, g, nv, ws, st, elem);
  return half ? launch_tp_t<float, 2>(a, nt, g, nv, ws, st, elem)
              : launch_tp_t<float, 4>(a, nt, g, nv, ws, st, elem);
}

}  // namespace

size_t twopass_workspace_bytes(int ntensors, int64_t slices, int64_t per_slice, int64_t groups,
                               bool nv) {
  if (slices <= 0 || per_slice <= 0) return 0;
  const int64_t wf = wgs_per_slice(per_slice, false), wb = wgs_per_slice(per_slice, true);
  const int64_t W = wf > wb ? wf : wb;  // the larger of the two input types' counts
  const int64_t fin = nv ? kNvFinal : groups;
  return 4 * (size_t)ntensors * (size_t)slices * ((size_t)groups * (size_t)W + (size_t)fin);
}

hipError_t launch_tensor_fp8(const void* const* x, bool bf16, int ntensors, int64_t slices,
                             int64_t per_slice, uint8_t* const* codes, float* const* scales,
                             float* ws, hipStream_t st, int elem) {
  TpArgs a{};
  for (int i = 0; i < ntensors; ++i) {
    a.x[i] = x[i];
    a.codes[i] = codes[i];
    a.scales[i] = scales[i];
    a.mode[i] = kKvLayer;
  }
  TpGeo g{};
  g.per_slice = per_slice;
  g.slices = slices;
  g.W = (int32_t)wgs_per_slice(per_slice, bf16);
  g.G = 1;
  g.row_units = 1;
  g.head_magic = 0;
  return launch_tp(a, ntensors, bf16, g, false, ws, st, elem);
}

hipError_t launch_nvfp4(const void* x, bool bf16, int64_t batch, int64_t per_slice,
                        uint8_t* codes, uint8_t* scales, float* gs, float* ws, hipStream_t st) {
  TpArgs a{};
  a.x[0] = x;
  a.codes[0] = codes;
  a.scales[0] = scales;
  a.gs[0] = gs;
  a.mode[0] = kKvLayer;
  TpGeo g{};
  g.per_slice = per_slice;
  g.slices = batch;
  g.W = (int32_t)wgs_per_slice(per_slice, bf16);
  g.G = 1;
  g.row_units = 1;
  return launch_tp(a, 1, bf16, g, true, ws, st);
}

hipError_t launch_kv_fp8(const KvTensor* t, int ntensors, bool bf16, int64_t layers,
                         int64_t tokens, int64_t heads, int64_t head_dim, float* ws,
                         hipStream_t st) {
  TpArgs a{};
  bool head = false;
  for (int i = 0; i < ntensors; ++i) {
    a.x[i] = t[i].x;
    a.codes[i] = t[i].codes;
    a.scales[i] = t[i].scales;
    a.mode[i] = t[i].mode;
    head |= t[i].mode == kKvHead;
  }
  TpGeo g{};
  g.per_slice = tokens * heads * head_dim;
  g.slices = layers;
  g.W = (int32_t)wgs_per_slice(g.per_slice, bf16);
  g.G = head ? (int32_t)heads : 1;
  g.row_units = (int32_t)(heads * head_dim / 8);
  g.head_magic = head_magic(head_dim / 8);
  return launch_tp(a, ntensors, bf16, g, false, ws, st);
}

size_t kv_workspace_bytes(int64_t layers, int64_t tokens, int64_t heads, int64_t head_dim) {
  // two tensors, per-head groups (the largest any mode combination needs)
  return twopass_workspace_bytes(2, layers, tokens * heads * head_dim, heads, false);
}

}  // namespace pqb
