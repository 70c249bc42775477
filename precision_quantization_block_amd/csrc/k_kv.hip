// FP8 KV-cache write with a scale mode per tensor (page "量化部署实战", section
// KV Cache 量化：误差要和信号比): K and V are quantized by independent
// quantizers, each with one scale per layer, one per (layer, head) over the
// tokens and head_dim (the page's per_head), or a static per-layer scale
// calibrated offline, for which the clamp to +-448 can bind.
//
// Layout [layers, tokens, heads, head_dim] (token-major).  One slice = one
// layer of K or V.  Both passes stream a slice grid-stride with a stride that
// is a multiple of the row width (heads * head_dim / 8 units), so a thread
// keeps one column, and so one head, for the whole slice: pass 1 keeps a
// running max per thread and folds it into its head's LDS slot once; pass 2
// looks its scale up once.
#include "launch.h"
#include "quant.h"

namespace pqb {
namespace {

struct KvArgs {
  const void* x[2];
  uint8_t* codes[2];
  float* scales[2];  // LAYER / HEAD: written; STATIC: read
  int32_t mode[2];
};

struct KvGeom {
  int64_t per_layer;  // elements of one slice (multiple of 8)
  int64_t layers;
  int32_t row_units;  // heads * head_dim / 8
  int32_t head_units; // head_dim / 8
  int32_t heads;
  int32_t P;          // pass-1 workgroups per slice (with a HEAD tensor, P * 256 is a
                      // multiple of row_units)
};

// Scope of this thread's (fixed) column: its head, or 0 for a per-layer scale.
__device__ __forceinline__ int kv_scope(int mode, int64_t u0, const KvGeom& g) {
  return mode == kKvHead ? (int)(u0 % g.row_units) / g.head_units : 0;
}

template <typename T>
__global__ __launch_bounds__(kBlockThreads) void k_kv_partial(KvArgs a, KvGeom g,
                                                              uint32_t* __restrict__ partials) {
  __shared__ uint32_t red[kMaxKvHeads];
  const int tz = blockIdx.z, mode = a.mode[tz];
  if (mode == kKvStatic) return;  // uniform over the workgroup
  const int64_t layer = blockIdx.y;
  const int G = mode == kKvHead ? g.heads : 1;
  for (int i = threadIdx.x; i < G; i += kBlockThreads) red[i] = 0;
  __syncthreads();
  const T* xs = reinterpret_cast<const T*>(a.x[tz]) + layer * g.per_layer;
  const int64_t nunits = g.per_layer / 8;
  const int64_t stride = (int64_t)gridDim.x * kBlockThreads;
  int64_t u = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x;
  const int scope = kv_scope(mode, u, g);
  uint32_t m = 0;
  for (; u + 3 * stride < nunits; u += 4 * stride) {
    const Raw8 r0 = load_raw8(xs + u * 8), r1 = load_raw8(xs + (u + stride) * 8);
    const Raw8 r2 = load_raw8(xs + (u + 2 * stride) * 8);
    const Raw8 r3 = load_raw8(xs + (u + 3 * stride) * 8);
    float v[8];
    widen8(r0, xs, v); m = max(m, as_u(absmax8(v)));
    widen8(r1, xs, v); m = max(m, as_u(absmax8(v)));
    widen8(r2, xs, v); m = max(m, as_u(absmax8(v)));
    widen8(r3, xs, v); m = max(m, as_u(absmax8(v)));
  }
  for (; u < nunits; u += stride) {
    float v[8];
    widen8(load_raw8(xs + u * 8), xs, v);
    m = max(m, as_u(absmax8(v)));
  }
  if (G == 1) m = wave_umax(m);
  if (G > 1 || (threadIdx.x & (kWave - 1)) == 0) atomicMax(&red[scope], m);
  __syncthreads();
  uint32_t* out = partials + (((int64_t)tz * g.layers + layer) * g.P + blockIdx.x) * g.heads;
  for (int i = threadIdx.x; i < G; i += kBlockThreads) out[i] = red[i];
}

// Eight codes from x with the static-scale clamp: |x| is first limited to
// 512 s (so x * RN(1/s) cannot overflow; any |x/s| >= 512 saturates anyway),
// then the correctly rounded quotient is clamped to +-448.
__device__ __forceinline__ uint2 fp8_pack8_clamped(const float v[8], float s, float y, float lim) {
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    q[i] = __builtin_amdgcn_fmed3f(div_rn(__builtin_amdgcn_fmed3f(v[i], -lim, lim), s, y), -448.0f,
                                   448.0f);
  return make_uint2(e4m3_bytes4(q[0], q[1], q[2], q[3]), e4m3_bytes4(q[4], q[5], q[6], q[7]));
}

template <typename T, bool kStatic>
__device__ __forceinline__ void kv_stream(const T* __restrict__ xs, uint8_t* __restrict__ cs,
                                          int64_t u, int64_t nunits, int64_t stride, float s,
                                          float y) {
  const float lim = s * 512.0f;
  auto pack = [&](const float v[8]) {
    if constexpr (kStatic)
      return fp8_pack8_clamped(v, s, y, lim);
    else
      return fp8_pack8(v, s, y);
  };
  for (; u + stride < nunits; u += 2 * stride) {
    const Raw8 r0 = load_raw8(xs + u * 8), r1 = load_raw8(xs + (u + stride) * 8);
    float v[8];
    widen8(r0, xs, v);
    store_codes8(cs + u * 8, pack(v));
    widen8(r1, xs, v);
    store_codes8(cs + (u + stride) * 8, pack(v));
  }
  for (; u < nunits; u += stride) {
    float v[8];
    widen8(load_raw8(xs + u * 8), xs, v);
    store_codes8(cs + u * 8, pack(v));
  }
}

template <typename T>
__global__ __launch_bounds__(kBlockThreads) void k_kv_quant(KvArgs a, KvGeom g,
                                                            const uint32_t* __restrict__ partials) {
  __shared__ uint32_t red[kMaxKvHeads];
  __shared__ float ss[kMaxKvHeads], ys[kMaxKvHeads];
  const int tz = blockIdx.z, mode = a.mode[tz];
  const int64_t layer = blockIdx.y;
  const int G = mode == kKvHead ? g.heads : 1;
  if (mode == kKvStatic) {
    if (threadIdx.x == 0) {
      const float s = a.scales[tz][layer];
      ss[0] = s;
      ys[0] = recip_rn(s);
    }
  } else {
    for (int i = threadIdx.x; i < G; i += kBlockThreads) red[i] = 0;
    __syncthreads();
    const uint32_t* p = partials + ((int64_t)tz * g.layers + layer) * g.P * g.heads;
    const int64_t n = (int64_t)g.P * g.heads;
    for (int64_t i = threadIdx.x; i < n; i += kBlockThreads) {
      const int h = (int)(i % g.heads);
      if (h < G) atomicMax(&red[h], p[i]);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < G; i += kBlockThreads) {
      const float s = fp8_scale_bits(red[i]);
      ss[i] = s;
      ys[i] = recip_rn(s);
      if (blockIdx.x == 0) a.scales[tz][layer * G + i] = s;
    }
  }
  __syncthreads();
  const int64_t nunits = g.per_layer / 8;
  const int64_t stride = (int64_t)gridDim.x * kBlockThreads;
  const int64_t u = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x;
  const int scope = kv_scope(mode, u, g);
  const float s = ss[scope], y = ys[scope];
  const T* xs = reinterpret_cast<const T*>(a.x[tz]) + layer * g.per_layer;
  uint8_t* cs = a.codes[tz] + layer * g.per_layer;
  if (mode == kKvStatic)
    kv_stream<T, true>(xs, cs, u, nunits, stride, s, y);
  else
    kv_stream<T, false>(xs, cs, u, nunits, stride, s, y);
}

int64_t gcd64(int64_t a, int64_t b) {
  while (b) {
    const int64_t t = a % b;
    a = b;
    b = t;
  }
  return a;
}

int64_t kv_blocks(int64_t work, int64_t per_block, int64_t cap) {
  const int64_t g = (work + per_block - 1) / per_block;
  return g < 1 ? 1 : (g > cap ? cap : g);
}

// Workgroups per slice for either pass, rounded up so that the grid stride
// (count * 256 units) is a multiple of the row width.
int64_t kv_round(int64_t count, int64_t row_units) {
  const int64_t m = row_units / gcd64(row_units, kBlockThreads);
  return (count + m - 1) / m * m;
}

}  // namespace

int64_t kv_stride_multiple(int64_t row_units) { return row_units / gcd64(row_units, kBlockThreads); }

int kv_partials_per_slice(int64_t layers, int64_t per_layer, int64_t row_units, int ntensors,
                          bool head) {
  const int64_t p = amax_partials_per_slice(layers, per_layer, ntensors);
  return (int)(head ? kv_round(p, row_units) : p);
}

hipError_t launch_kv_fp8(const KvTensor* t, int ntensors, bool bf16, int64_t layers,
                         int64_t tokens, int64_t heads, int64_t head_dim, uint32_t* partials,
                         hipStream_t st) {
  KvArgs a{};
  bool dynamic = false, head = false;
  for (int i = 0; i < ntensors; ++i) {
    a.x[i] = t[i].x;
    a.codes[i] = t[i].codes;
    a.scales[i] = t[i].scales;
    a.mode[i] = t[i].mode;
    dynamic |= t[i].mode != kKvStatic;
    head |= t[i].mode == kKvHead;
  }
  KvGeom g{};
  g.per_layer = tokens * heads * head_dim;
  g.layers = layers;
  g.row_units = (int32_t)(heads * head_dim / 8);
  g.head_units = (int32_t)(head_dim / 8);
  g.heads = (int32_t)heads;
  g.P = kv_partials_per_slice(layers, g.per_layer, g.row_units, ntensors, head);
  if (dynamic) {
    const dim3 g1((unsigned)g.P, (unsigned)layers, ntensors);
    if (bf16)
      hipLaunchKernelGGL(k_kv_partial<uint16_t>, g1, dim3(kBlockThreads), 0, st, a, g, partials);
    else
      hipLaunchKernelGGL(k_kv_partial<float>, g1, dim3(kBlockThreads), 0, st, a, g, partials);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // pass 2: about 8 units per thread, at most about 1024 workgroups per slice
  int64_t q = kv_blocks(g.per_layer / 8, (int64_t)kBlockThreads * 8, 1024);
  if (head) q = kv_round(q, g.row_units);
  const dim3 g2((unsigned)q, (unsigned)layers, ntensors);
  if (bf16)
    hipLaunchKernelGGL(k_kv_quant<uint16_t>, g2, dim3(kBlockThreads), 0, st, a, g, partials);
  else
    hipLaunchKernelGGL(k_kv_quant<float>, g2, dim3(kBlockThreads), 0, st, a, g, partials);
  return hipGetLastError();
}

}  // namespace pqb
