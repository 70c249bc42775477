// W4A16 product, the consumer of the INT4 group-128 codes (page "14. 量化：让
// 每一步搬更少的字节", 路线一: the 4-bit weights are read from memory,
// unpacked and dequantized to 16 bits, and multiplied, which is what cuts
// decode time):
//
//   y[m, n] = sum_k x[m, k] * (q[n, k] - z[n, g]) * s[n, g],   g = k / 128,
//
// for bf16 activations x [M, K], M <= 8 (decode), and a weight in the layout
// pqb_quantize writes for INT4_ASYM x GRP_128: codes [N, K / 2] (element 2i in
// the low nibble of byte i, two's complement), bf16 scales [N, K / 128],
// zero-point nibbles over the flat group index n * K / 128 + g.
//
// With q + 8 = (nibble ^ 8) in 0 .. 15, the weight w = 128 + q + 8 is an exact
// bf16 whose high byte is 0x43 and whose low byte is q + 8.  A unit of 32
// weights inside one group then contributes s * (sum x w - (136 + z) sum x),
// and both sums are packed bf16 dot products (v_dot2c_f32_bf16: two exact
// products per instruction added into a float32 accumulator; sum x is the dot
// with (1, 1)).  Unpacking costs, per 8 weights, one mask and one shift-mask
// (both with the sign flip) that split the nibbles into bytes, then one byte
// permute per pair that places two of them under the 0x43 byte.  The same
// permute pairs up the activations, once per unit for all rows.
//
// Lane l of a wave handles code units u = l, l + 64, ... (16 bytes = 32
// weights each) of kR consecutive rows; every wave load instruction reads 1
// KiB of one row.  The units are walked as items of kSteps units per lane, and
// the codes of the next item are loaded before the current one is computed.
// The activations are read once per unit and reused for the kR rows.  A
// wave-wide sum ends each row.
// One launch serves up to kW4MaxJobs independent products (the projections
// that share an input, or any batch of weights): workgroup b belongs to the
// job whose range of workgroups holds b.
#include "device.h"
#include "launch.h"

namespace pqb {
namespace {

constexpr int kWThreads = 256;  // 4 waves
// Launch shapes chosen by the rows one launch covers (measured on the
// Llama-3.1-8B-shaped weights): 2 rows per wave when a launch holds a few
// projections (more waves: with 2 units per lane in flight at M = 1), more
// rows per wave when it holds many (the activations then serve more rows per
// load): 8 at M <= 2 from 2^16 rows, 4 at M = 3 .. 5 from 2^13 rows.
constexpr int kBigLaunchRows = 1 << 16;
constexpr int kMidLaunchRows = 1 << 13;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x2v as_bf2(uint32_t v) { return __builtin_bit_cast(bf16x2v, v); }
constexpr uint32_t kBf16Ones = 0x3F803F80u;    // (1.0, 1.0)
constexpr uint32_t kBf16Hi128 = 0x43434343u;   // high byte of bf16 128 .. 255

template <int kM, bool kBf16Out, int kR, int kSteps>
__global__ __launch_bounds__(kWThreads) void k_w4a16(const W4Args a) {
  constexpr int kBlocks = 1;
  int jb = 0;
  while (jb + 1 < a.njobs && a.wg_begin[jb + 1] <= (int)blockIdx.x) ++jb;
  const uint16_t* __restrict__ x = a.job[jb].x;
  const uint8_t* __restrict__ codes = a.job[jb].codes;
  const uint16_t* __restrict__ scales = a.job[jb].scales;
  const uint8_t* __restrict__ zeros = a.job[jb].zeros;
  void* __restrict__ y = a.job[jb].y;
  const int N = a.job[jb].N, K = a.job[jb].K;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  // This wave's rows: kBlocks blocks of kR, walked as items (block, chunk of
  // kSteps units per lane); the codes of item i + 1 are loaded before item i
  // is computed.
  const int nw0 = (((int)blockIdx.x - a.wg_begin[jb]) * (kWThreads / 64) + wave) * kR * kBlocks;
  if (nw0 >= N) return;
  if (K == 0) {   // the empty sum: this wave's rows of y are zero
    for (int i = lane; i < kM * kR * kBlocks; i += 64) {
      const int m = i / (kR * kBlocks), n = nw0 + i % (kR * kBlocks);
      if (n < N) {
        if constexpr (kBf16Out)
          reinterpret_cast<uint16_t*>(y)[(int64_t)m * N + n] = 0;
        else
          reinterpret_cast<float*>(y)[(int64_t)m * N + n] = 0.0f;
      }
    }
    return;
  }
  const int U = K / 32, G = K / 128;
  const int chunks = (U + 64 * kSteps - 1) / (64 * kSteps);
  const int blocks = min(kBlocks, (N - nw0 + kR - 1) / kR);
  const int items = blocks * chunks;

  auto load_item = [&](int it, uint4 (&c)[kSteps][kR]) {
    const int b = it / chunks, u0 = (it - b * chunks) * 64 * kSteps;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const int u = u0 + 64 * s + lane;
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const int row = min(nw0 + b * kR + r, N - 1);   // rows past N are never stored
        c[s][r] = u < U ? ld_nt16(codes + (int64_t)row * (K / 2) + 16 * u) : uint4{0, 0, 0, 0};
      }
    }
  };

  float acc[kM][kR];
#pragma unroll
  for (int m = 0; m < kM; ++m)
#pragma unroll
    for (int r = 0; r < kR; ++r) acc[m][r] = 0.0f;
  uint4 cur[kSteps][kR], nxt[kSteps][kR];
  load_item(0, cur);
  for (int it = 0; it < items; ++it) {
    const int b = it / chunks, u0 = (it - b * chunks) * 64 * kSteps;
    const int n0 = nw0 + b * kR;
    // This item's activations, scales and zero-points are loaded before the
    // next item's codes: loads complete in issue order, so waiting for them
    // then does not wait for the prefetch.
    uint32_t xd[kSteps][kM][16];
    uint16_t sb[kSteps][kR];
    uint8_t zb[kSteps][kR];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const int u = min(u0 + 64 * s + lane, U - 1);   // lanes past U compute nothing
#pragma unroll
      for (int m = 0; m < kM; ++m) {
        const uint4* p = reinterpret_cast<const uint4*>(x + (int64_t)m * K + 32 * u);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 v = p[i];
          xd[s][m][4 * i] = v.x;
          xd[s][m][4 * i + 1] = v.y;
          xd[s][m][4 * i + 2] = v.z;
          xd[s][m][4 * i + 3] = v.w;
        }
      }
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const int gi = min(n0 + r, N - 1) * G + (u >> 2);
        sb[s][r] = scales[gi];
        zb[s][r] = zeros[gi >> 1];
      }
    }
    if (it + 1 < items) load_item(it + 1, nxt);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const int u = u0 + 64 * s + lane;
      if (u >= U) break;
      // Activation pairs matching the weight pairs below: for code dword d,
      // xp[4d + 2h + e] = (x[8d + 4h + e], x[8d + 4h + e + 2]) (e: nibble,
      // h: byte half); xs = sum of the unit's 32 x.
      bf16x2v xp[kM][16];
      float xs[kM];
#pragma unroll
      for (int m = 0; m < kM; ++m) {
        float t = 0.0f;
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const uint32_t lo = xd[s][m][4 * d + 2 * h], hi = xd[s][m][4 * d + 2 * h + 1];
              const bf16x2v v = as_bf2(__builtin_amdgcn_perm(hi, lo, e ? 0x07060302u : 0x05040100u));
              xp[m][4 * d + 2 * h + e] = v;
              t = __builtin_amdgcn_fdot2_f32_bf16(v, as_bf2(kBf16Ones), t, false);
            }
        xs[m] = t;
      }
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const int gi = min(n0 + r, N - 1) * G + (u >> 2);
        const float sc = as_f((uint32_t)sb[s][r] << 16);
        const int zn = (zb[s][r] >> (4 * (gi & 1))) & 0xF;
        const float cz = (float)(136 + (zn >= 8 ? zn - 16 : zn));    // 128 + 8 + z
        const uint32_t w4[4] = {cur[s][r].x, cur[s][r].y, cur[s][r].z, cur[s][r].w};
        float dot[kM];
#pragma unroll
        for (int m = 0; m < kM; ++m) dot[m] = 0.0f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          // q + 8 of the low (e = 0) and high (e = 1) nibble of each byte
          const uint32_t nb[2] = {(w4[d] & 0x0F0F0F0Fu) ^ 0x08080808u,
                                  ((w4[d] >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u};
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              // bytes 2h, 2h + 1 of nb[e] under the bf16 exponent byte 0x43:
              // the pair (128 + q + 8) of weights 8d + 4h + e, 8d + 4h + e + 2
              const bf16x2v wp = as_bf2(__builtin_amdgcn_perm(nb[e], kBf16Hi128, h ? 0x00070006u : 0x00050004u));
#pragma unroll
              for (int m = 0; m < kM; ++m)
                dot[m] = __builtin_amdgcn_fdot2_f32_bf16(xp[m][4 * d + 2 * h + e], wp, dot[m], false);
            }
        }
#pragma unroll
        for (int m = 0; m < kM; ++m)
          acc[m][r] = __builtin_fmaf(sc, __builtin_fmaf(-cz, xs[m], dot[m]), acc[m][r]);
      }
    }
    if (it - b * chunks == chunks - 1) {   // last chunk of block b: finish its rows
#pragma unroll
      for (int m = 0; m < kM; ++m)
#pragma unroll
        for (int r = 0; r < kR; ++r) {
          const float v = wave_sum(acc[m][r]);
          acc[m][r] = 0.0f;
          if (lane == 0 && n0 + r < N) {
            if constexpr (kBf16Out)
              reinterpret_cast<uint16_t*>(y)[(int64_t)m * N + n0 + r] = (uint16_t)bf16_rne_bits(v);
            else
              reinterpret_cast<float*>(y)[(int64_t)m * N + n0 + r] = v;
          }
        }
    }
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
#pragma unroll
      for (int r = 0; r < kR; ++r) cur[s][r] = nxt[s][r];
  }
}

template <int kM, int kR, int kSteps>
void launch_m(const W4Args& a, int wgs, bool out_bf16, hipStream_t st) {
  if (out_bf16)
    hipLaunchKernelGGL((k_w4a16<kM, true, kR, kSteps>), dim3((unsigned)wgs), dim3(kWThreads), 0, st,
                       a);
  else
    hipLaunchKernelGGL((k_w4a16<kM, false, kR, kSteps>), dim3((unsigned)wgs), dim3(kWThreads), 0,
                       st, a);
}

template <int kM, int kR, int kSteps>
hipError_t launch_shape(W4Args& a, bool out_bf16, hipStream_t st) {
  constexpr int rows_per_wg = (kWThreads / 64) * kR;
  int wg = 0;
  for (int i = 0; i < a.njobs; ++i) {
    a.wg_begin[i] = wg;
    wg += (a.job[i].N + rows_per_wg - 1) / rows_per_wg;
  }
  a.wg_begin[a.njobs] = wg;
  if (wg > 0) launch_m<kM, kR, kSteps>(a, wg, out_bf16, st);
  return hipGetLastError();
}

// Shapes per M that keep every instantiation free of register spills and at
// two or more waves per SIMD.
hipError_t launch_args(W4Args& a, int M, int64_t rows, bool out_bf16, hipStream_t st) {
  const bool big = rows >= kBigLaunchRows, mid = rows >= kMidLaunchRows;
  switch (M) {
    case 1: return big ? launch_shape<1, 8, 1>(a, out_bf16, st) : launch_shape<1, 2, 2>(a, out_bf16, st);
    case 2: return big ? launch_shape<2, 8, 1>(a, out_bf16, st) : launch_shape<2, 2, 1>(a, out_bf16, st);
    case 3: return mid ? launch_shape<3, 4, 1>(a, out_bf16, st) : launch_shape<3, 2, 1>(a, out_bf16, st);
    case 4: return mid ? launch_shape<4, 4, 1>(a, out_bf16, st) : launch_shape<4, 2, 1>(a, out_bf16, st);
    case 5: return mid ? launch_shape<5, 4, 1>(a, out_bf16, st) : launch_shape<5, 2, 1>(a, out_bf16, st);
    case 6: return launch_shape<6, 2, 1>(a, out_bf16, st);
    case 7: return launch_shape<7, 2, 1>(a, out_bf16, st);
    case 8: return launch_shape<8, 2, 1>(a, out_bf16, st);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------
// The same product on the matrix cores, for any M (v_mfma_f32_16x16x32_bf16).
// A workgroup owns kTiles tiles of 16 weight rows (the MFMA's N): four in
// launches of 2^14 rows or more, where sharing each activation load among the
// tiles pays, and one in smaller launches (most of a layer's projections),
// which need the workgroups.  Its 4 waves split K into four contiguous ranges of groups,
// so that one wave reads both halves of a 128-byte code line and a row's
// scales in consecutive steps.  For one group, lane l supplies row l & 15 of
// the activation block and of each weight tile, and K positions 32 (l >> 4)
// .. + 31 of the group, 8 per MFMA: its 16 code bytes of a tile are one load,
// and the activations of each MFMA one 16-byte load in the same K order,
// shared by the tiles.  The codes become exact bf16 w = 136 + q (high byte
// 0x43, low byte q + 8), so a group contributes s * (P - (136 + z) * S) with
// P = sum x w from four MFMAs per tile and S = sum x from four more against a
// B of ones; both are float32 accumulations of exact products.  The four
// waves' results meet in LDS and are added in wave order.  Activation rows
// come in blocks of 16 (kMB of them, up to 32 rows per launch); rows past M
// and weight rows past N are read clamped and never stored.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
constexpr int kMaxMB = 2;                    // 16-row activation blocks per launch
constexpr int kMfmaWaves = kWThreads / 64;

template <int kMB, int kTiles, bool kBf16Out>
__global__ __launch_bounds__(kWThreads) void k_w4a16_mfma(const W4Args a, int M) {
  constexpr int kMfmaRows = 16 * kTiles;
  int jb = 0;
  while (jb + 1 < a.njobs && a.wg_begin[jb + 1] <= (int)blockIdx.x) ++jb;
  const uint16_t* __restrict__ x = a.job[jb].x;
  const uint8_t* __restrict__ codes = a.job[jb].codes;
  const uint16_t* __restrict__ scales = a.job[jb].scales;
  const uint8_t* __restrict__ zeros = a.job[jb].zeros;
  void* __restrict__ y = a.job[jb].y;
  const int N = a.job[jb].N, K = a.job[jb].K;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int n0 = ((int)blockIdx.x - a.wg_begin[jb]) * kMfmaRows;
  const int col = lane & 15, kq = lane >> 4;
  const int G = K / 128;
  int nrow[kTiles];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) nrow[t] = min(n0 + 16 * t + col, N - 1);

  f32x4v acc[kMB][kTiles];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int t = 0; t < kTiles; ++t) acc[mb][t] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
  const int gb = wave * G / kMfmaWaves, ge = (wave + 1) * G / kMfmaWaves;   // this wave's groups
  if (gb < ge) {
    const uint16_t* xrow[kMB];
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) xrow[mb] = x + (int64_t)min(16 * mb + col, M - 1) * K + 32 * kq;
    // One group's weight data for this lane: the 16 code bytes of each tile
    // row, with its scale and zero-point byte; loaded one group ahead.
    struct Grp {
      uint4 c[kTiles];
      uint16_t s[kTiles];
      uint8_t z[kTiles];
    };
    auto load_grp = [&](int g, Grp& v) {
#pragma unroll
      for (int t = 0; t < kTiles; ++t) {
        v.c[t] = *reinterpret_cast<const uint4*>(codes + (int64_t)nrow[t] * (K / 2) + 64 * g + 16 * kq);
        const int gi = nrow[t] * G + g;
        v.s[t] = scales[gi];
        v.z[t] = zeros[gi >> 1];
      }
    };
    const uint4 ones4 = {kBf16Ones, kBf16Ones, kBf16Ones, kBf16Ones};
    const bf16x8v ones = __builtin_bit_cast(bf16x8v, ones4);
    // Group g is computed from one buffer while group g + 1 loads into the
    // other; the loop body takes two groups so that the buffers swap roles
    // without a register copy (a copy would wait for the prefetch).
    auto step = [&](int g, const Grp& cur, Grp& nxt) {
      uint4 xv[4][kMB];
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
          xv[st][mb] = *reinterpret_cast<const uint4*>(xrow[mb] + 128 * g + 8 * st);
      // The prefetch is unconditional (the last group reloads itself): under
      // a branch, the compiler's load counters would assume it absent and
      // wait for it before this group's last product.  The scheduling fences
      // keep the issue order activations, prefetch, products, so that the
      // products wait only for the activations.
      __builtin_amdgcn_sched_barrier(0);
      load_grp(min(g + 1, ge - 1), nxt);
      __builtin_amdgcn_sched_barrier(0);
      f32x4v p[kMB][kTiles], sx[kMB];
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) {
        sx[mb] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int t = 0; t < kTiles; ++t) p[mb][t] = sx[mb];
      }
#pragma unroll
      for (int st = 0; st < 4; ++st) {
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
          sx[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, xv[st][mb]),
                                                           ones, sx[mb], 0, 0, 0);
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
          // K positions 8 st + i: byte i / 2 of code dword st, low nibble for even i
          const uint32_t w = st == 0 ? cur.c[t].x : st == 1 ? cur.c[t].y : st == 2 ? cur.c[t].z : cur.c[t].w;
          const uint32_t lo = (w & 0x0F0F0F0Fu) ^ 0x08080808u;
          const uint32_t hi = ((w >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u;
          uint4 wb;
          wb.x = __builtin_amdgcn_perm(hi, lo, 0x0C040C00u) | 0x43004300u;
          wb.y = __builtin_amdgcn_perm(hi, lo, 0x0C050C01u) | 0x43004300u;
          wb.z = __builtin_amdgcn_perm(hi, lo, 0x0C060C02u) | 0x43004300u;
          wb.w = __builtin_amdgcn_perm(hi, lo, 0x0C070C03u) | 0x43004300u;
          const bf16x8v bv = __builtin_bit_cast(bf16x8v, wb);
#pragma unroll
          for (int mb = 0; mb < kMB; ++mb)
            p[mb][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, xv[st][mb]),
                                                               bv, p[mb][t], 0, 0, 0);
        }
      }
#pragma unroll
      for (int t = 0; t < kTiles; ++t) {
        const int gi = nrow[t] * G + g;
        const float sc = as_f((uint32_t)cur.s[t] << 16);
        const int zn = (cur.z[t] >> (4 * (gi & 1))) & 0xF;
        const float cz = (float)(136 + (zn >= 8 ? zn - 16 : zn));      // 128 + 8 + z
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[mb][t][r] = __builtin_fmaf(sc, __builtin_fmaf(-cz, sx[mb][r], p[mb][t][r]), acc[mb][t][r]);
      }
    };
    Grp b0, b1;
    load_grp(gb, b0);
    for (int g = gb; g < ge; g += 2) {
      step(g, b0, b1);
      if (g + 1 < ge) step(g + 1, b1, b0);
    }
  }
  // lane l holds rows 16 mb + 4 (l >> 4) + r of column n0 + 16 t + col
  __shared__ f32x4v part[kMfmaWaves][kMB][kTiles][64];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int t = 0; t < kTiles; ++t) part[wave][mb][t][lane] = acc[mb][t];
  __syncthreads();
  // wave w finishes tile w
  const int t = wave, n = n0 + 16 * t + col;
  if (t >= kTiles || n >= N) return;
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) {
    f32x4v v = part[0][mb][t][lane];
#pragma unroll
    for (int w = 1; w < kMfmaWaves; ++w) v += part[w][mb][t][lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 16 * mb + 4 * kq + r;
      if (m < M) {
        if constexpr (kBf16Out)
          reinterpret_cast<uint16_t*>(y)[(int64_t)m * N + n] = (uint16_t)bf16_rne_bits(v[r]);
        else
          reinterpret_cast<float*>(y)[(int64_t)m * N + n] = v[r];
      }
    }
  }
}

// Launches of this many weight rows or more take four tiles per workgroup:
// enough rows for 256 workgroups of 64, and each activation load then serves
// 4 tiles instead of 1 (a gate-up projection of 28672 rows: 27.7 -> 25.8 us
// per launch at M = 1, 32.0 -> 27.2 at M = 4, 45.7 -> 31.2 at M = 16, 140.0
// -> 76.3 at M = 64; one of 4096 rows, 64 workgroups of 4 tiles, is slower).
constexpr int64_t kMfmaBigLaunchRows = 1 << 14;

template <int kMB, int kTiles>
void launch_mfma_mb(const W4Args& a, int wgs, int M, bool out_bf16, hipStream_t st) {
  if (out_bf16)
    hipLaunchKernelGGL((k_w4a16_mfma<kMB, kTiles, true>), dim3((unsigned)wgs), dim3(kWThreads), 0,
                       st, a, M);
  else
    hipLaunchKernelGGL((k_w4a16_mfma<kMB, kTiles, false>), dim3((unsigned)wgs), dim3(kWThreads), 0,
                       st, a, M);
}

}  // namespace

hipError_t launch_w4a16(const W4Job* jobs, int njobs, int M, bool out_bf16, hipStream_t st) {
  for (int base = 0; base < njobs; base += kW4MaxJobs) {
    const int n = njobs - base < kW4MaxJobs ? njobs - base : kW4MaxJobs;
    W4Args a{};
    a.njobs = n;
    int64_t rows = 0;
    for (int i = 0; i < n; ++i) {
      a.job[i] = jobs[base + i];
      rows += a.job[i].N;
    }
    const hipError_t e = launch_args(a, M, rows, out_bf16, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_w4a16_mfma(const W4Job* jobs, int njobs, int64_t M, bool out_bf16,
                             hipStream_t st) {
  constexpr int kSlice = 16 * kMaxMB;
  for (int64_t m0 = 0; m0 < M; m0 += kSlice) {
    const int mr = (int)(M - m0 < kSlice ? M - m0 : kSlice);
    for (int base = 0; base < njobs; base += kW4MaxJobs) {
      const int n = njobs - base < kW4MaxJobs ? njobs - base : kW4MaxJobs;
      W4Args a{};
      a.njobs = n;
      int64_t rows = 0;
      for (int i = 0; i < n; ++i) rows += jobs[base + i].N;
      const int tiles = rows >= kMfmaBigLaunchRows ? 4 : 1, per_wg = 16 * tiles;
      int wg = 0;
      for (int i = 0; i < n; ++i) {
        W4Job j = jobs[base + i];
        j.x += m0 * j.K;
        j.y = static_cast<char*>(j.y) + m0 * j.N * (out_bf16 ? 2 : 4);
        a.job[i] = j;
        a.wg_begin[i] = wg;
        wg += (j.N + per_wg - 1) / per_wg;
      }
      a.wg_begin[n] = wg;
      if (wg == 0) continue;
      if (mr > 16)
        tiles == 4 ? launch_mfma_mb<2, 4>(a, wg, mr, out_bf16, st)
                   : launch_mfma_mb<2, 1>(a, wg, mr, out_bf16, st);
      else
        tiles == 4 ? launch_mfma_mb<1, 4>(a, wg, mr, out_bf16, st)
                   : launch_mfma_mb<1, 1>(a, wg, mr, out_bf16, st);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace pqb
