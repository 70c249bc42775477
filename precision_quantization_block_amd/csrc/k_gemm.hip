// Block-scaled FP8 GEMM, the consumer of the 1x128 activation codes and the
// 128x128 weight codes (page "量化部署实战", exercise section on FP8 blockwise
// scaling: within each 128-deep K block the FP8 products are multiplied and
// summed on the matrix cores, the block sum is multiplied by that block's
// activation and weight scales, and the result is accumulated in float32):
//
//   C[m, n] = sum_kb RN(sA[m, kb] * sB[n / 128, kb]) * P[m, n, kb],
//   P[m, n, kb] = sum_{k in kb} dec(a[m, k]) * dec(b[n, k]),
//
// accumulated with one fused multiply-add per block.  A [M, K] and B [N, K] are
// E4M3 codes, row-major; sA [M, K / 128], sB [N / 128, K / 128] float32.
//
// One workgroup of 4 waves owns a 128 x 128 tile of C; wave (wm, wn) owns the
// 64 x 64 quarter at (64 wm, 64 wn), as 4 x 4 tiles of 16 x 16.  One
// v_mfma_f32_16x16x128_f8f6f4 covers a whole 128-deep K block of one 16 x 16
// tile, so every MFMA result is promoted at once: acc = fma(P, sA sB, acc).
// The 128 x 128-byte tiles of A and B for one K block are staged through LDS,
// double buffered, with the next block's global loads in flight during the
// current block's MFMAs.  LDS rows hold 8 chunks of 16 bytes, chunk c of row r
// at position c ^ (r & 7), so the 8 lanes that read chunk c of 8 consecutive
// rows touch 8 distinct 16-byte bank groups.
//
// MFMA operand layout: lane l holds row (l & 15) of its 16-row A slice (and
// column (l & 15) of its B slice) and 32 bytes of K; A and B take the same 32
// bytes of the block, so the products pair up whatever order the matrix core
// sums them in.  Result layout: lane l, register r is C[4 (l >> 4) + r][l & 15].
#include "device.h"
#include "launch.h"

namespace pqb {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kGT = 128;                     // tile edge in M, N and K
constexpr int kGThreads = 256;               // 4 waves, 2 x 2
constexpr int kGTileBytes = kGT * kGT;       // one FP8 tile of A or B
constexpr int kGOutStride = 64 + 4;          // floats per row of a wave's staged 64 x 64 result
constexpr int kGOutBytes = 4 * 64 * kGOutStride * 4;
constexpr int kGLdsBytes = 4 * kGTileBytes > kGOutBytes ? 4 * kGTileBytes : kGOutBytes;

// Byte offset of 16-byte chunk c of row r in a staged 128 x 128-byte tile.
__device__ __forceinline__ int tile_off(int r, int c) { return r * kGT + ((c ^ (r & 7)) << 4); }

// The 32 bytes of K (chunks 2q, 2q + 1) of row r of a staged tile.
__device__ __forceinline__ v8i frag(const uint8_t* tile, int r, int q) {
  const uint4 lo = *reinterpret_cast<const uint4*>(tile + tile_off(r, 2 * q));
  const uint4 hi = *reinterpret_cast<const uint4*>(tile + tile_off(r, 2 * q + 1));
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

template <bool kBf16Out>
__global__ __launch_bounds__(kGThreads) void k_gemm_fp8_bs(const uint8_t* __restrict__ A,
                                                           const float* __restrict__ sA,
                                                           const uint8_t* __restrict__ B,
                                                           const float* __restrict__ sB, int M,
                                                           int N, int K, int tiles_n,
                                                           void* __restrict__ C) {
  // [A buf 0 | A buf 1 | B buf 0 | B buf 1], reused for the epilogue
  __shared__ __align__(16) uint8_t lds[kGLdsBytes];
  __shared__ __align__(16) float lds_s[2][kGT];
  auto lds_a = [&](int buf) { return lds + buf * kGTileBytes; };
  auto lds_b = [&](int buf) { return lds + (2 + buf) * kGTileBytes; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  const int m0 = tm * kGT, n0 = tn * kGT;
  const int nkb = K / kGT;

  // Staging: thread t moves chunk (t & 7) of rows (t >> 3) + 32 i, i < 4, of
  // both tiles, and (t < 128) the activation scale of row t.
  const int srow = tid >> 3, sc = tid & 7;
  uint4 ra[4], rb[4];
  float rs = 0.0f;
  auto load_block = [&](int kb) {
    const int64_t k0 = (int64_t)kb * kGT + 16 * sc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = srow + 32 * i;
      ra[i] = m0 + r < M ? *reinterpret_cast<const uint4*>(A + (int64_t)(m0 + r) * K + k0)
                         : uint4{0, 0, 0, 0};
      rb[i] = *reinterpret_cast<const uint4*>(B + (int64_t)(n0 + r) * K + k0);
    }
    if (tid < kGT) rs = m0 + tid < M ? sA[(int64_t)(m0 + tid) * nkb + kb] : 0.0f;
  };
  auto store_block = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = srow + 32 * i;
      *reinterpret_cast<uint4*>(lds_a(buf) + tile_off(r, sc)) = ra[i];
      *reinterpret_cast<uint4*>(lds_b(buf) + tile_off(r, sc)) = rb[i];
    }
    if (tid < kGT) lds_s[buf][tid] = rs;
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int r16 = lane & 15, q = lane >> 4;
  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  if (nkb > 0) {
    load_block(0);
    store_block(0);
  }
  __syncthreads();
  const float* sB_col = sB + (int64_t)(n0 / kGT) * nkb;
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) load_block(kb + 1);
    const float sb = sB_col[kb];
    v8i af[4];
    v4f sab[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      af[mt] = frag(lds_a(buf), wm * 64 + mt * 16 + r16, q);
      const v4f s4 = *reinterpret_cast<const v4f*>(&lds_s[buf][wm * 64 + mt * 16 + 4 * q]);
      sab[mt] = s4 * sb;
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const v8i bf = frag(lds_b(buf), wn * 64 + nt * 16 + r16, q);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            af[mt], bf, v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mt][nt][r] = __builtin_fmaf(p[r], sab[mt][r], acc[mt][nt][r]);
      }
    }
    if (kb + 1 < nkb) store_block(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: each wave stages its 64 x 64 floats in LDS (rows padded to 68
  // floats), then writes whole row segments: 256 bytes per row for float32,
  // 128 for bf16, with 16-byte stores.
  float* out_lds = reinterpret_cast<float*>(lds) + wave * 64 * kGOutStride;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        out_lds[(mt * 16 + 4 * q + r) * kGOutStride + nt * 16 + r16] = acc[mt][nt][r];
  __syncthreads();
  const int row0 = m0 + wm * 64, col0 = n0 + wn * 64;
  if constexpr (kBf16Out) {
    // 8 lanes per row, 8 rows per step
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int rr = s * 8 + (lane >> 3), cc = (lane & 7) * 8;
      if (row0 + rr < M) {
        const float* v = out_lds + rr * kGOutStride + cc;
        const v4f x0 = *reinterpret_cast<const v4f*>(v), x1 = *reinterpret_cast<const v4f*>(v + 4);
        uint16_t* dst = reinterpret_cast<uint16_t*>(C) + (int64_t)(row0 + rr) * N + col0 + cc;
        st_nt16(dst, bf16x2_rne(x0[0], x0[1]), bf16x2_rne(x0[2], x0[3]), bf16x2_rne(x1[0], x1[1]),
                bf16x2_rne(x1[2], x1[3]));
      }
    }
  } else {
    // 16 lanes per row, 4 rows per step
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int rr = s * 4 + (lane >> 4), cc = (lane & 15) * 4;
      if (row0 + rr < M) {
        const v4f x = *reinterpret_cast<const v4f*>(out_lds + rr * kGOutStride + cc);
        float* dst = reinterpret_cast<float*>(C) + (int64_t)(row0 + rr) * N + col0 + cc;
        st_nt16(dst, as_u(x[0]), as_u(x[1]), as_u(x[2]), as_u(x[3]));
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_fp8_bs(const uint8_t* a, const float* a_scales, const uint8_t* b,
                              const float* b_scales, int64_t M, int64_t N, int64_t K,
                              bool out_bf16, void* c, hipStream_t st) {
  const int tiles_m = (int)((M + kGT - 1) / kGT), tiles_n = (int)(N / kGT);
  const dim3 grid((unsigned)tiles_m * (unsigned)tiles_n);
  if (out_bf16)
    hipLaunchKernelGGL((k_gemm_fp8_bs<true>), grid, dim3(kGThreads), 0, st, a, a_scales, b,
                       b_scales, (int)M, (int)N, (int)K, tiles_n, c);
  else
    hipLaunchKernelGGL((k_gemm_fp8_bs<false>), grid, dim3(kGThreads), 0, st, a, a_scales, b,
                       b_scales, (int)M, (int)N, (int)K, tiles_n, c);
  return hipGetLastError();
}

}  // namespace pqb
