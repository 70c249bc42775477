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
// The products are taken transposed, weight rows as the matrix core's first
// operand, so that each lane's results share one activation row per tile and
// one scale product sA sB (4 multiplies per block instead of 16).  The four
// products of a column of tiles are issued before any of them is promoted,
// into distinct registers: with one result register set the compiler routed
// every product through the same accumulation registers and waited out each
// one's latency before the next could issue.
// The 128 x 128-byte tiles of A and B for one K block, and its 128 activation
// scales, go straight from global memory into LDS (global_load_lds_dwordx4:
// each wave instruction fills 1 KiB of LDS, lane l the 16 bytes at 16 l) in a
// ring of kGStages slots, so the loads of the next kGStages - 1 blocks are in
// flight while one block is multiplied.  The loads are issued from inline
// assembly and waited for with explicit vmcnt counts (every wave issues the
// same number of loads per block), since the compiler would otherwise wait for
// all of them before every LDS read.  LDS rows hold 8 chunks of 16 bytes, chunk c of
// row r at position c ^ (r & 7) (the lane filling position p loads chunk
// p ^ (r & 7)), so the 8 lanes that read chunk c of 8 consecutive rows touch
// 8 distinct 16-byte bank groups.
//
// MFMA operand layout: lane l holds row (l & 15) of its 16-row A slice (and
// column (l & 15) of its B slice) and 32 bytes of K, chunks q and q + 4 of
// the block for q = l >> 4 (two 16-byte LDS reads); A and B take the same 32
// bytes, so the products pair up whatever order the matrix core sums them in.
// Chunks 2q and 2q + 1 per lane group, the other obvious choice, stall the LDS
// on bank conflicts for about a fifth of the kernel's cycles (rocprofv3
// SQ_LDS_BANK_CONFLICT), against about 1% with chunks q, q + 4, the pattern
// the MXFP4 product also reads (5-6% faster).  Each 16-byte chunk is 16
// consecutive K elements either way, so the matrix core still sums aligned
// groups of 8 consecutive K elements.  Result layout: lane l, register r is
// D[4 (l >> 4) + r][l & 15] of D = (first operand) x (second operand)^T, i.e.
// C[l & 15][4 (l >> 4) + r] for the transposed FP8 products.
#include <atomic>

#include "launch.h"
#include "quant.h"

namespace pqb {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kGT = 128;                     // K block, B tile rows, B scale block edge
constexpr int kGTM = 128;                    // A tile rows (128 or 256)
constexpr int kGWaves = 2 * kGTM / 64;       // waves kGTM / 64 x 2, each 64 x 64 of C
constexpr int kGThreads = 64 * kGWaves;
constexpr int kGTileA = kGTM * kGT, kGTileB = kGT * kGT;   // FP8 tile bytes for one K block
constexpr int kGScaleBytes = 4 * 2 * kGTM;   // activation scales of one block (each row twice)
constexpr int kGSlotBytes = kGTileA + kGTileB + kGScaleBytes;
constexpr int kGStages = 2;                  // ring slots
constexpr int kGBInstr = kGT / kGWaves / 8;  // B DMA instructions per wave per block
constexpr int kGLoadsPerBlock = 4 + kGBInstr + 1;   // DMA instructions per wave per block
constexpr int kGOutStride = 64 + 4;          // floats per row of a wave's staged 64 x 64 result
constexpr int kGOutBytes = kGWaves * 64 * kGOutStride * 4;
constexpr int kGLdsBytes =
    kGStages * kGSlotBytes > kGOutBytes ? kGStages * kGSlotBytes : kGOutBytes;

// Byte offset of 16-byte chunk c of row r in a staged 128 x 128-byte tile.
__device__ __forceinline__ int tile_off(int r, int c) { return r * kGT + ((c ^ (r & 7)) << 4); }

// The 32 bytes of K (chunks q and q + 4) of row r of a staged tile.
__device__ __forceinline__ v8i frag(const uint8_t* tile, int r, int q) {
  const uint4 lo = *reinterpret_cast<const uint4*>(tile + tile_off(r, q));
  const uint4 hi = *reinterpret_cast<const uint4*>(tile + tile_off(r, q + 4));
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p);
}

// Wave-wide DMA of 16 (4) bytes per lane from g to LDS address lds + 16 l (4 l).
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds)
               : "memory");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds)
               : "memory");
}

// The same from a wave-uniform base g plus an unsigned 32-bit offset per lane
// (the scalar-base address form: the base in SGPRs, one VGPR per lane).
__device__ __forceinline__ void dma16s(const void* g, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(g),
               "s"(lds)
               : "memory");
}
__device__ __forceinline__ void dma4s(const void* g, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(g),
               "s"(lds)
               : "memory");
}

// Wait until at most `blocks` blocks of this wave's DMA are still in flight.
template <int kN>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kN) : "memory");
}
__device__ __forceinline__ void wait_blocks(int blocks) {
  if (blocks <= 0)
    wait_vmcnt<0>();
  else if (blocks == 1)
    wait_vmcnt<kGLoadsPerBlock>();
  else
    wait_vmcnt<2 * kGLoadsPerBlock>();
}

__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// The tile (row tm, column tn) that this workgroup computes.  Workgroups i,
// i + 8, ... run on one XCD: each XCD takes a contiguous run of tiles, walked
// down bands of up to 8 tile rows, so neighbouring workgroups on an XCD share
// A rows and B columns in its L2.  The grid is tiles_m x tiles_n workgroups.
__device__ __forceinline__ void gemm_tile(int tiles_n, int& tm, int& tn) {
  const int nwg = gridDim.x, per = nwg / 8;
  const int t = per * 8 == nwg ? (blockIdx.x & 7) * per + (blockIdx.x >> 3) : blockIdx.x;
  const int band = t / (8 * tiles_n), rem = t - band * 8 * tiles_n;
  const int band_rows = min(8, nwg / tiles_n - band * 8);
  tm = band * 8 + rem % band_rows;
  tn = rem / band_rows;
}

// Output forms: float32, bf16, or FP8 E4M3 codes with one scale per 128
// columns of a row (the 1x128 activation layout), quantized in the epilogue.
enum GemmOut { kOutF32 = 0, kOutBf16 = 1, kOutFp8 = 2 };

// Epilogue helpers.  Each wave stages its 64 x 64 floats in LDS (rows padded
// to 68 floats); the float32 / bf16 forms then write whole row segments, 256
// bytes per row for float32, 128 for bf16, with 16-byte stores.
__device__ __forceinline__ void stage_tile(const v4f (&acc)[4][4], uint8_t* lds, int wave, int lane) {
  const int r16 = lane & 15, q = lane >> 4;
  float* out_lds = reinterpret_cast<float*>(lds) + wave * 64 * kGOutStride;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        out_lds[(mt * 16 + 4 * q + r) * kGOutStride + nt * 16 + r16] = acc[mt][nt][r];
}

// The same for a wave whose products were taken transposed (weight rows as
// the matrix core's first operand): acc[mt][nt][r] is row 16 mt + (lane & 15),
// column 16 nt + 4 (lane >> 4) + r, so each lane writes 4 consecutive floats.
__device__ __forceinline__ void stage_tile_t(const v4f (&acc)[4][4], uint8_t* lds, int wave, int lane) {
  const int r16 = lane & 15, q = lane >> 4;
  float* out_lds = reinterpret_cast<float*>(lds) + wave * 64 * kGOutStride;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      *reinterpret_cast<v4f*>(&out_lds[(mt * 16 + r16) * kGOutStride + nt * 16 + 4 * q]) = acc[mt][nt];
}

// Writes kRows rows, from row r0 on, of the 64 x 64 floats staged at position
// pos to C at (row0 + r0, col0), rows at or past M skipped.
template <int kOut, int kRows = 64>
__device__ __forceinline__ void store_staged(const uint8_t* lds, int pos, int lane, int row0,
                                             int col0, int M, int N, void* C, int r0 = 0) {
  static_assert(kRows % 8 == 0, "whole steps of 8 rows");
  const float* out_lds = reinterpret_cast<const float*>(lds) + (pos * 64 + r0) * kGOutStride;
  row0 += r0;
  if constexpr (kOut == kOutBf16) {
#pragma unroll
    for (int s = 0; s < kRows / 8; ++s) {  // 8 lanes per row, 8 rows per step
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
#pragma unroll
    for (int s = 0; s < kRows / 4; ++s) {  // 16 lanes per row, 4 rows per step
      const int rr = s * 4 + (lane >> 4), cc = (lane & 15) * 4;
      if (row0 + rr < M) {
        const v4f x = *reinterpret_cast<const v4f*>(out_lds + rr * kGOutStride + cc);
        float* dst = reinterpret_cast<float*>(C) + (int64_t)(row0 + rr) * N + col0 + cc;
        st_nt16(dst, as_u(x[0]), as_u(x[1]), as_u(x[2]), as_u(x[3]));
      }
    }
  }
}

template <int kOut, bool kTransposed = false>
__device__ __forceinline__ void stage_and_store(const v4f (&acc)[4][4], uint8_t* lds, int wave,
                                                int lane, int m0, int n0, int M, int N, void* C) {
  if constexpr (kTransposed)
    stage_tile_t(acc, lds, wave, lane);
  else
    stage_tile(acc, lds, wave, lane);
  __syncthreads();
  store_staged<kOut>(lds, wave, lane, m0 + (wave >> 1) * 64, n0 + (wave & 1) * 64, M, N, C);
}

// FP8 1x128 quantization of a staged 128 x 128 tile's rows, each exactly one
// 128-column block, two threads per row (t >> 1): thread t takes columns
// 32 i + 16 (t & 1) + j (i < 4, j < 16), so that each 16-byte code store of the
// pair covers 32 contiguous bytes of the row (with 64-column halves per
// thread, every store covered half of a 32-byte sector, and the fused form
// wrote 1.77x its output bytes).  The pair's maxima meet by DPP, then the scale
// and codes follow the 1x128 quantizer's arithmetic.  Column c of row r is
// staged by wave (r / 64, c / 64).
__device__ __forceinline__ void quantize_tile_rows(const uint8_t* lds, int tid, int m0, int n0,
                                                   int M, int N, uint8_t* C, float* c_scales) {
  static_assert(kGTM == 128 && kGThreads == 256, "two threads per row of a 128-row tile");
  const int rr = tid >> 1, half = tid & 1;
  const float* stage = reinterpret_cast<const float*>(lds) + (rr & 63) * kGOutStride;
  auto piece = [&](int i) {   // the 16 staged floats of columns 32 i + 16 half ..
    return stage + ((rr >> 6) * 2 + (i >> 1)) * 64 * kGOutStride + 32 * (i & 1) + 16 * half;
  };
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float* v = piece(i);
#pragma unroll
    for (int j = 0; j < 16; j += 4) {
      const v4f x = *reinterpret_cast<const v4f*>(v + j);
      am = max(am, max(max(as_u(fabsf(x[0])), as_u(fabsf(x[1]))),
                       max(as_u(fabsf(x[2])), as_u(fabsf(x[3])))));
    }
  }
  const float s = fp8_scale_bits<kE4M3>(group_umax<2>(am));
  const float y = recip_rn(s);
  if (m0 + rr < M) {
    uint8_t* dst = C + (int64_t)(m0 + rr) * N + n0 + 16 * half;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float* v = piece(i);
      float w[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) w[j] = v[j];
      const uint2 lo = fp8_pack8<kE4M3>(w, s, y), hi = fp8_pack8<kE4M3>(w + 8, s, y);
      st_nt16(dst + 32 * i, lo.x, lo.y, hi.x, hi.y);
    }
    if (half == 0) c_scales[(int64_t)(m0 + rr) * (N / kGT) + n0 / kGT] = s;
  }
}

// The same for 64 staged rows, with all 256 threads: four per row (t >> 2).
// Thread t takes columns 64 i + 16 (t & 3) + j (i < 2, j < 16), so each
// 16-byte code store of the four covers 64 contiguous bytes of the row; the
// row's columns 0 .. 63 and 64 .. 127 are staged at positions 0 and 1.
__device__ __forceinline__ void quantize_half_tile_rows(const uint8_t* lds, int tid, int row0,
                                                        int n0, int M, int N, uint8_t* C,
                                                        float* c_scales) {
  static_assert(kGThreads == 256, "four threads per row of 64 rows");
  const int rr = tid >> 2, part = tid & 3;
  const float* stage = reinterpret_cast<const float*>(lds) + rr * kGOutStride + 16 * part;
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float* v = stage + i * 64 * kGOutStride;
#pragma unroll
    for (int j = 0; j < 16; j += 4) {
      const v4f x = *reinterpret_cast<const v4f*>(v + j);
      am = max(am, max(max(as_u(fabsf(x[0])), as_u(fabsf(x[1]))),
                       max(as_u(fabsf(x[2])), as_u(fabsf(x[3])))));
    }
  }
  const float s = fp8_scale_bits<kE4M3>(group_umax<4>(am));
  const float y = recip_rn(s);
  if (row0 + rr < M) {
    uint8_t* dst = C + (int64_t)(row0 + rr) * N + n0 + 16 * part;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float* v = stage + i * 64 * kGOutStride;
      float w[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) w[j] = v[j];
      const uint2 lo = fp8_pack8<kE4M3>(w, s, y), hi = fp8_pack8<kE4M3>(w + 8, s, y);
      st_nt16(dst + 64 * i, lo.x, lo.y, hi.x, hi.y);
    }
    if (part == 0) c_scales[(int64_t)(row0 + rr) * (N / kGT) + n0 / kGT] = s;
  }
}

template <int kOut>
__global__ __launch_bounds__(kGThreads) void k_gemm_fp8_bs(const uint8_t* __restrict__ A,
                                                           const float* __restrict__ sA,
                                                           const uint8_t* __restrict__ B,
                                                           const float* __restrict__ sB, int M,
                                                           int N, int K, int tiles_n,
                                                           void* __restrict__ C,
                                                           float* __restrict__ c_scales) {
  // kGStages slots of [A tile | B tile | scales], reused for the epilogue
  static_assert(kGStages <= 3, "wait_blocks counts at most 2 later blocks");
  __shared__ __align__(16) uint8_t lds[kGLdsBytes];
  auto slot = [&](int s) { return lds + s * kGSlotBytes; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn;
  gemm_tile(tiles_n, tm, tn);
  const int m0 = tm * kGTM, n0 = tn * kGT;
  const int nkb = K / kGT;

  // DMA of block kb into slot s.  Wave w fills rows 32 w .. 32 w + 31 of both
  // tiles (4 instructions of 8 rows each) and the scales of those rows (lanes
  // 32 .. 63 repeat lanes 0 .. 31, at scale slots 64 w .. 64 w + 63).  Rows of
  // A at or past M read row M - 1 instead; their results are never stored.
  const int drow = lane >> 3, dpos = lane & 7;
  auto issue_block = [&](int kb, int s) {
    const uint32_t base = lds_addr(slot(s));
    const int64_t k0 = (int64_t)kb * kGT;
#pragma unroll
    for (int j = 0; j < 4; ++j) {                      // A rows 32 w + 8 j + (l >> 3)
      const int r = wave * 32 + j * 8 + drow;
      dma16(A + (int64_t)min(m0 + r, M - 1) * K + k0 + 16 * (dpos ^ (r & 7)),
            __builtin_amdgcn_readfirstlane(base + (wave * 32 + j * 8) * kGT));
    }
#pragma unroll
    for (int j = 0; j < kGBInstr; ++j) {               // B rows 8 (kGBInstr w + j) + (l >> 3)
      const int r = (wave * kGBInstr + j) * 8 + drow;
      dma16(B + (int64_t)(n0 + r) * K + k0 + 16 * (dpos ^ (r & 7)),
            __builtin_amdgcn_readfirstlane(base + kGTileA + (wave * kGBInstr + j) * 8 * kGT));
    }
    const int sr = min(m0 + wave * 32 + (lane & 31), M - 1);
    dma4(sA + (int64_t)sr * nkb + kb,
         __builtin_amdgcn_readfirstlane(base + kGTileA + kGTileB + wave * 256));
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int r16 = lane & 15, q = lane >> 4;
  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  for (int s = 0; s < kGStages - 1 && s < nkb; ++s) issue_block(s, s);
  const float* sB_col = sB + (int64_t)(n0 / kGT) * nkb;
  for (int kb = 0; kb < nkb; ++kb) {
    // this block's DMA done (for every wave after the barrier), and every wave
    // done reading the slot the next issue overwrites
    wait_blocks(min(kGStages - 2, nkb - 1 - kb));
    barrier();
    if (kb + kGStages - 1 < nkb) issue_block(kb + kGStages - 1, (kb + kGStages - 1) % kGStages);
    const uint8_t* sl = slot(kb % kGStages);
    const float* ls = reinterpret_cast<const float*>(sl + kGTileA + kGTileB);
    const float sb = sB_col[kb];
    v8i af[4];
    float sab[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int r = wm * 64 + mt * 16 + r16;         // this lane's activation row
      af[mt] = frag(sl, r, q);
      sab[mt] = ls[(r >> 5) * 64 + (r & 31)] * sb;
    }
    // The wave that has reached its matrix products is served first: the
    // other waves of the CU are then mostly waiting on LDS reads or DMA.
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const v8i bf = frag(sl + kGTileA, wn * 64 + nt * 16 + r16, q);
      v4f p[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        p[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            bf, af[mt], v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mt][nt][r] = __builtin_fmaf(p[mt][r], sab[mt], acc[mt][nt][r]);
    }
    __builtin_amdgcn_s_setprio(0);
  }
  barrier();  // every wave done with the ring before it becomes the output stage

  if constexpr (kOut == kOutFp8) {
    stage_tile_t(acc, lds, wave, lane);
    __syncthreads();
    quantize_tile_rows(lds, tid, m0, n0, M, N, reinterpret_cast<uint8_t*>(C), c_scales);
  } else {
    stage_and_store<kOut, true>(acc, lds, wave, lane, m0, n0, M, N, C);
  }
}

// ---------------------------------------------------------------------------
// The same product with three workgroups per CU.  One wave per SIMD cannot
// keep the matrix core fed through its own promotions (the FMAs wait on each
// product's result), so what hides that latency is other waves on the SIMD:
// three workgroups give three.  That takes at most 168 VGPRs and 53 KiB of
// LDS per workgroup: a single ring slot, each block's fragments and scales
// read into registers right after its DMA has landed, a second barrier
// freeing the slot for the next block's DMA before the products, the DMA
// addressed from a wave-uniform tile origin plus a 32-bit lane offset (A: at
// most 127 K + 127 bytes, so K < 2^25), and the epilogue staged 64 rows at a
// time.  Same tile, layout, order of operations and results as above.
// ---------------------------------------------------------------------------
constexpr int kG3OutBytes = 2 * 64 * kGOutStride * 4;      // two staged 64 x 64 blocks
constexpr int kG3LdsBytes = kGSlotBytes > kG3OutBytes ? kGSlotBytes : kG3OutBytes;
static_assert(3 * kG3LdsBytes <= 160 * 1024, "three workgroups fit the CU's LDS");

template <int kOut>
__global__ __launch_bounds__(kGThreads, 3) void k_gemm_fp8_bs3(const uint8_t* __restrict__ A,
                                                               const float* __restrict__ sA,
                                                               const uint8_t* __restrict__ B,
                                                               const float* __restrict__ sB, int M,
                                                               int N, int K, int tiles_n,
                                                               void* __restrict__ C,
                                                               float* __restrict__ c_scales) {
  __shared__ __align__(16) uint8_t lds[kG3LdsBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn;
  gemm_tile(tiles_n, tm, tn);
  const int m0 = tm * kGTM, n0 = tn * kGT;
  const int nkb = K / kGT;

  // DMA of block kb: the rows of k_gemm_fp8_bs's issue_block, addressed as
  // tile origin + lane offset
  const int drow = lane >> 3, dpos = lane & 7;
  uint32_t a_off[4], b_off[kGBInstr];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = wave * 32 + j * 8 + drow;
    a_off[j] = (uint32_t)(min(m0 + r, M - 1) - m0) * (uint32_t)K + 16u * (dpos ^ (r & 7));
  }
#pragma unroll
  for (int j = 0; j < kGBInstr; ++j) {
    const int r = (wave * kGBInstr + j) * 8 + drow;
    b_off[j] = (uint32_t)r * (uint32_t)K + 16u * (dpos ^ (r & 7));
  }
  const uint32_t s_off = 4u * (uint32_t)(min(m0 + wave * 32 + (lane & 31), M - 1) - m0) * (uint32_t)nkb;
  const uint32_t base = lds_addr(lds);
  auto issue_block = [&](int kb) {
    const int64_t k0 = (int64_t)kb * kGT;
    const uint8_t* a_blk = A + (int64_t)m0 * K + k0;
    const uint8_t* b_blk = B + (int64_t)n0 * K + k0;
    const float* s_blk = sA + (int64_t)m0 * nkb + kb;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dma16s(a_blk, a_off[j], __builtin_amdgcn_readfirstlane(base + (wave * 32 + j * 8) * kGT));
#pragma unroll
    for (int j = 0; j < kGBInstr; ++j)
      dma16s(b_blk, b_off[j],
             __builtin_amdgcn_readfirstlane(base + kGTileA + (wave * kGBInstr + j) * 8 * kGT));
    dma4s(s_blk, s_off, __builtin_amdgcn_readfirstlane(base + kGTileA + kGTileB + wave * 256));
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int r16 = lane & 15, q = lane >> 4;
  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  const float* sB_col = sB + (int64_t)(n0 / kGT) * nkb;
  const float* ls = reinterpret_cast<const float*>(lds + kGTileA + kGTileB);
  if (nkb > 0) issue_block(0);
  for (int kb = 0; kb < nkb; ++kb) {
    wait_vmcnt<0>();                       // this wave's DMA of block kb
    barrier();                             // ... and every wave's
    const float sb = sB_col[kb];
    v8i af[4], bf[4];
    float sab[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 64 + i * 16 + r16;          // this lane's activation row
      af[i] = frag(lds, r, q);
      bf[i] = frag(lds + kGTileA, wn * 64 + i * 16 + r16, q);
      sab[i] = ls[(r >> 5) * 64 + (r & 31)] * sb;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    barrier();                             // every wave done reading the slot
    if (kb + 1 < nkb) issue_block(kb + 1);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      v4f p[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        p[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            bf[nt], af[mt], v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mt][nt][r] = __builtin_fmaf(p[mt][r], sab[mt], acc[mt][nt][r]);
    }
    __builtin_amdgcn_s_setprio(0);
  }
  barrier();  // every wave done with the slot before it becomes the output stage

  // Rows 64 pass .. 64 pass + 63 of the tile: waves (pass, 0) and (pass, 1)
  // stage their blocks at positions 0 and 1, then all four waves store them
  // (32 rows of one position each) or quantize them (four threads per row).
  for (int pass = 0; pass < 2; ++pass) {
    if (pass) __syncthreads();
    if (wm == pass) stage_tile_t(acc, lds, wn, lane);
    __syncthreads();
    if constexpr (kOut == kOutFp8) {
      quantize_half_tile_rows(lds, tid, m0 + 64 * pass, n0, M, N, reinterpret_cast<uint8_t*>(C),
                              c_scales);
    } else {                               // wave w: rows 32 (w >> 1) .. of position w & 1
      store_staged<kOut, 32>(lds, wave & 1, lane, m0 + 64 * pass, n0 + 64 * (wave & 1), M, N, C,
                             32 * (wave >> 1));
    }
  }
}

// ---------------------------------------------------------------------------
// MXFP4 x MXFP4 product C = dequant(A) dequant(B)^T on the block-scaled matrix
// cores: v_mfma_scale_f32_16x16x128_f8f6f4 with E2M1 operands takes each
// lane's 32 nibbles (16 bytes, one 32-element MX block: row l & 15, block
// l >> 4 of the 128-deep K step) and that lane's E8M0 scale byte, exactly the
// MXFP4 layout (codes [rows, K/2], scales [rows, K/32]).  The scales are
// powers of two applied by the matrix core, so the MFMAs accumulate straight
// into C, with no promotion step.  Same workgroup shape, DMA ring, swizzle and
// epilogue as the FP8 GEMM; one ring slot holds a 256-deep K stage: 128 rows x
// 128 bytes of codes for A and for B (the FP8 tile layout) and 8 scale bytes
// per row of each.
// ---------------------------------------------------------------------------
constexpr int kMxKS = 256;                                 // K elements per stage
constexpr int kMxScaleBytes = kGT * 8;                     // 8 E8M0 bytes per row and stage
constexpr int kMxSlotBytes = 2 * kGTileB + 2 * kMxScaleBytes;
static_assert(kGTM == 128 && kGThreads == 256, "the MX GEMM uses the 128 x 128 tile");
static_assert(kGStages * kMxSlotBytes <= kGLdsBytes, "ring fits the FP8 GEMM's LDS");

template <int kOut>
__global__ __launch_bounds__(kGThreads) void k_gemm_mxfp4(const uint8_t* __restrict__ A,
                                                          const uint8_t* __restrict__ sA,
                                                          const uint8_t* __restrict__ B,
                                                          const uint8_t* __restrict__ sB, int M,
                                                          int N, int K, int tiles_n,
                                                          void* __restrict__ C) {
  static_assert(kGStages == 2, "one stage in flight at each wait");
  __shared__ __align__(16) uint8_t lds[kGLdsBytes];
  auto slot = [&](int s) { return lds + s * kMxSlotBytes; };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn;
  gemm_tile(tiles_n, tm, tn);
  const int m0 = tm * kGT, n0 = tn * kGT;
  const int kb128 = K / 128, stages = (K + kMxKS - 1) / kMxKS;
  const int rowb = K / 2, srow = K / 32;                   // code and scale bytes per row

  // DMA of stage st into slot s.  Wave w fills code rows 32 w .. 32 w + 31 of
  // A and B (4 instructions of 8 rows each), and 64 scale rows (2 dwords per
  // row): waves 0, 1 those of A, waves 2, 3 those of B.  A second half past K
  // (K / 128 odd, last stage) reads the first half again and is never used.
  const int drow = lane >> 3, dpos = lane & 7;
  auto issue_stage = [&](int st, int s) {
    const uint32_t base = lds_addr(slot(s));
    const int64_t k0 = (int64_t)st * (kMxKS / 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wave * 32 + j * 8 + drow;
      int c = dpos ^ (r & 7);
      if (k0 + 16 * c >= rowb) c -= 4;
      const uint32_t dst = __builtin_amdgcn_readfirstlane(base + (wave * 32 + j * 8) * kGT);
      dma16(A + (int64_t)min(m0 + r, M - 1) * rowb + k0 + 16 * c, dst);
      dma16(B + (int64_t)(n0 + r) * rowb + k0 + 16 * c, dst + kGTileB);
    }
    // scale rows r = 64 (w & 1) + 32 i + (l >> 1), i < 2, dword (l & 1): LDS
    // dword 2 r + (l & 1), i.e. byte 512 (w & 1) + 256 i + 4 l
    const int half = lane & 1;
    const int hh = 8 * st + 4 * half < srow ? half : 0;
    const uint32_t sdst = base + 2 * kGTileB + (wave < 2 ? 0 : kMxScaleBytes) + (wave & 1) * 512;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int sr = (wave & 1) * 64 + 32 * i + (lane >> 1);
      const uint8_t* src = wave < 2 ? sA + (int64_t)min(m0 + sr, M - 1) * srow
                                    : sB + (int64_t)(n0 + sr) * srow;
      dma4(src + 8 * st + 4 * hh, __builtin_amdgcn_readfirstlane(sdst + 256 * i));
    }
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int r16 = lane & 15, q = lane >> 4;
  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  if (stages > 0) issue_stage(0, 0);
  for (int st = 0; st < stages; ++st) {
    // the only DMA in flight is this stage's (the next is issued after the
    // barrier), so wait for all of it
    wait_vmcnt<0>();
    barrier();
    if (st + 1 < stages) issue_stage(st + 1, (st + 1) & 1);
    const uint8_t* sl = slot(st & 1);
    const uint32_t* ls = reinterpret_cast<const uint32_t*>(sl + 2 * kGTileB);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (2 * st + h >= kb128) break;
      v8i af[4];
      int sa[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int r = wm * 64 + mt * 16 + r16;
        const uint4 v = *reinterpret_cast<const uint4*>(sl + tile_off(r, 4 * h + q));
        af[mt] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        // scale dword of row r: rows 32 w' + i of wave w' at dword 64 w' + 2 i + half
        sa[mt] = (ls[(r >> 5) * 64 + 2 * (r & 31) + h] >> (8 * q)) & 0xFF;
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int r = wn * 64 + nt * 16 + r16;
        const uint4 v = *reinterpret_cast<const uint4*>(sl + kGTileB + tile_off(r, 4 * h + q));
        const v8i bf = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        const int sb = (ls[kMxScaleBytes / 4 + (r >> 5) * 64 + 2 * (r & 31) + h] >> (8 * q)) & 0xFF;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[mt], bf, acc[mt][nt], 4,
                                                                         4, 0, sa[mt], 0, sb);
      }
    }
  }
  barrier();
  stage_and_store<kOut>(acc, lds, wave, lane, m0, n0, M, N, C);
}

// ---------------------------------------------------------------------------
// NVFP4 x NVFP4 product C = g * sum_k A'[m, k] B'[n, k] with A' = V(a) dec(sa)
// over 16-element blocks and g = float32(gsA gsB).  The matrix core's own
// scales are E8M0 per 32 elements, so they cannot carry NVFP4's E4M3 scales per
// 16; instead each wave widens its fragments to f16 between LDS and the matrix
// core.  v_cvt_scalef32_pk_f16_fp4 turns two nibbles into two halves times 2^8
// (the instruction takes only the exponent of its scale operand), and one
// packed f16 multiply by the half whose bits are the scale byte shifted left by
// 7 (the E4M3 value times 2^-8; E4M3's subnormals land on f16 subnormals) gives
// V dec(s) exactly: at most 6 significant bits, between 2^-10 and 2688.
// v_mfma_f32_16x16x32_f16 then forms exact products and accumulates them in
// float32, and g multiplies each result once.  Workgroup shape, DMA ring and
// swizzle are the MXFP4 product's: a stage is 256 deep in K (128 code bytes per
// row); its scales are 16 bytes per row.  Lane l of a fragment holds row l & 15
// and the 32 elements of 16-byte chunk q = l >> 4 of the 128-deep half (blocks
// 2q and 2q + 1); its dword t holds the 8 elements of K step t, and A and B
// take the same elements, so the products pair up.
// ---------------------------------------------------------------------------
constexpr int kNvScaleBytes = kGT * 16;                    // 16 E4M3 bytes per row and stage
constexpr int kNvSlotBytes = 2 * kGTileB + 2 * kNvScaleBytes;
constexpr int kNvLdsBytes = 2 * kNvSlotBytes > kGOutBytes ? 2 * kNvSlotBytes : kGOutBytes;

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

// dec(s) * 2^-8 in both halves, for a scale byte s (sign bit cleared).
__device__ __forceinline__ h2 nv_scale(uint32_t s) {
  return __builtin_bit_cast(h2, s * 0x00800080u);
}

// The 8 nibbles of w (low nibble first) as V * dec(s) in halves.
__device__ __forceinline__ h8 nv_widen8(uint32_t w, h2 s) {
  const h2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0) * s;
  const h2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1) * s;
  const h2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2) * s;
  const h2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3) * s;
  return h8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Fragment of row r in half h of a staged stage: the lane's 16 code bytes
// (chunk 4 h + q) and its two block scales (bytes 8 h + 2 q, + 1 of the row).
__device__ __forceinline__ void nv_frag(const uint8_t* tile, const uint32_t* scales, int r, int h,
                                        int q, h8 (&f)[4]) {
  const uint4 v = *reinterpret_cast<const uint4*>(tile + tile_off(r, 4 * h + q));
  const uint32_t sw = scales[4 * r + 2 * h + (q >> 1)] >> (16 * (q & 1));
  const h2 s0 = nv_scale(sw & 0x7Fu), s1 = nv_scale((sw >> 8) & 0x7Fu);
  f[0] = nv_widen8(v.x, s0);
  f[1] = nv_widen8(v.y, s0);
  f[2] = nv_widen8(v.z, s1);
  f[3] = nv_widen8(v.w, s1);
}

template <int kOut>
__global__ __launch_bounds__(kGThreads) void k_gemm_nvfp4(const uint8_t* __restrict__ A,
                                                          const uint8_t* __restrict__ sA,
                                                          const float* __restrict__ gA,
                                                          const uint8_t* __restrict__ B,
                                                          const uint8_t* __restrict__ sB,
                                                          const float* __restrict__ gB, int M,
                                                          int N, int K, int tiles_n,
                                                          void* __restrict__ C) {
  static_assert(kGTM == 128 && kGThreads == 256, "the NVFP4 GEMM uses the 128 x 128 tile");
  __shared__ __align__(16) uint8_t lds[kNvLdsBytes];
  auto slot = [&](int s) { return lds + s * kNvSlotBytes; };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn;
  gemm_tile(tiles_n, tm, tn);
  const int m0 = tm * kGT, n0 = tn * kGT;
  const int kb128 = K / 128, stages = (K + kMxKS - 1) / kMxKS;
  const int rowb = K / 2, srow = K / 16;                   // code and scale bytes per row

  // DMA of stage st into slot s: code rows as in the MXFP4 product; scale
  // rows r = 64 (w & 1) + 16 i + (l >> 2), dword l & 3 (LDS byte 16 r + 4 (l & 3)),
  // waves 0, 1 those of A, waves 2, 3 those of B.  A second half past K
  // (K / 128 odd, last stage) reads the first half again and is never used.
  const int drow = lane >> 3, dpos = lane & 7;
  auto issue_stage = [&](int st, int s) {
    const uint32_t base = lds_addr(slot(s));
    const int64_t k0 = (int64_t)st * (kMxKS / 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wave * 32 + j * 8 + drow;
      int c = dpos ^ (r & 7);
      if (k0 + 16 * c >= rowb) c -= 4;
      const uint32_t dst = __builtin_amdgcn_readfirstlane(base + (wave * 32 + j * 8) * kGT);
      dma16(A + (int64_t)min(m0 + r, M - 1) * rowb + k0 + 16 * c, dst);
      dma16(B + (int64_t)(n0 + r) * rowb + k0 + 16 * c, dst + kGTileB);
    }
    const int dw = 16 * st + 4 * (lane & 3) < srow ? (lane & 3) : (lane & 1);
    const uint32_t sdst = base + 2 * kGTileB + (wave < 2 ? 0 : kNvScaleBytes) + (wave & 1) * 64 * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sr = (wave & 1) * 64 + 16 * i + (lane >> 2);
      const uint8_t* src = wave < 2 ? sA + (int64_t)min(m0 + sr, M - 1) * srow
                                    : sB + (int64_t)(n0 + sr) * srow;
      dma4(src + 16 * st + 4 * dw, __builtin_amdgcn_readfirstlane(sdst + 256 * i));
    }
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int r16 = lane & 15, q = lane >> 4;
  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  if (stages > 0) issue_stage(0, 0);
  for (int st = 0; st < stages; ++st) {
    // the only DMA in flight is this stage's (the next is issued after the
    // barrier), so wait for all of it
    wait_vmcnt<0>();
    barrier();
    if (st + 1 < stages) issue_stage(st + 1, (st + 1) & 1);
    const uint8_t* sl = slot(st & 1);
    const uint32_t* lsa = reinterpret_cast<const uint32_t*>(sl + 2 * kGTileB);
    const uint32_t* lsb = lsa + kNvScaleBytes / 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (2 * st + h >= kb128) break;
      h8 af[4][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) nv_frag(sl, lsa, wm * 64 + mt * 16 + r16, h, q, af[mt]);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        h8 bf[4];
        nv_frag(sl + kGTileB, lsb, wn * 64 + nt * 16 + r16, h, q, bf);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mt][ks], bf[ks], acc[mt][nt], 0, 0, 0);
      }
    }
  }
  barrier();
  const float g = K > 0 ? gA[0] * gB[0] : 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = acc[i][j] * g;
  stage_and_store<kOut>(acc, lds, wave, lane, m0, n0, M, N, C);
}

}  // namespace

// Compute units of the current device, read once per device (concurrent
// first calls store the same value).
static int gemm_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int v = 0;
    n = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0
            ? v
            : 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

hipError_t launch_gemm_fp8_bs(const uint8_t* a, const float* a_scales, const uint8_t* b,
                              const float* b_scales, int64_t M, int64_t N, int64_t K, int out,
                              void* c, float* c_scales, hipStream_t st) {
  const int tiles_m = (int)((M + kGTM - 1) / kGTM), tiles_n = (int)(N / kGT);
  const dim3 grid((unsigned)tiles_m * (unsigned)tiles_n);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kGThreads), 0, st, a, a_scales, b, b_scales, (int)M,
                       (int)N, (int)K, tiles_n, c, c_scales);
  };
  // Three workgroups per CU give each CU about 1.2x the throughput of two
  // (measured on 8192 x 7168 x 2048), but in rounds of three: with n tiles
  // per CU that is ceil(n / 3) rounds of 1.2 against ceil(n / 2) of 1.
  const int64_t n = ((int64_t)tiles_m * tiles_n + gemm_cus() - 1) / gemm_cus();
  const bool three = K < (1 << 25) && 6 * ((n + 2) / 3) < 5 * ((n + 1) / 2);
  if (three) {
    if (out == kOutBf16)
      go(k_gemm_fp8_bs3<kOutBf16>);
    else if (out == kOutFp8)
      go(k_gemm_fp8_bs3<kOutFp8>);
    else
      go(k_gemm_fp8_bs3<kOutF32>);
  } else if (out == kOutBf16) {
    go(k_gemm_fp8_bs<kOutBf16>);
  } else if (out == kOutFp8) {
    go(k_gemm_fp8_bs<kOutFp8>);
  } else {
    go(k_gemm_fp8_bs<kOutF32>);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_mxfp4(const uint8_t* a, const uint8_t* a_scales, const uint8_t* b,
                             const uint8_t* b_scales, int64_t M, int64_t N, int64_t K,
                             bool out_bf16, void* c, hipStream_t st) {
  const int tiles_m = (int)((M + kGT - 1) / kGT), tiles_n = (int)(N / kGT);
  const dim3 grid((unsigned)tiles_m * (unsigned)tiles_n);
  if (out_bf16)
    hipLaunchKernelGGL(k_gemm_mxfp4<kOutBf16>, grid, dim3(kGThreads), 0, st, a, a_scales, b, b_scales,
                       (int)M, (int)N, (int)K, tiles_n, c);
  else
    hipLaunchKernelGGL(k_gemm_mxfp4<kOutF32>, grid, dim3(kGThreads), 0, st, a, a_scales, b, b_scales,
                       (int)M, (int)N, (int)K, tiles_n, c);
  return hipGetLastError();
}

hipError_t launch_gemm_nvfp4(const uint8_t* a, const uint8_t* a_scales, const float* a_gs,
                             const uint8_t* b, const uint8_t* b_scales, const float* b_gs, int64_t M,
                             int64_t N, int64_t K, bool out_bf16, void* c, hipStream_t st) {
  const int tiles_m = (int)((M + kGT - 1) / kGT), tiles_n = (int)(N / kGT);
  const dim3 grid((unsigned)tiles_m * (unsigned)tiles_n);
  if (out_bf16)
    hipLaunchKernelGGL(k_gemm_nvfp4<kOutBf16>, grid, dim3(kGThreads), 0, st, a, a_scales, a_gs, b,
                       b_scales, b_gs, (int)M, (int)N, (int)K, tiles_n, c);
  else
    hipLaunchKernelGGL(k_gemm_nvfp4<kOutF32>, grid, dim3(kGThreads), 0, st, a, a_scales, a_gs, b,
                       b_scales, b_gs, (int)M, (int)N, (int)K, tiles_n, c);
  return hipGetLastError();
}

}  // namespace pqb
