// Fused quantization of several tensors in one launch (pqb_quantize_batch).
//
// Every job gets a contiguous range of workgroups; a workgroup finds its job
// by scanning the prefix table in the kernel arguments (uniform, scalar) and
// runs that job's body from quant.h with its local workgroup index.  One
// dispatch then covers, e.g., a weight's 128x128 tiles and an activation's
// 1x128 blocks, or a whole decoder's INT4 weights.  (Per-row FP8 jobs keep a
// whole row in registers; they get launches of their own so that this kernel's
// register budget, and with it the occupancy of the streaming kinds, stays low.)
#include "launch.h"
#include "quant.h"

namespace pqb {
namespace {

enum : int32_t { kJobFp8Blk = 0, kJobFp8Tile = 1, kJobMx = 2, kJobInt4 = 3 };

constexpr int kMultiWaves = 8;  // 512-thread workgroups (a 128x128 tile: 4 rows per lane)
constexpr int kMultiThreads = kMultiWaves * kWave;
constexpr int kUnrFlat = 4;     // tiles per wave per chunk (flat kinds)
constexpr int kMxIters = 4;     // MXFP4 chunks per wave, to amortize the table fill

struct Job {
  const void* x;
  uint8_t* codes;
  void* scales;
  uint8_t* aux;
  int64_t rows;    // tiles: rows of one slice
  int64_t cols;
  int64_t nunits;  // flat kinds
  int32_t kind;
  int32_t bf16;
  int32_t br;      // tiles: min(128, rows)
  int32_t iters;   // flat kinds: chunks per wave
};

struct MultiArgs {
  int32_t njobs;
  int32_t pad;
  int64_t wg_begin[kMaxBatchJobs + 1];
  Job job[kMaxBatchJobs];
};

template <typename T, int kIters, typename Body>
__device__ __forceinline__ void flat_job(int64_t local, int64_t nunits, Body body) {
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
#pragma unroll 1
  for (int it = 0; it < kIters; ++it) {
    const int64_t chunk = (local * kIters + it) * kMultiWaves + wave;
    const int64_t u0 = chunk * kUnrFlat * kWave;
    if (u0 >= nunits) break;
    if (u0 + kUnrFlat * kWave <= nunits)
      body(u0, std::integral_constant<bool, false>{});
    else
      body(u0, std::integral_constant<bool, true>{});
  }
}

template <typename T>
__device__ __forceinline__ void run_job(const Job& jb, int64_t local, uint8_t* lut, uint32_t* red) {
  const T* x = reinterpret_cast<const T*>(jb.x);
  switch (jb.kind) {
    case kJobFp8Blk:
      flat_job<T, 1>(local, jb.nunits, [&](int64_t u0, auto g) {
        fp8_1x128_chunk<T, kUnrFlat, decltype(g)::value>(x, u0, jb.nunits, jb.codes,
                                                          reinterpret_cast<float*>(jb.scales));
      });
      break;
    case kJobFp8Tile:
      fp8_tile_128x128<T, kMultiWaves>(x, jb.rows, jb.cols, jb.br, local, jb.codes,
                                       reinterpret_cast<float*>(jb.scales), red);
      break;
    case kJobMx:
      e2m1_lut_fill(lut, 0);
      __syncthreads();
      flat_job<T, kMxIters>(local, jb.nunits, [&](int64_t u0, auto g) {
        mx_chunk<T, kUnrFlat, decltype(g)::value>(x, u0, jb.nunits, jb.codes,
                                                   reinterpret_cast<uint8_t*>(jb.scales), lut);
      });
      break;
    case kJobInt4:
      flat_job<T, 1>(local, jb.nunits, [&](int64_t u0, auto g) {
        int4_chunk<T, kUnrFlat, decltype(g)::value>(x, u0, jb.nunits, jb.codes,
                                                     reinterpret_cast<uint16_t*>(jb.scales),
                                                     jb.aux);
      });
      break;
  }
}

__global__ __launch_bounds__(kMultiThreads) void k_multi(MultiArgs a) {
  __shared__ __align__(16) uint8_t lut[kE2M1LutSize];
  __shared__ uint32_t red[kMultiWaves];
  const int64_t wg = blockIdx.x;
  int j = 0;
  while (j + 1 < a.njobs && wg >= a.wg_begin[j + 1]) ++j;
  const Job& jb = a.job[j];
  const int64_t local = wg - a.wg_begin[j];
  if (jb.bf16)
    run_job<uint16_t>(jb, local, lut, red);
  else
    run_job<float>(jb, local, lut, red);
}

}  // namespace

hipError_t launch_multi(const MultiJob* jobs, int njobs, hipStream_t st) {
  for (int base = 0; base < njobs; base += kMaxBatchJobs) {
    const int n = njobs - base < kMaxBatchJobs ? njobs - base : kMaxBatchJobs;
    MultiArgs a{};
    a.njobs = n;
    int64_t wg = 0;
    for (int i = 0; i < n; ++i) {
      const MultiJob& m = jobs[base + i];
      Job& jb = a.job[i];
      jb.x = m.x;
      jb.codes = m.codes;
      jb.scales = m.scales;
      jb.aux = m.aux;
      jb.bf16 = m.bf16;
      jb.cols = m.cols;
      const int64_t n_el = m.batch * m.rows * m.cols;
      const int64_t nunits = n_el / 8;
      const int64_t nchunks = (nunits + kUnrFlat * kWave - 1) / (kUnrFlat * kWave);
      const int64_t waves = kMultiWaves;
      int64_t wgs = 0;
      switch (m.kind) {
        case kMultiFp8Blk:
          jb.kind = kJobFp8Blk;
          jb.nunits = nunits;
          wgs = (nchunks + waves - 1) / waves;
          break;
        case kMultiFp8Tile: {
          jb.kind = kJobFp8Tile;
          jb.rows = m.rows;
          jb.br = (int32_t)(m.rows < 128 ? m.rows : 128);
          wgs = m.batch * (m.rows / jb.br) * (m.cols / 128);
          break;
        }
        case kMultiMx:
          jb.kind = kJobMx;
          jb.nunits = nunits;
          wgs = (nchunks + waves * kMxIters - 1) / (waves * kMxIters);
          break;
        case kMultiInt4:
          jb.kind = kJobInt4;
          jb.nunits = nunits;
          wgs = (nchunks + waves - 1) / waves;
          break;
      }
      a.wg_begin[i] = wg;
      wg += wgs;
    }
    a.wg_begin[n] = wg;
    if (wg > 0) hipLaunchKernelGGL(k_multi, dim3((unsigned)wg), dim3(kMultiThreads), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pqb
