// Fused quantization of several tensors per launch (pqb_quantize_batch).
//
// Jobs are grouped by family, one kernel per family: FP8 E4M3 / E5M2 (1x128
// blocks and 128x128 tiles together, 512-thread workgroups because a tile is
// 8 waves), MXFP4 with MXFP8, and INT4 (256-thread workgroups, longer chunks
// per wave).  Within a
// launch every job gets a contiguous range of workgroups; a workgroup finds its
// job by scanning the prefix table in the kernel arguments (uniform, scalar)
// and runs that job's body from quant.h with its local workgroup index.  One
// dispatch then covers, e.g., a weight's 128x128 tiles and an activation's
// 1x128 blocks, or a whole decoder's INT4 weights.  Each family kernel only
// holds the registers of its own bodies.  (Per-row FP8 jobs keep a whole row in
// registers; they get launches of their own.)
#include <vector>

#include "launch.h"
#include "quant.h"

namespace pqb {
namespace {

enum : int32_t { kJobFp8Blk = 0, kJobFp8Tile = 1, kJobMx = 2, kJobInt4 = 3, kJobMx8 = 4 };
enum Family : int { kFamFp8 = 0, kFamMx = 1, kFamInt4 = 2 };

constexpr int kFp8Waves = 8;  // 512 threads: a 128x128 tile holds 4 rows per lane
constexpr int kFp8Unr = 2;    // tiles per wave per 1x128 chunk (W8A8 step: 4 -> 2 took
                               // 36.8 -> 35.8 us; the last round of workgroups is shorter)
constexpr int kFp4Waves = 4;  // MXFP4 / INT4: 256 threads
// MXFP4 / INT4 chunk: 8 tiles of bf16 or 4 of float32 (8 KiB per wave either way)
template <typename T>
constexpr int kFp4Unr = sizeof(T) == 2 ? 8 : 4;

template <int kFam>
constexpr int kThreads = (kFam == kFamFp8 ? kFp8Waves : kFp4Waves) * kWave;

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
  int32_t elem;    // FP8 kinds: kE4M3 or kE5M2
};

struct MultiArgs {
  int32_t njobs;
  int32_t pad;
  int64_t wg_begin[kMaxBatchJobs + 1];
  Job job[kMaxBatchJobs];
};

// One chunk of kUnr tiles per wave: chunk = local * kWaves + wave.
template <int kWaves, int kUnr, typename Body>
__device__ __forceinline__ void flat_job(int64_t local, int64_t nunits, Body body) {
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int64_t u0 = (local * kWaves + wave) * kUnr * kWave;
  if (u0 >= nunits) return;
  if (u0 + kUnr * kWave <= nunits)
    body(u0, std::integral_constant<bool, false>{});
  else
    body(u0, std::integral_constant<bool, true>{});
}

template <typename T, int kElem>
__device__ __forceinline__ void fp8_job(const Job& jb, const T* x, int64_t local, uint32_t* red) {
  if (jb.kind == kJobFp8Blk) {
    flat_job<kFp8Waves, kFp8Unr>(local, jb.nunits, [&](int64_t u0, auto g) {
      fp8_1x128_chunk<T, kFp8Unr, decltype(g)::value, kElem>(x, u0, jb.nunits, jb.codes,
                                                              reinterpret_cast<float*>(jb.scales));
    });
  } else {
    fp8_tile_128x128<T, kFp8Waves, kElem>(x, jb.rows, jb.cols, jb.br, local, jb.codes,
                                          reinterpret_cast<float*>(jb.scales), red);
  }
}

template <int kFam, typename T>
__device__ __forceinline__ void run_job(const Job& jb, int64_t local, uint8_t* lut, uint32_t* red) {
  const T* x = reinterpret_cast<const T*>(jb.x);
  if constexpr (kFam == kFamFp8) {
    if (jb.elem == kE5M2)
      fp8_job<T, kE5M2>(jb, x, local, red);
    else
      fp8_job<T, kE4M3>(jb, x, local, red);
  } else if constexpr (kFam == kFamMx) {
    if (jb.kind == kJobMx8) {
      flat_job<kFp4Waves, kFp4Unr<T>>(local, jb.nunits, [&](int64_t u0, auto g) {
        mx8_chunk<T, kFp4Unr<T>, decltype(g)::value>(x, u0, jb.nunits, jb.codes,
                                                      reinterpret_cast<uint8_t*>(jb.scales));
      });
    } else {
      flat_job<kFp4Waves, kFp4Unr<T>>(local, jb.nunits, [&](int64_t u0, auto g) {
        mx_chunk<T, kFp4Unr<T>, decltype(g)::value>(x, u0, jb.nunits, jb.codes,
                                                     reinterpret_cast<uint8_t*>(jb.scales), lut);
      });
    }
  } else {
    flat_job<kFp4Waves, kFp4Unr<T>>(local, jb.nunits, [&](int64_t u0, auto g) {
      int4_chunk<T, kFp4Unr<T>, decltype(g)::value>(x, u0, jb.nunits, jb.codes,
                                                     reinterpret_cast<uint16_t*>(jb.scales),
                                                     jb.aux);
    });
  }
}

template <int kFam>
__global__ __launch_bounds__(kThreads<kFam>) void k_multi(MultiArgs a) {
  __shared__ __align__(16) uint8_t lut[kFam == kFamMx ? kE2M1LutSize : 16];
  __shared__ uint32_t red[kFp8Waves];
  if constexpr (kFam == kFamMx) {
    e2m1_lut_fill(lut, 0);
    __syncthreads();
  }
  const int64_t wg = blockIdx.x;
  int j = 0;
  while (j + 1 < a.njobs && wg >= a.wg_begin[j + 1]) ++j;
  const Job& jb = a.job[j];
  const int64_t local = wg - a.wg_begin[j];
  if (jb.bf16)
    run_job<kFam, uint16_t>(jb, local, lut, red);
  else
    run_job<kFam, float>(jb, local, lut, red);
}

int family_of(int kind) {
  return (kind == kMultiMx || kind == kMultiMx8) ? kFamMx : kind == kMultiInt4 ? kFamInt4 : kFamFp8;
}

// Workgroups one job needs in its family's kernel; fills the kernel-side job.
int64_t describe(const MultiJob& m, Job& jb) {
  jb = Job{};
  jb.x = m.x;
  jb.codes = m.codes;
  jb.scales = m.scales;
  jb.aux = m.aux;
  jb.bf16 = m.bf16;
  jb.elem = m.elem;
  jb.cols = m.cols;
  jb.nunits = m.batch * m.rows * m.cols / 8;
  auto flat_wgs = [&](int waves, int unr) {
    const int64_t nchunks = (jb.nunits + (int64_t)unr * kWave - 1) / ((int64_t)unr * kWave);
    return (nchunks + waves - 1) / waves;
  };
  const int fp4_unr = m.bf16 ? kFp4Unr<uint16_t> : kFp4Unr<float>;
  switch (m.kind) {
    case kMultiFp8Blk:
      jb.kind = kJobFp8Blk;
      return flat_wgs(kFp8Waves, kFp8Unr);
    case kMultiFp8Tile:
      jb.kind = kJobFp8Tile;
      jb.rows = m.rows;
      jb.br = (int32_t)(m.rows < 128 ? m.rows : 128);
      return m.batch * (m.rows / jb.br) * (m.cols / 128);
    case kMultiMx:
      jb.kind = kJobMx;
      return flat_wgs(kFp4Waves, fp4_unr);
    case kMultiMx8:
      jb.kind = kJobMx8;
      return flat_wgs(kFp4Waves, fp4_unr);
    default:
      jb.kind = kJobInt4;
      return flat_wgs(kFp4Waves, fp4_unr);
  }
}

template <int kFam>
hipError_t launch_family(const std::vector<const MultiJob*>& jobs, hipStream_t st) {
  for (size_t base = 0; base < jobs.size(); base += kMaxBatchJobs) {
    const int n = (int)(jobs.size() - base < (size_t)kMaxBatchJobs ? jobs.size() - base
                                                                    : (size_t)kMaxBatchJobs);
    MultiArgs a{};
    a.njobs = n;
    // whole-tile jobs (the heaviest workgroups) first, so that they are not
    // the last to be dispatched
    Job tmp[kMaxBatchJobs];
    int64_t cnt[kMaxBatchJobs];
    for (int i = 0; i < n; ++i) cnt[i] = describe(*jobs[base + i], tmp[i]);
    int order[kMaxBatchJobs], k = 0;
    for (int i = 0; i < n; ++i) if (tmp[i].kind == kJobFp8Tile) order[k++] = i;
    for (int i = 0; i < n; ++i) if (tmp[i].kind != kJobFp8Tile) order[k++] = i;
    int64_t wg = 0;
    for (int i = 0; i < n; ++i) {
      a.wg_begin[i] = wg;
      a.job[i] = tmp[order[i]];
      wg += cnt[order[i]];
    }
    a.wg_begin[n] = wg;
    if (wg > 0)
      hipLaunchKernelGGL(k_multi<kFam>, dim3((unsigned)wg), dim3(kThreads<kFam>), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_multi(const MultiJob* jobs, int njobs, hipStream_t st) {
  std::vector<const MultiJob*> fam[3];
  for (int i = 0; i < njobs; ++i) fam[family_of(jobs[i].kind)].push_back(&jobs[i]);
  hipError_t e = hipSuccess;
  if (!fam[kFamFp8].empty()) e = launch_family<kFamFp8>(fam[kFamFp8], st);
  if (e == hipSuccess && !fam[kFamMx].empty()) e = launch_family<kFamMx>(fam[kFamMx], st);
  if (e == hipSuccess && !fam[kFamInt4].empty()) e = launch_family<kFamInt4>(fam[kFamInt4], st);
  return e;
}

}  // namespace pqb
