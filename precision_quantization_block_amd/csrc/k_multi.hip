// Fused quantization of several tensors per launch (pqb_quantize_batch).
//
// Jobs are grouped by family, one kernel per family: FP8 E4M3 / E5M2 (1x128
// blocks and 128x128 tiles together, 512-thread workgroups because a tile is
// 8 waves), MXFP4 with MXFP8 (256-thread workgroups), and INT4 (512-thread
// workgroups).  Within a
// launch every job gets a contiguous range of workgroups; a workgroup finds its
// job by a binary search of the prefix table in the kernel arguments (uniform,
// scalar) and runs that job's body from quant.h with its local workgroup index.  One
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
constexpr int kFp4Waves = 4;  // MXFP4: 256 threads
constexpr int kInt4Waves = 8; // INT4: 512 threads (224 Llama-3.1-8B weights: +1.4% against 4 waves,
                              // level with 16)
// MXFP4 / INT4 chunk: 8 tiles of bf16 or 4 of float32 (8 KiB per wave either way)
template <typename T>
constexpr int kFp4Unr = sizeof(T) == 2 ? 8 : 4;

template <int kFam>
constexpr int kThreads =
    (kFam == kFamFp8 ? kFp8Waves : kFam == kFamInt4 ? kInt4Waves : kFp4Waves) * kWave;

// Kernel-side job, 48 bytes: a launch's argument block (njobs, the workgroup
// prefix table and the jobs) stays within 4 KiB for kMaxBatchJobs jobs.
struct Job {
  const void* x;
  uint8_t* codes;
  void* scales;
  uint8_t* aux;
  int64_t n;      // flat kinds: units (8 elements each); tiles: columns
  uint32_t meta;  // kind | bf16 << 4 | elem << 5 | br << 8 (tiles: min(128, rows))
  uint32_t pad;
};
__host__ __device__ constexpr uint32_t job_kind(uint32_t m) { return m & 15u; }
__host__ __device__ constexpr bool job_bf16(uint32_t m) { return (m >> 4) & 1u; }
__host__ __device__ constexpr int job_elem(uint32_t m) { return (int)((m >> 5) & 7u); }
__host__ __device__ constexpr int job_br(uint32_t m) { return (int)(m >> 8); }

struct MultiArgs {
  int32_t njobs;
  int32_t pad;
  int64_t wg_begin[kMaxBatchJobs + 1];
  Job job[kMaxBatchJobs];
};
static_assert(sizeof(Job) == 48, "kernel-side job layout");
static_assert(sizeof(MultiArgs) <= 4096, "kernel arguments must stay within 4 KiB");

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
  if (job_kind(jb.meta) == kJobFp8Blk) {
    flat_job<kFp8Waves, kFp8Unr>(local, jb.n, [&](int64_t u0, auto g) {
      fp8_1x128_chunk<T, kFp8Unr, decltype(g)::value, kElem>(x, u0, jb.n, jb.codes,
                                                              reinterpret_cast<float*>(jb.scales));
    });
  } else {
    fp8_tile_128x128<T, kFp8Waves, kElem>(x, 0, jb.n, job_br(jb.meta), local, jb.codes,
                                          reinterpret_cast<float*>(jb.scales), red);
  }
}

template <int kFam, typename T>
__device__ __forceinline__ void run_job(const Job& jb, int64_t local, uint8_t* lut, uint32_t* red) {
  const T* x = reinterpret_cast<const T*>(jb.x);
  if constexpr (kFam == kFamFp8) {
    if (job_elem(jb.meta) == kE5M2)
      fp8_job<T, kE5M2>(jb, x, local, red);
    else
      fp8_job<T, kE4M3>(jb, x, local, red);
  } else if constexpr (kFam == kFamMx) {
    if (job_kind(jb.meta) == kJobMx8) {
      flat_job<kFp4Waves, kFp4Unr<T>>(local, jb.n, [&](int64_t u0, auto g) {
        mx8_chunk<T, kFp4Unr<T>, decltype(g)::value>(x, u0, jb.n, jb.codes,
                                                      reinterpret_cast<uint8_t*>(jb.scales));
      });
    } else {
      flat_job<kFp4Waves, kFp4Unr<T>>(local, jb.n, [&](int64_t u0, auto g) {
        mx_chunk<T, kFp4Unr<T>, decltype(g)::value>(x, u0, jb.n, jb.codes,
                                                     reinterpret_cast<uint8_t*>(jb.scales), lut);
      });
    }
  } else {
    flat_job<kInt4Waves, kFp4Unr<T>>(local, jb.n, [&](int64_t u0, auto g) {
      int4_chunk<T, kFp4Unr<T>, decltype(g)::value>(x, u0, jb.n, jb.codes,
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
  // this workgroup's job: the last j with wg_begin[j] <= wg (binary search,
  // uniform over the workgroup)
  const int64_t wg = blockIdx.x;
  int lo = 0, hi = a.njobs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.wg_begin[mid] <= wg)
      lo = mid;
    else
      hi = mid - 1;
  }
  const Job& jb = a.job[lo];
  const int64_t local = wg - a.wg_begin[lo];
  if (job_bf16(jb.meta))
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
  const int64_t nunits = m.batch * m.rows * m.cols / 8;
  jb.n = nunits;
  uint32_t kind;
  auto flat_wgs = [&](int waves, int unr) {
    const int64_t nchunks = (nunits + (int64_t)unr * kWave - 1) / ((int64_t)unr * kWave);
    return (nchunks + waves - 1) / waves;
  };
  const int fp4_unr = m.bf16 ? kFp4Unr<uint16_t> : kFp4Unr<float>;
  int64_t wgs;
  uint32_t br = 0;
  switch (m.kind) {
    case kMultiFp8Blk:
      kind = kJobFp8Blk;
      wgs = flat_wgs(kFp8Waves, kFp8Unr);
      break;
    case kMultiFp8Tile:
      kind = kJobFp8Tile;
      br = (uint32_t)(m.rows < 128 ? m.rows : 128);
      jb.n = m.cols;
      wgs = m.batch * (m.rows / br) * (m.cols / 128);
      break;
    case kMultiMx:
      kind = kJobMx;
      wgs = flat_wgs(kFp4Waves, fp4_unr);
      break;
    case kMultiMx8:
      kind = kJobMx8;
      wgs = flat_wgs(kFp4Waves, fp4_unr);
      break;
    default:
      kind = kJobInt4;
      wgs = flat_wgs(kInt4Waves, fp4_unr);
  }
  jb.meta = kind | (m.bf16 ? 1u : 0u) << 4 | (uint32_t)m.elem << 5 | br << 8;
  return wgs;
}

struct Launch {
  int fam;
  int64_t wgs;
  MultiArgs args;
};

// Splits one family's jobs into launches of at most kMaxBatchJobs jobs, as
// even in job count as possible; false if a launch would exceed the grid
// limit (2^32 - 1 threads), in which case nothing is planned to be launched.
template <int kFam>
bool plan_family(const std::vector<const MultiJob*>& jobs, std::vector<Launch>& out) {
  const size_t n = jobs.size();
  if (n == 0) return true;
  const size_t nl = (n + kMaxBatchJobs - 1) / kMaxBatchJobs, per = (n + nl - 1) / nl;
  for (size_t base = 0; base < n; base += per) {
    const int cnt_jobs = (int)(n - base < per ? n - base : per);
    Launch L;
    L.fam = kFam;
    L.args = MultiArgs{};
    L.args.njobs = cnt_jobs;
    // whole-tile jobs (the heaviest workgroups) first, so that they are not
    // the last to be dispatched
    Job tmp[kMaxBatchJobs];
    int64_t cnt[kMaxBatchJobs];
    for (int i = 0; i < cnt_jobs; ++i) cnt[i] = describe(*jobs[base + i], tmp[i]);
    int order[kMaxBatchJobs], k = 0;
    for (int i = 0; i < cnt_jobs; ++i)
      if (job_kind(tmp[i].meta) == kJobFp8Tile) order[k++] = i;
    for (int i = 0; i < cnt_jobs; ++i)
      if (job_kind(tmp[i].meta) != kJobFp8Tile) order[k++] = i;
    int64_t wg = 0;
    for (int i = 0; i < cnt_jobs; ++i) {
      L.args.wg_begin[i] = wg;
      L.args.job[i] = tmp[order[i]];
      wg += cnt[order[i]];
    }
    L.args.wg_begin[cnt_jobs] = wg;
    L.wgs = wg;
    if (wg > (int64_t)(0xFFFFFFFFu / (uint32_t)kThreads<kFam>)) return false;
    if (wg > 0) out.push_back(L);
  }
  return true;
}

bool plan_multi(const MultiJob* jobs, int njobs, std::vector<Launch>& out) {
  std::vector<const MultiJob*> fam[3];
  for (int i = 0; i < njobs; ++i) fam[family_of(jobs[i].kind)].push_back(&jobs[i]);
  return plan_family<kFamFp8>(fam[kFamFp8], out) && plan_family<kFamMx>(fam[kFamMx], out) &&
         plan_family<kFamInt4>(fam[kFamInt4], out);
}

}  // namespace

int64_t multi_launches(const MultiJob* jobs, int njobs) {
  std::vector<Launch> plan;
  if (!plan_multi(jobs, njobs, plan)) return -1;
  return (int64_t)plan.size();
}

hipError_t launch_multi(const MultiJob* jobs, int njobs, hipStream_t st) {
  std::vector<Launch> plan;
  if (!plan_multi(jobs, njobs, plan)) return hipErrorInvalidConfiguration;
  for (const Launch& L : plan) {
    const dim3 grid((unsigned)L.wgs);
    switch (L.fam) {
      case kFamFp8:
        hipLaunchKernelGGL(k_multi<kFamFp8>, grid, dim3(kThreads<kFamFp8>), 0, st, L.args);
        break;
      case kFamMx:
        hipLaunchKernelGGL(k_multi<kFamMx>, grid, dim3(kThreads<kFamMx>), 0, st, L.args);
        break;
      default:
        hipLaunchKernelGGL(k_multi<kFamInt4>, grid, dim3(kThreads<kFamInt4>), 0, st, L.args);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pqb
