// The C ABI declared in include/pqb.h: argument validation, buffer sizes and
// dispatch to the kernel launchers.  Nothing here allocates or synchronizes.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/pqb.h"
#include "launch.h"

namespace {

using namespace pqb;

bool valid_dtype(int d) { return d == PQB_F32 || d == PQB_BF16; }

bool valid_pair(int fmt, int gran) {
  switch (fmt) {
    case PQB_FP8_E4M3:
    case PQB_FP8_E5M2:
      return gran == PQB_TENSOR || gran == PQB_ROW || gran == PQB_BLK_1x128 ||
             gran == PQB_BLK_128x128;
    case PQB_INT8_SYM:
      return gran == PQB_TENSOR || gran == PQB_ROW;
    case PQB_MXFP4:
    case PQB_MXFP8:
      return gran == PQB_BLK_32;
    case PQB_NVFP4:
      return gran == PQB_BLK_16;
    case PQB_INT4_ASYM:
      return gran == PQB_GRP_128;
  }
  return false;
}

bool known_format(int f) { return f >= PQB_FP8_E4M3 && f <= PQB_INT8_SYM; }

// Formats with one byte per element and float32 scales over the FP8 scopes,
// and their element kind for the launchers (0 E4M3, 1 E5M2, 2 INT8).
bool one_byte(int f) { return f == PQB_FP8_E4M3 || f == PQB_FP8_E5M2 || f == PQB_INT8_SYM; }
int elem_of(int f) { return f == PQB_FP8_E5M2 ? 1 : f == PQB_INT8_SYM ? 2 : 0; }
bool known_gran(int g) { return g >= PQB_TENSOR && g <= PQB_GRP_128; }

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

constexpr int64_t kMaxGridY = 65535;
// KIVI kernels use one-dimensional grids of up to n / 32 threads.
constexpr int64_t kKiviMaxElems = (int64_t)1 << 36;

// Shape rules of one (format, granularity) pair; also bounds the grid sizes
// the launchers will form.
pqb_status check_shape(int fmt, int gran, int64_t b, int64_t r, int64_t c) {
  if (b < 0 || r < 0 || c < 0) return PQB_ERR_SHAPE;
  if (r > 0 && c > INT64_MAX / r) return PQB_ERR_SHAPE;
  if (b > 0 && r * c > INT64_MAX / 4 / b) return PQB_ERR_SHAPE;
  switch (gran) {
    case PQB_TENSOR:
      if (b > kMaxGridY) return PQB_ERR_SHAPE;
      break;
    case PQB_ROW:
      // one wave per row, 4 rows per 256-thread workgroup: the grid must stay
      // within 2^32 - 1 threads
      if (c > 0 && (b * r + 3) / 4 > (int64_t)(0xFFFFFFFFu / 256u)) return PQB_ERR_SHAPE;
      break;
    case PQB_BLK_1x128:
    case PQB_GRP_128:
      if (c % 128) return PQB_ERR_SHAPE;
      break;
    case PQB_BLK_128x128: {
      if (c % 128) return PQB_ERR_SHAPE;
      if (r > 128 && r % 128) return PQB_ERR_SHAPE;
      const int64_t br = r < 128 ? r : 128;
      if (br > 0 && b * (r / br) * (c / 128) > 0xFFFFFFFFll) return PQB_ERR_SHAPE;
      break;
    }
    case PQB_BLK_32:
      if (c % 32) return PQB_ERR_SHAPE;
      break;
    case PQB_BLK_16:
      if (c % 16 || b > kMaxGridY) return PQB_ERR_SHAPE;
      break;
  }
  (void)fmt;
  return PQB_OK;
}

int64_t fp8_num_scales(int gran, int64_t b, int64_t r, int64_t c) {
  switch (gran) {
    case PQB_TENSOR: return b;
    case PQB_ROW: return b * r;
    case PQB_BLK_1x128: return b * r * (c / 128);
    default: {
      const int64_t br = r < 128 ? r : 128;
      return br == 0 ? 0 : b * (r / br) * (c / 128);
    }
  }
}

// Workspace of the per-tensor FP8 passes over `nt` tensors of `slices` slices.
size_t tensor_workspace(int nt, int64_t slices, int64_t per_slice) {
  if (slices <= 0 || per_slice <= 0) return 0;
  if (per_slice % 8 == 0) return twopass_workspace_bytes(nt, slices, per_slice, 1, false);
  return 4 * (size_t)nt * (size_t)slices * (size_t)amax_partials_per_slice(slices, per_slice, nt);
}

pqb_sizes sizes_of(int fmt, int gran, int64_t b, int64_t r, int64_t c) {
  pqb_sizes s{0, 0, 0, 0};
  const int64_t n = b * r * c;
  switch (fmt) {
    case PQB_FP8_E4M3:
    case PQB_FP8_E5M2:
    case PQB_INT8_SYM:
      s.codes = (size_t)n;
      s.scales = 4 * (size_t)fp8_num_scales(gran, b, r, c);
      if (gran == PQB_TENSOR && n > 0) s.workspace = tensor_workspace(1, b, r * c);
      break;
    case PQB_MXFP8:
      s.codes = (size_t)n;
      s.scales = (size_t)n / 32;
      break;
    case PQB_MXFP4:
      s.codes = (size_t)n / 2;
      s.scales = (size_t)n / 32;
      break;
    case PQB_NVFP4:
      s.codes = (size_t)n / 2;
      s.scales = (size_t)n / 16;
      s.aux = 4 * (size_t)b;
      if (n > 0) s.workspace = twopass_workspace_bytes(1, b, r * c, 1, true);
      break;
    case PQB_INT4_ASYM:
      s.codes = (size_t)n / 2;
      s.scales = 2 * (size_t)(n / 128);
      s.aux = (size_t)(n / 128 + 1) / 2;
      break;
  }
  return s;
}

pqb_status hip_status(hipError_t e) { return e == hipSuccess ? PQB_OK : PQB_ERR_HIP; }

}  // namespace

// ---------------------------------------------------------------------------
// Fixed scratch for pqb_quantize_noalloc: one array per GPU, resolved once per
// device with hipGetSymbolAddress (host code never passes the symbol itself,
// which is only a host-side stand-in) and kept until the process ends.
// ---------------------------------------------------------------------------
static_assert(PQB_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) uint8_t scratch[PQB_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch array; PQB_ERR_HIP when
// `stream` runs on another device, where that address would not be valid.
pqb_status scratch_of_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PQB_ERR_HIP;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess || sdev != dev) return PQB_ERR_HIP;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PQB_ERR_HIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return PQB_OK;
}
}  // namespace

extern "C" {

int pqb_abi_version(void) { return PQB_ABI_VERSION; }

#ifndef PQB_SOURCE_HASH
#define PQB_SOURCE_HASH "unknown"
#endif
const char* pqb_source_hash(void) { return PQB_SOURCE_HASH; }

const char* pqb_status_string(pqb_status s) {
  switch (s) {
    case PQB_OK: return "ok";
    case PQB_ERR_NULL: return "a required pointer is NULL";
    case PQB_ERR_ENUM: return "unknown dtype, format or granularity";
    case PQB_ERR_COMBO: return "format and granularity do not go together";
    case PQB_ERR_SHAPE: return "shape rejected by the block rules";
    case PQB_ERR_ALIGN: return "pointer alignment rule broken";
    case PQB_ERR_WORKSPACE: return "workspace too small";
    case PQB_ERR_HIP: return "HIP launch failed";
    case PQB_ERR_SCRATCH: return "needs more scratch than the fixed buffer of pqb_quantize_noalloc";
  }
  return "unknown status";
}

pqb_status pqb_query_sizes(pqb_format fmt, pqb_gran gran, int64_t batch, int64_t rows,
                           int64_t cols, pqb_sizes* out) {
  if (!out) return PQB_ERR_NULL;
  if (!known_format(fmt) || !known_gran(gran)) return PQB_ERR_ENUM;
  if (!valid_pair(fmt, gran)) return PQB_ERR_COMBO;
  const pqb_status st = check_shape(fmt, gran, batch, rows, cols);
  if (st != PQB_OK) return st;
  *out = sizes_of(fmt, gran, batch, rows, cols);
  return PQB_OK;
}

// Validation shared by pqb_quantize and pqb_quantize_batch; fills `need`.
static pqb_status check_quantize(const void* x, int dtype, int64_t batch, int64_t rows,
                                 int64_t cols, int fmt, int gran, const void* codes,
                                 const void* scales, const void* aux, const void* workspace,
                                 size_t workspace_bytes, pqb_sizes* need,
                                 bool check_workspace = true) {
  if (!valid_dtype(dtype) || !known_format(fmt) || !known_gran(gran)) return PQB_ERR_ENUM;
  if (!valid_pair(fmt, gran)) return PQB_ERR_COMBO;
  pqb_status st = check_shape(fmt, gran, batch, rows, cols);
  if (st != PQB_OK) return st;
  *need = sizes_of(fmt, gran, batch, rows, cols);
  if (batch * rows * cols == 0) return PQB_OK;
  if (!x || !codes || !scales) return PQB_ERR_NULL;
  if (need->aux && !aux) return PQB_ERR_NULL;
  if (check_workspace) {
    if (need->workspace && !workspace) return PQB_ERR_NULL;
    if (workspace_bytes < need->workspace) return PQB_ERR_WORKSPACE;
    if (need->workspace && !aligned(workspace, 16)) return PQB_ERR_ALIGN;
  }
  if (!aligned(x, 16) || !aligned(codes, 16)) return PQB_ERR_ALIGN;
  if (one_byte(fmt) && !aligned(scales, 4)) return PQB_ERR_ALIGN;
  if (fmt == PQB_INT4_ASYM && !aligned(scales, 2)) return PQB_ERR_ALIGN;
  if (fmt == PQB_NVFP4 && !aligned(aux, 4)) return PQB_ERR_ALIGN;
  return PQB_OK;
}

pqb_status pqb_quantize(const void* x, pqb_dtype dtype, int64_t batch, int64_t rows, int64_t cols,
                        pqb_format fmt, pqb_gran gran, void* codes, void* scales, void* aux,
                        void* workspace, size_t workspace_bytes, void* stream) {
  pqb_sizes need;
  const pqb_status st = check_quantize(x, dtype, batch, rows, cols, fmt, gran, codes, scales, aux,
                                       workspace, workspace_bytes, &need);
  if (st != PQB_OK) return st;
  const int64_t n = batch * rows * cols;
  if (n == 0) return PQB_OK;
  const bool bf16 = dtype == PQB_BF16;
  hipStream_t s = (hipStream_t)stream;
  uint8_t* c8 = (uint8_t*)codes;
  switch (fmt) {
    case PQB_FP8_E4M3:
    case PQB_FP8_E5M2:
    case PQB_INT8_SYM: {
      float* sc = (float*)scales;
      const int el = elem_of(fmt);
      switch (gran) {
        case PQB_TENSOR: {
          const void* xs[1] = {x};
          uint8_t* cs[1] = {c8};
          float* ss[1] = {sc};
          return hip_status(launch_fp8_tensor(xs, bf16, 1, batch, rows * cols, cs, ss,
                                              (float*)workspace, s, el));
        }
        case PQB_ROW:
          return hip_status(launch_fp8_row(x, bf16, batch * rows, cols, c8, sc, s, el));
        case PQB_BLK_1x128:
          return hip_status(launch_fp8_1x128(x, bf16, n, c8, sc, s, el));
        default:
          return hip_status(launch_fp8_128x128(x, bf16, batch, rows, cols, c8, sc, s, el));
      }
    }
    case PQB_MXFP8:
      return hip_status(launch_mxfp8(x, bf16, n, c8, (uint8_t*)scales, s));
    case PQB_MXFP4:
      return hip_status(launch_mxfp4(x, bf16, n, c8, (uint8_t*)scales, s));
    case PQB_NVFP4:
      return hip_status(launch_nvfp4(x, bf16, batch, rows * cols, c8, (uint8_t*)scales,
                                     (float*)aux, (float*)workspace, s));
    case PQB_INT4_ASYM:
      return hip_status(
          launch_int4(x, bf16, n, c8, (uint16_t*)scales, (uint8_t*)aux, s));
  }
  return PQB_ERR_ENUM;
}

pqb_status pqb_quantize_noalloc(const void* x, pqb_dtype dtype, int64_t batch, int64_t rows,
                                int64_t cols, pqb_format fmt, pqb_gran gran, void* codes,
                                void* scales, void* aux, void* stream) {
  pqb_sizes need;
  // every rule of pqb_quantize except the workspace's, which the fixed
  // scratch replaces
  pqb_status st = check_quantize(x, dtype, batch, rows, cols, fmt, gran, codes, scales, aux,
                                 nullptr, 0, &need, false);
  if (st != PQB_OK) return st;
  if (need.workspace > PQB_NOALLOC_SCRATCH_BYTES) return PQB_ERR_SCRATCH;
  if (batch * rows * cols == 0) return PQB_OK;
  void* ws = nullptr;
  if (need.workspace) {
    st = scratch_of_current_device((hipStream_t)stream, &ws);
    if (st != PQB_OK) return st;
  }
  return pqb_quantize(x, dtype, batch, rows, cols, fmt, gran, codes, scales, aux, ws,
                      need.workspace ? (size_t)PQB_NOALLOC_SCRATCH_BYTES : 0, stream);
}

// Validates a batch and sorts its jobs: one-pass jobs for the fused launches
// into `fused`, per-row one-byte jobs into `rows`; `launches` receives the
// number of kernel launches the batch takes.  Every check happens here, before
// anything is enqueued.
static pqb_status prepare_batch(const pqb_job* jobs, int64_t njobs, std::vector<MultiJob>& fused,
                                std::vector<int64_t>& rows, int64_t* launches) {
  *launches = 0;
  if (njobs < 0) return PQB_ERR_SHAPE;
  if (njobs == 0) return PQB_OK;
  if (!jobs) return PQB_ERR_NULL;
  for (int64_t i = 0; i < njobs; ++i) {
    const pqb_job& j = jobs[i];
    if (j.reserved != 0) return PQB_ERR_ENUM;
    pqb_sizes need;
    const pqb_status st = check_quantize(j.x, j.dtype, j.batch, j.rows, j.cols, j.fmt, j.gran,
                                         j.codes, j.scales, j.aux, nullptr, 0, &need);
    if (st == PQB_ERR_NULL && need.workspace) return PQB_ERR_COMBO;  // two-pass format
    if (st != PQB_OK) return st;
    if (need.workspace) return PQB_ERR_COMBO;
  }
  fused.reserve((size_t)njobs);
  for (int64_t i = 0; i < njobs; ++i) {
    const pqb_job& j = jobs[i];
    if (j.batch * j.rows * j.cols == 0) continue;
    if (one_byte(j.fmt) && j.gran == PQB_ROW) {  // a launch of its own
      rows.push_back(i);
      continue;
    }
    MultiJob m{j.x, (uint8_t*)j.codes, j.scales, (uint8_t*)j.aux, j.batch, j.rows, j.cols, 0,
               j.dtype == PQB_BF16, elem_of(j.fmt)};
    if (one_byte(j.fmt))  // E4M3 or E5M2 (INT8 has only ROW here)
      m.kind = j.gran == PQB_BLK_1x128 ? kMultiFp8Blk : kMultiFp8Tile;
    else if (j.fmt == PQB_MXFP4)
      m.kind = kMultiMx;
    else if (j.fmt == PQB_MXFP8)
      m.kind = kMultiMx8;
    else
      m.kind = kMultiInt4;
    fused.push_back(m);
  }
  const int64_t nl = fused.empty() ? 0 : multi_launches(fused.data(), (int)fused.size());
  if (nl < 0) return PQB_ERR_SHAPE;
  *launches = nl + (int64_t)rows.size();
  return PQB_OK;
}

int64_t pqb_quantize_batch_launches(const pqb_job* jobs, int64_t njobs) {
  std::vector<MultiJob> fused;
  std::vector<int64_t> rows;
  int64_t launches;
  const pqb_status st = prepare_batch(jobs, njobs, fused, rows, &launches);
  return st == PQB_OK ? launches : (int64_t)st;
}

pqb_status pqb_quantize_batch(const pqb_job* jobs, int64_t njobs, void* stream) {
  std::vector<MultiJob> fused;
  std::vector<int64_t> rows;
  int64_t launches;
  const pqb_status st = prepare_batch(jobs, njobs, fused, rows, &launches);
  if (st != PQB_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (!fused.empty()) {
    const hipError_t e = launch_multi(fused.data(), (int)fused.size(), s);
    if (e != hipSuccess) return PQB_ERR_HIP;
  }
  for (const int64_t i : rows) {
    const pqb_job& j = jobs[i];
    const hipError_t e = launch_fp8_row(j.x, j.dtype == PQB_BF16, j.batch * j.rows, j.cols,
                                        (uint8_t*)j.codes, (float*)j.scales, s, elem_of(j.fmt));
    if (e != hipSuccess) return PQB_ERR_HIP;
  }
  return PQB_OK;
}

// Validation shared by pqb_dequantize and pqb_dequantize_batch.
static pqb_status check_dequantize(const void* codes, const void* scales, const void* aux, int fmt,
                                   int gran, int64_t batch, int64_t rows, int64_t cols,
                                   int out_dtype, const void* out) {
  if (!valid_dtype(out_dtype) || !known_format(fmt) || !known_gran(gran)) return PQB_ERR_ENUM;
  if (!valid_pair(fmt, gran)) return PQB_ERR_COMBO;
  const pqb_status st = check_shape(fmt, gran, batch, rows, cols);
  if (st != PQB_OK) return st;
  if (batch * rows * cols == 0) return PQB_OK;
  const pqb_sizes need = sizes_of(fmt, gran, batch, rows, cols);
  if (!codes || !scales || !out || (need.aux && !aux)) return PQB_ERR_NULL;
  if (!aligned(codes, 16) || !aligned(out, 16)) return PQB_ERR_ALIGN;
  if (one_byte(fmt) && !aligned(scales, 4)) return PQB_ERR_ALIGN;
  if (fmt == PQB_INT4_ASYM && !aligned(scales, 2)) return PQB_ERR_ALIGN;
  if (fmt == PQB_NVFP4 && !aligned(aux, 4)) return PQB_ERR_ALIGN;
  if (one_byte(fmt) && batch * rows > 0 && (cols > 0x7FFFFFFF)) return PQB_ERR_SHAPE;
  return PQB_OK;
}

pqb_status pqb_dequantize(const void* codes, const void* scales, const void* aux, pqb_format fmt,
                          pqb_gran gran, int64_t batch, int64_t rows, int64_t cols,
                          pqb_dtype out_dtype, void* out, void* stream) {
  const pqb_status st =
      check_dequantize(codes, scales, aux, fmt, gran, batch, rows, cols, out_dtype, out);
  if (st != PQB_OK) return st;
  const int64_t n = batch * rows * cols;
  if (n == 0) return PQB_OK;
  const bool bf16 = out_dtype == PQB_BF16;
  hipStream_t s = (hipStream_t)stream;
  switch (fmt) {
    case PQB_FP8_E4M3:
    case PQB_FP8_E5M2:
    case PQB_INT8_SYM:
      return hip_status(launch_fp8_dequant((const uint8_t*)codes, (const float*)scales, gran,
                                           batch, rows, cols, bf16, out, s, elem_of(fmt)));
    case PQB_MXFP8:
      return hip_status(launch_mxfp8_dequant((const uint8_t*)codes, (const uint8_t*)scales, n,
                                             bf16, out, s));
    case PQB_MXFP4:
      return hip_status(launch_mxfp4_dequant((const uint8_t*)codes, (const uint8_t*)scales, n,
                                             bf16, out, s));
    case PQB_NVFP4:
      return hip_status(launch_nvfp4_dequant((const uint8_t*)codes, (const uint8_t*)scales,
                                             (const float*)aux, batch, rows * cols, bf16, out,
                                             s));
    case PQB_INT4_ASYM:
      return hip_status(launch_int4_dequant((const uint8_t*)codes, (const uint16_t*)scales,
                                            (const uint8_t*)aux, n, bf16, out, s));
  }
  return PQB_ERR_ENUM;
}

// The fused kind of a dequantization job, or -1 for the scopes that keep a
// launch of their own (FP8 / E5M2 / INT8 per tensor, per row, 128x128).
static int dq_kind_of(int fmt, int gran) {
  switch (fmt) {
    case PQB_FP8_E4M3: return gran == PQB_BLK_1x128 ? kDqFp8 : -1;
    case PQB_FP8_E5M2: return gran == PQB_BLK_1x128 ? kDqE5m2 : -1;
    case PQB_MXFP4: return kDqMx4;
    case PQB_MXFP8: return kDqMx8;
    case PQB_NVFP4: return kDqNv;
    case PQB_INT4_ASYM: return kDqInt4;
  }
  return -1;
}

pqb_status pqb_dequantize_batch(const pqb_dq_job* jobs, int64_t njobs, void* stream) {
  if (njobs < 0) return PQB_ERR_SHAPE;
  if (njobs == 0) return PQB_OK;
  if (!jobs) return PQB_ERR_NULL;
  std::vector<DqMultiJob> fused;
  std::vector<int64_t> own;
  for (int64_t i = 0; i < njobs; ++i) {
    const pqb_dq_job& j = jobs[i];
    if (j.reserved != 0) return PQB_ERR_ENUM;
    const pqb_status st = check_dequantize(j.codes, j.scales, j.aux, j.fmt, j.gran, j.batch,
                                           j.rows, j.cols, j.out_dtype, j.out);
    if (st != PQB_OK) return st;
  }
  for (int64_t i = 0; i < njobs; ++i) {
    const pqb_dq_job& j = jobs[i];
    const int64_t n = j.batch * j.rows * j.cols;
    if (n == 0) continue;
    const int kind = dq_kind_of(j.fmt, j.gran);
    if (kind < 0) {
      own.push_back(i);
      continue;
    }
    const bool bf16 = j.out_dtype == PQB_BF16;
    if (kind == kDqNv) {  // one job per slice, each with its own tensor scale
      const int64_t per = j.rows * j.cols;
      const size_t ob = bf16 ? 2 : 4;
      for (int64_t b = 0; b < j.batch; ++b)
        fused.push_back(DqMultiJob{(const uint8_t*)j.codes + b * (per / 2),
                                   (const uint8_t*)j.scales + b * (per / 16),
                                   (const float*)j.aux + b, (uint8_t*)j.out + (size_t)(b * per) * ob,
                                   per / 8, kind, bf16});
    } else {
      fused.push_back(DqMultiJob{(const uint8_t*)j.codes, j.scales, j.aux, j.out, n / 8, kind,
                                 bf16});
    }
  }
  if (!fused.empty() && dq_multi_launches(fused.data(), (int)fused.size()) < 0)
    return PQB_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  if (!fused.empty() && launch_dq_multi(fused.data(), (int)fused.size(), s) != hipSuccess)
    return PQB_ERR_HIP;
  for (const int64_t i : own) {
    const pqb_dq_job& j = jobs[i];
    const pqb_status st = pqb_dequantize(j.codes, j.scales, j.aux, (pqb_format)j.fmt,
                                         (pqb_gran)j.gran, j.batch, j.rows, j.cols,
                                         (pqb_dtype)j.out_dtype, j.out, stream);
    if (st != PQB_OK) return st;
  }
  return PQB_OK;
}

size_t pqb_kv_workspace_bytes(int64_t layers, int64_t elems_per_layer) {
  if (layers <= 0 || elems_per_layer <= 0) return 0;
  return tensor_workspace(2, layers, elems_per_layer);
}

pqb_status pqb_kv_write_fp8(const void* k, const void* v, pqb_dtype dtype, int64_t layers,
                            int64_t elems_per_layer, uint8_t* k_codes, uint8_t* v_codes,
                            float* k_scales, float* v_scales, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (!valid_dtype(dtype)) return PQB_ERR_ENUM;
  if (layers < 0 || elems_per_layer < 0 || layers > kMaxGridY) return PQB_ERR_SHAPE;
  if (elems_per_layer > 0 && layers > INT64_MAX / 4 / elems_per_layer) return PQB_ERR_SHAPE;
  if (layers == 0 || elems_per_layer == 0) return PQB_OK;
  if (!k || !v || !k_codes || !v_codes || !k_scales || !v_scales || !workspace)
    return PQB_ERR_NULL;
  if (workspace_bytes < pqb_kv_workspace_bytes(layers, elems_per_layer)) return PQB_ERR_WORKSPACE;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) ||
      !aligned(k_scales, 4) || !aligned(v_scales, 4) || !aligned(workspace, 16))
    return PQB_ERR_ALIGN;
  const void* xs[2] = {k, v};
  uint8_t* cs[2] = {k_codes, v_codes};
  float* ss[2] = {k_scales, v_scales};
  return hip_status(launch_fp8_tensor(xs, dtype == PQB_BF16, 2, layers, elems_per_layer, cs, ss,
                                      (float*)workspace, (hipStream_t)stream));
}

static bool kv_dims_ok(int64_t layers, int64_t tokens, int64_t heads, int64_t head_dim) {
  if (layers < 0 || tokens < 0 || heads < 0 || head_dim < 0 || head_dim % 8) return false;
  if (layers > kMaxGridY) return false;
  if (heads > 0 && head_dim > INT32_MAX / 8 / heads) return false;  // row width fits int32
  const int64_t row = heads * head_dim;
  if (row > 0 && tokens > INT64_MAX / 4 / row) return false;
  if (row * tokens > 0 && layers > INT64_MAX / 4 / (row * tokens)) return false;
  return true;
}

// Per head: the LDS tables hold kMaxKvHeads entries, and the head of a column
// c < heads * hu (hu = head_dim / 8) is the multiply-high of c by
// ceil(2^32 / hu), exact while heads * hu * hu < 2^32.
static bool kv_head_ok(int64_t heads, int64_t head_dim) {
  const int64_t hu = head_dim / 8;
  return heads <= kMaxKvHeads && hu < (int64_t)1 << 16 && heads * hu * hu < (int64_t)1 << 32;
}

size_t pqb_kv_workspace_bytes_ex(int64_t layers, int64_t tokens, int64_t heads,
                                 int64_t head_dim) {
  if (!kv_dims_ok(layers, tokens, heads, head_dim)) return 0;
  if (layers == 0 || tokens == 0 || heads == 0 || head_dim == 0) return 0;
  return kv_workspace_bytes(layers, tokens, heads, head_dim);
}

pqb_status pqb_kv_write_fp8_ex(const void* k, const void* v, pqb_dtype dtype, int64_t layers,
                               int64_t tokens, int64_t heads, int64_t head_dim,
                               pqb_kv_mode k_mode, pqb_kv_mode v_mode, uint8_t* k_codes,
                               uint8_t* v_codes, float* k_scales, float* v_scales,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_dtype(dtype)) return PQB_ERR_ENUM;
  const int modes[2] = {(int)k_mode, (int)v_mode};
  for (int m : modes)
    if (m < PQB_KV_LAYER || m > PQB_KV_STATIC) return PQB_ERR_ENUM;
  if (!kv_dims_ok(layers, tokens, heads, head_dim)) return PQB_ERR_SHAPE;
  const void* xs[2] = {k, v};
  uint8_t* cs[2] = {k_codes, v_codes};
  float* ss[2] = {k_scales, v_scales};
  KvTensor t[2];
  int nt = 0;
  bool dynamic = false;
  for (int i = 0; i < 2; ++i) {
    if (!xs[i]) continue;
    if (modes[i] == PQB_KV_HEAD && !kv_head_ok(heads, head_dim)) return PQB_ERR_SHAPE;
    t[nt++] = KvTensor{xs[i], cs[i], ss[i], modes[i]};
    dynamic |= modes[i] != PQB_KV_STATIC;
  }
  if (nt == 0) return PQB_ERR_NULL;
  if (layers == 0 || tokens == 0 || heads == 0 || head_dim == 0) return PQB_OK;
  for (int i = 0; i < nt; ++i)
    if (!t[i].codes || !t[i].scales) return PQB_ERR_NULL;
  if (dynamic && !workspace) return PQB_ERR_NULL;
  if (dynamic && workspace_bytes < pqb_kv_workspace_bytes_ex(layers, tokens, heads, head_dim))
    return PQB_ERR_WORKSPACE;
  for (int i = 0; i < nt; ++i)
    if (!aligned(t[i].x, 16) || !aligned(t[i].codes, 16) || !aligned(t[i].scales, 4))
      return PQB_ERR_ALIGN;
  if (dynamic && !aligned(workspace, 16)) return PQB_ERR_ALIGN;
  return hip_status(launch_kv_fp8(t, nt, dtype == PQB_BF16, layers, tokens, heads, head_dim,
                                  (float*)workspace, (hipStream_t)stream));
}

// KIVI shape rules; `with_k` adds the 32-token groups of K.
static bool kivi_dims_ok(int64_t layers, int64_t tokens, int64_t heads, int64_t head_dim,
                         bool with_k) {
  if (layers < 0 || tokens < 0 || heads < 0 || head_dim < 0 || head_dim % 32) return false;
  if (with_k && tokens % 32) return false;
  int64_t n = 1;
  for (int64_t d : {layers, tokens, heads, head_dim}) {
    if (d == 0) return true;
    if (d > (kKiviMaxElems - 1) / n) return false;  // n * d < 2^36
    n *= d;
  }
  return true;
}

pqb_status pqb_kv_write_kivi(const void* k, const void* v, pqb_dtype dtype, int64_t layers,
                             int64_t tokens, int64_t heads, int64_t head_dim, int bits,
                             uint8_t* k_codes, uint8_t* v_codes, float* k_scales, float* k_mins,
                             float* v_scales, float* v_mins, void* stream) {
  if (!valid_dtype(dtype) || (bits != 2 && bits != 4)) return PQB_ERR_ENUM;
  if (!k && !v) return PQB_ERR_NULL;
  if (!kivi_dims_ok(layers, tokens, heads, head_dim, k != nullptr)) return PQB_ERR_SHAPE;
  const int64_t n = layers * tokens * heads * head_dim;
  if (n == 0) return PQB_OK;
  if ((k && (!k_codes || !k_scales || !k_mins)) || (v && (!v_codes || !v_scales || !v_mins)))
    return PQB_ERR_NULL;
  if (k && !(aligned(k, 16) && aligned(k_codes, 16) && aligned(k_scales, 16) && aligned(k_mins, 16)))
    return PQB_ERR_ALIGN;
  if (v && !(aligned(v, 16) && aligned(v_codes, 16) && aligned(v_scales, 16) && aligned(v_mins, 16)))
    return PQB_ERR_ALIGN;
  const bool bf16 = dtype == PQB_BF16;
  const hipStream_t st = (hipStream_t)stream;
  if (k) {
    const hipError_t e = launch_kivi_k(k, bf16, layers, tokens, heads, head_dim, bits, k_codes,
                                       k_scales, k_mins, st);
    if (e != hipSuccess) return hip_status(e);
  }
  if (v) return hip_status(launch_kivi_v(v, bf16, n, bits, v_codes, v_scales, v_mins, st));
  return PQB_OK;
}

pqb_status pqb_kv_read_kivi(const uint8_t* k_codes, const uint8_t* v_codes,
                            const float* k_scales, const float* k_mins, const float* v_scales,
                            const float* v_mins, int64_t layers, int64_t tokens, int64_t heads,
                            int64_t head_dim, int bits, pqb_dtype out_dtype, void* k_out,
                            void* v_out, void* stream) {
  if (!valid_dtype(out_dtype) || (bits != 2 && bits != 4)) return PQB_ERR_ENUM;
  if (!k_codes && !v_codes) return PQB_ERR_NULL;
  if (!kivi_dims_ok(layers, tokens, heads, head_dim, k_codes != nullptr)) return PQB_ERR_SHAPE;
  const int64_t n = layers * tokens * heads * head_dim;
  if (n == 0) return PQB_OK;
  if ((k_codes && (!k_scales || !k_mins || !k_out)) ||
      (v_codes && (!v_scales || !v_mins || !v_out)))
    return PQB_ERR_NULL;
  if (k_codes && !(aligned(k_codes, 16) && aligned(k_scales, 16) && aligned(k_mins, 16) &&
                   aligned(k_out, 16)))
    return PQB_ERR_ALIGN;
  if (v_codes && !(aligned(v_codes, 16) && aligned(v_scales, 16) && aligned(v_mins, 16) &&
                   aligned(v_out, 16)))
    return PQB_ERR_ALIGN;
  const bool bf16 = out_dtype == PQB_BF16;
  const hipStream_t st = (hipStream_t)stream;
  if (k_codes) {
    const hipError_t e = launch_kivi_k_dequant(k_codes, k_scales, k_mins, layers, tokens, heads,
                                               head_dim, bits, bf16, k_out, st);
    if (e != hipSuccess) return hip_status(e);
  }
  if (v_codes)
    return hip_status(launch_kivi_v_dequant(v_codes, v_scales, v_mins, n, bits, bf16, v_out, st));
  return PQB_OK;
}

// Shape, code-pointer and output rules shared by the GEMM entry points (each
// checks its own scale pointers).
static pqb_status check_gemm(const uint8_t* a, const uint8_t* b, int64_t m, int64_t n, int64_t k,
                             const void* c) {
  if (m < 0 || n < 0 || k < 0 || k % 128 || n % 128) return PQB_ERR_SHAPE;
  if (m > INT32_MAX || n > INT32_MAX || k > INT32_MAX) return PQB_ERR_SHAPE;
  if ((m + 127) / 128 * (n / 128) > INT32_MAX) return PQB_ERR_SHAPE;
  if (m == 0 || n == 0) return PQB_OK;
  if (!c || (k > 0 && (!a || !b))) return PQB_ERR_NULL;
  if (!aligned(c, 16)) return PQB_ERR_ALIGN;
  if (k > 0 && !(aligned(a, 16) && aligned(b, 16))) return PQB_ERR_ALIGN;
  return PQB_OK;
}

pqb_status pqb_gemm_fp8_blockscaled(const uint8_t* a, const float* a_scales, const uint8_t* b,
                                    const float* b_scales, int64_t m, int64_t n, int64_t k,
                                    pqb_dtype out_dtype, void* c, void* stream) {
  if (!valid_dtype(out_dtype)) return PQB_ERR_ENUM;
  const pqb_status e = check_gemm(a, b, m, n, k, c);
  if (e != PQB_OK || m == 0 || n == 0) return e;
  if (k > 0 && (!a_scales || !b_scales)) return PQB_ERR_NULL;
  if (k > 0 && !(aligned(a_scales, 4) && aligned(b_scales, 4))) return PQB_ERR_ALIGN;
  return hip_status(launch_gemm_fp8_bs(a, a_scales, b, b_scales, m, n, k,
                                       out_dtype == PQB_BF16 ? 1 : 0, c, nullptr,
                                       (hipStream_t)stream));
}

pqb_status pqb_gemm_mxfp4(const uint8_t* a, const uint8_t* a_scales, const uint8_t* b,
                          const uint8_t* b_scales, int64_t m, int64_t n, int64_t k,
                          pqb_dtype out_dtype, void* c, void* stream) {
  if (!valid_dtype(out_dtype)) return PQB_ERR_ENUM;
  const pqb_status e = check_gemm(a, b, m, n, k, c);
  if (e != PQB_OK || m == 0 || n == 0) return e;
  if (k > 0 && (!a_scales || !b_scales)) return PQB_ERR_NULL;
  if (k > 0 && !(aligned(a_scales, 4) && aligned(b_scales, 4))) return PQB_ERR_ALIGN;
  return hip_status(launch_gemm_mxfp4(a, a_scales, b, b_scales, m, n, k, out_dtype == PQB_BF16, c,
                                      (hipStream_t)stream));
}

pqb_status pqb_stream_reference(const void* src, int64_t read_bytes, int reads_per_write,
                                int tiles_per_wave, void* dst, void* stream) {
  if (reads_per_write != 1 && reads_per_write != 2 && reads_per_write != 4) return PQB_ERR_ENUM;
  if (tiles_per_wave != 4 && tiles_per_wave != 8) return PQB_ERR_ENUM;
  if (read_bytes < 0 || read_bytes % 8192 || read_bytes > ((int64_t)1 << 38)) return PQB_ERR_SHAPE;
  if (read_bytes == 0) return PQB_OK;
  if (!src || !dst) return PQB_ERR_NULL;
  if (!aligned(src, 16) || !aligned(dst, 16)) return PQB_ERR_ALIGN;
  return hip_status(launch_stream_ref(src, read_bytes, reads_per_write, tiles_per_wave, dst,
                                     (hipStream_t)stream));
}

pqb_status pqb_gemm_nvfp4(const uint8_t* a, const uint8_t* a_scales, const float* a_gs,
                          const uint8_t* b, const uint8_t* b_scales, const float* b_gs, int64_t m,
                          int64_t n, int64_t k, pqb_dtype out_dtype, void* c, void* stream) {
  if (!valid_dtype(out_dtype)) return PQB_ERR_ENUM;
  const pqb_status e = check_gemm(a, b, m, n, k, c);
  if (e != PQB_OK || m == 0 || n == 0) return e;
  if (k > 0 && (!a_scales || !b_scales || !a_gs || !b_gs)) return PQB_ERR_NULL;
  if (k > 0 && !(aligned(a_scales, 4) && aligned(b_scales, 4) && aligned(a_gs, 4) &&
                 aligned(b_gs, 4)))
    return PQB_ERR_ALIGN;
  return hip_status(launch_gemm_nvfp4(a, a_scales, a_gs, b, b_scales, b_gs, m, n, k,
                                      out_dtype == PQB_BF16, c, (hipStream_t)stream));
}

pqb_status pqb_gemm_fp8_blockscaled_quant(const uint8_t* a, const float* a_scales,
                                          const uint8_t* b, const float* b_scales, int64_t m,
                                          int64_t n, int64_t k, uint8_t* c_codes,
                                          float* c_scales, void* stream) {
  const pqb_status e = check_gemm(a, b, m, n, k, c_codes);
  if (e != PQB_OK || m == 0 || n == 0) return e;
  if (k > 0 && (!a_scales || !b_scales)) return PQB_ERR_NULL;
  if (k > 0 && !(aligned(a_scales, 4) && aligned(b_scales, 4))) return PQB_ERR_ALIGN;
  if (!c_scales) return PQB_ERR_NULL;
  if (!aligned(c_scales, 4)) return PQB_ERR_ALIGN;
  return hip_status(launch_gemm_fp8_bs(a, a_scales, b, b_scales, m, n, k, 2, c_codes, c_scales,
                                       (hipStream_t)stream));
}

// Rules of one W4A16 product (m is checked by the caller); fills `job` when
// there is work (n > 0, m > 0), else sets job->N = 0.
static pqb_status check_w4a16(const void* x, int64_t m, const uint8_t* codes, const void* scales,
                              const uint8_t* zeros, int64_t n, int64_t k, void* y, W4Job* job) {
  job->N = 0;
  if (n < 0 || k < 0 || k % 128 || k > INT32_MAX) return PQB_ERR_SHAPE;
  if (k > 0 && n > INT32_MAX / (k / 128)) return PQB_ERR_SHAPE;
  if (m == 0 || n == 0) return PQB_OK;
  if (!y || (k > 0 && (!x || !codes || !scales || !zeros))) return PQB_ERR_NULL;
  if (!aligned(y, 4)) return PQB_ERR_ALIGN;
  if (k > 0 && !(aligned(x, 16) && aligned(codes, 16) && aligned(scales, 2))) return PQB_ERR_ALIGN;
  *job = W4Job{(const uint16_t*)x, codes, (const uint16_t*)scales, zeros, y, (int32_t)n, (int32_t)k};
  return PQB_OK;
}

pqb_status pqb_gemv_w4a16(const void* x, int64_t m, const uint8_t* codes, const void* scales,
                          const uint8_t* zeros, int64_t n, int64_t k, pqb_dtype out_dtype,
                          void* y, void* stream) {
  if (!valid_dtype(out_dtype)) return PQB_ERR_ENUM;
  if (m < 0 || m > 8) return PQB_ERR_SHAPE;
  W4Job job;
  const pqb_status e = check_w4a16(x, m, codes, scales, zeros, n, k, y, &job);
  if (e != PQB_OK || job.N == 0) return e;
  return hip_status(launch_w4a16(&job, 1, (int)m, out_dtype == PQB_BF16, (hipStream_t)stream));
}

pqb_status pqb_gemv_w4a16_batch(const pqb_w4a16_job* jobs, int64_t njobs, int64_t m,
                                pqb_dtype out_dtype, void* stream) {
  if (!valid_dtype(out_dtype)) return PQB_ERR_ENUM;
  if (m < 0 || m > 8 || njobs < 0 || njobs > INT32_MAX) return PQB_ERR_SHAPE;
  if (njobs == 0 || m == 0) return PQB_OK;
  if (!jobs) return PQB_ERR_NULL;
  std::vector<W4Job> w;
  w.reserve((size_t)njobs);
  for (int64_t i = 0; i < njobs; ++i) {
    const pqb_w4a16_job& j = jobs[i];
    W4Job job;
    const pqb_status e = check_w4a16(j.x, m, j.codes, j.scales, j.zeros, j.n, j.k, j.y, &job);
    if (e != PQB_OK) return e;
    if (job.N > 0) w.push_back(job);
  }
  if (w.empty()) return PQB_OK;
  return hip_status(
      launch_w4a16(w.data(), (int)w.size(), (int)m, out_dtype == PQB_BF16, (hipStream_t)stream));
}

pqb_status pqb_gemm_w4a16(const void* x, int64_t m, const uint8_t* codes, const void* scales,
                          const uint8_t* zeros, int64_t n, int64_t k, pqb_dtype out_dtype,
                          void* y, void* stream) {
  if (!valid_dtype(out_dtype)) return PQB_ERR_ENUM;
  if (m < 0 || m > INT32_MAX) return PQB_ERR_SHAPE;
  W4Job job;
  const pqb_status e = check_w4a16(x, m, codes, scales, zeros, n, k, y, &job);
  if (e != PQB_OK || job.N == 0) return e;
  return hip_status(launch_w4a16_mfma(&job, 1, m, out_dtype == PQB_BF16, (hipStream_t)stream));
}

pqb_status pqb_gemm_w4a16_batch(const pqb_w4a16_job* jobs, int64_t njobs, int64_t m,
                                pqb_dtype out_dtype, void* stream) {
  if (!valid_dtype(out_dtype)) return PQB_ERR_ENUM;
  if (m < 0 || m > INT32_MAX || njobs < 0 || njobs > INT32_MAX) return PQB_ERR_SHAPE;
  if (njobs == 0 || m == 0) return PQB_OK;
  if (!jobs) return PQB_ERR_NULL;
  std::vector<W4Job> w;
  w.reserve((size_t)njobs);
  for (int64_t i = 0; i < njobs; ++i) {
    const pqb_w4a16_job& j = jobs[i];
    W4Job job;
    const pqb_status e = check_w4a16(j.x, m, j.codes, j.scales, j.zeros, j.n, j.k, j.y, &job);
    if (e != PQB_OK) return e;
    if (job.N > 0) w.push_back(job);
  }
  if (w.empty()) return PQB_OK;
  return hip_status(
      launch_w4a16_mfma(w.data(), (int)w.size(), m, out_dtype == PQB_BF16, (hipStream_t)stream));
}

pqb_status pqb_encode_e4m3(const float* y, int64_t n, uint8_t* out, void* stream) {
  if (n < 0) return PQB_ERR_SHAPE;
  if (n == 0) return PQB_OK;
  if (!y || !out) return PQB_ERR_NULL;
  if (!aligned(y, 4)) return PQB_ERR_ALIGN;
  return hip_status(launch_encode_elem(y, n, out, (hipStream_t)stream, 0));
}

pqb_status pqb_encode_e5m2(const float* y, int64_t n, uint8_t* out, void* stream) {
  if (n < 0) return PQB_ERR_SHAPE;
  if (n == 0) return PQB_OK;
  if (!y || !out) return PQB_ERR_NULL;
  if (!aligned(y, 4)) return PQB_ERR_ALIGN;
  return hip_status(launch_encode_elem(y, n, out, (hipStream_t)stream, 1));
}

pqb_status pqb_encode_e2m1(const float* y, int64_t n, uint8_t* out, void* stream) {
  if (n < 0) return PQB_ERR_SHAPE;
  if (n == 0) return PQB_OK;
  if (!y || !out) return PQB_ERR_NULL;
  if (!aligned(y, 4)) return PQB_ERR_ALIGN;
  return hip_status(launch_encode_e2m1(y, n, out, (hipStream_t)stream));
}

pqb_status pqb_check_recip(uint32_t first_bits, int64_t n, float* out, void* stream) {
  if (n < 0 || (uint64_t)first_bits + (uint64_t)n > ((uint64_t)1 << 32)) return PQB_ERR_SHAPE;
  if (n == 0) return PQB_OK;
  if (!out) return PQB_ERR_NULL;
  if (!aligned(out, 4)) return PQB_ERR_ALIGN;
  return hip_status(launch_check_recip(first_bits, n, out, (hipStream_t)stream));
}

pqb_status pqb_check_div(const float* s, int64_t ns, uint32_t x_first_bits, int64_t nx,
                         float* out, void* stream) {
  if (ns < 0 || nx < 0 || (uint64_t)x_first_bits + (uint64_t)nx > ((uint64_t)1 << 32))
    return PQB_ERR_SHAPE;
  if (nx > 0 && ns > INT64_MAX / nx) return PQB_ERR_SHAPE;
  if (ns == 0 || nx == 0) return PQB_OK;
  if (!s || !out) return PQB_ERR_NULL;
  if (!aligned(s, 4) || !aligned(out, 4)) return PQB_ERR_ALIGN;
  return hip_status(launch_check_div(s, ns, x_first_bits, nx, out, (hipStream_t)stream));
}

}  // extern "C"
