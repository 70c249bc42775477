// The engine's division routines (device.h) on generated arguments, so that
// tests can compare them with IEEE division over whole ranges of floats: every
// code of the FP8, NVFP4, INT4, INT8 and KIVI quantizers rests on x / s being
// the correctly rounded quotient (page "量化部署实战", section 伪量化实现,
// divides by the scale before rounding).
#include "launch.h"
#include "device.h"

namespace pqb {
namespace {

// out[i] = recip_rn(s) for s = the float with bit pattern first + i.
__global__ __launch_bounds__(kBlockThreads) void k_check_recip(uint32_t first, int64_t n,
                                                                float* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kBlockThreads;
  for (int64_t i = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x; i < n; i += stride)
    out[i] = recip_rn(as_f(first + (uint32_t)i));
}

// out[j * nx + i] = div_rn(x, s[j], recip_rn(s[j])) for x = the float with
// bit pattern x_first + i: the quotient as the quantizers form it.
__global__ __launch_bounds__(kBlockThreads) void k_check_div(const float* __restrict__ s, int64_t ns,
                                                              uint32_t x_first, int64_t nx,
                                                              float* __restrict__ out) {
  const int64_t n = ns * nx, stride = (int64_t)gridDim.x * kBlockThreads;
  for (int64_t i = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x; i < n; i += stride) {
    const int64_t j = i / nx, k = i - j * nx;
    const float sj = s[j];
    out[i] = div_rn(as_f(x_first + (uint32_t)k), sj, recip_rn(sj));
  }
}

int grid_of(int64_t n) {
  const int64_t g = (n + kBlockThreads - 1) / kBlockThreads;
  return (int)(g < 1 ? 1 : g > 65536 ? 65536 : g);
}

}  // namespace

hipError_t launch_check_recip(uint32_t first, int64_t n, float* out, hipStream_t st) {
  hipLaunchKernelGGL(k_check_recip, dim3(grid_of(n)), dim3(kBlockThreads), 0, st, first, n, out);
  return hipGetLastError();
}

hipError_t launch_check_div(const float* s, int64_t ns, uint32_t x_first, int64_t nx, float* out,
                            hipStream_t st) {
  hipLaunchKernelGGL(k_check_div, dim3(grid_of(ns * nx)), dim3(kBlockThreads), 0, st, s, ns,
                     x_first, nx, out);
  return hipGetLastError();
}

}  // namespace pqb
