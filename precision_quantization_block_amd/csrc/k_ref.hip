// Streaming reference: the quantizers' own memory pattern with nothing
// computed, to measure the bandwidth ceiling their read:write mixes can reach
// on this GPU.  Each wave takes an 8 KiB chunk of the source as 8 tiles of
// 1 KiB (lane l holds bytes 16 l .. 16 l + 15 of each tile, one 16-byte
// non-temporal load per tile, as the quantizers load bf16 units) and writes
// 8 / R tiles of 1 KiB with 16-byte non-temporal stores: output tile j of the
// chunk is the XOR of its input tiles R j .. R j + R - 1, which keeps every
// load live.
#include "device.h"
#include "launch.h"

namespace pqb {
namespace {

template <int R>
__global__ __launch_bounds__(kBlockThreads) void k_stream_ref(const uint8_t* __restrict__ src,
                                                              int64_t nchunks,
                                                              uint8_t* __restrict__ dst) {
  const int64_t w = wave_index();
  if (w >= nchunks) return;  // whole waves
  const int lane = threadIdx.x & (kWave - 1);
  const uint8_t* s = src + w * 8192 + 16 * lane;
  uint8_t* d = dst + w * (8192 / R) + 16 * lane;
  uint4 v[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) v[t] = ld_nt16(s + 1024 * t);
#pragma unroll
  for (int j = 0; j < 8 / R; ++j) {
    uint4 x = v[R * j];
#pragma unroll
    for (int r = 1; r < R; ++r) {
      x.x ^= v[R * j + r].x;
      x.y ^= v[R * j + r].y;
      x.z ^= v[R * j + r].z;
      x.w ^= v[R * j + r].w;
    }
    st_nt16(d + 1024 * j, x.x, x.y, x.z, x.w);
  }
}

}  // namespace

hipError_t launch_stream_ref(const void* src, int64_t read_bytes, int reads_per_write, void* dst,
                             hipStream_t st) {
  const int64_t nchunks = read_bytes / 8192;
  const int waves = kBlockThreads / kWave;
  const dim3 grid((unsigned)((nchunks + waves - 1) / waves));
  const uint8_t* s = (const uint8_t*)src;
  uint8_t* d = (uint8_t*)dst;
  if (reads_per_write == 1)
    hipLaunchKernelGGL(k_stream_ref<1>, grid, dim3(kBlockThreads), 0, st, s, nchunks, d);
  else if (reads_per_write == 2)
    hipLaunchKernelGGL(k_stream_ref<2>, grid, dim3(kBlockThreads), 0, st, s, nchunks, d);
  else
    hipLaunchKernelGGL(k_stream_ref<4>, grid, dim3(kBlockThreads), 0, st, s, nchunks, d);
  return hipGetLastError();
}

}  // namespace pqb
