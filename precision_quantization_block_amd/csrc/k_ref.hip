// Streaming reference: the quantizers' own memory pattern with nothing
// computed, to measure the bandwidth ceiling their read:write mixes can reach
// on this GPU.  Each wave takes a chunk of kT tiles of 1 KiB (lane l holds
// bytes 16 l .. 16 l + 15 of each tile, one 16-byte non-temporal load per
// tile, as the quantizers load bf16 units) and writes kT / R tiles of 1 KiB
// with 16-byte non-temporal stores: output tile j of the chunk is the XOR of
// its input tiles R j .. R j + R - 1, which keeps every load live.  The
// quantizers take 8 tiles per wave; 4 tiles is the faster stream at 4 bytes
// read per byte written.
#include "device.h"
#include "launch.h"

namespace pqb {
namespace {

template <int R, int kT>
__global__ __launch_bounds__(kBlockThreads) void k_stream_ref(const uint8_t* __restrict__ src,
                                                              int64_t nchunks,
                                                              uint8_t* __restrict__ dst) {
  const int64_t w = wave_index();
  if (w >= nchunks) return;  // whole waves
  const int lane = threadIdx.x & (kWave - 1);
  const uint8_t* s = src + w * (1024 * kT) + 16 * lane;
  uint8_t* d = dst + w * (1024 * kT / R) + 16 * lane;
  uint4 v[kT];
#pragma unroll
  for (int t = 0; t < kT; ++t) v[t] = ld_nt16(s + 1024 * t);
#pragma unroll
  for (int j = 0; j < kT / R; ++j) {
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

template <int kT>
static void launch_stream_ref_t(const uint8_t* s, int64_t read_bytes, int reads_per_write, uint8_t* d,
                         hipStream_t st) {
  const int64_t nchunks = read_bytes / (1024 * kT);
  const int waves = kBlockThreads / kWave;
  const dim3 grid((unsigned)((nchunks + waves - 1) / waves));
  if (reads_per_write == 1)
    hipLaunchKernelGGL((k_stream_ref<1, kT>), grid, dim3(kBlockThreads), 0, st, s, nchunks, d);
  else if (reads_per_write == 2)
    hipLaunchKernelGGL((k_stream_ref<2, kT>), grid, dim3(kBlockThreads), 0, st, s, nchunks, d);
  else
    hipLaunchKernelGGL((k_stream_ref<4, kT>), grid, dim3(kBlockThreads), 0, st, s, nchunks, d);
}

hipError_t launch_stream_ref(const void* src, int64_t read_bytes, int reads_per_write,
                             int tiles_per_wave, void* dst, hipStream_t st) {
  if (tiles_per_wave == 4)
    launch_stream_ref_t<4>((const uint8_t*)src, read_bytes, reads_per_write, (uint8_t*)dst, st);
  else
    launch_stream_ref_t<8>((const uint8_t*)src, read_bytes, reads_per_write, (uint8_t*)dst, st);
  return hipGetLastError();
}

}  // namespace pqb
