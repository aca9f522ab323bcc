// Measurement aid (gfx950): the achievable streaming-read rate of the device,
// the ceiling the decode split kernels are compared with besides the HBM
// peak.  The grid sweeps the buffer together: pass k of workgroup b reads the
// 16 KiB tile (k * gridDim.x + b) (each wavefront 1 KiB contiguous per load,
// four loads in flight per thread) with non-temporal loads, so that the
// addresses in flight at any moment stay close (on MI355X this reads ~5 %
// faster than giving each workgroup its own contiguous range); each workgroup
// folds the words it read into one so that no load can be dropped.

#include "tg_device.h"

namespace tg_dev {
namespace {

__global__ __launch_bounds__(256) void read_kernel(const TG_GLOBAL u32x4_t* __restrict__ src, int64_t n16,
                                                   TG_GLOBAL uint32_t* __restrict__ sink) {
  constexpr int kLoads = 4;  // 16-byte loads in flight per thread
  const int64_t tile = 256 * kLoads;
  const int64_t step = static_cast<int64_t>(gridDim.x) * tile;
  uint32_t acc = 0;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * tile + threadIdx.x; base < n16; base += step) {
    u32x4_t v[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int64_t j = base + u * 256;
      v[u] = j < n16 ? __builtin_nontemporal_load(src + j) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kLoads; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (static_cast<int>(threadIdx.x) < k) red[threadIdx.x] ^= red[threadIdx.x + k];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

}  // namespace
}  // namespace tg_dev

using namespace tg_dev;

extern "C" int tg_bench_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16) return TG_EINVAL;
  if (bytes == 0) return TG_OK;
  hipLaunchKernelGGL(read_kernel, dim3(TG_BENCH_READ_BLOCKS), dim3(256), 0, static_cast<hipStream_t>(stream),
                     (const TG_GLOBAL u32x4_t*)(src), static_cast<int64_t>(bytes / 16),
                     (TG_GLOBAL uint32_t*)(sink));
  return hipGetLastError() == hipSuccess ? TG_OK : TG_EDEVICE;
}
