// Measurement aid (gfx950): the achievable streaming-read rate of the device,
// the ceiling the decode split kernels are compared with besides the HBM
// peak.  Workgroup b reads its own contiguous 1/nblocks of the buffer, 16 KiB
// per step (each wavefront 1 KiB contiguous per load, four loads in flight per
// thread), with non-temporal loads, and folds the words into one per
// workgroup so that no load can be dropped.

#include "tg_device.h"

namespace tg_dev {
namespace {

__global__ __launch_bounds__(256) void read_kernel(const TG_GLOBAL u32x4_t* __restrict__ src, int64_t n16,
                                                   TG_GLOBAL uint32_t* __restrict__ sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t hi = lo + per < n16 ? lo + per : n16;
  uint32_t acc = 0;
  int64_t i = lo + threadIdx.x;
  for (; i + 3 * 256 < hi; i += 4 * 256) {
    const u32x4_t a = __builtin_nontemporal_load(src + i);
    const u32x4_t b = __builtin_nontemporal_load(src + i + 256);
    const u32x4_t c = __builtin_nontemporal_load(src + i + 512);
    const u32x4_t d = __builtin_nontemporal_load(src + i + 768);
    acc ^= (a[0] ^ a[1] ^ a[2] ^ a[3]) ^ (b[0] ^ b[1] ^ b[2] ^ b[3]) ^ (c[0] ^ c[1] ^ c[2] ^ c[3]) ^
           (d[0] ^ d[1] ^ d[2] ^ d[3]);
  }
  for (; i < hi; i += 256) {
    const u32x4_t a = __builtin_nontemporal_load(src + i);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
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
