// Measurement aid (gfx950): the achievable streaming-read rate of the device,
// the ceiling the decode split kernels are compared with besides the HBM
// peak.  The grid sweeps the buffer together: pass k of workgroup b reads the
// 16 KiB tile (k * gridDim.x + b) (each wavefront 1 KiB contiguous per load,
// four loads in flight per thread) with non-temporal loads, so that the
// addresses in flight at any moment stay close (on MI355X this reads ~5 %
// faster than giving each workgroup its own contiguous range); each workgroup
// folds the words it read into one so that no load can be dropped.
//
// A second aid reads in the split kernels' own pattern instead: independent
// streams, one wavefront each, every stream a list of 8 KiB chunks read in
// order with two chunks (sixteen 1 KiB wave loads) in flight, as a decode item
// reads its pages.  Timing it over the chunk counts of a plan gives the rate
// that pattern allows on this device, with no arithmetic at all.

#include <hip/hip_ext.h>
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

// Stream w reads chunks chunk[off[w]] .. chunk[off[w + 1] - 1] of src (chunk
// c: 16-byte words 512 c .. 512 c + 511), ids taken modulo n_chunks, in
// windows of 64 chunk ids (one per lane); sink[w] = XOR of every 32-bit word
// it read.
__global__ __launch_bounds__(256) void streams_kernel(const TG_GLOBAL u32x4_t* __restrict__ src, int64_t n_chunks,
                                                      const TG_GLOBAL int32_t* __restrict__ chunk,
                                                      const TG_GLOBAL int32_t* __restrict__ off, int n_streams,
                                                      TG_GLOBAL uint32_t* __restrict__ sink) {
  constexpr int kDepth = 16;  // 1 KiB wave loads in flight: two 8 KiB chunks
  const int wave = uniform(static_cast<int>(blockIdx.x) * kWavesPerBlock + (static_cast<int>(threadIdx.x) >> 6));
  if (wave >= n_streams) return;
  const int lane = threadIdx.x & 63;
  const int p0 = uniform(off[wave]);
  const int np = uniform(off[wave + 1]) - p0;
  uint32_t acc = 0;
  for (int w0 = 0; w0 < np; w0 += 64) {
    const int nw = min(64, np - w0);
    int64_t c = chunk[p0 + w0 + min(lane, nw - 1)] % n_chunks;
    if (c < 0) c += n_chunks;
    const int cid_lane = static_cast<int>(c);
    const int nloads = nw * 8;
    auto at = [&](int k) {  // load k of the window: 1 KiB k % 8 of chunk k / 8
      const int64_t cid = __builtin_amdgcn_readlane(cid_lane, min(k, nloads - 1) >> 3);
      return src + cid * 512 + (min(k, nloads - 1) & 7) * 64 + lane;
    };
    u32x4_t v[kDepth];
#pragma unroll
    for (int u = 0; u < kDepth; ++u) v[u] = __builtin_nontemporal_load(at(u));
    for (int k = 0; k < nloads; k += kDepth) {
#pragma unroll
      for (int u = 0; u < kDepth; ++u) {
        if (k + u < nloads) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
        if (k + u + kDepth < nloads) v[u] = __builtin_nontemporal_load(at(k + u + kDepth));
      }
    }
  }
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) acc ^= __shfl_xor(acc, m, 64);
  if (lane == 0) sink[wave] = acc;
}

}  // namespace
}  // namespace tg_dev

using namespace tg_dev;

extern "C" int tg_bench_read(const void* src, size_t bytes, uint32_t* sink, void* start_event, void* stop_event,
                             void* stream) {
  if (!src || !sink || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16) return TG_EINVAL;
  if (bytes == 0) return TG_OK;
  hipExtLaunchKernelGGL(read_kernel, dim3(TG_BENCH_READ_BLOCKS), dim3(256), 0, static_cast<hipStream_t>(stream),
                        static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event), 0,
                     (const TG_GLOBAL u32x4_t*)(src), static_cast<int64_t>(bytes / 16),
                     (TG_GLOBAL uint32_t*)(sink));
  return hipGetLastError() == hipSuccess ? TG_OK : TG_EDEVICE;
}

extern "C" int tg_bench_streams(const void* src, size_t bytes, const int32_t* chunk, const int32_t* off,
                                int32_t n_streams, uint32_t* sink, void* start_event, void* stop_event,
                                void* stream) {
  if (!src || reinterpret_cast<uintptr_t>(src) % 16 || bytes == 0 || bytes % 8192 || n_streams < 0) return TG_EINVAL;
  if (n_streams == 0) return TG_OK;
  if (!chunk || !off || !sink) return TG_EINVAL;
  const int blocks = (n_streams + kWavesPerBlock - 1) / kWavesPerBlock;
  hipExtLaunchKernelGGL(streams_kernel, dim3(blocks), dim3(64 * kWavesPerBlock), 0, static_cast<hipStream_t>(stream),
                        static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event), 0,
                     (const TG_GLOBAL u32x4_t*)(src), static_cast<int64_t>(bytes / 8192),
                     (const TG_GLOBAL int32_t*)(chunk), (const TG_GLOBAL int32_t*)(off), n_streams,
                     (TG_GLOBAL uint32_t*)(sink));
  return hipGetLastError() == hipSuccess ? TG_OK : TG_EDEVICE;
}
