// Lossless bf16 exponent codec (gfx950), SplitZip page ("Die SplitZip-
// Strategie", "Warum es schnell ist"): the 16 most frequent exponents get
// 4-bit codes packed two per byte, sign and mantissa go to one byte per value,
// and values with any other exponent are listed in an escape stream
// (position, exponent) that decoding writes over its first result.  Buffer
// format in include/tg.h.
//
// Encode: exponent histogram (16 LDS copies per workgroup so that lanes with
// the same exponent rarely hit the same counter, then global atomics) ->
// codebook (one workgroup ranks the 256 counts) -> streams, with each
// workgroup's escapes staged in the workspace (up to kStage of them) ->
// exclusive scan of the per-workgroup counts -> escape records placed in
// position order (staged ones sorted by position; a workgroup with more
// re-reads its values).  Decode: one pass over the streams, then one thread
// per escape.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "tg.h"

namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 8;                           // values per thread and step (16 bytes)
constexpr int kSteps = 16;                              // steps per workgroup
constexpr int kStage = 128;                             // escapes staged per workgroup
constexpr int kCopies = 16;                             // LDS histogram copies
constexpr int kLoads = 4;                               // 16-byte loads in flight per thread
constexpr int64_t kPerBlock = kThreads * kPerThread * kSteps;  // values per encode workgroup
constexpr int64_t kHeader = 256;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

struct Work {  // device workspace
  uint32_t hist[256];
  uint32_t code_of[256];  // code, or 16 for an escaped exponent
  int64_t n_esc;
  // then block counts [nb], block offsets [nb] (uint32), staged escape
  // positions [nb][kStage] (uint32) and exponents [nb][kStage] (uint8)
};

__global__ void zero_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
    p[i] = 0;
}

__device__ __forceinline__ uint32_t exp_of(uint32_t v) { return (v >> 7) & 0xFFu; }

__global__ __launch_bounds__(kThreads) void hist_kernel(const u32x4_t* __restrict__ src, int64_t n16,
                                                        Work* __restrict__ ws) {
  __shared__ uint32_t h[kCopies][257];  // padded so that copies sit on different banks
  for (int k = threadIdx.x; k < kCopies * 257; k += kThreads) (&h[0][0])[k] = 0;
  __syncthreads();
  uint32_t* mine = h[threadIdx.x % kCopies];
  // workgroup b reads tiles b, b + grid, ... of kLoads * 256 words, kLoads
  // loads in flight per thread
  const int64_t tile = int64_t(kThreads) * kLoads;
  for (int64_t base = blockIdx.x * tile + threadIdx.x; base < n16; base += int64_t(gridDim.x) * tile) {
    u32x4_t x[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u)
      if (base + u * kThreads < n16) x[u] = __builtin_nontemporal_load(src + base + u * kThreads);
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      if (base + u * kThreads >= n16) break;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        atomicAdd(&mine[exp_of(x[u][k])], 1u);
        atomicAdd(&mine[exp_of(x[u][k] >> 16)], 1u);
      }
    }
  }
  __syncthreads();
  uint32_t t = 0;
  for (int c = 0; c < kCopies; ++c) t += h[c][threadIdx.x];
  if (t) atomicAdd(&ws->hist[threadIdx.x], t);
}

// Rank of exponent e: count descending, then exponent ascending.
__global__ __launch_bounds__(256) void book_kernel(Work* __restrict__ ws, uint8_t* __restrict__ dst, int64_t n) {
  __shared__ uint32_t c[256];
  const int e = threadIdx.x;
  c[e] = ws->hist[e];
  __syncthreads();
  int rank = 0;
  for (int f = 0; f < 256; ++f) rank += (c[f] > c[e]) || (c[f] == c[e] && f < e);
  ws->code_of[e] = rank < 16 ? rank : 16;
  if (rank < 16) dst[16 + rank] = static_cast<uint8_t>(e);
  if (e < 224) dst[32 + e] = 0;
  if (e == 0) {
    ws->n_esc = 0;
    *reinterpret_cast<int64_t*>(dst) = n;
  }
}

// Streams of kPerBlock values per workgroup; escape count per workgroup.
__global__ __launch_bounds__(kThreads) void encode_kernel(const u32x4_t* __restrict__ src, int64_t n,
                                                          const Work* __restrict__ ws, uint8_t* __restrict__ dst,
                                                          uint32_t* __restrict__ block_count,
                                                          uint32_t* __restrict__ stage_pos,
                                                          uint8_t* __restrict__ stage_exp) {
  __shared__ uint32_t code_of[256];
  __shared__ uint32_t n_staged;
  code_of[threadIdx.x] = ws->code_of[threadIdx.x];
  if (threadIdx.x == 0) n_staged = 0;
  __syncthreads();
  uint32_t* spos = stage_pos + static_cast<int64_t>(blockIdx.x) * kStage;
  uint8_t* sexp = stage_exp + static_cast<int64_t>(blockIdx.x) * kStage;
  const int64_t base16 = blockIdx.x * (kPerBlock / kPerThread);
  static_assert(kSteps % kLoads == 0, "steps go in groups of kLoads");
  for (int step0 = 0; step0 < kSteps; step0 += kLoads) {
    u32x4_t xs[kLoads];  // the group's loads first: kLoads in flight per thread
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int64_t i = base16 + (step0 + u) * kThreads + threadIdx.x;
      if (i * kPerThread < n) xs[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
    const int64_t i = base16 + (step0 + u) * kThreads + threadIdx.x;  // 8-value group
    if (i * kPerThread >= n) break;
    const u32x4_t x = xs[u];
    uint32_t sm[2] = {0, 0}, codes = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t v = (x[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
      const uint32_t c = code_of[exp_of(v)];
      if (c == 16) {  // rare: stage (position, exponent), in any order
        const uint32_t at = atomicAdd(&n_staged, 1u);
        if (at < kStage) {
          spos[at] = static_cast<uint32_t>(i * kPerThread + k);
          sexp[at] = static_cast<uint8_t>(exp_of(v));
        }
      }
      codes |= (c & 15u) << (4 * k);
      sm[k >> 2] |= (((v >> 15) << 7) | (v & 0x7Fu)) << (8 * (k & 3));
    }
    *reinterpret_cast<u32x2_t*>(dst + kHeader + i * 8) = u32x2_t{sm[0], sm[1]};
    *reinterpret_cast<uint32_t*>(dst + kHeader + n + i * 4) = codes;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) block_count[blockIdx.x] = n_staged;
}

// Exclusive scan of the block counts (one workgroup of 16 wavefronts), total
// into the header.  Wavefront w owns a contiguous segment of the counts and
// walks it 64 at a time with coalesced loads and a wavefront scan; the 16
// segment totals are scanned in LDS, and a second walk writes the offsets.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

__global__ __launch_bounds__(1024) void scan_kernel(const uint32_t* __restrict__ count, uint32_t* __restrict__ off,
                                                    int64_t nb, Work* __restrict__ ws, uint8_t* __restrict__ dst) {
  __shared__ uint32_t seg_total[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t per = ((nb + 15) / 16 + 63) / 64 * 64;  // segment length, a multiple of 64
  const int64_t lo = wave * per, hi = lo + per < nb ? lo + per : nb;
  constexpr int U = 8;  // loads in flight per lane
  uint32_t total = 0;
  for (int64_t b0 = lo + lane; b0 - lane < hi; b0 += 64 * U) {
    uint32_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = b0 + 64 * u < hi ? count[b0 + 64 * u] : 0u;
    uint32_t t = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) t += v[u];
    total += t;
  }
  // a wavefront sum: every lane's partial folded
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) total += __shfl_xor(total, d, 64);
  if (lane == 0) seg_total[wave] = total;
  __syncthreads();
  uint32_t base = 0;
  for (int k = 0; k < wave; ++k) base += seg_total[k];
  for (int64_t b0 = lo + lane; b0 - lane < hi; b0 += 64 * U) {
    uint32_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = b0 + 64 * u < hi ? count[b0 + 64 * u] : 0u;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t inc = wave_inclusive_scan(v[u]);
      if (b0 + 64 * u < hi) off[b0 + 64 * u] = base + inc - v[u];
      base += __shfl(inc, 63, 64);
    }
  }
  if (threadIdx.x == 1023) {
    uint32_t all = 0;
    for (int k = 0; k < 16; ++k) all += seg_total[k];
    ws->n_esc = all;
    *reinterpret_cast<int64_t*>(dst + 8) = all;
  }
}

// Escape records of a workgroup's values, in position order: the staged
// ones ranked by position, or (more than kStage) found again by re-reading.
__global__ __launch_bounds__(kThreads) void escape_kernel(const u32x4_t* __restrict__ src, int64_t n,
                                                          const Work* __restrict__ ws,
                                                          const uint32_t* __restrict__ block_count,
                                                          const uint32_t* __restrict__ block_off,
                                                          const uint32_t* __restrict__ stage_pos,
                                                          const uint8_t* __restrict__ stage_exp,
                                                          uint8_t* __restrict__ dst) {
  const uint32_t count = block_count[blockIdx.x];
  if (count == 0) return;
  __shared__ uint32_t code_of[256];
  __shared__ uint32_t scan[kThreads];
  const int64_t n_esc = ws->n_esc;
  uint32_t* pos = reinterpret_cast<uint32_t*>(dst + kHeader + n + n / 2);
  uint8_t* exps = reinterpret_cast<uint8_t*>(pos + n_esc);
  uint32_t at = block_off[blockIdx.x];
  if (count <= kStage) {
    const uint32_t* sp = stage_pos + static_cast<int64_t>(blockIdx.x) * kStage;
    const uint8_t* se = stage_exp + static_cast<int64_t>(blockIdx.x) * kStage;
    if (threadIdx.x < count) scan[threadIdx.x] = sp[threadIdx.x];
    __syncthreads();
    if (threadIdx.x < count) {
      const uint32_t p = scan[threadIdx.x];
      uint32_t rank = 0;  // positions are distinct
      for (uint32_t j = 0; j < count; ++j) rank += scan[j] < p;
      pos[at + rank] = p;
      exps[at + rank] = se[threadIdx.x];
    }
    return;
  }
  code_of[threadIdx.x] = ws->code_of[threadIdx.x];
  __syncthreads();
  const int64_t base16 = blockIdx.x * (kPerBlock / kPerThread);
  for (int step = 0; step < kSteps; ++step) {
    const int64_t i = base16 + step * kThreads + threadIdx.x;
    u32x4_t x = {0, 0, 0, 0};
    const bool in = i * kPerThread < n;
    if (in) x = src[i];
    uint32_t mine = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) mine += in ? code_of[exp_of(x[k >> 1] >> (16 * (k & 1)))] >> 4 : 0;
    scan[threadIdx.x] = mine;
    __syncthreads();
    for (int k = 1; k < kThreads; k <<= 1) {
      const uint32_t v = threadIdx.x >= static_cast<unsigned>(k) ? scan[threadIdx.x - k] : 0u;
      __syncthreads();
      scan[threadIdx.x] += v;
      __syncthreads();
    }
    uint32_t w = at + scan[threadIdx.x] - mine;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t e = exp_of(x[k >> 1] >> (16 * (k & 1)));
      if (in && code_of[e] == 16) {
        pos[w] = static_cast<uint32_t>(i * kPerThread + k);
        exps[w] = static_cast<uint8_t>(e);
        ++w;
      }
    }
    at += scan[kThreads - 1];
    __syncthreads();
  }
}

__global__ __launch_bounds__(kThreads) void decode_kernel(const uint8_t* __restrict__ src, int64_t n,
                                                          u32x4_t* __restrict__ out) {
  __shared__ uint32_t book[16];
  if (threadIdx.x < 16) book[threadIdx.x] = src[16 + threadIdx.x];
  __syncthreads();
  const int64_t groups = n / kPerThread;
  const int64_t tile = int64_t(kThreads) * kLoads;
  for (int64_t base = blockIdx.x * tile + threadIdx.x; base < groups; base += int64_t(gridDim.x) * tile) {
    u32x2_t sms[kLoads];
    uint32_t cs[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int64_t i = base + u * kThreads;
      if (i < groups) {
        sms[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(src + kHeader) + i);
        cs[u] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(src + kHeader + n) + i);
      }
    }
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int64_t i = base + u * kThreads;
      if (i >= groups) break;
      const u32x2_t sm = sms[u];
      const uint32_t codes = cs[u];
      uint32_t v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t b = (sm[k >> 2] >> (8 * (k & 3))) & 0xFFu;
        v[k] = ((b >> 7) << 15) | (book[(codes >> (4 * k)) & 15u] << 7) | (b & 0x7Fu);
      }
      out[i] = u32x4_t{v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16)};
    }
  }
}

__global__ __launch_bounds__(kThreads) void patch_kernel(const uint8_t* __restrict__ src, int64_t n,
                                                         uint16_t* __restrict__ out) {
  const int64_t n_esc = *reinterpret_cast<const int64_t*>(src + 8);
  const uint32_t* pos = reinterpret_cast<const uint32_t*>(src + kHeader + n + n / 2);
  const uint8_t* exps = reinterpret_cast<const uint8_t*>(pos + n_esc);
  for (int64_t j = blockIdx.x * int64_t(kThreads) + threadIdx.x; j < n_esc; j += int64_t(gridDim.x) * kThreads) {
    const uint32_t p = pos[j];
    if (p < n) out[p] = static_cast<uint16_t>((out[p] & 0x807Fu) | (static_cast<uint32_t>(exps[j]) << 7));
  }
}

int64_t n_blocks(int64_t n) { return (n + kPerBlock - 1) / kPerBlock; }

}  // namespace

extern "C" size_t tg_zip_bound(int64_t n) {
  return n < 0 ? 0 : static_cast<size_t>(kHeader + n + n / 2 + 5 * n);
}

extern "C" size_t tg_zip_workspace_bytes(int64_t n) {
  return n < 0 ? 0 : sizeof(Work) + (8 + 5 * kStage) * static_cast<size_t>(n_blocks(n));
}

extern "C" int tg_zip_encode(const uint16_t* src, int64_t n, void* dst, size_t dst_bytes, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (!src || !dst || !workspace || n < 8 || n % 8 || n > (int64_t(1) << 32)) return TG_EINVAL;
  if (dst_bytes < tg_zip_bound(n) || workspace_bytes < tg_zip_workspace_bytes(n)) return TG_EINVAL;
  if (reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16 ||
      reinterpret_cast<uintptr_t>(workspace) % 16)
    return TG_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Work* ws = static_cast<Work*>(workspace);
  const int64_t nb = n_blocks(n);
  uint32_t* count = reinterpret_cast<uint32_t*>(ws + 1);
  uint32_t* off = count + nb;
  uint32_t* spos = off + nb;
  uint8_t* sexp = reinterpret_cast<uint8_t*>(spos + nb * kStage);
  uint8_t* out = static_cast<uint8_t*>(dst);
  const u32x4_t* in = reinterpret_cast<const u32x4_t*>(src);
  const int64_t n16 = n / 8;
  hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(256), 0, st, reinterpret_cast<uint32_t*>(ws->hist), int64_t(256));
  const int64_t hb = (n16 + kThreads * kLoads - 1) / (kThreads * kLoads);
  hipLaunchKernelGGL(hist_kernel, dim3(static_cast<unsigned>(hb < 4096 ? hb : 4096)), dim3(kThreads), 0, st, in, n16,
                     ws);
  hipLaunchKernelGGL(book_kernel, dim3(1), dim3(256), 0, st, ws, out, n);
  hipLaunchKernelGGL(encode_kernel, dim3(static_cast<unsigned>(nb)), dim3(kThreads), 0, st, in, n, ws, out, count,
                     spos, sexp);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, count, off, nb, ws, out);
  hipLaunchKernelGGL(escape_kernel, dim3(static_cast<unsigned>(nb)), dim3(kThreads), 0, st, in, n, ws, count, off,
                     spos, sexp, out);
  return hipGetLastError() == hipSuccess ? TG_OK : TG_EDEVICE;
}

extern "C" int tg_zip_decode(const void* src, int64_t n, uint16_t* dst, void* stream) {
  if (!src || !dst || n < 8 || n % 8 || n > (int64_t(1) << 32)) return TG_EINVAL;
  if (reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16) return TG_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint8_t* in = static_cast<const uint8_t*>(src);
  const int64_t groups = n / 8;
  const int64_t gb = (groups + kThreads * kLoads - 1) / (kThreads * kLoads);
  hipLaunchKernelGGL(decode_kernel, dim3(static_cast<unsigned>(gb < 4096 ? gb : 4096)), dim3(kThreads), 0, st, in, n,
                     reinterpret_cast<u32x4_t*>(dst));
  hipLaunchKernelGGL(patch_kernel, dim3(256), dim3(kThreads), 0, st, in, n, dst);
  return hipGetLastError() == hipSuccess ? TG_OK : TG_EDEVICE;
}
