// Split kernels of the decode step (gfx950).  The plan's leading n_gitems
// entries are group items: workgroup b < n_gitems runs entry b on all four
// wavefronts together (bf16_group_coop); every later workgroup runs four
// entries, one per wavefront.  A cache with an INT8 tier runs every item of
// both tiers in one launch (the longest-first plan then balances the two
// tiers together, and there is one tail instead of two); a bf16-only cache
// runs the bf16 kernel.  Launches go through hipExtLaunchKernelGGL so that a
// measurement can have the kernel's own start and end recorded into two
// events (null events: an ordinary launch).

#include <cstdlib>

#include <hip/hip_ext.h>

#include "tg_device.h"
#include "tg_item_bf16.h"
#include "tg_item_i8.h"

namespace tg_dev {
namespace {

// Plan entry of wavefront `wave` of workgroup `b` outside the cooperative
// workgroups (ng of them), or -1 past the plan.
__device__ __forceinline__ int single_item(const SplitArgs& a, int ng, int b, int wave) {
  const int item = ng + (b - ng) * kWavesPerBlock + wave;
  return item < a.n_items ? item : -1;
}

template <int D, int G, bool QF32, int DEPTH>
__global__ __launch_bounds__(64 * kWavesPerBlock) __attribute__((amdgpu_waves_per_eu(2))) void split_bf16_kernel(
    SplitArgs a) {
  __shared__ __attribute__((aligned(16))) char coop[kCoopLdsBytes<D>];
  const int b = static_cast<int>(blockIdx.x);
  const int wave = uniform(static_cast<int>(threadIdx.x) >> 6);
  const int ng = min(a.n_gitems, a.n_items);
  if (b < ng) {
    const TG_GLOBAL int32_t* w = a.work + static_cast<int64_t>(b) * 6;
    if (uniform(w[0]) < 0) {
      bf16_group_coop<D, G, QF32>(a, w, (TG_LDS char*)coop);
    } else if (wave == 0 && uniform(w[2]) == TG_TIER_BF16) {
      bf16_dispatch<D, G, QF32, DEPTH>(a, w);  // not a group item: one wavefront runs it
    }
    return;
  }
  const int item = uniform(single_item(a, ng, b, wave));
  if (item < 0) return;
  const TG_GLOBAL int32_t* w = a.work + static_cast<int64_t>(item) * 6;
  if (uniform(w[2]) != TG_TIER_BF16) return;  // no INT8 pages in this cache
  bf16_dispatch<D, G, QF32, DEPTH>(a, w);
}

template <int D, int G, bool QF32, int BITS>
__global__ __launch_bounds__(64 * kWavesPerBlock) __attribute__((amdgpu_waves_per_eu(2))) void split_tiered_kernel(
    SplitArgs a) {
  // LDS: the INT8 items' accumulators, or the pages of a cooperative group item
  constexpr int kI8Bytes = kWavesPerBlock * kI8LdsFloats<D> * 4;
  __shared__ __attribute__((aligned(16))) char smem[kI8Bytes > kCoopLdsBytes<D> ? kI8Bytes : kCoopLdsBytes<D>];
  float(*lds)[kI8LdsFloats<D>] = reinterpret_cast<float(*)[kI8LdsFloats<D>]>(smem);
  const int b = static_cast<int>(blockIdx.x);
  const int wave = uniform(static_cast<int>(threadIdx.x) >> 6);
  const int ng = min(a.n_gitems, a.n_items);
  if (b < ng) {
    const TG_GLOBAL int32_t* w = a.work + static_cast<int64_t>(b) * 6;
    if (uniform(w[0]) < 0) {
      bf16_group_coop<D, G, QF32>(a, w, (TG_LDS char*)smem);
    } else if (wave == 0) {  // not a group item: one wavefront runs it
      if (uniform(w[2]) == TG_TIER_I8)
        i8_dispatch<D, G, QF32, BITS == 4 ? 4 : 2, BITS>(a, w, lds[0]);
      else
        bf16_dispatch<D, G, QF32, 2>(a, w);
    }
    return;
  }
  const int item = uniform(single_item(a, ng, b, wave));
  if (item < 0) return;
  const TG_GLOBAL int32_t* w = a.work + static_cast<int64_t>(item) * 6;
  if (uniform(w[2]) == TG_TIER_I8)
    i8_dispatch<D, G, QF32, BITS == 4 ? 4 : 2, BITS>(a, w, lds[wave]);
  else
    bf16_dispatch<D, G, QF32, 2>(a, w);
}

template <int D, int G, bool QF32>
hipError_t launch(const SplitArgs& a, bool has_i8, int old_bits, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int ng = a.n_gitems < a.n_items ? a.n_gitems : a.n_items;
  const int blocks = ng + (a.n_items - ng + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks == 0) return hipSuccess;
  const dim3 grid(blocks), block(64 * kWavesPerBlock);
  if (has_i8) {
    if (old_bits == 4) {
      if constexpr (D == 128)
        hipExtLaunchKernelGGL((split_tiered_kernel<D, G, QF32, 4>), grid, block, 0, s, e0, e1, 0, a);
      else
        return hipErrorInvalidValue;
    } else {
      hipExtLaunchKernelGGL((split_tiered_kernel<D, G, QF32, 8>), grid, block, 0, s, e0, e1, 0, a);
    }
    return hipGetLastError();
  }
  static const int depth = [] {
    const char* e = getenv("TG_SPLIT_DEPTH");  // tuning knob: 2 or 3 page buffers
    return (e && atoi(e) == 3) ? 3 : 2;
  }();
  if (depth == 3)
    hipExtLaunchKernelGGL((split_bf16_kernel<D, G, QF32, 3>), grid, block, 0, s, e0, e1, 0, a);
  else
    hipExtLaunchKernelGGL((split_bf16_kernel<D, G, QF32, 2>), grid, block, 0, s, e0, e1, 0, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const SplitArgs& a, int G, bool qf32, bool has_i8, int old_bits, hipStream_t s, hipEvent_t e0,
                    hipEvent_t e1) {
  switch (G * 2 + (qf32 ? 1 : 0)) {
    case 2: return launch<D, 1, false>(a, has_i8, old_bits, s, e0, e1);
    case 3: return launch<D, 1, true>(a, has_i8, old_bits, s, e0, e1);
    case 4: return launch<D, 2, false>(a, has_i8, old_bits, s, e0, e1);
    case 5: return launch<D, 2, true>(a, has_i8, old_bits, s, e0, e1);
    case 8: return launch<D, 4, false>(a, has_i8, old_bits, s, e0, e1);
    case 9: return launch<D, 4, true>(a, has_i8, old_bits, s, e0, e1);
    case 16: return launch<D, 8, false>(a, has_i8, old_bits, s, e0, e1);
    case 17: return launch<D, 8, true>(a, has_i8, old_bits, s, e0, e1);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_split(const SplitArgs& a, int d, int G, bool qf32, bool has_i8, int old_bits, hipStream_t s,
                        hipEvent_t e0, hipEvent_t e1) {
  if (d == 128) return launch_d<128>(a, G, qf32, has_i8, old_bits, s, e0, e1);
  if (d == 64) return launch_d<64>(a, G, qf32, has_i8, old_bits, s, e0, e1);
  return hipErrorInvalidValue;
}

}  // namespace tg_dev
