// Split kernels of the decode step (gfx950): one wavefront per plan item,
// four wavefronts per workgroup.  A cache with an INT8 tier runs every item
// of both tiers in one launch (the longest-first plan then balances the two
// tiers together, and there is one tail instead of two); a bf16-only cache
// runs the bf16 kernel, which needs no LDS.

#include <cstdlib>

#include "tg_device.h"
#include "tg_item_bf16.h"
#include "tg_item_i8.h"

namespace tg_dev {
namespace {

template <int D, int G, bool QF32, int DEPTH>
__global__ __launch_bounds__(64 * kWavesPerBlock) void split_bf16_kernel(SplitArgs a) {
  const int item = uniform(static_cast<int>(blockIdx.x) * kWavesPerBlock + (static_cast<int>(threadIdx.x) >> 6));
  if (item >= a.n_items) return;
  const TG_GLOBAL int32_t* w = a.work + static_cast<int64_t>(item) * 6;
  if (uniform(w[2]) != TG_TIER_BF16) return;  // no INT8 pages in this cache
  bf16_dispatch<D, G, QF32, DEPTH>(a, w);
}

template <int D, int G, bool QF32, int BITS>
__global__ __launch_bounds__(64 * kWavesPerBlock) void split_tiered_kernel(SplitArgs a) {
  __shared__ float lds[kWavesPerBlock][kI8LdsFloats<D>];
  const int wave = uniform(static_cast<int>(threadIdx.x) >> 6);
  const int item = uniform(static_cast<int>(blockIdx.x) * kWavesPerBlock + wave);
  if (item >= a.n_items) return;
  const TG_GLOBAL int32_t* w = a.work + static_cast<int64_t>(item) * 6;
  if (uniform(w[2]) == TG_TIER_I8)
    i8_dispatch<D, G, QF32, 2, BITS>(a, w, lds[wave]);
  else
    bf16_dispatch<D, G, QF32, 2>(a, w);
}

template <int D, int G, bool QF32>
hipError_t launch(const SplitArgs& a, bool has_i8, int old_bits, hipStream_t s) {
  const int blocks = (a.n_items + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks == 0) return hipSuccess;
  const dim3 grid(blocks), block(64 * kWavesPerBlock);
  if (has_i8) {
    if (old_bits == 4) {
      if constexpr (D == 128)
        hipLaunchKernelGGL((split_tiered_kernel<D, G, QF32, 4>), grid, block, 0, s, a);
      else
        return hipErrorInvalidValue;
    } else {
      hipLaunchKernelGGL((split_tiered_kernel<D, G, QF32, 8>), grid, block, 0, s, a);
    }
    return hipGetLastError();
  }
  static const int depth = [] {
    const char* e = getenv("TG_SPLIT_DEPTH");  // tuning knob: 2 or 3 page buffers
    return (e && atoi(e) == 3) ? 3 : 2;
  }();
  if (depth == 3)
    hipLaunchKernelGGL((split_bf16_kernel<D, G, QF32, 3>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((split_bf16_kernel<D, G, QF32, 2>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const SplitArgs& a, int G, bool qf32, bool has_i8, int old_bits, hipStream_t s) {
  switch (G * 2 + (qf32 ? 1 : 0)) {
    case 2: return launch<D, 1, false>(a, has_i8, old_bits, s);
    case 3: return launch<D, 1, true>(a, has_i8, old_bits, s);
    case 4: return launch<D, 2, false>(a, has_i8, old_bits, s);
    case 5: return launch<D, 2, true>(a, has_i8, old_bits, s);
    case 8: return launch<D, 4, false>(a, has_i8, old_bits, s);
    case 9: return launch<D, 4, true>(a, has_i8, old_bits, s);
    case 16: return launch<D, 8, false>(a, has_i8, old_bits, s);
    case 17: return launch<D, 8, true>(a, has_i8, old_bits, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_split(const SplitArgs& a, int d, int G, bool qf32, bool has_i8, int old_bits, hipStream_t s) {
  if (d == 128) return launch_d<128>(a, G, qf32, has_i8, old_bits, s);
  if (d == 64) return launch_d<64>(a, G, qf32, has_i8, old_bits, s);
  return hipErrorInvalidValue;
}

}  // namespace tg_dev
