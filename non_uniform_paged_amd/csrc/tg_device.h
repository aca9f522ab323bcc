// Internal device-side declarations shared by the decode kernels (gfx950).
// Not part of the C ABI.
#ifndef TG_DEVICE_H_
#define TG_DEVICE_H_

#include <hip/hip_runtime.h>

#include <cstdint>

#include "tg.h"
#include "tg_layout.h"

// Every device pointer the kernels touch is kept in the global address space:
// pointers read from a struct are otherwise generic, and flat loads also count
// against lgkmcnt, which serialises the waits of the streaming loops.
#define TG_GLOBAL __attribute__((address_space(1)))
// LDS pointers are kept in the local address space for the same reason.
#define TG_LDS __attribute__((address_space(3)))

namespace tg_dev {

typedef const TG_GLOBAL char* gptr;

constexpr int kWavesPerBlock = 4;   // wavefronts per workgroup of the split kernels
constexpr int kPage = 16;           // bf16 page: token slots per head
constexpr int kQBlock = 64;         // INT8 block: token slots per head
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Reference-max slack (base 2): weights are 2^(s - m_ref) <= 2^kSlack, and the
// accumulators are rescaled only when a score exceeds m_ref + kSlack.  Any
// reference gives the same merged result; the slack only saves rescales.
constexpr float kSlack = 8.f;

struct SplitArgs {
  gptr pool[TG_MAX_CLUSTERS][2];
  int32_t page_bytes[TG_MAX_CLUSTERS][2];  // between page ids; < 2^31 (checked on the host)
  int64_t head_stride[TG_MAX_CLUSTERS][2];  // between the head slots of one page
  const TG_GLOBAL int32_t* bt[TG_MAX_CLUSTERS][2];
  int32_t stride[TG_MAX_CLUSTERS][2];
  const TG_GLOBAL int32_t* cluster_of_head;
  const TG_GLOBAL int32_t* slot_in_cluster;
  const TG_GLOBAL int32_t* len;      // [B*H*2] live (n_i8, n_bf): items are clipped to them
  const TG_GLOBAL int32_t* n_fixed;  // [B] or null
  const TG_GLOBAL int32_t* ring;     // [B*C] bf16 ring pages, or null (no ring)
  const TG_GLOBAL int32_t* bf_base;  // [B*H] ring row of logical bf16 row 0 (with ring)
  gptr q;
  const TG_GLOBAL int32_t* work;
  const TG_GLOBAL int32_t* gitems;  // [n_gitems][TG_GROUP_WIDTH][2] (request, slot)
  TG_GLOBAL float* ws_acc;  // [n_slots][G][D]
  TG_GLOBAL float* ws_ml;   // [n_slots][G][2]
  int32_t n_items;
  int32_t n_gitems;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t n_clusters;
  float scale_log2;
};

// Partial of an item with no live rows (m = -inf, l = 0, acc = 0): the merge
// gives it no weight.
template <int D, int G>
__device__ __forceinline__ void write_empty_partial(const SplitArgs& a, int slot) {
  const int lane = threadIdx.x & 63;
  TG_GLOBAL float* acc = a.ws_acc + static_cast<int64_t>(slot) * G * D;
  for (int i = lane; i < G * D; i += 64) acc[i] = 0.f;
  if (lane < G) {
    a.ws_ml[(static_cast<int64_t>(slot) * G + lane) * 2 + 0] = -INFINITY;
    a.ws_ml[(static_cast<int64_t>(slot) * G + lane) * 2 + 1] = 0.f;
  }
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ T uniform(T x) {
  return __builtin_amdgcn_readfirstlane(x);
}

// Page loads: rows that only one sequence reads are streamed with
// non-temporal loads (they are not reused, and keeping them out of the caches
// measurably raises HBM read throughput); rows on a shared radix path use
// ordinary loads so that the sequences sharing them hit in L2 / MALL.
template <bool STREAM>
__device__ __forceinline__ u32x4_t ldpage(gptr p) {
  if constexpr (STREAM) return __builtin_nontemporal_load((const TG_GLOBAL u32x4_t*)(p));
  else return *(const TG_GLOBAL u32x4_t*)(p);
}
__device__ __forceinline__ u32x4_t ldv16(gptr p) { return *(const TG_GLOBAL u32x4_t*)(p); }
__device__ __forceinline__ void st16(TG_GLOBAL float* p, float a, float b, float c, float d) {
  f32x4_t x = {a, b, c, d};
  *(TG_GLOBAL f32x4_t*)(p) = x;
}

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}
// split x into bf16 hi + lo (x - hi - lo is ~2^-17 |x|)
__device__ __forceinline__ void split_bf16(float x, uint32_t& hi, uint32_t& lo) {
  hi = bf16_rne(x);
  lo = bf16_rne(x - __uint_as_float(hi << 16));
}
// split x into fp16 hi + lo bits (round to nearest even)
__device__ __forceinline__ void split_f16(float x, uint32_t& hi, uint32_t& lo) {
  const _Float16 h = static_cast<_Float16>(x);
  const _Float16 l = static_cast<_Float16>(x - static_cast<float>(h));
  hi = __builtin_bit_cast(uint16_t, h);
  lo = __builtin_bit_cast(uint16_t, l);
}

// Butterfly steps across the 16-lane rows of a wavefront (v_permlane*_swap
// with both operands the same value returns the lane's and its partner's).
__device__ __forceinline__ float xor16_max(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Matrix-core tiles (16x16 fp32 accumulators; lane l holds rows 4(l/16)..+3
// of column l%16).  A operands: lane l holds row l%16, k-slice l/16.
__device__ __forceinline__ f32x4_t mfma_bf16_k32(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_bf16_k16(const u32x2_t& a, const u32x2_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_f16_k32(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_f16_k16(const u32x2_t& a, const u32x2_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a), __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
}

// Split-kernel launch over every plan item; has_i8: the cache has INT8 (or,
// with old_bits 4, INT4) pages.  Returns hipErrorInvalidValue for an unsupported (d, G).
hipError_t launch_split(const SplitArgs& a, int d, int G, bool qf32, bool has_i8, int old_bits, hipStream_t s,
                        hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);

}  // namespace tg_dev

#endif  // TG_DEVICE_H_
