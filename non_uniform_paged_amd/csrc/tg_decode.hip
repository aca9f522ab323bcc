// Decode attention over the ragged, tiered, paged cache (gfx950): the C-ABI
// entry points of the decode step and the log-sum-exp merge kernel.
//
// tg_decode_split launches one split kernel per tier present in the cache
// (tg_split_bf16.hip, tg_split_i8.hip); each writes, per plan item, the
// online-normaliser partial (m, l, acc) of the item's rows.  tg_merge_partials
// combines the partials of each (r, h) with the weights e^{m_s - M} (CAP survey
// page, section 2.4.3 "Distributed acceleration", online normaliser [88]) and
// writes o in fp32.  tg_decode_attn is the two in sequence.

#include <cmath>
#include <cstdint>

#include "tg_device.h"

namespace tg_dev {
namespace {

// ---------------------------------------------------------------- merge kernel
// One wavefront per (pair, g).  The wave finds M = max_s m_s and the
// denominator sum_s e^{m_s - M} l_s with one slot per lane, then sums the
// weighted accumulators with NG = 64/(D/8) slots in flight at once (lane
// group q takes slots q, q + NG, ...; each lane owns 8 channels) and folds
// the groups together.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const TG_GLOBAL float* __restrict__ ws_acc,
                                                    const TG_GLOBAL float* __restrict__ ws_ml,
                                                    const TG_GLOBAL int32_t* __restrict__ part_off,
                                                    int32_t n_pairs, int32_t G,
                                                    TG_GLOBAL float* __restrict__ out) {
  constexpr int LPR = D / 8;   // lanes per channel row
  constexpr int NG = 64 / LPR; // slots merged concurrently
  const int lane = threadIdx.x & 63;
  const int64_t rowid = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (rowid >= static_cast<int64_t>(n_pairs) * G) return;
  const int64_t pair = rowid / G;
  const int g = static_cast<int>(rowid % G);
  const int s0 = part_off[pair], s1 = part_off[pair + 1];
  const int q = lane / LPR, c8 = lane % LPR;
  TG_GLOBAL float* dst = out + rowid * D + 8 * c8;
  auto ml = [&](int s, int k) { return ws_ml[(static_cast<int64_t>(s) * G + g) * 2 + k]; };
  auto accp = [&](int s) { return ws_acc + (static_cast<int64_t>(s) * G + g) * D + 8 * c8; };
  if (s1 - s0 <= 1) {
    if (q == 0) {
      if (s1 == s0) {
        st16(dst, 0.f, 0.f, 0.f, 0.f);
        st16(dst + 4, 0.f, 0.f, 0.f, 0.f);
      } else {
        const float inv = 1.f / ml(s0, 1);
        const f32x4_t x0 = *(const TG_GLOBAL f32x4_t*)(accp(s0));
        const f32x4_t x1 = *(const TG_GLOBAL f32x4_t*)(accp(s0) + 4);
        st16(dst, x0[0] * inv, x0[1] * inv, x0[2] * inv, x0[3] * inv);
        st16(dst + 4, x1[0] * inv, x1[1] * inv, x1[2] * inv, x1[3] * inv);
      }
    }
    return;
  }
  float mx = -INFINITY;
  for (int s = s0 + lane; s < s1; s += 64) mx = fmaxf(mx, ml(s, 0));
#pragma unroll
  for (int k = 1; k < 64; k <<= 1) mx = fmaxf(mx, __shfl_xor(mx, k, 64));
  float den = 0.f;
  for (int s = s0 + lane; s < s1; s += 64) den += __expf(ml(s, 0) - mx) * ml(s, 1);
#pragma unroll
  for (int k = 1; k < 64; k <<= 1) den += __shfl_xor(den, k, 64);
  float num[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s = s0 + q; s < s1; s += NG) {
    const float wgt = __expf(ml(s, 0) - mx);
    const f32x4_t x0 = *(const TG_GLOBAL f32x4_t*)(accp(s));
    const f32x4_t x1 = *(const TG_GLOBAL f32x4_t*)(accp(s) + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      num[e] = fmaf(wgt, x0[e], num[e]);
      num[e + 4] = fmaf(wgt, x1[e], num[e + 4]);
    }
  }
#pragma unroll
  for (int k = LPR; k < 64; k <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) num[e] += __shfl_xor(num[e], k, 64);
  if (q == 0) {
    const float inv = 1.f / den;
    st16(dst, num[0] * inv, num[1] * inv, num[2] * inv, num[3] * inv);
    st16(dst + 4, num[4] * inv, num[5] * inv, num[6] * inv, num[7] * inv);
  }
}

hipError_t launch_merge(const float* ws_acc, const float* ws_ml, const int32_t* part_off,
                        int32_t n_pairs, int32_t G, int32_t d, float* out, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(n_pairs) * G;
  if (rows == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((rows + 3) / 4));
  auto acc = (const TG_GLOBAL float*)(ws_acc);
  auto ml = (const TG_GLOBAL float*)(ws_ml);
  auto po = (const TG_GLOBAL int32_t*)(part_off);
  auto o = (TG_GLOBAL float*)(out);
  if (d == 128)
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(256), 0, s, acc, ml, po, n_pairs, G, o);
  else
    hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(256), 0, s, acc, ml, po, n_pairs, G, o);
  return hipGetLastError();
}

bool supported(int32_t d, int32_t G) {
  return (d == 64 || d == 128) && (G == 1 || G == 2 || G == 4 || G == 8);
}

}  // namespace
}  // namespace tg_dev

using namespace tg_dev;

extern "C" size_t tg_decode_workspace_bytes(int32_t n_slots, int32_t G, int32_t d) {
  if (n_slots < 0 || G < 1 || d < 1) return 0;
  return static_cast<size_t>(n_slots) * G * (d + 2) * sizeof(float);
}

extern "C" int tg_merge_partials(const float* workspace, int32_t n_slots, int32_t n_pairs, int32_t G,
                                 int32_t d, const int32_t* part_off, float* out, void* stream) {
  if (!supported(d, G) ) return TG_EUNSUPPORTED;
  if (n_slots < 0 || n_pairs < 0 || (n_pairs > 0 && (!part_off || !out)) || (n_slots > 0 && !workspace))
    return TG_EINVAL;
  const float* ws_ml = workspace + static_cast<int64_t>(n_slots) * G * d;
  hipError_t e = launch_merge(workspace, ws_ml, part_off, n_pairs, G, d, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TG_OK : TG_EDEVICE;
}

namespace {

int decode_split(const tg_cache* c, const tg_decode_args* a, void* stream, bool merge) {
  if (!c || !a) return TG_EINVAL;
  if (c->B < 1 || c->n_kv_heads < 1 || c->n_clusters < 1 || c->n_clusters > TG_MAX_CLUSTERS)
    return TG_EINVAL;
  if (a->n_q_heads < 1 || a->n_q_heads % c->n_kv_heads) return TG_EINVAL;
  const int32_t G = a->n_q_heads / c->n_kv_heads;
  const int32_t d = c->head_dim;
  if (!supported(d, G) || c->page_size != kPage || c->quant_block != kQBlock) return TG_EUNSUPPORTED;
  if (a->q_dtype != TG_Q_F32 && a->q_dtype != TG_Q_BF16) return TG_EINVAL;
  if (a->n_items < 0 || a->n_gitems < 0 || a->n_slots < 0 || !a->q || !c->cluster_of_head ||
      !c->slot_in_cluster || !c->len)
    return TG_EINVAL;
  if (merge && (!a->out || !a->part_off)) return TG_EINVAL;
  if (a->n_items > 0 && (!a->work || !a->workspace || a->n_slots == 0)) return TG_EINVAL;
  if (a->n_gitems > 0 && !a->gitems) return TG_EINVAL;
  if (a->workspace_bytes < tg_decode_workspace_bytes(a->n_slots, G, d)) return TG_EINVAL;
  for (int32_t cl = 0; cl < c->n_clusters; ++cl)
    for (int t = 0; t < 2; ++t) {
      if (c->stride[cl][t] < 0 || c->n_pages[cl][t] < 0) return TG_EINVAL;
      if (c->stride[cl][t] > 0 && (!c->bt[cl][t] || !c->pool[cl][t] || c->page_bytes[cl][t] <= 0))
        return TG_EINVAL;
      if (reinterpret_cast<uintptr_t>(c->pool[cl][t]) % 16) return TG_EINVAL;
    }
  SplitArgs s{};
  for (int32_t cl = 0; cl < c->n_clusters; ++cl)
    for (int t = 0; t < 2; ++t) {
      s.pool[cl][t] = (gptr)(c->pool[cl][t]);
      s.page_bytes[cl][t] = c->page_bytes[cl][t];
      s.bt[cl][t] = (const TG_GLOBAL int32_t*)(c->bt[cl][t]);
      s.stride[cl][t] = c->stride[cl][t];
    }
  s.len = (const TG_GLOBAL int32_t*)(c->len);
  s.n_fixed = (const TG_GLOBAL int32_t*)(c->n_fixed);
  s.n_kv_heads = c->n_kv_heads;
  s.cluster_of_head = (const TG_GLOBAL int32_t*)(c->cluster_of_head);
  s.slot_in_cluster = (const TG_GLOBAL int32_t*)(c->slot_in_cluster);
  s.q = (gptr)(a->q);
  s.work = (const TG_GLOBAL int32_t*)(a->work);
  s.ws_acc = (TG_GLOBAL float*)(a->workspace);
  s.ws_ml = (TG_GLOBAL float*)(a->workspace + static_cast<int64_t>(a->n_slots) * G * d);
  s.n_items = a->n_items;
  s.gitems = (const TG_GLOBAL int32_t*)(a->gitems);
  s.n_gitems = a->n_gitems;
  s.n_q_heads = a->n_q_heads;
  const float scale = a->sm_scale != 0.f ? a->sm_scale : 1.f / std::sqrt(static_cast<float>(d));
  s.scale_log2 = scale * kLog2e;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // one launch per tier present in the cache (a tier whose tables are all
  // empty has no items)
  bool has_i8 = false, has_bf = false;
  for (int32_t cl = 0; cl < c->n_clusters; ++cl) {
    has_i8 |= c->stride[cl][TG_TIER_I8] > 0;
    has_bf |= c->stride[cl][TG_TIER_BF16] > 0;
  }
  const bool qf32 = a->q_dtype == TG_Q_F32;
  hipError_t e = hipSuccess;
  if (has_i8) e = launch_split_i8(s, d, G, qf32, st);
  if (e == hipSuccess && has_bf) e = launch_split_bf16(s, d, G, qf32, st);
  if (e != hipSuccess) return TG_EDEVICE;
  if (!merge) return TG_OK;
  e = launch_merge(a->workspace, a->workspace + static_cast<int64_t>(a->n_slots) * G * d, a->part_off,
                   c->B * c->n_kv_heads, G, d, a->out, st);
  return e == hipSuccess ? TG_OK : TG_EDEVICE;
}

}  // namespace

extern "C" int tg_decode_attn(const tg_cache* c, const tg_decode_args* a, void* stream) {
  return decode_split(c, a, stream, true);
}

extern "C" int tg_decode_split(const tg_cache* c, const tg_decode_args* a, void* stream) {
  return decode_split(c, a, stream, false);
}
