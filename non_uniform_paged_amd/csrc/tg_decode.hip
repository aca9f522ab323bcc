// Decode attention over the ragged, tiered, paged cache (gfx950): the C-ABI
// entry points of the decode step and the log-sum-exp merge kernel.
//
// tg_decode_split launches the split kernel (tg_split.hip, with the work
// items of tg_item_bf16.h and tg_item_i8.h), which writes, per plan item, the
// online-normaliser partial (m, l, acc) of the item's rows.  tg_merge_partials
// combines the partials of each (r, h) with the weights e^{m_s - M} (CAP survey
// page, section 2.4.3 "Distributed acceleration", online normaliser [88]) and
// writes o in fp32.  tg_decode_attn is the two in sequence.

#include <cmath>
#include <algorithm>
#include <cstdint>
#include <map>
#include <mutex>
#include <vector>

#include "tg_device.h"

namespace tg_dev {
namespace {

// ---------------------------------------------------------------- merge kernel
// WPR wavefronts per (pair, g) row.  Lanes form NG = 64/(D/8) groups of D/8
// lanes; each lane owns 8 channels.  Group q of wave w takes slots
// s0 + (w*NG + q), stepping by WPR*NG, and keeps its own running maximum:
//   m <- max(m, m_s);  den = sum e^{m_s - m} l_s;  num = sum e^{m_s - m} acc_s
// rescaling den and num when m grows, so every slot is read once.  The groups
// (then the waves, through LDS) are folded with the same rescaling, and
// o = num / den.
template <int D, int WPR>
__global__ __launch_bounds__(256) void merge_kernel(const TG_GLOBAL float* __restrict__ ws_acc,
                                                    const TG_GLOBAL float* __restrict__ ws_ml,
                                                    const TG_GLOBAL int32_t* __restrict__ part_off,
                                                    int32_t n_pairs, int32_t G,
                                                    TG_GLOBAL float* __restrict__ out) {
  constexpr int LPR = D / 8;    // lanes per channel row
  constexpr int NG = 64 / LPR;  // slot groups per wave
  constexpr int RPB = 4 / WPR;  // rows per 256-thread block
  __shared__ float red[WPR > 1 ? 4 : 1][WPR > 1 ? LPR : 1][10];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int w = wave % WPR;
  const int64_t rowid = static_cast<int64_t>(blockIdx.x) * RPB + wave / WPR;
  if (rowid >= static_cast<int64_t>(n_pairs) * G) return;  // uniform per block when WPR > 1
  const int64_t pair = rowid / G;
  const int g = static_cast<int>(rowid % G);
  const int s0 = part_off[pair], s1 = part_off[pair + 1];
  const int q = lane / LPR, c8 = lane % LPR;
  TG_GLOBAL float* dst = out + rowid * D + 8 * c8;
  float m = -INFINITY, den = 0.f;
  float num[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](float ms, float ls, const f32x4_t& x0, const f32x4_t& x1) {
    if (ms == -INFINITY) return;  // a partial with no rows
    if (ms > m) {
      const float sc = __expf(m - ms);
      den *= sc;
#pragma unroll
      for (int e = 0; e < 8; ++e) num[e] *= sc;
      m = ms;
    }
    const float wgt = __expf(ms - m);
    den = fmaf(wgt, ls, den);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      num[e] = fmaf(wgt, x0[e], num[e]);
      num[e + 4] = fmaf(wgt, x1[e], num[e + 4]);
    }
  };
  constexpr int STEP = WPR * NG;
  // U slots an iteration (four with many slots a pair), all loaded before
  // any is folded in; folded in slot order
  constexpr int U = WPR > 1 ? 4 : 2;
  for (int s = s0 + w * NG + q; s < s1; s += U * STEP) {
    float ms[U], ls[U];
    f32x4_t x0[U], x1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {  // past s1: slot s again, not folded
      const int64_t b = static_cast<int64_t>(s + u * STEP < s1 ? s + u * STEP : s) * G + g;
      ms[u] = ws_ml[b * 2 + 0];
      ls[u] = ws_ml[b * 2 + 1];
      x0[u] = *(const TG_GLOBAL f32x4_t*)(ws_acc + b * D + 8 * c8);
      x1[u] = *(const TG_GLOBAL f32x4_t*)(ws_acc + b * D + 8 * c8 + 4);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (s + u * STEP < s1) add(ms[u], ls[u], x0[u], x1[u]);
  }
  auto fold = [&](float mo, float dno, const float* nmo) {
    const float mn = fmaxf(m, mo);
    const float a = m == -INFINITY ? 0.f : __expf(m - mn);
    const float b = mo == -INFINITY ? 0.f : __expf(mo - mn);
    den = a * den + b * dno;
#pragma unroll
    for (int e = 0; e < 8; ++e) num[e] = a * num[e] + b * nmo[e];
    m = mn;
  };
#pragma unroll
  for (int k = LPR; k < 64; k <<= 1) {
    float nmo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) nmo[e] = __shfl_xor(num[e], k, 64);
    fold(__shfl_xor(m, k, 64), __shfl_xor(den, k, 64), nmo);
  }
  if constexpr (WPR > 1) {
    if (q == 0) {
      float* r = red[w][c8];
      r[0] = m;
      r[1] = den;
#pragma unroll
      for (int e = 0; e < 8; ++e) r[2 + e] = num[e];
    }
    __syncthreads();
    if (w != 0) return;
    for (int o = 1; o < WPR; ++o) {
      const float* r = red[o][c8];
      fold(r[0], r[1], r + 2);
    }
  }
  if (q == 0) {
    if (s1 == s0) {
      st16(dst, 0.f, 0.f, 0.f, 0.f);
      st16(dst + 4, 0.f, 0.f, 0.f, 0.f);
    } else {
      const float inv = 1.f / den;
      st16(dst, num[0] * inv, num[1] * inv, num[2] * inv, num[3] * inv);
      st16(dst + 4, num[4] * inv, num[5] * inv, num[6] * inv, num[7] * inv);
    }
  }
}

template <int D>
void launch_merge_d(const TG_GLOBAL float* acc, const TG_GLOBAL float* ml, const TG_GLOBAL int32_t* po,
                    int32_t n_pairs, int32_t G, TG_GLOBAL float* o, int64_t n_slots, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(n_pairs) * G;
  // many slots per pair (long sequences split into many items): a block of
  // four waves per row; otherwise one wave per row
  if (n_slots >= 16 * static_cast<int64_t>(n_pairs))
    hipLaunchKernelGGL((merge_kernel<D, 4>), dim3(static_cast<unsigned>(rows)), dim3(256), 0, s, acc, ml,
                       po, n_pairs, G, o);
  else
    hipLaunchKernelGGL((merge_kernel<D, 1>), dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, s,
                       acc, ml, po, n_pairs, G, o);
}

hipError_t launch_merge(const float* ws_acc, const float* ws_ml, const int32_t* part_off,
                        int32_t n_pairs, int32_t G, int32_t d, float* out, int64_t n_slots, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(n_pairs) * G;
  if (rows == 0) return hipSuccess;
  auto acc = (const TG_GLOBAL float*)(ws_acc);
  auto ml = (const TG_GLOBAL float*)(ws_ml);
  auto po = (const TG_GLOBAL int32_t*)(part_off);
  auto o = (TG_GLOBAL float*)(out);
  if (d == 128)
    launch_merge_d<128>(acc, ml, po, n_pairs, G, o, n_slots, s);
  else
    launch_merge_d<64>(acc, ml, po, n_pairs, G, o, n_slots, s);
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
  hipError_t e =
      launch_merge(workspace, ws_ml, part_off, n_pairs, G, d, out, n_slots, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TG_OK : TG_EDEVICE;
}

namespace {

// Code width of the slow tier (0 in an older cache struct means 8).
int old_bits_of(const tg_cache* c) { return c->old_bits == 4 ? 4 : 8; }

// Validates a decode call and fills the split-kernel arguments.
int make_split_args(const tg_cache* c, const tg_decode_args* a, bool merge, SplitArgs* out, int32_t* G_out) {
  if (!c || !a) return TG_EINVAL;
  if (c->B < 1 || c->n_kv_heads < 1 || c->n_clusters < 1 || c->n_clusters > TG_MAX_CLUSTERS)
    return TG_EINVAL;
  if (a->n_q_heads < 1 || a->n_q_heads % c->n_kv_heads) return TG_EINVAL;
  const int32_t G = a->n_q_heads / c->n_kv_heads;
  const int32_t d = c->head_dim;
  if (!supported(d, G) || c->page_size != kPage || c->quant_block != kQBlock) return TG_EUNSUPPORTED;
  if (a->q_dtype != TG_Q_F32 && a->q_dtype != TG_Q_BF16) return TG_EINVAL;
  if (!(a->sm_scale >= 0.f) || !std::isfinite(a->sm_scale)) return TG_EINVAL;
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
      if (c->page_bytes[cl][t] > INT32_MAX) return TG_EUNSUPPORTED;
      if (reinterpret_cast<uintptr_t>(c->pool[cl][t]) % 16) return TG_EINVAL;
    }
  if (c->ring != nullptr && c->bf_base == nullptr) return TG_EINVAL;
  if (c->old_bits != 0 && c->old_bits != 8 && c->old_bits != 4) return TG_EINVAL;
  if (c->old_bits == 4 && d != 128) return TG_EUNSUPPORTED;
  if (!layout_flags_valid(c)) return TG_EINVAL;
  SplitArgs& s = *out;
  s = SplitArgs{};
  for (int32_t cl = 0; cl < c->n_clusters; ++cl)
    for (int t = 0; t < 2; ++t) {
      int64_t page_stride = 0, head_stride = 0;
      pool_strides(c, cl, t, &page_stride, &head_stride);
      if (c->stride[cl][t] > 0 && c->page_bytes[cl][t] % head_slot_bytes(c, t)) return TG_EINVAL;
      s.pool[cl][t] = (gptr)(c->pool[cl][t]);
      s.page_bytes[cl][t] = static_cast<int32_t>(page_stride);
      s.head_stride[cl][t] = head_stride;
      s.bt[cl][t] = (const TG_GLOBAL int32_t*)(c->bt[cl][t]);
      s.stride[cl][t] = c->stride[cl][t];
    }
  s.len = (const TG_GLOBAL int32_t*)(c->len);
  s.ring = (const TG_GLOBAL int32_t*)(c->ring);
  s.bf_base = (const TG_GLOBAL int32_t*)(c->bf_base);
  s.n_clusters = c->n_clusters;
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
  *G_out = G;
  return TG_OK;
}

int decode_split(const tg_cache* c, const tg_decode_args* a, void* stream, bool merge, hipEvent_t e0 = nullptr,
                 hipEvent_t e1 = nullptr) {
  SplitArgs s;
  int32_t G = 0;
  const int st_code = make_split_args(c, a, merge, &s, &G);
  if (st_code) return st_code;
  const int32_t d = c->head_dim;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // one launch over both tiers when the cache has INT8 pages
  bool has_i8 = false;
  for (int32_t cl = 0; cl < c->n_clusters; ++cl) has_i8 |= c->stride[cl][TG_TIER_I8] > 0;
  hipError_t e = launch_split(s, d, G, a->q_dtype == TG_Q_F32, has_i8, old_bits_of(c), st, e0, e1);
  if (e != hipSuccess) return TG_EDEVICE;
  if (!merge) return TG_OK;
  e = launch_merge(a->workspace, a->workspace + static_cast<int64_t>(a->n_slots) * G * d, a->part_off,
                   c->B * c->n_kv_heads, G, d, a->out, a->n_slots, st);
  return e == hipSuccess ? TG_OK : TG_EDEVICE;
}

// ---------------------------------------------------------------- host-DRAM INT8 tier
// INT8 pages of request r in cluster c: the leading non-negative entries of
// its host table row.
int64_t i8_pages_of(const tg_tables* t, int32_t c, int32_t r) {
  const int32_t stride = t->stride[c][TG_TIER_I8];
  if (stride == 0) return 0;
  const int32_t* row = t->bt[c][TG_TIER_I8] + static_cast<int64_t>(r) * stride;
  int64_t n = 0;
  while (n < stride && row[n] >= 0) ++n;
  return n;
}

// Staging slot layout: per cluster, room for the INT8 pages of the largest
// request, clusters one after another; two slots.
size_t slot_layout(const tg_cache* c, const tg_tables* t, size_t* off /*[C]*/) {
  size_t at = 0;
  for (int32_t cl = 0; cl < c->n_clusters; ++cl) {
    int64_t most = 0;
    for (int32_t r = 0; r < c->B; ++r) most = std::max(most, i8_pages_of(t, cl, r));
    off[cl] = at;
    at += static_cast<size_t>(most) * static_cast<size_t>(c->page_bytes[cl][TG_TIER_I8]);
    at = (at + 255) & ~static_cast<size_t>(255);
  }
  return at;
}

// The copy stream and events of the streamed decode, one set per device,
// created on a device's first call and kept until the process ends.  Calls on
// one device must not overlap in time (they share the set); calls on
// different devices may.
struct StreamState {
  hipStream_t copy = nullptr;
  std::vector<hipEvent_t> events;
};

int stream_state(int32_t n_events, StreamState** out) {
  static std::mutex mu;
  static std::map<int, StreamState> states;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TG_EDEVICE;
  std::lock_guard<std::mutex> lock(mu);
  StreamState& state = states[dev];
  if (state.copy == nullptr &&
      hipStreamCreateWithFlags(&state.copy, hipStreamNonBlocking) != hipSuccess)
    return TG_EDEVICE;
  while (static_cast<int32_t>(state.events.size()) < n_events) {
    hipEvent_t e;
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return TG_EDEVICE;
    state.events.push_back(e);
  }
  *out = &state;
  return TG_OK;
}

}  // namespace

extern "C" size_t tg_stream_staging_bytes(const tg_cache* c, const tg_tables* t) {
  if (!c || !t || c->n_clusters < 1 || c->n_clusters > TG_MAX_CLUSTERS) return 0;
  size_t off[TG_MAX_CLUSTERS];
  return 2 * slot_layout(c, t, off);
}

extern "C" int tg_decode_streamed(const tg_cache* c, const tg_tables* t, const tg_decode_args* a,
                                  const int32_t* chunk_off, void* staging, size_t staging_bytes,
                                  void* stream) {
  SplitArgs s;
  int32_t G = 0;
  int code = make_split_args(c, a, true, &s, &G);
  if (code) return code;
  if (!t || !chunk_off || !staging) return TG_EINVAL;
  const int32_t B = c->B, d = c->head_dim;
  for (int32_t cl = 0; cl < c->n_clusters; ++cl)
    if (c->head_major[cl][TG_TIER_I8]) return TG_EUNSUPPORTED;  // staged pages are copied whole
  if (chunk_off[0] < 0 || chunk_off[B] != a->n_items) return TG_EINVAL;
  for (int32_t r = 0; r < B; ++r)
    if (chunk_off[r + 1] < chunk_off[r]) return TG_EINVAL;
  size_t off[TG_MAX_CLUSTERS];
  const size_t slot_bytes = slot_layout(c, t, off);
  if (staging_bytes < 2 * slot_bytes || reinterpret_cast<uintptr_t>(staging) % 256) return TG_EINVAL;
  StreamState* ss = nullptr;
  if ((code = stream_state(2 * B + 1, &ss))) return code;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipEvent_t ev_start = ss->events[2 * B];
  const bool qf32 = a->q_dtype == TG_Q_F32;
  // the staging slots are free once earlier work on the compute stream is done
  if (hipEventRecord(ev_start, st) != hipSuccess || hipStreamWaitEvent(ss->copy, ev_start, 0) != hipSuccess)
    return TG_EDEVICE;
  // bf16 items (HBM-resident pages) first: they run while the first pages cross
  SplitArgs sb = s;
  sb.n_items = chunk_off[0];
  if (launch_split(sb, d, G, qf32, false, 8, st) != hipSuccess) return TG_EDEVICE;
  char* stage = static_cast<char*>(staging);
  for (int32_t r = 0; r < B; ++r) {
    char* slot = stage + (r % 2) * slot_bytes;
    hipEvent_t copied = ss->events[2 * r], done = ss->events[2 * r + 1];
    if (r >= 2 && hipStreamWaitEvent(ss->copy, ss->events[2 * (r - 2) + 1], 0) != hipSuccess) return TG_EDEVICE;
    for (int32_t cl = 0; cl < c->n_clusters; ++cl) {
      const int64_t n = i8_pages_of(t, cl, r);
      const int32_t* row = t->bt[cl][TG_TIER_I8] + static_cast<int64_t>(r) * t->stride[cl][TG_TIER_I8];
      const size_t pb = static_cast<size_t>(c->page_bytes[cl][TG_TIER_I8]);
      const char* host = static_cast<const char*>(c->pool[cl][TG_TIER_I8]);
      for (int64_t j0 = 0; j0 < n;) {  // one copy per run of consecutive page ids
        int64_t j1 = j0 + 1;
        while (j1 < n && row[j1] == row[j1 - 1] + 1) ++j1;
        if (hipMemcpyAsync(slot + off[cl] + j0 * pb, host + static_cast<size_t>(row[j0]) * pb, (j1 - j0) * pb,
                           hipMemcpyHostToDevice, ss->copy) != hipSuccess)
          return TG_EDEVICE;
        j0 = j1;
      }
    }
    if (hipEventRecord(copied, ss->copy) != hipSuccess || hipStreamWaitEvent(st, copied, 0) != hipSuccess)
      return TG_EDEVICE;
    SplitArgs sr = s;
    for (int32_t cl = 0; cl < c->n_clusters; ++cl) {
      sr.pool[cl][TG_TIER_I8] = (gptr)(slot + off[cl]);
      sr.bt[cl][TG_TIER_I8] = nullptr;  // block j of the request is staged page j
    }
    sr.work = s.work + static_cast<int64_t>(chunk_off[r]) * 6;
    sr.n_items = chunk_off[r + 1] - chunk_off[r];
    sr.n_gitems = 0;  // INT8 items only: no cooperative workgroups
    if (launch_split(sr, d, G, qf32, true, old_bits_of(c), st) != hipSuccess) return TG_EDEVICE;
    if (hipEventRecord(done, st) != hipSuccess) return TG_EDEVICE;
  }
  const hipError_t e = launch_merge(a->workspace, a->workspace + static_cast<int64_t>(a->n_slots) * G * d,
                                    a->part_off, B * c->n_kv_heads, G, d, a->out, a->n_slots, st);
  return e == hipSuccess ? TG_OK : TG_EDEVICE;
}

extern "C" int tg_decode_attn(const tg_cache* c, const tg_decode_args* a, void* stream) {
  return decode_split(c, a, stream, true);
}

// ---------------------------------------------------------------- decode without allocation
// Partials of tg_decode_attn_noalloc: a fixed device array of the library.
// Each device the library runs on holds its own copy until the process ends.
// Host code never passes `scratch` itself to a kernel (in host code the name
// is a stand-in, not a device address): it takes the address that
// hipGetSymbolAddress gives on each device, once per device.
static __device__ __align__(256) char scratch[TG_NOALLOC_SCRATCH_BYTES];

namespace {

int scratch_address(void** out) {
  static std::mutex mu;
  static std::map<int, void*> addr;  // device -> its copy of `scratch`
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TG_EDEVICE;
  std::lock_guard<std::mutex> lock(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return TG_EDEVICE;
    it = addr.emplace(dev, p).first;
  }
  *out = it->second;
  return TG_OK;
}

}  // namespace

extern "C" int tg_decode_attn_noalloc(const tg_cache* c, const tg_decode_args* a, void* stream) {
  if (!c || !a || c->n_kv_heads < 1 || a->n_q_heads < 1 || a->n_q_heads % c->n_kv_heads || a->n_slots < 0)
    return TG_EINVAL;
  const size_t need = tg_decode_workspace_bytes(a->n_slots, a->n_q_heads / c->n_kv_heads, c->head_dim);
  if (need > TG_NOALLOC_SCRATCH_BYTES) return TG_EOVERFLOW;
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st) return st;
  tg_decode_args b = *a;
  b.workspace = static_cast<float*>(ws);
  b.workspace_bytes = TG_NOALLOC_SCRATCH_BYTES;
  return decode_split(c, &b, stream, true);
}

extern "C" int tg_decode_split(const tg_cache* c, const tg_decode_args* a, void* stream) {
  return decode_split(c, a, stream, false);
}

extern "C" int tg_decode_split_timed(const tg_cache* c, const tg_decode_args* a, void* start_event,
                                     void* stop_event, void* stream) {
  if (!start_event || !stop_event) return TG_EINVAL;
  return decode_split(c, a, stream, false, static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event));
}
