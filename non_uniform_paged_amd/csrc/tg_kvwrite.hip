// Cache fill: scatter logical K/V rows into their ragged pages, quantising the
// oldest rows into the INT8 tier (gfx950).
//
// TTKV page (arXiv 2604.19769 explainer): "Tier Layout" (slow tier holds older
// KV states at INT8), "Tier Content" (the newest share stays high precision)
// and "Tier Interaction" (the slow tier is quantised block by block).  The
// quantiser is symmetric absmax per (64-token block, channel), computed in
// fp32:  s = fp16_rne(absmax / 127) (+inf saturates to 65504),
//        q8 = s > 0 ? clamp(rint_even(x / s), -127, 127) : 0.
// Page layouts are the ones documented in include/tg.h (the bf16 one is
// arranged so that each 1 KiB wave load in the decode kernel is one MFMA
// operand).

#include <hip/hip_runtime.h>

#include <cstdint>

#include "tg.h"
#include "tg_layout.h"

namespace {

constexpr int kPage = 16;
constexpr int kQBlock = 64;

struct WriteArgs {
  char* pool[TG_MAX_CLUSTERS][2];
  int64_t page_bytes[TG_MAX_CLUSTERS][2];   // between page ids
  int64_t head_stride[TG_MAX_CLUSTERS][2];  // between the head slots of a page
  const int32_t* bt[TG_MAX_CLUSTERS][2];
  int32_t stride[TG_MAX_CLUSTERS][2];
  const int32_t* cluster_of_head;
  const int32_t* slot_in_cluster;
  const int32_t* len;
  const uint16_t* rows;
  const int32_t* index;
  const int64_t* offsets;
  int32_t H;
  int32_t pairs;  // B * H; the grid's y dimension strides over them
};

// One thread per 8 channels of one bf16-tier row; 256 threads = 256/(D/8) rows.
template <int D>
__device__ __forceinline__ void write_bf16_rows(const WriteArgs& a, int rh) {
  constexpr int LPR = D / 8;
  constexpr int RPB = 256 / LPR;
  const int r = rh / a.H, h = rh % a.H;
  const int n_i8 = a.len[2 * rh], n_bf = a.len[2 * rh + 1];
  const int u = blockIdx.x * RPB + threadIdx.x / LPR;
  const int c8 = threadIdx.x % LPR;
  if (u >= n_bf) return;
  const int cl = a.cluster_of_head[h], hs = a.slot_in_cluster[h];
  const int64_t src_row = a.index[a.offsets[rh] + n_i8 + u];
  const uint16_t* src = a.rows + src_row * 2 * D + 8 * c8;
  const int pid = a.bt[cl][TG_TIER_BF16][static_cast<int64_t>(r) * a.stride[cl][TG_TIER_BF16] + u / kPage];
  char* head = a.pool[cl][TG_TIER_BF16] + static_cast<int64_t>(pid) * a.page_bytes[cl][TG_TIER_BF16] +
               static_cast<int64_t>(hs) * a.head_stride[cl][TG_TIER_BF16];
  const int t = u % kPage;
  // K: channels 8c8..8c8+7 of row t are one contiguous 16-byte group
  *reinterpret_cast<uint4*>(head + (((c8 >> 2) * 64 + (c8 & 3) * 16 + t) * 16)) =
      *reinterpret_cast<const uint4*>(src);
  // V: channel d of row t sits with the same channel of rows t^1..t^3
  uint16_t* vblk = reinterpret_cast<uint16_t*>(head + kPage * D * 2);
  const uint16_t* vsrc = src + D;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int d = 8 * c8 + e;
    const int off = (((d >> 5) * 64 + (t >> 2) * 16 + (d & 15)) * 16 + ((d >> 4) & 1) * 8 + (t & 3) * 2) / 2;
    vblk[off] = vsrc[e];
  }
}
template <int D>
__global__ __launch_bounds__(256) void write_bf16_kernel(WriteArgs a) {
  for (int rh = blockIdx.y; rh < a.pairs; rh += gridDim.y) write_bf16_rows<D>(a, rh);
}

// One block of 2*D threads per (r, h, 64-row INT8 block): thread = (K|V, channel).
template <int D>
__device__ __forceinline__ void write_i8_block(const WriteArgs& a, int rh) {
  const int r = rh / a.H, h = rh % a.H;
  const int n_i8 = a.len[2 * rh];
  const int b = blockIdx.x;
  if (b * kQBlock >= n_i8) return;
  const int kv = threadIdx.x / D, ch = threadIdx.x % D;
  const int cl = a.cluster_of_head[h], hs = a.slot_in_cluster[h];
  const int64_t base = a.offsets[rh] + static_cast<int64_t>(b) * kQBlock;
  float amax = 0.f;
  for (int t = 0; t < kQBlock; ++t) {
    const int64_t row = a.index[base + t];
    const float x = __uint_as_float(static_cast<uint32_t>(a.rows[row * 2 * D + kv * D + ch]) << 16);
    amax = fmaxf(amax, fabsf(x));
  }
  _Float16 s16 = static_cast<_Float16>(amax / 127.0f);
  if (__builtin_isinf(static_cast<float>(s16))) s16 = static_cast<_Float16>(65504.0f);
  const float sf = static_cast<float>(s16);
  const int pid = a.bt[cl][TG_TIER_I8][static_cast<int64_t>(r) * a.stride[cl][TG_TIER_I8] + b];
  char* head = a.pool[cl][TG_TIER_I8] + static_cast<int64_t>(pid) * a.page_bytes[cl][TG_TIER_I8] +
               static_cast<int64_t>(hs) * a.head_stride[cl][TG_TIER_I8];
  int8_t* codes = reinterpret_cast<int8_t*>(head + kv * kQBlock * D);
  constexpr int NL = D / 64;
  for (int t = 0; t < kQBlock; ++t) {
    const int64_t row = a.index[base + t];
    const float x = __uint_as_float(static_cast<uint32_t>(a.rows[row * 2 * D + kv * D + ch]) << 16);
    int q = 0;
    if (sf > 0.f) q = static_cast<int>(fminf(fmaxf(__builtin_rintf(x / sf), -127.f), 127.f));
    // matrix-core operand order of the decode kernel (include/tg.h)
    const int c = ch;
    const int off = kv == 0
        ? ((t >> 4) * NL + (c >> 6)) * 1024 + (((c >> 3) & 3) * 16 + (t & 15)) * 16 + ((c >> 5) & 1) * 8 + (c & 7)
        : ((t >> 4) * NL + (c >> 6)) * 1024 + (((t >> 2) & 3) * 16 + (c & 15)) * 16 + ((c >> 4) & 3) * 4 + (t & 3);
    codes[off] = static_cast<int8_t>(q);
  }
  reinterpret_cast<_Float16*>(head + 2 * kQBlock * D + kv * D * 2)[ch] = s16;
}
template <int D>
__global__ __launch_bounds__(2 * D) void write_i8_kernel(WriteArgs a) {
  for (int rh = blockIdx.y; rh < a.pairs; rh += gridDim.y) write_i8_block<D>(a, rh);
}

// Packs the codes of one head's block (LDS, int8 [2][kQBlock][D], K then V,
// values in [-7, 7]) into the INT4 page layout of include/tg.h at `head`:
// 32-bit words, nibble p = bits 4p..4p+3 holding u = q4 + 8.  Called by all
// 2*D threads of the workgroup after the codes are in LDS.
template <int D>
__device__ void store_i4_words(const int8_t (*codes)[kQBlock][D], char* head) {
  constexpr int WORDS = kQBlock * D / 8;  // per K (and per V)
  for (int wi = threadIdx.x; wi < 2 * WORDS; wi += 2 * D) {
    const int kv = wi / WORDS, x = wi % WORDS;
    const int g = x / 256, l = (x % 256) / 4, m = x % 4;
    uint32_t word = 0;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      int t, c;
      if (kv == 0) {  // K: row 16g + l%16, channel 32m + 8(l/16) + e
        t = 16 * g + (l & 15);
        c = 32 * m + 8 * (l >> 4) + (((p & 3) << 1) | (p >> 2));
      } else {        // V: rows 16g + 4(l/16) + i, channel l%16 of tile 2m + q
        t = 16 * g + 4 * (l >> 4) + (((p & 1) << 1) | (p >> 2));
        c = (l & 15) + 16 * (2 * m + ((p >> 1) & 1));
      }
      word |= static_cast<uint32_t>(codes[kv][t][c] + 8) << (4 * p);
    }
    *reinterpret_cast<uint32_t*>(head + kv * (kQBlock * D / 2) + x * 4) = word;
  }
}

// One block of 2*D threads per (r, h, 64-row block), thread = (K|V, channel):
// the INT4 slow tier (codes in [-7, 7], scale absmax / 7).
template <int D>
__device__ __forceinline__ void write_i4_block(const WriteArgs& a, int rh, int8_t (*codes)[kQBlock][D]) {
  const int r = rh / a.H, h = rh % a.H;
  const int n_i8 = a.len[2 * rh];
  const int b = blockIdx.x;
  if (b * kQBlock >= n_i8) return;
  const int kv = threadIdx.x / D, ch = threadIdx.x % D;
  const int cl = a.cluster_of_head[h], hs = a.slot_in_cluster[h];
  const int64_t base = a.offsets[rh] + static_cast<int64_t>(b) * kQBlock;
  float amax = 0.f;
  for (int t = 0; t < kQBlock; ++t) {
    const int64_t row = a.index[base + t];
    amax = fmaxf(amax, fabsf(__uint_as_float(static_cast<uint32_t>(a.rows[row * 2 * D + kv * D + ch]) << 16)));
  }
  _Float16 s16 = static_cast<_Float16>(amax / 7.0f);
  if (__builtin_isinf(static_cast<float>(s16))) s16 = static_cast<_Float16>(65504.0f);
  const float sf = static_cast<float>(s16);
  for (int t = 0; t < kQBlock; ++t) {
    const int64_t row = a.index[base + t];
    const float x = __uint_as_float(static_cast<uint32_t>(a.rows[row * 2 * D + kv * D + ch]) << 16);
    codes[kv][t][ch] = sf > 0.f ? static_cast<int8_t>(fminf(fmaxf(__builtin_rintf(x / sf), -7.f), 7.f)) : 0;
  }
  const int pid = a.bt[cl][TG_TIER_I8][static_cast<int64_t>(r) * a.stride[cl][TG_TIER_I8] + b];
  char* head = a.pool[cl][TG_TIER_I8] + static_cast<int64_t>(pid) * a.page_bytes[cl][TG_TIER_I8] +
               static_cast<int64_t>(hs) * a.head_stride[cl][TG_TIER_I8];
  reinterpret_cast<_Float16*>(head + kQBlock * D + kv * D * 2)[ch] = s16;
  __syncthreads();
  store_i4_words<D>(codes, head);
  __syncthreads();  // the codes are read before the next pair overwrites them
}
template <int D>
__global__ __launch_bounds__(2 * D) void write_i4_kernel(WriteArgs a) {
  __shared__ int8_t codes[2][kQBlock][D];
  // (rh, blockIdx.x) is uniform over the workgroup, so are the early exits
  // of write_i4_block and its barriers
  for (int rh = blockIdx.y; rh < a.pairs; rh += gridDim.y) write_i4_block<D>(a, rh, codes);
}

// ---------------------------------------------------------------- decode-step append
struct AppendArgs {
  char* pool[TG_MAX_CLUSTERS][2];
  int64_t page_bytes[TG_MAX_CLUSTERS][2];   // between page ids
  int64_t head_stride[TG_MAX_CLUSTERS][2];  // between the head slots of a page
  const int32_t* bt[TG_MAX_CLUSTERS][2];
  int32_t stride[TG_MAX_CLUSTERS][2];
  const int32_t* cluster_of_head;
  const int32_t* slot_in_cluster;
  const int32_t* ring;
  int32_t* len;
  int32_t* bf_base;
  const uint16_t* rows;
  int32_t* status;
  int32_t H, C, recent_ppm;
};

__device__ __forceinline__ int64_t i8_rows(int64_t L, int64_t recent_ppm) {
  const int64_t recent = (L * recent_ppm + 999999) / 1000000;
  return ((L - recent) / kQBlock) * kQBlock;
}

// Byte offset of (row t, channel c) inside a head's bf16 page (K, or V at
// +2*kPage*D), the layout of include/tg.h.
template <int D>
__device__ __forceinline__ int bf16_offset(int kv, int t, int c) {
  return kv == 0 ? (((c >> 5) * 64 + ((c >> 3) & 3) * 16 + t) * 16 + (c & 7) * 2)
                 : 2 * kPage * D + (((c >> 5) * 64 + (t >> 2) * 16 + (c & 15)) * 16 + ((c >> 4) & 1) * 8 + (t & 3) * 2);
}

// One workgroup of 2*D threads per (r, h), thread = (K|V, channel): writes
// the new row as the newest bf16 row (ring row base + n_bf) and, when the
// tier split of the new length moves the INT8 boundary, quantises the oldest
// kQBlock bf16 rows into INT8 block n_i8 / kQBlock and advances the ring.
template <int D, int BITS>
__global__ __launch_bounds__(2 * D) void append_kernel(AppendArgs a) {
  __shared__ int8_t lcodes[BITS == 4 ? 2 : 1][BITS == 4 ? kQBlock : 1][BITS == 4 ? D : 1];
  const int rh = blockIdx.x;
  const int r = rh / a.H, h = rh % a.H;
  const int kv = threadIdx.x / D, ch = threadIdx.x % D;
  const int cl = a.cluster_of_head[h], hs = a.slot_in_cluster[h];
  // Thread 0 reads the lengths and the ring base into LDS and every thread
  // takes them from there after the barrier: thread 0 updates them in memory
  // at the end of the step, and a wavefront reading memory itself could see
  // the new values (no order holds between wavefronts without the barrier).
  __shared__ int state[3];
  if (threadIdx.x == 0) {
    state[0] = a.len[2 * rh];
    state[1] = a.len[2 * rh + 1];
    state[2] = a.bf_base[rh];
  }
  __syncthreads();
  const int n_i8 = state[0], n_bf = state[1];
  const int base = state[2];
  const int ring_rows = a.ring[r * a.C + cl] * kPage;
  const bool age = i8_rows(static_cast<int64_t>(n_i8) + n_bf + 1, a.recent_ppm) > n_i8;
  const int blk = n_i8 / kQBlock;
  const int32_t* bt_i8 = a.bt[cl][TG_TIER_I8] + static_cast<int64_t>(r) * a.stride[cl][TG_TIER_I8];
  bool ok = n_bf + 1 <= ring_rows;
  if (age) ok = ok && blk < a.stride[cl][TG_TIER_I8] && bt_i8[blk] >= 0;
  if (!ok) {  // past the capacity reserved at admission: nothing is written
    if (threadIdx.x == 0 && a.status != nullptr) atomicOr(a.status, 1);
    return;
  }
  const int32_t* bt_bf = a.bt[cl][TG_TIER_BF16] + static_cast<int64_t>(r) * a.stride[cl][TG_TIER_BF16];
  auto bf_head = [&](int ring_row) {
    const int pid = bt_bf[ring_row / kPage];
    return a.pool[cl][TG_TIER_BF16] + static_cast<int64_t>(pid) * a.page_bytes[cl][TG_TIER_BF16] +
           static_cast<int64_t>(hs) * a.head_stride[cl][TG_TIER_BF16];
  };
  {
    const int pos = (base + n_bf) % ring_rows;
    *reinterpret_cast<uint16_t*>(bf_head(pos) + bf16_offset<D>(kv, pos % kPage, ch)) =
        a.rows[static_cast<int64_t>(rh) * 2 * D + kv * D + ch];
  }
  if (!age) {
    if (threadIdx.x == 0) a.len[2 * rh + 1] = n_bf + 1;
    return;
  }
  __syncthreads();  // the new row may be one of the rows that age
  auto value = [&](int t) {
    const int pos = (base + t) % ring_rows;
    const uint16_t x = *reinterpret_cast<const uint16_t*>(bf_head(pos) + bf16_offset<D>(kv, pos % kPage, ch));
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
  };
  constexpr float kQMax = BITS == 8 ? 127.f : 7.f;
  constexpr int CODE_BYTES = kQBlock * D * BITS / 8;
  float amax = 0.f;
  for (int t = 0; t < kQBlock; ++t) amax = fmaxf(amax, fabsf(value(t)));
  _Float16 s16 = static_cast<_Float16>(amax / kQMax);
  if (__builtin_isinf(static_cast<float>(s16))) s16 = static_cast<_Float16>(65504.0f);
  const float sf = static_cast<float>(s16);
  char* head = a.pool[cl][TG_TIER_I8] + static_cast<int64_t>(bt_i8[blk]) * a.page_bytes[cl][TG_TIER_I8] +
               static_cast<int64_t>(hs) * a.head_stride[cl][TG_TIER_I8];
  constexpr int NL = D / 64;
  for (int t = 0; t < kQBlock; ++t) {
    const float x = value(t);
    int q = 0;
    if (sf > 0.f) q = static_cast<int>(fminf(fmaxf(__builtin_rintf(x / sf), -kQMax), kQMax));
    if constexpr (BITS == 4) {
      lcodes[kv][t][ch] = static_cast<int8_t>(q);
    } else {
      const int c = ch;
      const int off = kv == 0
          ? ((t >> 4) * NL + (c >> 6)) * 1024 + (((c >> 3) & 3) * 16 + (t & 15)) * 16 + ((c >> 5) & 1) * 8 + (c & 7)
          : ((t >> 4) * NL + (c >> 6)) * 1024 + (((t >> 2) & 3) * 16 + (c & 15)) * 16 + ((c >> 4) & 3) * 4 + (t & 3);
      reinterpret_cast<int8_t*>(head + kv * CODE_BYTES)[off] = static_cast<int8_t>(q);
    }
  }
  reinterpret_cast<_Float16*>(head + 2 * CODE_BYTES + kv * D * 2)[ch] = s16;
  if constexpr (BITS == 4) {
    __syncthreads();
    store_i4_words<D>(lcodes, head);
  }
  if (threadIdx.x == 0) {
    a.len[2 * rh] = n_i8 + kQBlock;
    a.len[2 * rh + 1] = n_bf + 1 - kQBlock;
    a.bf_base[rh] = (base + kQBlock) % ring_rows;
  }
}

}  // namespace

extern "C" int tg_append_kv(const tg_cache* c, const uint16_t* rows, int32_t* status, void* stream) {
  if (!c || !rows || !c->len || !c->ring || !c->bf_base || !c->cluster_of_head || !c->slot_in_cluster)
    return TG_EINVAL;
  if (c->B < 1 || c->n_kv_heads < 1 || c->n_clusters < 1 || c->n_clusters > TG_MAX_CLUSTERS)
    return TG_EINVAL;
  if (c->head_dim != 64 && c->head_dim != 128) return TG_EUNSUPPORTED;
  if (c->page_size != kPage || c->quant_block != kQBlock) return TG_EUNSUPPORTED;
  if (c->recent_ppm < 0 || c->recent_ppm > 1000000) return TG_EINVAL;
  if (!tg_dev::layout_flags_valid(c)) return TG_EINVAL;
  AppendArgs a{};
  for (int32_t cl = 0; cl < c->n_clusters; ++cl)
    for (int t = 0; t < 2; ++t) {
      if (c->stride[cl][t] > 0 && (!c->bt[cl][t] || !c->pool[cl][t])) return TG_EINVAL;
      a.pool[cl][t] = static_cast<char*>(c->pool[cl][t]);
      if (c->stride[cl][t] > 0 && c->page_bytes[cl][t] % tg_dev::head_slot_bytes(c, t)) return TG_EINVAL;
      tg_dev::pool_strides(c, cl, t, &a.page_bytes[cl][t], &a.head_stride[cl][t]);
      a.bt[cl][t] = c->bt[cl][t];
      a.stride[cl][t] = c->stride[cl][t];
    }
  a.cluster_of_head = c->cluster_of_head;
  a.slot_in_cluster = c->slot_in_cluster;
  a.ring = c->ring;
  a.len = c->len;
  a.bf_base = c->bf_base;
  a.rows = rows;
  a.status = status;
  a.H = c->n_kv_heads;
  a.C = c->n_clusters;
  a.recent_ppm = c->recent_ppm;
  const int64_t pairs = static_cast<int64_t>(c->B) * c->n_kv_heads;
  if (pairs > INT32_MAX) return TG_EUNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(pairs));
  if (c->old_bits == 4) {
    if (c->head_dim != 128) return TG_EUNSUPPORTED;
    hipLaunchKernelGGL((append_kernel<128, 4>), grid, dim3(256), 0, st, a);
  } else if (c->head_dim == 128) {
    hipLaunchKernelGGL((append_kernel<128, 8>), grid, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((append_kernel<64, 8>), grid, dim3(128), 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? TG_OK : TG_EDEVICE;
}

extern "C" int tg_write_kv(const tg_cache* c, const uint16_t* rows, const int32_t* index,
                           const int64_t* offsets, void* stream) {
  if (!c || !rows || !index || !offsets || !c->len || !c->cluster_of_head || !c->slot_in_cluster)
    return TG_EINVAL;
  if (c->B < 1 || c->n_kv_heads < 1 || c->n_clusters < 1 || c->n_clusters > TG_MAX_CLUSTERS)
    return TG_EINVAL;
  if (c->head_dim != 64 && c->head_dim != 128) return TG_EUNSUPPORTED;
  if (c->page_size != kPage || c->quant_block != kQBlock) return TG_EUNSUPPORTED;
  if (!tg_dev::layout_flags_valid(c)) return TG_EINVAL;
  WriteArgs a{};
  int32_t max_bf = 0, max_i8 = 0;
  for (int32_t cl = 0; cl < c->n_clusters; ++cl)
    for (int t = 0; t < 2; ++t) {
      if (c->stride[cl][t] > 0 && (!c->bt[cl][t] || !c->pool[cl][t])) return TG_EINVAL;
      a.pool[cl][t] = static_cast<char*>(c->pool[cl][t]);
      if (c->stride[cl][t] > 0 && c->page_bytes[cl][t] % tg_dev::head_slot_bytes(c, t)) return TG_EINVAL;
      tg_dev::pool_strides(c, cl, t, &a.page_bytes[cl][t], &a.head_stride[cl][t]);
      a.bt[cl][t] = c->bt[cl][t];
      a.stride[cl][t] = c->stride[cl][t];
      if (t == TG_TIER_BF16) max_bf = c->stride[cl][t] > max_bf ? c->stride[cl][t] : max_bf;
      else max_i8 = c->stride[cl][t] > max_i8 ? c->stride[cl][t] : max_i8;
    }
  a.cluster_of_head = c->cluster_of_head;
  a.slot_in_cluster = c->slot_in_cluster;
  a.len = c->len;
  a.rows = rows;
  a.index = index;
  a.offsets = offsets;
  a.H = c->n_kv_heads;
  const int64_t pairs = static_cast<int64_t>(c->B) * c->n_kv_heads;
  if (pairs > INT32_MAX) return TG_EOVERFLOW;
  a.pairs = static_cast<int32_t>(pairs);
  // gridDim.y is at most 65535: the kernels stride over the pairs past it
  const unsigned gy = static_cast<unsigned>(pairs < 65535 ? pairs : 65535);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int d = c->head_dim;
  const int rpb = 256 / (d / 8);
  if (max_bf > 0) {
    const dim3 grid(static_cast<unsigned>((static_cast<int64_t>(max_bf) * kPage + rpb - 1) / rpb), gy);
    if (d == 128) hipLaunchKernelGGL(write_bf16_kernel<128>, grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL(write_bf16_kernel<64>, grid, dim3(256), 0, st, a);
    if (hipGetLastError() != hipSuccess) return TG_EDEVICE;
  }
  if (max_i8 > 0) {
    const dim3 grid(static_cast<unsigned>(max_i8), gy);
    if (c->old_bits == 4) {
      if (d != 128) return TG_EUNSUPPORTED;
      hipLaunchKernelGGL(write_i4_kernel<128>, grid, dim3(256), 0, st, a);
    } else if (d == 128) {
      hipLaunchKernelGGL(write_i8_kernel<128>, grid, dim3(256), 0, st, a);
    } else {
      hipLaunchKernelGGL(write_i8_kernel<64>, grid, dim3(128), 0, st, a);
    }
    if (hipGetLastError() != hipSuccess) return TG_EDEVICE;
  }
  return TG_OK;
}
