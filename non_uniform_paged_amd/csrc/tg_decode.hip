// Decode attention over the ragged, tiered, paged cache (gfx950).
//
// Two kernels per step:
//   split_kernel  -- one wavefront per plan item (r, h, tier, [t0, t1)):
//                    streams the item's pages with 16-byte (bf16) or 8-byte
//                    (INT8) coalesced loads, computes the G scores of every
//                    row, and keeps the online-normaliser state (m, l, acc)
//                    of the G q-heads in registers.  INT8 rows are
//                    dequantised in registers: the block's K scale is folded
//                    into q, the V scale into each value.
//   merge_kernel  -- combines the partials of each (r, h) with the
//                    log-sum-exp weights and writes o in fp32.
//
// The maths is the online normaliser (CAP survey page, section 2.4.3
// "Distributed acceleration", online normaliser [88]): per chunk keep
// m = max s, l = sum e^{s-m}, acc = sum e^{s-m} v; chunks merge exactly with
// weights e^{m_i - M}.  Scores are kept in base 2 (s * log2 e) inside the
// kernel; partial m is stored in natural-log units.
//
// Lane mapping inside a wavefront (64 lanes).  A row of d values is LPR =
// d/8 lanes wide (8 values per lane); a wave covers ROWS = 64/LPR rows per
// load.  Lane (j, c) = (lane / LPR, lane % LPR) owns channels [8c, 8c+8) of
// rows j, j + ROWS, ...  Row dot products are summed across the LPR lanes
// with DPP row permutations; the row max and the final accumulator sums
// cross rows with lane shuffles.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "tg.h"

namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kPage = 16;   // bf16 page: token slots per head
constexpr int kQBlock = 64; // INT8 block: token slots per head
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct SplitArgs {
  const char* pool[TG_MAX_CLUSTERS][2];
  int64_t page_bytes[TG_MAX_CLUSTERS][2];
  const int32_t* bt[TG_MAX_CLUSTERS][2];
  int32_t stride[TG_MAX_CLUSTERS][2];
  const int32_t* cluster_of_head;
  const int32_t* slot_in_cluster;
  const void* q;
  const int32_t* work;
  float* ws_acc;  // [n_items][G][D]
  float* ws_ml;   // [n_items][G][2]
  int32_t n_items;
  int32_t n_q_heads;
  float scale_log2;
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the LPR lanes of a row (LPR = 8 or 16), result in every lane.
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  if constexpr (LPR == 16) x += dpp<0x140>(x);  // row_mirror
  return x;
}

// Max / sum across the rows of a wave (lane bits >= log2(LPR)).
template <int LPR>
__device__ __forceinline__ float cross_max(float x) {
#pragma unroll
  for (int m = LPR; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}
template <int LPR>
__device__ __forceinline__ float cross_sum(float x) {
#pragma unroll
  for (int m = LPR; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

template <int D, int G>
struct State {
  float m[G];       // running max (base-2 scaled score), uniform over the wave
  float l[G];       // this lane's share of sum e^{s-m} (its rows)
  float acc[G][8];  // this lane's share of sum e^{s-m} v over its 8 channels
};

// Online-normaliser update for NS row groups whose base-2 scores are sc[s][g]
// (-inf where masked).  Returns the weights in sc (p = e^{s - m_new}) and
// rescales l and acc; the caller then adds p * v.
template <int D, int G, int NS>
__device__ __forceinline__ void softmax_update(State<D, G>& st, float (&sc)[NS][G]) {
  constexpr int LPR = D / 8;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float pm = sc[0][g];
#pragma unroll
    for (int s = 1; s < NS; ++s) pm = fmaxf(pm, sc[s][g]);
    pm = cross_max<LPR>(pm);
    const float mn = fmaxf(st.m[g], pm);
    const float alpha = __builtin_amdgcn_exp2f(st.m[g] - mn);
    st.m[g] = mn;
    float ps = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      sc[s][g] = __builtin_amdgcn_exp2f(sc[s][g] - mn);
      ps += sc[s][g];
    }
    st.l[g] = fmaf(st.l[g], alpha, ps);
#pragma unroll
    for (int e = 0; e < 8; ++e) st.acc[g][e] *= alpha;
  }
}

template <int D, int G>
__device__ __forceinline__ void accumulate(State<D, G>& st, const float (&p)[G], const float (&v)[8]) {
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) st.acc[g][e] = fmaf(p[g], v[e], st.acc[g][e]);
}

// Query channels [8c, 8c+8) of the lane for each of the G heads: fp32, or
// bf16 pairs (packed, fed to the bf16 dot2 instruction).
template <int G, bool QF32>
struct Query;
template <int G>
struct Query<G, true> {
  float f[G][8];
  __device__ __forceinline__ float get(int g, int e) const { return f[g][e]; }
};
template <int G>
struct Query<G, false> {
  uint32_t b[G][4];
  __device__ __forceinline__ float get(int g, int e) const {
    return (e & 1) ? bf_hi(b[g][e >> 1]) : bf_lo(b[g][e >> 1]);
  }
};

template <int G>
__device__ __forceinline__ float dot8(const Query<G, true>& q, int g, const uint4& k) {
  float a = q.f[g][0] * bf_lo(k.x);
  a = fmaf(q.f[g][1], bf_hi(k.x), a);
  a = fmaf(q.f[g][2], bf_lo(k.y), a);
  a = fmaf(q.f[g][3], bf_hi(k.y), a);
  a = fmaf(q.f[g][4], bf_lo(k.z), a);
  a = fmaf(q.f[g][5], bf_hi(k.z), a);
  a = fmaf(q.f[g][6], bf_lo(k.w), a);
  a = fmaf(q.f[g][7], bf_hi(k.w), a);
  return a;
}
template <int G>
__device__ __forceinline__ float dot8(const Query<G, false>& q, int g, const uint4& k) {
  float a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.b[g][0]), __builtin_bit_cast(bf16x2_t, k.x), 0.f, false);
  a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.b[g][1]), __builtin_bit_cast(bf16x2_t, k.y), a, false);
  a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.b[g][2]), __builtin_bit_cast(bf16x2_t, k.z), a, false);
  a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.b[g][3]), __builtin_bit_cast(bf16x2_t, k.w), a, false);
  return a;
}

__device__ __forceinline__ uint4 ld16(const char* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 ld8(const char* p) { return *reinterpret_cast<const uint2*>(p); }

template <typename T>
__device__ __forceinline__ T uniform(T x) {
  return __builtin_amdgcn_readfirstlane(x);
}
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const char*>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ void bf8(const uint4& x, float (&v)[8]) {
  v[0] = bf_lo(x.x); v[1] = bf_hi(x.x);
  v[2] = bf_lo(x.y); v[3] = bf_hi(x.y);
  v[4] = bf_lo(x.z); v[5] = bf_hi(x.z);
  v[6] = bf_lo(x.w); v[7] = bf_hi(x.w);
}

__device__ __forceinline__ float i8f(uint32_t w, int b) {
  return static_cast<float>(static_cast<int32_t>(w << (24 - 8 * b)) >> 24);
}

__device__ __forceinline__ void half8(const uint4& x, float (&f)[8]) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i] & 0xffff)));
    f[2 * i + 1] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i] >> 16)));
  }
}

// ---------------------------------------------------------------- split kernel
template <int D, int G, bool QF32>
__global__ __launch_bounds__(64 * kWavesPerBlock) void split_kernel(SplitArgs a) {
  constexpr int LPR = D / 8;          // lanes per row
  constexpr int ROWS = 64 / LPR;      // rows per wave-wide load
  constexpr int NS = kPage / ROWS;    // loads per 16-row group
  const int lane = threadIdx.x & 63;
  const int j = lane / LPR;
  const int c8 = lane % LPR;
  const int item = uniform(static_cast<int>(blockIdx.x) * kWavesPerBlock + (static_cast<int>(threadIdx.x) >> 6));
  if (item >= a.n_items) return;
  const int32_t* w = a.work + static_cast<int64_t>(item) * 6;
  const int r = uniform(w[0]), h = uniform(w[1]), tier = uniform(w[2]);
  const int t0 = uniform(w[3]), t1 = uniform(w[4]), slot = uniform(w[5]);
  const int cl = uniform(a.cluster_of_head[h]);
  const int hs = uniform(a.slot_in_cluster[h]);
  const int32_t* bt_row = a.bt[cl][tier] + static_cast<int64_t>(r) * a.stride[cl][tier];
  const char* pool = a.pool[cl][tier];
  const int64_t pbytes = a.page_bytes[cl][tier];

  Query<G, QF32> q;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int64_t row = static_cast<int64_t>(r) * a.n_q_heads + h * G + g;
    if constexpr (QF32) {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.q) + row * D + 8 * c8);
      const float4 x0 = p[0], x1 = p[1];
      q.f[g][0] = x0.x; q.f[g][1] = x0.y; q.f[g][2] = x0.z; q.f[g][3] = x0.w;
      q.f[g][4] = x1.x; q.f[g][5] = x1.y; q.f[g][6] = x1.z; q.f[g][7] = x1.w;
    } else {
      const uint4 x = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + row * D + 8 * c8);
      q.b[g][0] = x.x; q.b[g][1] = x.y; q.b[g][2] = x.z; q.b[g][3] = x.w;
    }
  }

  State<D, G> st;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    st.m[g] = -INFINITY;
    st.l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) st.acc[g][e] = 0.f;
  }

  if (tier == TG_TIER_BF16) {
    // page i: K at +0, V at +kPage*D*2 (bytes) inside the head's block
    const int64_t head_off = static_cast<int64_t>(hs) * (4 * kPage * D);
    const int lane_off = (j * D + 8 * c8) * 2;
    const int p0 = t0 / kPage;
    const int np = (t1 - t0 + kPage - 1) / kPage;
    auto page_ptr = [&](int i) {
      const int pid = uniform(bt_row[p0 + i]);
      return uniform_ptr(pool + static_cast<int64_t>(pid) * pbytes + head_off);
    };
    uint4 kr[NS], vr[NS];
    const char* pp = page_ptr(0);
#pragma unroll
    for (int s = 0; s < NS; ++s) kr[s] = ld16(pp + lane_off + s * ROWS * D * 2);
#pragma unroll
    for (int s = 0; s < NS; ++s) vr[s] = ld16(pp + kPage * D * 2 + lane_off + s * ROWS * D * 2);
    for (int i = 0; i < np; ++i) {
      const int valid = t1 - (t0 + i * kPage);  // rows of this page inside the item
      float sc[NS][G];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bool ok = s * ROWS + j < valid;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float dsum = row_sum<LPR>(dot8(q, g, kr[s]));
          sc[s][g] = ok ? dsum * a.scale_log2 : -INFINITY;
        }
      }
      const char* pn = i + 1 < np ? page_ptr(i + 1) : pp;
      if (i + 1 < np) {
#pragma unroll
        for (int s = 0; s < NS; ++s) kr[s] = ld16(pn + lane_off + s * ROWS * D * 2);
      }
      softmax_update<D, G, NS>(st, sc);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        float v[8];
        bf8(vr[s], v);
        if (s * ROWS + j >= valid) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = 0.f;
        }
        float p[G];
#pragma unroll
        for (int g = 0; g < G; ++g) p[g] = sc[s][g];
        accumulate<D, G>(st, p, v);
      }
      if (i + 1 < np) {
#pragma unroll
        for (int s = 0; s < NS; ++s) vr[s] = ld16(pn + kPage * D * 2 + lane_off + s * ROWS * D * 2);
      }
      pp = pn;
    }
  } else {
    // INT8 block: K codes at +0, V codes at +kQBlock*D, K scales at
    // +2*kQBlock*D, V scales at +2*kQBlock*D + 2*D (bytes)
    const int64_t head_off = static_cast<int64_t>(hs) * (2 * kQBlock * D + 4 * D);
    const int lane_off = j * D + 8 * c8;
    constexpr int GR = kQBlock / kPage;  // 16-row groups per block
    const int b0 = t0 / kQBlock;
    const int ng = (t1 - t0) / kPage;    // groups in the item
    auto blk_ptr = [&](int gi) {
      const int pid = uniform(bt_row[b0 + gi / GR]);
      return uniform_ptr(pool + static_cast<int64_t>(pid) * pbytes + head_off);
    };
    uint2 kr[NS], vr[NS];
    const char* bp = blk_ptr(0);
#pragma unroll
    for (int s = 0; s < NS; ++s) kr[s] = ld8(bp + lane_off + s * ROWS * D);
#pragma unroll
    for (int s = 0; s < NS; ++s) vr[s] = ld8(bp + kQBlock * D + lane_off + s * ROWS * D);
    float qs[G][8], sv[8];
    for (int gi = 0; gi < ng; ++gi) {
      const int grp = gi % GR;
      if (grp == 0) {
        float sk[8];
        half8(ld16(bp + 2 * kQBlock * D + 16 * c8), sk);
        half8(ld16(bp + 2 * kQBlock * D + 2 * D + 16 * c8), sv);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int e = 0; e < 8; ++e) qs[g][e] = q.get(g, e) * sk[e];
      }
      float sc[NS][G];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        float k[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          k[e] = i8f(kr[s].x, e);
          k[e + 4] = i8f(kr[s].y, e);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float acc = qs[g][0] * k[0];
#pragma unroll
          for (int e = 1; e < 8; ++e) acc = fmaf(qs[g][e], k[e], acc);
          sc[s][g] = row_sum<LPR>(acc) * a.scale_log2;
        }
      }
      const char* bn = bp;
      int on = (grp + 1) * kPage * D;
      if (gi + 1 < ng) {
        if (grp + 1 == GR) {
          bn = blk_ptr(gi + 1);
          on = 0;
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) kr[s] = ld8(bn + on + lane_off + s * ROWS * D);
      }
      softmax_update<D, G, NS>(st, sc);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = i8f(vr[s].x, e) * sv[e];
          v[e + 4] = i8f(vr[s].y, e) * sv[e + 4];
        }
        float p[G];
#pragma unroll
        for (int g = 0; g < G; ++g) p[g] = sc[s][g];
        accumulate<D, G>(st, p, v);
      }
      if (gi + 1 < ng) {
#pragma unroll
        for (int s = 0; s < NS; ++s) vr[s] = ld8(bn + kQBlock * D + on + lane_off + s * ROWS * D);
      }
      bp = bn;
    }
  }

  // combine rows and write the partial
  float* acc_out = a.ws_acc + static_cast<int64_t>(slot) * G * D;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = cross_sum<LPR>(st.acc[g][e]);
    const float l = cross_sum<LPR>(st.l[g]);
    if (j == 0) {
      float4* dst = reinterpret_cast<float4*>(acc_out + g * D + 8 * c8);
      dst[0] = make_float4(o[0], o[1], o[2], o[3]);
      dst[1] = make_float4(o[4], o[5], o[6], o[7]);
    }
    if (lane == 0) {
      a.ws_ml[(static_cast<int64_t>(slot) * G + g) * 2 + 0] = st.m[g] * kLn2;
      a.ws_ml[(static_cast<int64_t>(slot) * G + g) * 2 + 1] = l;
    }
  }
}

// ---------------------------------------------------------------- merge kernel
// One wavefront per (pair, g); lanes hold d/64 consecutive channels.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ ws_acc,
                                                    const float* __restrict__ ws_ml,
                                                    const int32_t* __restrict__ part_off,
                                                    int32_t n_pairs, int32_t G,
                                                    float* __restrict__ out) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t rowid = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (rowid >= static_cast<int64_t>(n_pairs) * G) return;
  const int64_t pair = rowid / G;
  const int g = static_cast<int>(rowid % G);
  const int s0 = part_off[pair], s1 = part_off[pair + 1];
  float M = -INFINITY;
  for (int s = s0; s < s1; ++s) M = fmaxf(M, ws_ml[(static_cast<int64_t>(s) * G + g) * 2]);
  float den = 0.f;
  float num[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) num[e] = 0.f;
  for (int s = s0; s < s1; ++s) {
    const float* ml = ws_ml + (static_cast<int64_t>(s) * G + g) * 2;
    const float wgt = __builtin_amdgcn_exp2f((ml[0] - M) * kLog2e);
    den = fmaf(wgt, ml[1], den);
    const float* acc = ws_acc + (static_cast<int64_t>(s) * G + g) * D + PER * lane;
#pragma unroll
    for (int e = 0; e < PER; ++e) num[e] = fmaf(wgt, acc[e], num[e]);
  }
  float* dst = out + rowid * D + PER * lane;
  const float inv = s1 > s0 ? 1.f / den : 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) dst[e] = s1 > s0 ? num[e] * inv : 0.f;
}

template <int D, int G, bool QF32>
hipError_t launch_split(const SplitArgs& a, hipStream_t s) {
  const int blocks = (a.n_items + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((split_kernel<D, G, QF32>), dim3(blocks), dim3(64 * kWavesPerBlock), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_split_d(const SplitArgs& a, int G, bool qf32, hipStream_t s) {
  switch (G * 2 + (qf32 ? 1 : 0)) {
    case 2: return launch_split<D, 1, false>(a, s);
    case 3: return launch_split<D, 1, true>(a, s);
    case 4: return launch_split<D, 2, false>(a, s);
    case 5: return launch_split<D, 2, true>(a, s);
    case 8: return launch_split<D, 4, false>(a, s);
    case 9: return launch_split<D, 4, true>(a, s);
    case 16: return launch_split<D, 8, false>(a, s);
    case 17: return launch_split<D, 8, true>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_merge(const float* ws_acc, const float* ws_ml, const int32_t* part_off,
                        int32_t n_pairs, int32_t G, int32_t d, float* out, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(n_pairs) * G;
  if (rows == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((rows + 3) / 4));
  if (d == 128)
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(256), 0, s, ws_acc, ws_ml, part_off, n_pairs, G, out);
  else
    hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(256), 0, s, ws_acc, ws_ml, part_off, n_pairs, G, out);
  return hipGetLastError();
}

bool supported(int32_t d, int32_t G) {
  return (d == 64 || d == 128) && (G == 1 || G == 2 || G == 4 || G == 8);
}

}  // namespace

extern "C" size_t tg_decode_workspace_bytes(int32_t n_items, int32_t G, int32_t d) {
  if (n_items < 0 || G < 1 || d < 1) return 0;
  return static_cast<size_t>(n_items) * G * (d + 2) * sizeof(float);
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
  if (a->n_items < 0 || !a->q || !c->cluster_of_head || !c->slot_in_cluster) return TG_EINVAL;
  if (merge && (!a->out || !a->part_off)) return TG_EINVAL;
  if (a->n_items > 0 && (!a->work || !a->workspace)) return TG_EINVAL;
  if (a->workspace_bytes < tg_decode_workspace_bytes(a->n_items, G, d)) return TG_EINVAL;
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
      s.pool[cl][t] = static_cast<const char*>(c->pool[cl][t]);
      s.page_bytes[cl][t] = c->page_bytes[cl][t];
      s.bt[cl][t] = c->bt[cl][t];
      s.stride[cl][t] = c->stride[cl][t];
    }
  s.cluster_of_head = c->cluster_of_head;
  s.slot_in_cluster = c->slot_in_cluster;
  s.q = a->q;
  s.work = a->work;
  s.ws_acc = a->workspace;
  s.ws_ml = a->workspace + static_cast<int64_t>(a->n_items) * G * d;
  s.n_items = a->n_items;
  s.n_q_heads = a->n_q_heads;
  const float scale = a->sm_scale != 0.f ? a->sm_scale : 1.f / std::sqrt(static_cast<float>(d));
  s.scale_log2 = scale * kLog2e;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = d == 128 ? launch_split_d<128>(s, G, a->q_dtype == TG_Q_F32, st)
                          : launch_split_d<64>(s, G, a->q_dtype == TG_Q_F32, st);
  if (e != hipSuccess) return TG_EDEVICE;
  if (!merge) return TG_OK;
  e = launch_merge(s.ws_acc, s.ws_ml, a->part_off, c->B * c->n_kv_heads, G, d, a->out, st);
  return e == hipSuccess ? TG_OK : TG_EDEVICE;
}

}  // namespace

extern "C" int tg_decode_attn(const tg_cache* c, const tg_decode_args* a, void* stream) {
  return decode_split(c, a, stream, true);
}

extern "C" int tg_decode_split(const tg_cache* c, const tg_decode_args* a, void* stream) {
  return decode_split(c, a, stream, false);
}
