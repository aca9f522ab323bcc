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
#include <cstdlib>

#include "tg.h"

// Every device pointer the kernels touch is kept in the global address space:
// pointers read from a struct are otherwise generic, and flat loads also count
// against lgkmcnt, which serialises the waits of the streaming loop.
#define TG_GLOBAL __attribute__((address_space(1)))

namespace {

typedef const TG_GLOBAL char* gptr;

constexpr int kWavesPerBlock = 4;
constexpr int kPage = 16;   // bf16 page: token slots per head
constexpr int kQBlock = 64; // INT8 block: token slots per head
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct SplitArgs {
  gptr pool[TG_MAX_CLUSTERS][2];
  int64_t page_bytes[TG_MAX_CLUSTERS][2];
  const TG_GLOBAL int32_t* bt[TG_MAX_CLUSTERS][2];
  int32_t stride[TG_MAX_CLUSTERS][2];
  const TG_GLOBAL int32_t* cluster_of_head;
  const TG_GLOBAL int32_t* slot_in_cluster;
  const TG_GLOBAL int32_t* len;      // [B*H*2] (n_i8, n_bf)
  const TG_GLOBAL int32_t* n_fixed;  // [B] or null
  gptr q;
  const TG_GLOBAL int32_t* work;
  TG_GLOBAL float* ws_acc;  // [n_items][G][D]
  TG_GLOBAL float* ws_ml;   // [n_items][G][2]
  int32_t n_items;
  int32_t n_q_heads;
  int32_t n_kv_heads;
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

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16(gptr p) {
  const u32x4_t x = *(const TG_GLOBAL u32x4_t*)(p);
  return make_uint4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ uint2 ld8(gptr p) {
  const u32x2_t x = *(const TG_GLOBAL u32x2_t*)(p);
  return make_uint2(x[0], x[1]);
}
__device__ __forceinline__ void st16(TG_GLOBAL float* p, float a, float b, float c, float d) {
  f32x4_t x = {a, b, c, d};
  *(TG_GLOBAL f32x4_t*)(p) = x;
}

// ------------------------------------------------------------ MFMA helpers
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_qk(const u32x4_t& k, const u32x4_t& q, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, k), __builtin_bit_cast(bf16x8_t, q), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_pv(const u32x2_t& p, const u32x2_t& v, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, p), __builtin_bit_cast(s16x4_t, v), c, 0, 0, 0);
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

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}
// split x into hi + lo bf16 parts (x - hi - lo is ~2^-17 |x|)
__device__ __forceinline__ void split_bf16(float x, uint32_t& hi, uint32_t& lo) {
  hi = bf16_rne(x);
  lo = bf16_rne(x - __uint_as_float(hi << 16));
}
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

template <typename T>
__device__ __forceinline__ T uniform(T x) {
  return __builtin_amdgcn_readfirstlane(x);
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

// ---------------------------------------------------------------- bf16 tier (MFMA)
// One item of the bf16 tier on one wavefront.  Per 16-row page the scores of
// the G heads are one MFMA tile S^T = K Q^T (16 rows x G columns, padded to
// 16) and the value update is P V over 16-row k-slices (bf16 P split into a
// high and a low part so the weights keep ~16 significant bits).  The page
// layout is chosen so that each contiguous 1 KiB wave load is exactly one
// MFMA operand (include/tg.h documents it):
//   K: byte ((d>>5)*64 + ((d>>3)&3)*16 + t)*16 + (d&7)*2
//   V: byte ((d>>5)*64 + (t>>2)*16 + (d&15))*16 + ((d>>4)&1)*8 + (t&3)*2
// Lane l = 16*lj + lg: in S^T it holds rows (tokens) 4lj..4lj+3 of column
// (head) lg; in the P V accumulators rows (heads) 4lj..4lj+3 of channel lg of
// each 16-channel tile.  The online-normaliser state m, l of head lg is kept
// in the lanes of column lg.
// Reference-max slack (base 2): weights are e^(s - m_ref) <= 2^kSlack, and the
// accumulators are rescaled only when a page max exceeds m_ref + kSlack.  Any
// reference gives the same merged result; the slack only saves rescales.
constexpr float kSlack = 8.f;

// One 16-row page of the bf16 tier (see bf16_item).  TAIL masks rows at or
// past `valid`, both in the scores and in the V operand.
template <int NK, int NT, int NQ, bool TAIL>
__device__ __forceinline__ void bf16_page(const u32x4_t (&kb)[NK], const u32x4_t (&vb)[NK],
                                          const u32x4_t (&qop)[NQ][NK], f32x4_t (&acc)[NT],
                                          float& m_ref, float& l_run, float scale_log2, int valid,
                                          int lj) {
  f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NK; ++s)
#pragma unroll
    for (int qp = 0; qp < NQ; ++qp) sacc = mfma_qk(kb[s], qop[qp][s], sacc);
  float sc[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    sc[rr] = sacc[rr] * scale_log2;
    if (TAIL && 4 * lj + rr >= valid) sc[rr] = -INFINITY;
  }
  float pm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
  pm = xor32_max(xor16_max(pm));
  if (__builtin_amdgcn_ballot_w64(pm > m_ref + kSlack) != 0) {
    const float mn = fmaxf(m_ref, pm);
    const float alpha = __builtin_amdgcn_exp2f(m_ref - mn);
    l_run *= alpha;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float ar = __shfl(alpha, 4 * lj + rr, 64);  // alpha of head 4lj+rr
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n][rr] *= ar;
    }
    m_ref = mn;
  }
  float pw[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    pw[rr] = __builtin_amdgcn_exp2f(sc[rr] - m_ref);
    l_run += pw[rr];
  }
  uint32_t ph[4], pl[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) split_bf16(pw[rr], ph[rr], pl[rr]);
  const u32x2_t Ph = {ph[0] | (ph[1] << 16), ph[2] | (ph[3] << 16)};
  const u32x2_t Pl = {pl[0] | (pl[1] << 16), pl[2] | (pl[3] << 16)};
  // V rows 4lj..4lj+3; in a tail page the rows past the item end are zeroed
  // so that whatever the page holds there cannot reach the sums
  uint32_t keep01 = 0xFFFFFFFFu, keep23 = 0xFFFFFFFFu;
  if (TAIL) {
    const int v0 = valid - 4 * lj;
    keep01 = (v0 > 0 ? 0x0000FFFFu : 0u) | (v0 > 1 ? 0xFFFF0000u : 0u);
    keep23 = (v0 > 2 ? 0x0000FFFFu : 0u) | (v0 > 3 ? 0xFFFF0000u : 0u);
  }
#pragma unroll
  for (int s = 0; s < NK; ++s) {
    const u32x4_t x = vb[s];
    const u32x2_t v0 = TAIL ? u32x2_t{x[0] & keep01, x[1] & keep23} : u32x2_t{x[0], x[1]};
    const u32x2_t v1 = TAIL ? u32x2_t{x[2] & keep01, x[3] & keep23} : u32x2_t{x[2], x[3]};
    acc[2 * s] = mfma_pv(Ph, v0, acc[2 * s]);
    acc[2 * s] = mfma_pv(Pl, v0, acc[2 * s]);
    acc[2 * s + 1] = mfma_pv(Ph, v1, acc[2 * s + 1]);
    acc[2 * s + 1] = mfma_pv(Pl, v1, acc[2 * s + 1]);
  }
}

template <int D, int G, bool QF32, int DEPTH, bool STREAM>
__device__ __forceinline__ void bf16_item(const SplitArgs& a, int r, int h, int t0, int t1, int slot,
                                          int hs, const TG_GLOBAL int32_t* bt_row, gptr pool,
                                          int64_t pbytes) {
  constexpr int NK = D / 32;           // 1 KiB loads per K (and per V) block
  constexpr int NT = D / 16;           // 16-channel tiles of V
  constexpr int NQ = QF32 ? 2 : 1;     // bf16 pieces of q
  static_assert(G <= 16, "G must fit one MFMA tile");
  const int lane = threadIdx.x & 63;
  const int lg = lane & 15;
  const int lj = lane >> 4;

  // Q^T operand of step s: lane (lg, lj) holds q[lg][32 s + 8 lj + e], e < 8
  u32x4_t qop[NQ][NK];
  {
    const bool has = lg < G;
    const int64_t row = static_cast<int64_t>(r) * a.n_q_heads + h * G + (has ? lg : 0);
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      if constexpr (QF32) {
        const u32x4_t x0 = ldv16(a.q + (row * D + 32 * s + 8 * lj) * 4);
        const u32x4_t x1 = ldv16(a.q + (row * D + 32 * s + 8 * lj + 4) * 4);
        const float f[8] = {__uint_as_float(x0[0]), __uint_as_float(x0[1]), __uint_as_float(x0[2]),
                            __uint_as_float(x0[3]), __uint_as_float(x1[0]), __uint_as_float(x1[1]),
                            __uint_as_float(x1[2]), __uint_as_float(x1[3])};
        uint32_t hi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) split_bf16(f[e], hi[e], lo[e]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qop[0][s][e] = has ? (hi[2 * e] | (hi[2 * e + 1] << 16)) : 0u;
          qop[1][s][e] = has ? (lo[2 * e] | (lo[2 * e + 1] << 16)) : 0u;
        }
      } else {
        const u32x4_t x = ldv16(a.q + (row * D + 32 * s + 8 * lj) * 2);
#pragma unroll
        for (int e = 0; e < 4; ++e) qop[0][s][e] = has ? x[e] : 0u;
      }
    }
  }

  const int64_t head_off = static_cast<int64_t>(hs) * (4 * kPage * D);
  const int lane_off = lane * 16;
  f32x4_t acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;  // reference max of head lg (base-2 scaled score)
  float l_run = 0.f;        // sum of weights of head lg over this lane's rows
  const int p0 = t0 / kPage;
  const int np = (t1 - t0 + kPage - 1) / kPage;
  u32x4_t kb[DEPTH][NK], vb[DEPTH][NK];

  for (int w0 = 0; w0 < np; w0 += 64) {
    const int nw = min(64, np - w0);
    const int pid_lane = bt_row[p0 + w0 + min(lane, nw - 1)];
    auto issue = [&](u32x4_t (&kk)[NK], u32x4_t (&vv)[NK], int i) {
      const int pid = __builtin_amdgcn_readlane(pid_lane, min(i, nw - 1));
      gptr pp = pool + static_cast<int64_t>(pid) * pbytes + head_off + lane_off;
#pragma unroll
      for (int s = 0; s < NK; ++s) kk[s] = ldpage<STREAM>(pp + s * 1024);
#pragma unroll
      for (int s = 0; s < NK; ++s) vv[s] = ldpage<STREAM>(pp + kPage * D * 2 + s * 1024);
    };
#pragma unroll
    for (int u = 0; u < DEPTH - 1; ++u) issue(kb[u], vb[u], u);
    for (int base = 0; base < nw; base += DEPTH) {
#pragma unroll
      for (int u = 0; u < DEPTH; ++u) {
        const int i = base + u;
        const int nxt = (u + DEPTH - 1) % DEPTH;
        issue(kb[nxt], vb[nxt], i + DEPTH - 1);
        __builtin_amdgcn_sched_barrier(0);
        if (i < nw) {
          const int valid = t1 - (t0 + (w0 + i) * kPage);  // rows of this page in the item
          if (valid >= kPage)
            bf16_page<NK, NT, NQ, false>(kb[u], vb[u], qop, acc, m_ref, l_run, a.scale_log2, kPage, lj);
          else
            bf16_page<NK, NT, NQ, true>(kb[u], vb[u], qop, acc, m_ref, l_run, a.scale_log2, valid, lj);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // partial of the item: m and l of head lg, accumulator rows 4lj+rr
  const float l_tot = xor32_sum(xor16_sum(l_run));
  TG_GLOBAL float* acc_out = a.ws_acc + static_cast<int64_t>(slot) * G * D;
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int g = 4 * lj + rr;
    if (g < G) {
#pragma unroll
      for (int n = 0; n < NT; ++n) acc_out[g * D + 16 * n + lg] = acc[n][rr];
    }
  }
  if (lj == 0 && lg < G) {
    a.ws_ml[(static_cast<int64_t>(slot) * G + lg) * 2 + 0] = m_ref * kLn2;
    a.ws_ml[(static_cast<int64_t>(slot) * G + lg) * 2 + 1] = l_tot;
  }
}

// ---------------------------------------------------------------- split kernel
template <int D, int G, bool QF32, int TIER, int DEPTH>
__global__ __launch_bounds__(64 * kWavesPerBlock) void split_kernel(SplitArgs a) {
  constexpr int LPR = D / 8;          // lanes per row
  constexpr int ROWS = 64 / LPR;      // rows per wave-wide load
  constexpr int NS = kPage / ROWS;    // loads per 16-row group
  const int lane = threadIdx.x & 63;
  const int j = lane / LPR;
  const int c8 = lane % LPR;
  const int item = uniform(static_cast<int>(blockIdx.x) * kWavesPerBlock + (static_cast<int>(threadIdx.x) >> 6));
  if (item >= a.n_items) return;
  const TG_GLOBAL int32_t* w = a.work + static_cast<int64_t>(item) * 6;
  const int r = uniform(w[0]), h = uniform(w[1]), tier = uniform(w[2]);
  if (tier != TIER) return;  // the other tier's kernel takes this item
  const int t0 = uniform(w[3]), t1 = uniform(w[4]), slot = uniform(w[5]);
  const int cl = uniform(a.cluster_of_head[h]);
  const int hs = uniform(a.slot_in_cluster[h]);
  const TG_GLOBAL int32_t* bt_row = a.bt[cl][tier] + static_cast<int64_t>(r) * a.stride[cl][tier];
  gptr pool = a.pool[cl][tier];
  const int64_t pbytes = a.page_bytes[cl][tier];

  Query<G, QF32> q;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int64_t row = static_cast<int64_t>(r) * a.n_q_heads + h * G + g;
    if constexpr (QF32) {
      const uint4 x0 = ld16(a.q + (row * D + 8 * c8) * 4);
      const uint4 x1 = ld16(a.q + (row * D + 8 * c8 + 4) * 4);
      q.f[g][0] = __uint_as_float(x0.x); q.f[g][1] = __uint_as_float(x0.y);
      q.f[g][2] = __uint_as_float(x0.z); q.f[g][3] = __uint_as_float(x0.w);
      q.f[g][4] = __uint_as_float(x1.x); q.f[g][5] = __uint_as_float(x1.y);
      q.f[g][6] = __uint_as_float(x1.z); q.f[g][7] = __uint_as_float(x1.w);
    } else {
      const uint4 x = ld16(a.q + (row * D + 8 * c8) * 2);
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

  if constexpr (TIER == TG_TIER_BF16) {
    // an item that starts on the shared radix path reads through the caches
    bool shared = false;
    if (a.n_fixed) {
      const int n_i8 = uniform(a.len[2 * (r * a.n_kv_heads + h)]);
      shared = n_i8 + t0 + kPage <= uniform(a.n_fixed[r]);
    }
    if (shared)
      bf16_item<D, G, QF32, DEPTH, false>(a, r, h, t0, t1, slot, hs, bt_row, pool, pbytes);
    else
      bf16_item<D, G, QF32, DEPTH, true>(a, r, h, t0, t1, slot, hs, bt_row, pool, pbytes);
    return;
  } else {
    // INT8 block: K codes at +0, V codes at +kQBlock*D, K scales at
    // +2*kQBlock*D, V scales at +2*kQBlock*D + 2*D (bytes).  Processed in
    // 16-row groups, prefetching the next group like the bf16 loop.
    const int64_t head_off = static_cast<int64_t>(hs) * (2 * kQBlock * D + 4 * D);
    const int lane_off = j * D + 8 * c8;
    constexpr int GR = kQBlock / kPage;  // 16-row groups per block
    const int b0 = t0 / kQBlock;
    const int nb = (t1 - t0) / kQBlock;
    auto blk_ptr = [&](int pid) { return pool + static_cast<int64_t>(pid) * pbytes + head_off; };
    uint2 kr[NS], vr[NS];
    gptr bp = blk_ptr(uniform(bt_row[b0]));
#pragma unroll
    for (int s = 0; s < NS; ++s) kr[s] = ld8(bp + lane_off + s * ROWS * D);
#pragma unroll
    for (int s = 0; s < NS; ++s) vr[s] = ld8(bp + kQBlock * D + lane_off + s * ROWS * D);
    int pid_next = uniform(bt_row[b0 + min(1, nb - 1)]);
    for (int b = 0; b < nb; ++b) {
      const int pid_after = uniform(bt_row[b0 + min(b + 2, nb - 1)]);
      gptr bn = blk_ptr(pid_next);
      float qs[G][8], sv[8];
      {
        float sk[8];
        half8(ld16(bp + 2 * kQBlock * D + 16 * c8), sk);
        half8(ld16(bp + 2 * kQBlock * D + 2 * D + 16 * c8), sv);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int e = 0; e < 8; ++e) qs[g][e] = q.get(g, e) * sk[e];
      }
#pragma unroll
      for (int grp = 0; grp < GR; ++grp) {
        // the group after this one: the next group of this block, or the
        // first group of the next block
        gptr np_ = grp + 1 < GR ? bp : bn;
        const int on = grp + 1 < GR ? (grp + 1) * kPage * D : 0;
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
#pragma unroll
        for (int s = 0; s < NS; ++s) kr[s] = ld8(np_ + on + lane_off + s * ROWS * D);
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
#pragma unroll
        for (int s = 0; s < NS; ++s) vr[s] = ld8(np_ + kQBlock * D + on + lane_off + s * ROWS * D);
      }
      bp = bn;
      pid_next = pid_after;
    }
  }

  // combine rows and write the partial
  TG_GLOBAL float* acc_out = a.ws_acc + static_cast<int64_t>(slot) * G * D;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = cross_sum<LPR>(st.acc[g][e]);
    const float l = cross_sum<LPR>(st.l[g]);
    if (j == 0) {
      st16(acc_out + g * D + 8 * c8, o[0], o[1], o[2], o[3]);
      st16(acc_out + g * D + 8 * c8 + 4, o[4], o[5], o[6], o[7]);
    }
    if (lane == 0) {
      a.ws_ml[(static_cast<int64_t>(slot) * G + g) * 2 + 0] = st.m[g] * kLn2;
      a.ws_ml[(static_cast<int64_t>(slot) * G + g) * 2 + 1] = l;
    }
  }
}

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

// One launch per tier present in the cache (a tier whose tables are all
// empty has no items).  Each kernel skips the other tier's items.
template <int D, int G, bool QF32>
hipError_t launch_split(const SplitArgs& a, bool has_i8, bool has_bf, hipStream_t s) {
  const int blocks = (a.n_items + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks == 0) return hipSuccess;
  static const int depth = [] {
    const char* e = getenv("TG_SPLIT_DEPTH");  // tuning knob: 2 or 3 page buffers
    return (e && atoi(e) == 3) ? 3 : 2;
  }();
  const dim3 grid(blocks), block(64 * kWavesPerBlock);
  if (has_i8) hipLaunchKernelGGL((split_kernel<D, G, QF32, TG_TIER_I8, 2>), grid, block, 0, s, a);
  if (has_bf) {
    if (depth == 3)
      hipLaunchKernelGGL((split_kernel<D, G, QF32, TG_TIER_BF16, 3>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((split_kernel<D, G, QF32, TG_TIER_BF16, 2>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_split_d(const SplitArgs& a, int G, bool qf32, bool i8, bool bf, hipStream_t s) {
  switch (G * 2 + (qf32 ? 1 : 0)) {
    case 2: return launch_split<D, 1, false>(a, i8, bf, s);
    case 3: return launch_split<D, 1, true>(a, i8, bf, s);
    case 4: return launch_split<D, 2, false>(a, i8, bf, s);
    case 5: return launch_split<D, 2, true>(a, i8, bf, s);
    case 8: return launch_split<D, 4, false>(a, i8, bf, s);
    case 9: return launch_split<D, 4, true>(a, i8, bf, s);
    case 16: return launch_split<D, 8, false>(a, i8, bf, s);
    case 17: return launch_split<D, 8, true>(a, i8, bf, s);
    default: return hipErrorInvalidValue;
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
  if (a->n_items < 0 || !a->q || !c->cluster_of_head || !c->slot_in_cluster || !c->len) return TG_EINVAL;
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
  s.ws_ml = (TG_GLOBAL float*)(a->workspace + static_cast<int64_t>(a->n_items) * G * d);
  s.n_items = a->n_items;
  s.n_q_heads = a->n_q_heads;
  const float scale = a->sm_scale != 0.f ? a->sm_scale : 1.f / std::sqrt(static_cast<float>(d));
  s.scale_log2 = scale * kLog2e;
  hipStream_t st = static_cast<hipStream_t>(stream);
  bool has_i8 = false, has_bf = false;
  for (int32_t cl = 0; cl < c->n_clusters; ++cl) {
    has_i8 |= c->stride[cl][TG_TIER_I8] > 0;
    has_bf |= c->stride[cl][TG_TIER_BF16] > 0;
  }
  const bool qf32 = a->q_dtype == TG_Q_F32;
  hipError_t e = d == 128 ? launch_split_d<128>(s, G, qf32, has_i8, has_bf, st)
                          : launch_split_d<64>(s, G, qf32, has_i8, has_bf, st);
  if (e != hipSuccess) return TG_EDEVICE;
  if (!merge) return TG_OK;
  e = launch_merge(a->workspace, a->workspace + static_cast<int64_t>(a->n_items) * G * d, a->part_off,
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
