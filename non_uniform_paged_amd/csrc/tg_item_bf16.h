#ifndef TG_ITEM_BF16_H_
#define TG_ITEM_BF16_H_
// Split work item, bf16 tier (gfx950): one wavefront per plan item
// (r, h, bf16, [t0, t1)) computes the online-normaliser partial of the G
// q-heads of KV-head h over rows [t0, t1) of the bf16 tier.  A group item
// does the same for the requests that share those pages (radix prefix), one
// set of G score columns per member, in one pass over the pages: the four
// wavefronts of a workgroup take up to 32 / G members each (two 16-column score
// tiles) and share the page loads through LDS (bf16_group_coop).
//
// The maths is the online normaliser (CAP survey page, section 2.4.3
// "Distributed acceleration", online normaliser [88]): per chunk keep
// m = max s, l = sum e^{s-m}, acc = sum e^{s-m} v; chunks merge exactly with
// weights e^{m_i - M}.  Scores are kept in base 2 (s * log2 e) inside the
// kernel; partial m is stored in natural-log units.
//
// Per 16-row page the scores of the G heads are one matrix-core tile
// S^T = K Q^T (16 rows x G columns, padded to 16) and the value update is P V
// over 16-row k-slices (bf16 P split into a high and a low part so that the
// weights keep ~16 significant bits).  The page layout (include/tg.h) is
// chosen so that each contiguous 1 KiB wave load is exactly one MFMA operand:
//   K: byte ((c>>5)*64 + ((c>>3)&3)*16 + t)*16 + (c&7)*2
//   V: byte ((c>>5)*64 + (t>>2)*16 + (c&15))*16 + ((c>>4)&1)*8 + (t&3)*2
// Lane l = 16*lj + lg: in S^T it holds rows (tokens) 4lj..4lj+3 of column
// (head) lg; in the P V accumulators rows (heads) 4lj..4lj+3 of channel lg of
// each 16-channel tile.  The online-normaliser state m, l of head lg is kept
// in the lanes of column lg.

#include <cmath>

#include "tg_device.h"

namespace tg_dev {

// One 16-row page.  TAIL masks rows at or past `valid`, both in the scores
// and in the V operand.
template <int NK, int NT, int NQ, bool TAIL>
__device__ __forceinline__ void bf16_page(const u32x4_t (&kb)[NK], const u32x4_t (&vb)[NK],
                                          const u32x4_t (&qop)[NQ][NK], f32x4_t (&acc)[NT],
                                          float& m_ref, float& l_run, float scale_log2, int valid,
                                          int lj) {
  f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NK; ++s)
#pragma unroll
    for (int qp = 0; qp < NQ; ++qp) sacc = mfma_bf16_k32(kb[s], qop[qp][s], sacc);
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
    acc[2 * s] = mfma_bf16_k16(Ph, v0, acc[2 * s]);
    acc[2 * s] = mfma_bf16_k16(Pl, v0, acc[2 * s]);
    acc[2 * s + 1] = mfma_bf16_k16(Ph, v1, acc[2 * s + 1]);
    acc[2 * s + 1] = mfma_bf16_k16(Pl, v1, acc[2 * s + 1]);
  }
}

// Two 16-row pages a, b as one 32-token step for one score tile, the pages
// read from LDS (`pg`: page a of the pair slot at this lane's 16-byte offset,
// page b PAGE bytes on): both pages' scores against one reference max, then
// P V over both pages in one K = 32 matrix-core product per 16-channel tile
// (about 40 % less matrix-core time than two K = 16 products on gfx950).
// K-slots 8lj..8lj+3 carry rows 4lj..4lj+3 of page a and k-slots 8lj+4..8lj+7
// the same rows of page b, in the P and the V operand alike.  Operands are
// read from LDS next to their use.  TAIL masks rows at or past valid_a
// (page a) and valid_b (page b; <= 0: the whole page), in the scores and in V.
template <int NK, int NT, int NQ, int PAGE, bool TAIL>
__device__ __forceinline__ void bf16_pair_lds(const TG_LDS char* pg, const u32x4_t (&qop)[NQ][NK],
                                              f32x4_t (&acc)[NT], float& m_ref, float& l_run, float scale_log2,
                                              int valid_a, int valid_b, int lj) {
  f32x4_t sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NK; ++s) {
    const u32x4_t ka = *(const TG_LDS u32x4_t*)(pg + s * 1024);
    const u32x4_t kb = *(const TG_LDS u32x4_t*)(pg + PAGE + s * 1024);
#pragma unroll
    for (int qp = 0; qp < NQ; ++qp) {
      sa = mfma_bf16_k32(ka, qop[qp][s], sa);
      sb = mfma_bf16_k32(kb, qop[qp][s], sb);
    }
  }
  float sc[8];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    sc[rr] = sa[rr] * scale_log2;
    sc[4 + rr] = sb[rr] * scale_log2;
    if (TAIL && 4 * lj + rr >= valid_a) sc[rr] = -INFINITY;
    if (TAIL && 4 * lj + rr >= valid_b) sc[4 + rr] = -INFINITY;
  }
  float pm = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
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
  uint32_t ph[8], pl[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float pw = __builtin_amdgcn_exp2f(sc[e] - m_ref);
    l_run += pw;
    split_bf16(pw, ph[e], pl[e]);
  }
  const u32x4_t Ph = {ph[0] | (ph[1] << 16), ph[2] | (ph[3] << 16), ph[4] | (ph[5] << 16), ph[6] | (ph[7] << 16)};
  const u32x4_t Pl = {pl[0] | (pl[1] << 16), pl[2] | (pl[3] << 16), pl[4] | (pl[5] << 16), pl[6] | (pl[7] << 16)};
  uint32_t a01 = 0xFFFFFFFFu, a23 = 0xFFFFFFFFu, b01 = 0xFFFFFFFFu, b23 = 0xFFFFFFFFu;
  if (TAIL) {
    const int ra = valid_a - 4 * lj, rb = valid_b - 4 * lj;
    a01 = (ra > 0 ? 0x0000FFFFu : 0u) | (ra > 1 ? 0xFFFF0000u : 0u);
    a23 = (ra > 2 ? 0x0000FFFFu : 0u) | (ra > 3 ? 0xFFFF0000u : 0u);
    b01 = (rb > 0 ? 0x0000FFFFu : 0u) | (rb > 1 ? 0xFFFF0000u : 0u);
    b23 = (rb > 2 ? 0x0000FFFFu : 0u) | (rb > 3 ? 0xFFFF0000u : 0u);
  }
#pragma unroll
  for (int s = 0; s < NK; ++s) {
    const u32x4_t x = *(const TG_LDS u32x4_t*)(pg + (NK + s) * 1024);
    const u32x4_t y = *(const TG_LDS u32x4_t*)(pg + PAGE + (NK + s) * 1024);
    const u32x4_t v0 = TAIL ? u32x4_t{x[0] & a01, x[1] & a23, y[0] & b01, y[1] & b23} : u32x4_t{x[0], x[1], y[0], y[1]};
    const u32x4_t v1 = TAIL ? u32x4_t{x[2] & a01, x[3] & a23, y[2] & b01, y[3] & b23} : u32x4_t{x[2], x[3], y[2], y[3]};
    acc[2 * s] = mfma_bf16_k32(Ph, v0, acc[2 * s]);
    acc[2 * s] = mfma_bf16_k32(Pl, v0, acc[2 * s]);
    acc[2 * s + 1] = mfma_bf16_k32(Ph, v1, acc[2 * s + 1]);
    acc[2 * s + 1] = mfma_bf16_k32(Pl, v1, acc[2 * s + 1]);
  }
}

// Score columns of NTILE tiles: column c = lg + 16 * tile belongs to member
// mbase + c / G (its q-head c % G).  A plain item (gm null) has the one
// member (r, slot) in columns 0..G-1 of tile 0; a group item's members come
// from `gm`, the (request, slot) pairs of its member table row.  Unused
// columns get slot -1 (and zero q).
template <int G, int NTILE>
__device__ __forceinline__ void tile_members(int r, int slot, const TG_GLOBAL int32_t* gm, int mbase,
                                             int (&col_r)[NTILE], int (&col_slot)[NTILE]) {
  const int lg = threadIdx.x & 15;
#pragma unroll
  for (int tile = 0; tile < NTILE; ++tile) {
    col_r[tile] = r;
    col_slot[tile] = (tile == 0 && lg < G) ? slot : -1;
    if (gm != nullptr) {
      const int mu = mbase + (lg + 16 * tile) / G;
      const int mr = mu < TG_GROUP_WIDTH ? gm[2 * mu] : -1;
      col_r[tile] = mr < 0 ? r : mr;
      col_slot[tile] = mr < 0 ? -1 : gm[2 * mu + 1];
    }
  }
}

// Q^T operand of step s: lane (lg, lj) holds q[column lg][32 s + 8 lj + e]
template <int D, int G, bool QF32, int NTILE>
__device__ __forceinline__ void load_qop(const SplitArgs& a, int h, const int (&col_r)[NTILE],
                                         const int (&col_slot)[NTILE],
                                         u32x4_t (&qop)[NTILE][QF32 ? 2 : 1][D / 32]) {
  constexpr int NK = D / 32;
  const int lane = threadIdx.x & 63;
  const int lg = lane & 15;
  const int lj = lane >> 4;
#pragma unroll
  for (int tile = 0; tile < NTILE; ++tile) {
    const bool has = col_slot[tile] >= 0;
    const int64_t row = static_cast<int64_t>(col_r[tile]) * a.n_q_heads + h * G + lg % G;
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
          qop[tile][0][s][e] = has ? (hi[2 * e] | (hi[2 * e + 1] << 16)) : 0u;
          qop[tile][1][s][e] = has ? (lo[2 * e] | (lo[2 * e + 1] << 16)) : 0u;
        }
      } else {
        const u32x4_t x = ldv16(a.q + (row * D + 32 * s + 8 * lj) * 2);
#pragma unroll
        for (int e = 0; e < 4; ++e) qop[tile][0][s][e] = has ? x[e] : 0u;
      }
    }
  }
}

// Partials of NTILE tiles: m and l of column lg, accumulator rows (columns)
// 4lj+rr, each to its column's slot.
template <int D, int G, int NTILE>
__device__ __forceinline__ void write_partials(const SplitArgs& a, const int (&col_slot)[NTILE],
                                               const f32x4_t (&acc)[NTILE][D / 16], const float (&m_ref)[NTILE],
                                               const float (&l_run)[NTILE]) {
  constexpr int NT = D / 16;
  const int lane = threadIdx.x & 63;
  const int lg = lane & 15;
  const int lj = lane >> 4;
#pragma unroll
  for (int tile = 0; tile < NTILE; ++tile) {
    const float l_tot = xor32_sum(xor16_sum(l_run[tile]));
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int cslot = __shfl(col_slot[tile], 4 * lj + rr, 64);  // lane 4lj+rr owns that column
      if (cslot >= 0) {
        TG_GLOBAL float* acc_out = a.ws_acc + (static_cast<int64_t>(cslot) * G + (4 * lj + rr) % G) * D;
#pragma unroll
        for (int n = 0; n < NT; ++n) acc_out[16 * n + lg] = acc[tile][n][rr];
      }
    }
    if (lj == 0 && col_slot[tile] >= 0) {
      a.ws_ml[(static_cast<int64_t>(col_slot[tile]) * G + lg % G) * 2 + 0] = m_ref[tile] * kLn2;
      a.ws_ml[(static_cast<int64_t>(col_slot[tile]) * G + lg % G) * 2 + 1] = l_tot;
    }
  }
}

// One item on one wavefront.  A register pipeline of DEPTH page buffers: page
// i + DEPTH - 1 is requested before page i is consumed.  Requests past the
// last page repeat the last page (an L2 hit), so every request is
// unconditional and the waits before a page's use cover exactly that page's
// loads.  Page ids of up to 64 pages sit one per lane and are read with
// readlane.  The members are those of tile_members (a group item that runs
// here takes the 16 / G members from mbase).  With ring_pg > 0 the tier's
// pages form a ring: logical page p is table entry (ring_base + p) mod ring_pg.
template <int D, int G, bool QF32, int DEPTH, bool STREAM>
__device__ __forceinline__ void bf16_item(const SplitArgs& a, int r, int h, int t0, int t1, int slot,
                                          const TG_GLOBAL int32_t* gm, int mbase, int64_t head_off,
                                          const TG_GLOBAL int32_t* bt_row, int ring_base, int ring_pg,
                                          gptr pool, int64_t pbytes) {
  constexpr int NK = D / 32;           // 1 KiB loads per K (and per V) block
  constexpr int NT = D / 16;           // 16-channel tiles of V
  constexpr int NQ = QF32 ? 2 : 1;     // bf16 pieces of q
  static_assert(G <= 16, "G must fit one MFMA tile");
  const int lane = threadIdx.x & 63;
  const int lj = lane >> 4;

  int col_r[1], col_slot[1];
  tile_members<G, 1>(r, slot, gm, mbase, col_r, col_slot);
  u32x4_t qop[1][NQ][NK];
  load_qop<D, G, QF32, 1>(a, h, col_r, col_slot, qop);

  const int lane_off = lane * 16;
  f32x4_t acc[1][NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[0][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref[1] = {-INFINITY}, l_run[1] = {0.f};  // reference max (base-2 scaled score), weight sum
  const int p0 = t0 / kPage;
  const int np = (t1 - t0 + kPage - 1) / kPage;
  u32x4_t kb[DEPTH][NK], vb[DEPTH][NK];

  for (int w0 = 0; w0 < np; w0 += 64) {
    const int nw = min(64, np - w0);
    int lp = p0 + w0 + min(lane, nw - 1);
    if (ring_pg > 0) lp = (ring_base + lp) % ring_pg;
    const int pid_lane = bt_row[lp];
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
            bf16_page<NK, NT, NQ, false>(kb[u], vb[u], qop[0], acc[0], m_ref[0], l_run[0], a.scale_log2, kPage,
                                         lj);
          else
            bf16_page<NK, NT, NQ, true>(kb[u], vb[u], qop[0], acc[0], m_ref[0], l_run[0], a.scale_log2, valid,
                                        lj);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  write_partials<D, G, 1>(a, col_slot, acc, m_ref, l_run);
}

// LDS ring of a cooperative group item, in page pairs: kCoopPairs - 1 pairs
// are in flight while one is consumed.
constexpr int kCoopPairs = 3;
template <int D>
constexpr int kCoopLdsBytes = kCoopPairs * 2 * 4 * kPage * D;

// vector-memory wait for at most n outstanding operations (expcnt and
// lgkmcnt left free)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier across which the compiler moves no memory access.  (Not
// __syncthreads: its fences would also wait for the page loads in flight.)
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// A group item on the four wavefronts of a workgroup (every wavefront calls
// this with the same item).  The item's page range is read once, two pages a
// step: pages 2j, 2j + 1 go to LDS pair slot j % kCoopPairs by direct-to-LDS
// 16-byte loads, wavefront w loading 1 KiB blocks w, w + 4, ... of each
// head page (K blocks then V blocks, the pool's own order), so a page is one
// contiguous 4 kPage D bytes in LDS too.  After its own loads of pair j have
// landed (vmcnt) every wavefront meets the barrier; past it, pair j is
// complete in LDS and every wavefront has finished reading pair j - 1, whose
// slot then takes the load of pair j + kCoopPairs - 1.  Requests past the
// last page repeat the last page, so the wait count is the same at every
// step.  Wavefront w scores the members pass + w * M .. (M = 32 / G in two
// 16-column tiles; one tile, M = 2, for G = 8 with fp32 q, whose two-part q
// operands would not fit the registers) of each pass; members past the 4 M
// of a pass take another pass over the pages.
template <int D, int G, bool QF32>
__device__ __forceinline__ void bf16_group_coop(const SplitArgs& a, const TG_GLOBAL int32_t* w,
                                                TG_LDS char* lds) {
  constexpr int NK = D / 32;
  constexpr int NT = D / 16;
  constexpr int NQ = QF32 ? 2 : 1;
  constexpr int PAGE = 4 * kPage * D;             // bytes of one head's page (K then V)
  constexpr int BLKS = PAGE / 1024;               // 1 KiB blocks per head page
  constexpr int PER = BLKS / kWavesPerBlock;      // blocks each wavefront loads per page
  constexpr int CT = (QF32 && G == 8) ? 1 : 2;    // score tiles per wavefront (register budget)
  constexpr int M = 16 * CT / G;                  // members per wavefront and pass
  static_assert(BLKS % kWavesPerBlock == 0, "page blocks must split over the wavefronts");
  const int wave = static_cast<int>(threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  const int lj = lane >> 4;
  const int k = -1 - uniform(w[0]);
  if (k < 0 || k >= a.n_gitems) return;  // the same test in every wavefront
  const int h = uniform(w[1]);
  const int t0 = uniform(w[3]), t1 = uniform(w[4]);
  const TG_GLOBAL int32_t* gm = a.gitems + static_cast<int64_t>(k) * (2 * TG_GROUP_WIDTH);
  const int r0 = uniform(gm[0]);
  const int cl = uniform(a.cluster_of_head[h]);
  const int hs = uniform(a.slot_in_cluster[h]);
  const TG_GLOBAL int32_t* bt_row = a.bt[cl][TG_TIER_BF16] + static_cast<int64_t>(r0) * a.stride[cl][TG_TIER_BF16];
  gptr pool = a.pool[cl][TG_TIER_BF16];
  const int64_t pbytes = a.page_bytes[cl][TG_TIER_BF16];
  const int64_t head_off = static_cast<int64_t>(hs) * a.head_stride[cl][TG_TIER_BF16];
  const int p0 = t0 / kPage;
  const int np = (t1 - t0 + kPage - 1) / kPage;

  for (int pass = 0; pass < TG_GROUP_WIDTH; pass += kWavesPerBlock * M) {
    if (pass > 0 && uniform(gm[2 * pass]) < 0) break;  // no members left (same in every wavefront)
    // the previous pass's partial stores share the vector-memory counter with
    // the page loads: let them drain so that the counts below cover loads only
    wait_vmcnt<0>();
    int col_r[CT], col_slot[CT];
    tile_members<G, CT>(r0, -1, gm, pass + wave * M, col_r, col_slot);
    // a wavefront without members only helps load the pages (uniform)
    bool mine = false;
#pragma unroll
    for (int t = 0; t < CT; ++t) mine = mine || col_slot[t] >= 0;
    const bool any = __builtin_amdgcn_ballot_w64(mine) != 0;
    u32x4_t qop[CT][NQ][NK];
    load_qop<D, G, QF32, CT>(a, h, col_r, col_slot, qop);
    f32x4_t acc[CT][NT];
    float m_ref[CT], l_run[CT];
#pragma unroll
    for (int t = 0; t < CT; ++t) {
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[t][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      m_ref[t] = -INFINITY;
      l_run[t] = 0.f;
    }

    for (int w0 = 0; w0 < np; w0 += 64) {  // windows of 64 pages (an even count): pairs never straddle
      const int nw = min(64, np - w0);
      const int npair = (nw + 1) / 2;
      const int pid_lane = bt_row[p0 + w0 + min(lane, nw - 1)];
      auto issue = [&](int j) {  // pair j of the window into its slot
        TG_LDS char* dst = lds + (j % kCoopPairs) * (2 * PAGE);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int pid = __builtin_amdgcn_readlane(pid_lane, min(2 * j + e, nw - 1));
          gptr src = pool + static_cast<int64_t>(pid) * pbytes + head_off + lane * 16;
#pragma unroll
          for (int b = 0; b < PER; ++b) {
            const int blk = wave + kWavesPerBlock * b;
            __builtin_amdgcn_global_load_lds((const TG_GLOBAL void*)(src + blk * 1024),
                                             (TG_LDS void*)(dst + e * PAGE + blk * 1024), 16, 0, 0);
          }
        }
      };
      // every wavefront is done with the slots before they are loaded again
      wg_barrier();
#pragma unroll
      for (int u = 0; u < kCoopPairs - 1; ++u) issue(u);
      for (int j = 0; j < npair; ++j) {
        wait_vmcnt<(kCoopPairs - 2) * 2 * PER>();
        wg_barrier();
        issue(j + kCoopPairs - 1);
        const TG_LDS char* pg = lds + (j % kCoopPairs) * (2 * PAGE) + lane * 16;
        const int valid_a = t1 - (t0 + (w0 + 2 * j) * kPage);  // rows of page 2j in the item
        const int valid_b = valid_a - kPage;
        if (!any) continue;
#pragma unroll
        for (int t = 0; t < CT; ++t) {  // one tile after the other (fewer live registers)
          if (valid_b >= kPage)
            bf16_pair_lds<NK, NT, NQ, PAGE, false>(pg, qop[t], acc[t], m_ref[t], l_run[t], a.scale_log2, kPage,
                                                   kPage, lj);
          else
            bf16_pair_lds<NK, NT, NQ, PAGE, true>(pg, qop[t], acc[t], m_ref[t], l_run[t], a.scale_log2, valid_a,
                                                  valid_b, lj);
        }
      }
      wait_vmcnt<0>();  // the repeated requests past the last page have landed
    }
    write_partials<D, G, CT>(a, col_slot, acc, m_ref, l_run);
  }
}

// Runs plan item `w` on one wavefront: reads its fields and tables and calls
// bf16_item with the load flavour of its pages.  A group item met here (a
// plan whose group items do not lead) runs its members 16 / G at a time, one
// pass over the pages each.
template <int D, int G, bool QF32, int DEPTH>
__device__ __forceinline__ void bf16_dispatch(const SplitArgs& a, const TG_GLOBAL int32_t* w) {
  int r = uniform(w[0]);
  const int h = uniform(w[1]);
  const int t0 = uniform(w[3]), t1 = uniform(w[4]), slot = uniform(w[5]);
  const TG_GLOBAL int32_t* gm = nullptr;
  if (r < 0) {  // group item: rows [t0, t1) are the same pages for every member
    const int k = -1 - r;
    if (k >= a.n_gitems) return;
    gm = a.gitems + static_cast<int64_t>(k) * (2 * TG_GROUP_WIDTH);
    r = uniform(gm[0]);
  }
  const int cl = uniform(a.cluster_of_head[h]);
  const int hs = uniform(a.slot_in_cluster[h]);
  const int64_t head_off = static_cast<int64_t>(hs) * a.head_stride[cl][TG_TIER_BF16];
  const int rh = r * a.n_kv_heads + h;
  int t1c = t1;
  if (gm == nullptr) {
    // plans built for growth cover the reserved capacity: clip to the live rows
    t1c = min(t1, uniform(a.len[2 * rh + 1]));
    if (t0 >= t1c) {
      write_empty_partial<D, G>(a, slot);
      return;
    }
  }
  int ring_pg = 0, ring_base = 0;
  if (a.ring != nullptr) {
    ring_pg = uniform(a.ring[r * a.n_clusters + cl]);
    ring_base = uniform(a.bf_base[rh]) / kPage;
  }
  const TG_GLOBAL int32_t* bt_row = a.bt[cl][TG_TIER_BF16] + static_cast<int64_t>(r) * a.stride[cl][TG_TIER_BF16];
  gptr pool = a.pool[cl][TG_TIER_BF16];
  const int64_t pbytes = a.page_bytes[cl][TG_TIER_BF16];
  if (gm != nullptr) {
    for (int mbase = 0; mbase < TG_GROUP_WIDTH; mbase += 16 / G) {
      if (uniform(gm[2 * mbase]) < 0) break;
      bf16_item<D, G, QF32, DEPTH, false>(a, r, h, t0, t1c, -1, gm, mbase, head_off, bt_row, ring_base, ring_pg, pool,
                                          pbytes);
    }
    return;
  }
  // an item that starts on the shared radix path reads through the caches
  bool shared = false;
  if (a.n_fixed) {
    const int n_i8 = uniform(a.len[2 * rh]);
    shared = n_i8 + t0 + kPage <= uniform(a.n_fixed[r]);
  }
  if (shared)
    bf16_item<D, G, QF32, DEPTH, false>(a, r, h, t0, t1c, slot, nullptr, 0, head_off, bt_row, ring_base, ring_pg, pool,
                                        pbytes);
  else
    bf16_item<D, G, QF32, DEPTH, true>(a, r, h, t0, t1c, slot, nullptr, 0, head_off, bt_row, ring_base, ring_pg, pool,
                                       pbytes);
}

}  // namespace tg_dev

#endif  // TG_ITEM_BF16_H_
