#ifndef TG_ITEM_BF16_H_
#define TG_ITEM_BF16_H_
// Split work item, bf16 tier (gfx950): one wavefront per plan item
// (r, h, bf16, [t0, t1)) computes the online-normaliser partial of the G
// q-heads of KV-head h over rows [t0, t1) of the bf16 tier.  A group item
// does the same for up to 32 / G requests that share those pages (radix
// prefix), one set of G score columns per member (two 16-column score tiles
// past 16 / G members), in one pass over the pages.
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

// One item.  A register pipeline of DEPTH page buffers: page i + DEPTH - 1 is
// requested before page i is consumed.  Requests past the last page repeat the
// last page (an L2 hit), so every request is unconditional and the waits
// before a page's use cover exactly that page's loads.  Page ids of up to 64
// pages sit one per lane and are read with readlane.
//
// NTILE score tiles of 16 columns share every page load.  Column
// c = lg + 16 * tile belongs to member c / G (its q-head c % G).  A plain
// item has one member (r, slot); a group item's members come from `gm`, the
// (request, slot) pairs of its member table row.  With ring_pg > 0 the
// tier's pages form a ring: logical page p is table entry
// (ring_base + p) mod ring_pg.
template <int D, int G, bool QF32, int DEPTH, bool STREAM, int NTILE>
__device__ __forceinline__ void bf16_item(const SplitArgs& a, int r, int h, int t0, int t1, int slot,
                                          const TG_GLOBAL int32_t* gm, int hs,
                                          const TG_GLOBAL int32_t* bt_row, int ring_base, int ring_pg,
                                          gptr pool, int64_t pbytes) {
  constexpr int NK = D / 32;           // 1 KiB loads per K (and per V) block
  constexpr int NT = D / 16;           // 16-channel tiles of V
  constexpr int NQ = QF32 ? 2 : 1;     // bf16 pieces of q
  static_assert(G <= 16, "G must fit one MFMA tile");
  static_assert(16 * NTILE <= 2 * TG_GROUP_WIDTH, "member table too narrow");
  const int lane = threadIdx.x & 63;
  const int lg = lane & 15;
  const int lj = lane >> 4;

  // column lg + 16 tile: member request and partial slot (-1: unused column)
  int col_r[NTILE], col_slot[NTILE];
#pragma unroll
  for (int tile = 0; tile < NTILE; ++tile) {
    col_r[tile] = r;
    col_slot[tile] = (tile == 0 && lg < G) ? slot : -1;
    if (gm != nullptr) {
      const int mu = (lg + 16 * tile) / G;  // < TG_GROUP_WIDTH
      const int mr = gm[2 * mu], ms = gm[2 * mu + 1];
      col_r[tile] = mr < 0 ? r : mr;
      col_slot[tile] = mr < 0 ? -1 : ms;
    }
  }
  // Q^T operand of step s: lane (lg, lj) holds q[column lg][32 s + 8 lj + e]
  u32x4_t qop[NTILE][NQ][NK];
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

  const int64_t head_off = static_cast<int64_t>(hs) * (4 * kPage * D);
  const int lane_off = lane * 16;
  f32x4_t acc[NTILE][NT];
#pragma unroll
  for (int tile = 0; tile < NTILE; ++tile)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[tile][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref[NTILE], l_run[NTILE];  // per column: reference max (base-2 scaled score), weight sum
#pragma unroll
  for (int tile = 0; tile < NTILE; ++tile) {
    m_ref[tile] = -INFINITY;
    l_run[tile] = 0.f;
  }
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
#pragma unroll
          for (int tile = 0; tile < NTILE; ++tile) {
            if (valid >= kPage)
              bf16_page<NK, NT, NQ, false>(kb[u], vb[u], qop[tile], acc[tile], m_ref[tile], l_run[tile],
                                           a.scale_log2, kPage, lj);
            else
              bf16_page<NK, NT, NQ, true>(kb[u], vb[u], qop[tile], acc[tile], m_ref[tile], l_run[tile],
                                          a.scale_log2, valid, lj);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // partials: m and l of column lg, accumulator rows (columns) 4lj+rr
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

// Runs plan item `w` (a bf16-tier item): reads its fields and tables and
// calls bf16_item with the load flavour of its pages.
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
  // an item that starts on the shared radix path reads through the caches
  bool shared = gm != nullptr;
  if (!shared && a.n_fixed) {
    const int n_i8 = uniform(a.len[2 * rh]);
    shared = n_i8 + t0 + kPage <= uniform(a.n_fixed[r]);
  }
  // a group with members past the first 16 columns takes a second score tile
  const bool two = gm != nullptr && uniform(gm[2 * (16 / G)]) >= 0;
  if (two)
    bf16_item<D, G, QF32, DEPTH, false, 2>(a, r, h, t0, t1c, slot, gm, hs, bt_row, ring_base, ring_pg, pool,
                                           pbytes);
  else if (shared)
    bf16_item<D, G, QF32, DEPTH, false, 1>(a, r, h, t0, t1c, slot, gm, hs, bt_row, ring_base, ring_pg, pool,
                                           pbytes);
  else
    bf16_item<D, G, QF32, DEPTH, true, 1>(a, r, h, t0, t1c, slot, gm, hs, bt_row, ring_base, ring_pg, pool,
                                          pbytes);
}

}  // namespace tg_dev

#endif  // TG_ITEM_BF16_H_
