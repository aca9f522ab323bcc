#ifndef TG_ITEM_I8_H_
#define TG_ITEM_I8_H_
// Split work item, INT8 tier (gfx950): one wavefront per plan item
// (r, h, INT8, [t0, t1)) computes the online-normaliser partial of the G
// q-heads of KV-head h over rows [t0, t1) of the INT8 tier, dequantising in
// registers (TTKV page, "Tier Layout" / "Tier Interaction": the slow tier is
// block-quantised; here every 64-row block has one fp16 scale per channel for
// K and one for V).
//
// Matrix-core form of a 16-row group:
//   * codes q8 become the exact fp16 values 1152 + q8 with one byte permute
//     (0x64 high byte, q8 ^ 0x80 low byte);
//   * S^T = K' Q'^T where Q' = q * s_K (per block, split into fp16 high + low
//     parts) and K' = 1152 + q8; the constant part 1152 * sum_c Q'[g][c] is
//     one extra tile per block against a constant-1152 operand and is
//     subtracted from the scores;
//   * the value sum uses V' = 1152 + q8 with the weights P split into fp16 high
//     + low parts; the constant part 1152 * sum_t P[g][t] is accumulated by the
//     same tiles against a constant-1152 operand; at the end of a block
//     acc += s_V[c] * (sum P V' - bias) folds in the per-channel V scale.
// The running accumulator lives in LDS (32 KiB per workgroup at d = 128); the
// per-block tiles live in registers.
//
// INT8 page layout per head slot (64 rows, d channels; include/tg.h):
//   K codes: row t, channel c at
//     ((t>>4)*(d/64) + (c>>6))*1024 + (((c>>3)&3)*16 + (t&15))*16 + ((c>>5)&1)*8 + (c&7)
//   V codes (at +64*d):
//     ((t>>4)*(d/64) + (c>>6))*1024 + (((t>>2)&3)*16 + (c&15))*16 + ((c>>4)&3)*4 + (t&3)
//   K scales [d] fp16 at +128*d, V scales [d] fp16 at +130*d
// so that each contiguous 1 KiB wave load holds matrix-core operands.
//
// INT4 page (d = 128): codes u = q4 + 8 in nibbles; K codes of group g (rows
// 16g..16g+15), lane l, step s (channels 32s + 8(l/16) + e) are 32-bit word
// (64g + l)*4 + s, nibble ((e&1)<<2) | (e>>1); V codes (at +32d) of lane l
// (channel l%16 of tile n, rows 16g + 4(l/16) + i) are word (64g + l)*4 + n/2,
// nibble ((i&1)<<2) | ((n&1)<<1) | (i>>1); scales at +64d (K) and +66d (V).
// A word of 8 codes becomes four fp16 operand words with one and-or each
// (and a shift per K word, one per two V words): K as 24 + q4, V as 1032 + q4
// or 72 + q4 by word.  q' goes in as two fp16 parts packed into one score
// tile (columns g and g + 8); the weights P as one fp16 part.

#include <cmath>

#include "tg_device.h"

namespace tg_dev {

constexpr uint32_t kF16x2_1152 = 0x64806480u;  // two fp16 1152.0
constexpr uint32_t kF16x2_1032 = 0x64086408u;  // two fp16 1032.0
constexpr uint32_t kF16x2_72 = 0x54805480u;    // two fp16 72.0

// 4 int8 codes (one dword) -> 4 fp16 values 1152 + q8 (two dwords)
__device__ __forceinline__ u32x2_t codes_to_f16(uint32_t w) {
  const uint32_t x = w ^ 0x80808080u;
  return u32x2_t{__builtin_amdgcn_perm(0x64646464u, x, 0x04010400u),
                 __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u)};
}

// 8 INT4 codes u = q4 + 8 (one dword, nibble k = bits 4k..4k+3) -> 8 exact
// fp16 values; word k of the result holds nibbles k and k + 4.  A nibble in
// bits 0..3 of a 16-bit half is the low mantissa of fp16 1024 (value
// 1024 + u = 1032 + q4); one in bits 4..7 sits in mantissa bits 4..7 of fp16
// 64 (value 64 + u = 72 + q4); a byte shift brings nibbles 2, 3, 6, 7 to
// those places.  Words 0 and 2 are offset by 1032, words 1 and 3 by 72.
// (x & mask) | base as one instruction.  gfx9 VOP3 encodings take no
// literal, so the compiler otherwise spends an AND and an OR (each with a
// literal) on it; here the mask comes in a scalar register and the base in a
// vector register (one scalar operand: the constant-bus limit).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t base) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(base));
  return r;
}

__device__ __forceinline__ u32x4_t nibbles_to_f16(uint32_t x) {
  const uint32_t y = x >> 8;
  return u32x4_t{and_or(x, 0x000F000Fu, 0x64006400u), and_or(x, 0x00F000F0u, 0x54005400u),
                 and_or(y, 0x000F000Fu, 0x64006400u), and_or(y, 0x00F000F0u, 0x54005400u)};
}

// The same 8 codes with every nibble in mantissa bits 6..9 of fp16 16, so
// that each value is 16 + u = 24 + q4 (word k again nibbles k and k + 4).
// Used for K: the scores subtract 24 * sum_c q'_c from sum_c (24 + q4) q'_c,
// and the small offset keeps that difference to within a few units of fp32
// rounding of the score itself at any score scale (the 1032 offset of the
// cheaper form cost ~8 bits there).
constexpr uint32_t kF16x2_24 = 0x4E004E00u;  // two fp16 24.0
__device__ __forceinline__ u32x4_t nibbles_to_f16_k(uint32_t x) {
  constexpr uint32_t kMask = 0x03C003C0u, kBase = 0x4C004C00u;  // mantissa bits 6..9 of fp16 16.0
  return u32x4_t{and_or(x << 6, kMask, kBase), and_or(x << 2, kMask, kBase), and_or(x >> 2, kMask, kBase),
                 and_or(x >> 6, kMask, kBase)};
}

// x of the lane 8 places on inside its 16-lane row (DPP row_ror:8)
__device__ __forceinline__ float ror8_in_row(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
}

__device__ __forceinline__ float half_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)));
}
__device__ __forceinline__ float half_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}

// BITS = 4: the INT4 page (include/tg.h): per 16-row group one 16-byte load
// per lane holds all d = 128 channels of K (and one all of V) as nibbles;
// K values 24 + q4 (nibbles_to_f16_k) and V values 1032 + q4 or 72 + q4 (by
// operand word, nibbles_to_f16) take the place of 1152 + q8, the constant
// tiles carry the same offsets, and the rest is unchanged.
template <int D, int G, bool QF32, int DEPTH, bool STREAM, int BITS>
__device__ __forceinline__ void i8_item(const SplitArgs& a, int r, int h, int t0, int t1, int slot,
                                        int64_t head_off, const TG_GLOBAL int32_t* bt_row, gptr pool,
                                        int64_t pbytes, float* lds) {
  static_assert(BITS == 8 || (BITS == 4 && D == 128), "INT4 pages are laid out for d = 128");
  constexpr int NL = BITS == 8 ? D / 64 : 1;  // 1 KiB loads per 16-row group (K codes, V codes)
  constexpr int CODE_BYTES = kQBlock * D * BITS / 8;  // K (or V) codes of one head's block
  // q' = q * s_K enters the matrix cores as fp16 high + low parts (~22
  // significant bits): a score's error then stays a small fraction of the
  // score at any score scale.  The weights P: two parts for INT8, one for
  // INT4 (P <= 2^kSlack, so one fp16 part bounds the relative error of every
  // weight by 2^-11 whatever the scores; the sum l takes the rounded weights).
  constexpr bool TWO = BITS == 8;  // two-part P
  // INT4: two 16-row groups form one 32-row step (one reference max, K = 32
  // products for P V), with DEPTH groups in the register pipeline, one pair
  // ahead.  (For INT8 the pair step measured slower: its two-part operands
  // already keep the matrix cores busier.)
  constexpr bool PAIR = BITS == 4;
  static_assert(!PAIR || (DEPTH % 2 == 0 && (kQBlock / kPage) % 2 == 0), "groups go in pairs");
  constexpr int NK = D / 32;           // score steps (32 channels each)
  constexpr int NT = D / 16;           // 16-channel tiles of V
  constexpr int GR = kQBlock / kPage;  // 16-row groups per block
  static_assert(G <= 16, "G must fit one MFMA tile");
  static_assert(GR % DEPTH == 0, "pipeline depth must divide the groups of a block");
  const int lane = threadIdx.x & 63;
  const int lg = lane & 15;
  const int lj = lane >> 4;
  const bool has = lg < G;
  // INT4 (PACKQ): the two fp16 parts of q' share one score tile, the high
  // part of head g in column g and the low part in column g + 8 (G <= 8), so
  // that one matrix-core product per step gives both; a rotation by 8 lanes
  // inside each 16-lane row then adds column g + 8 to column g (and g to
  // g + 8, a copy of head g that is never written out).
  constexpr bool PACKQ = BITS == 4;
  static_assert(!PACKQ || G <= 8, "packed q parts need 2G <= 16 columns");
  const int qhead = PACKQ ? (lg & 7) : lg;   // head whose q this lane holds
  const bool hasq = qhead < G;

  // q of head qhead, channels 32 s + 8 lj + e
  float qf[NK][8];
  {
    const int64_t row = static_cast<int64_t>(r) * a.n_q_heads + h * G + (hasq ? qhead : 0);
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      if constexpr (QF32) {
        const u32x4_t x0 = ldv16(a.q + (row * D + 32 * s + 8 * lj) * 4);
        const u32x4_t x1 = ldv16(a.q + (row * D + 32 * s + 8 * lj + 4) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qf[s][e] = hasq ? __uint_as_float(x0[e]) : 0.f;
          qf[s][e + 4] = hasq ? __uint_as_float(x1[e]) : 0.f;
        }
      } else {
        const u32x4_t x = ldv16(a.q + (row * D + 32 * s + 8 * lj) * 2);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qf[s][2 * e] = hasq ? __uint_as_float(x[e] << 16) : 0.f;
          qf[s][2 * e + 1] = hasq ? __uint_as_float(x[e] & 0xffff0000u) : 0.f;
        }
      }
    }
  }

  // running accumulator in LDS: this lane's rows 4lj+rr, channel 16n+lg
#pragma unroll
  for (int k = 0; k < NT * 4; ++k) lds[k * 64 + lane] = 0.f;
  float m_ref = -INFINITY;
  float l_run = 0.f;
  const int lane_off = lane * 16;
  // constant-offset operands: 1152 for every INT8 value; for INT4 the offsets
  // of the operand words (K: words 0-3 of a step; V: the two words of a tile)
  constexpr uint32_t kOffA = BITS == 8 ? kF16x2_1152 : kF16x2_1032;
  constexpr uint32_t kOffB = BITS == 8 ? kF16x2_1152 : kF16x2_72;
  constexpr uint32_t kOffK = BITS == 8 ? kF16x2_1152 : kF16x2_24;  // K operands (nibbles_to_f16_k)
  const u32x4_t c1152x8 = {kOffK, kOffK, kOffK, kOffK};
  const u32x2_t c1152x4 = {kOffA, kOffB};
  const int b0 = t0 / kQBlock;
  const int nb = (t1 - t0) / kQBlock;

  for (int w0 = 0; w0 < nb; w0 += 64) {
    const int nw = min(64, nb - w0);
    const int jb = b0 + w0 + min(lane, nw - 1);
    const int pid_lane = bt_row != nullptr ? bt_row[jb] : jb;  // no table: block j is page j
    auto blk_ptr = [&](int b) {
      const int pid = __builtin_amdgcn_readlane(pid_lane, min(b, nw - 1));
      return pool + static_cast<int64_t>(pid) * pbytes + head_off;
    };
    u32x4_t kc[DEPTH][NL], vc[DEPTH][NL];
    auto issue = [&](u32x4_t (&kk)[NL], u32x4_t (&vv)[NL], int b, int k) {
      gptr bp = blk_ptr(b) + lane_off;
#pragma unroll
      for (int L = 0; L < NL; ++L) kk[L] = ldpage<STREAM>(bp + (k * NL + L) * 1024);
#pragma unroll
      for (int L = 0; L < NL; ++L) vv[L] = ldpage<STREAM>(bp + CODE_BYTES + (k * NL + L) * 1024);
    };
    u32x4_t skraw[NK];  // K scales 32 s + 8 lj .. +8 of the next block to start
    uint32_t svraw[NT];  // V scale of channel 16 n + lg of the current block
    auto load_sk = [&](int b) {
      gptr bp = blk_ptr(b) + 2 * CODE_BYTES;
#pragma unroll
      for (int s = 0; s < NK; ++s) skraw[s] = ldv16(bp + (32 * s + 8 * lj) * 2);
    };
    load_sk(0);
#pragma unroll
    for (int u = 0; u < DEPTH - (PAIR ? 2 : 1); ++u) issue(kc[u], vc[u], 0, u);

    for (int blk = 0; blk < nw; ++blk) {
      // Q' = q * s_K as fp16 high + low parts, and the score bias of the block
      u32x4_t qop[2][NK];
#pragma unroll
      for (int s = 0; s < NK; ++s) {
        uint32_t hi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          split_f16(qf[s][2 * e] * half_lo(skraw[s][e]), hi[2 * e], lo[2 * e]);
          split_f16(qf[s][2 * e + 1] * half_hi(skraw[s][e]), hi[2 * e + 1], lo[2 * e + 1]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qop[0][s][e] = hi[2 * e] | (hi[2 * e + 1] << 16);
          qop[1][s][e] = lo[2 * e] | (lo[2 * e + 1] << 16);
          if constexpr (PACKQ) {  // columns 8.. take the low parts
            if (lg >= 8) qop[0][s][e] = qop[1][s][e];
          }
        }
      }
      f32x4_t qb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NK; ++s) {
        qb = mfma_f16_k32(c1152x8, qop[0][s], qb);
        if constexpr (!PACKQ) qb = mfma_f16_k32(c1152x8, qop[1][s], qb);
      }
      // offset * sum_c Q'[lg][c] (with PACKQ: of this column's part), the same
      // in every row
      const float qk_bias = qb[0];

      f32x4_t accb[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) accb[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      f32x4_t pbias = {0.f, 0.f, 0.f, 0.f};

      if constexpr (PAIR) {
#pragma unroll
      for (int k = 0; k < GR; k += 2) {  // groups k, k + 1 as one 32-row step
        const int kn = k + DEPTH - 2;    // groups requested now: kn, kn + 1
        issue(kc[kn % DEPTH], vc[kn % DEPTH], blk + kn / GR, kn % GR);
        issue(kc[(kn + 1) % DEPTH], vc[(kn + 1) % DEPTH], blk + (kn + 1) / GR, (kn + 1) % GR);
        if (k == 0) {
          gptr sp = blk_ptr(blk) + 2 * CODE_BYTES + 2 * D;
#pragma unroll
          for (int n = 0; n < NT; ++n) svraw[n] = *(const TG_GLOBAL uint16_t*)(sp + (16 * n + lg) * 2);
        }
        if (k == 2) load_sk(blk + 1);
        __builtin_amdgcn_sched_barrier(0);
        const int u0 = k % DEPTH, u1 = (k + 1) % DEPTH;
        f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NK; ++s) {
          u32x4_t A0, A1;
          if constexpr (BITS == 8) {
            const u32x4_t x0 = kc[u0][s / 2], x1 = kc[u1][s / 2];
            const u32x2_t c00 = codes_to_f16(x0[(s % 2) * 2]), c01 = codes_to_f16(x0[(s % 2) * 2 + 1]);
            const u32x2_t c10 = codes_to_f16(x1[(s % 2) * 2]), c11 = codes_to_f16(x1[(s % 2) * 2 + 1]);
            A0 = u32x4_t{c00[0], c00[1], c01[0], c01[1]};
            A1 = u32x4_t{c10[0], c10[1], c11[0], c11[1]};
          } else {
            A0 = nibbles_to_f16_k(kc[u0][0][s]);
            A1 = nibbles_to_f16_k(kc[u1][0][s]);
          }
          s0 = mfma_f16_k32(A0, qop[0][s], s0);
          s1 = mfma_f16_k32(A1, qop[0][s], s1);
          if constexpr (!PACKQ) {
            s0 = mfma_f16_k32(A0, qop[1][s], s0);
            s1 = mfma_f16_k32(A1, qop[1][s], s1);
          }
        }
        float sc[8];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          float d0 = s0[rr] - qk_bias, d1 = s1[rr] - qk_bias;
          if constexpr (PACKQ) {  // + the other part, 8 lanes on in the row
            d0 += ror8_in_row(d0);
            d1 += ror8_in_row(d1);
          }
          sc[rr] = d0 * a.scale_log2;
          sc[4 + rr] = d1 * a.scale_log2;
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
            for (int n = 0; n < NT; ++n) {
              accb[n][rr] *= ar;
              lds[(4 * n + rr) * 64 + lane] *= ar;
            }
            pbias[rr] *= ar;
          }
          m_ref = mn;
        }
        uint32_t ph[8], pl[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pw = __builtin_amdgcn_exp2f(sc[e] - m_ref);
          split_f16(pw, ph[e], pl[e]);
          l_run += TWO ? pw : static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(ph[e])));
        }
        const u32x4_t Ph = {ph[0] | (ph[1] << 16), ph[2] | (ph[3] << 16), ph[4] | (ph[5] << 16), ph[6] | (ph[7] << 16)};
        const u32x4_t Pl = {pl[0] | (pl[1] << 16), pl[2] | (pl[3] << 16), pl[4] | (pl[5] << 16), pl[6] | (pl[7] << 16)};
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          u32x2_t B0, B1;
          if constexpr (BITS == 8) {
            B0 = codes_to_f16(vc[u0][n / 4][n % 4]);
            B1 = codes_to_f16(vc[u1][n / 4][n % 4]);
          } else {
            const u32x4_t f0 = nibbles_to_f16(vc[u0][0][n / 2]), f1 = nibbles_to_f16(vc[u1][0][n / 2]);
            B0 = (n & 1) ? u32x2_t{f0[2], f0[3]} : u32x2_t{f0[0], f0[1]};
            B1 = (n & 1) ? u32x2_t{f1[2], f1[3]} : u32x2_t{f1[0], f1[1]};
          }
          const u32x4_t B = {B0[0], B0[1], B1[0], B1[1]};
          accb[n] = mfma_f16_k32(Ph, B, accb[n]);
          if constexpr (TWO) accb[n] = mfma_f16_k32(Pl, B, accb[n]);
        }
        const u32x4_t c2 = {c1152x4[0], c1152x4[1], c1152x4[0], c1152x4[1]};
        pbias = mfma_f16_k32(Ph, c2, pbias);
        if constexpr (TWO) pbias = mfma_f16_k32(Pl, c2, pbias);
        __builtin_amdgcn_sched_barrier(0);
      }
      } else {
#pragma unroll
      for (int k = 0; k < GR; ++k) {
        const int kn = k + DEPTH - 1;  // group requested now: block blk + kn/GR, group kn%GR
        issue(kc[kn % DEPTH], vc[kn % DEPTH], blk + kn / GR, kn % GR);
        if (k == 1) {
          gptr sp = blk_ptr(blk) + 2 * CODE_BYTES + 2 * D;
#pragma unroll
          for (int n = 0; n < NT; ++n) svraw[n] = *(const TG_GLOBAL uint16_t*)(sp + (16 * n + lg) * 2);
        }
        if (k == 2) load_sk(blk + 1);
        __builtin_amdgcn_sched_barrier(0);
        const int u = k % DEPTH;
        // scores of rows 4lj..4lj+3 for head lg
        f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NK; ++s) {
          u32x4_t A;
          if constexpr (BITS == 8) {
            const u32x4_t x = kc[u][s / 2];
            const u32x2_t c0 = codes_to_f16(x[(s % 2) * 2]);
            const u32x2_t c1 = codes_to_f16(x[(s % 2) * 2 + 1]);
            A = u32x4_t{c0[0], c0[1], c1[0], c1[1]};
          } else {
            A = nibbles_to_f16_k(kc[u][0][s]);  // channels 32 s + 8 lj + e, e < 8
          }
          sacc = mfma_f16_k32(A, qop[0][s], sacc);
          sacc = mfma_f16_k32(A, qop[1][s], sacc);
        }
        float sc[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) sc[rr] = (sacc[rr] - qk_bias) * a.scale_log2;
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
            for (int n = 0; n < NT; ++n) {
              accb[n][rr] *= ar;
              lds[(4 * n + rr) * 64 + lane] *= ar;
            }
            pbias[rr] *= ar;
          }
          m_ref = mn;
        }
        float pw[4];
        uint32_t ph[4], pl[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          pw[rr] = __builtin_amdgcn_exp2f(sc[rr] - m_ref);
          split_f16(pw[rr], ph[rr], pl[rr]);
          // with one part, the sum takes the rounded weights the products use
          l_run += TWO ? pw[rr] : static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(ph[rr])));
        }
        const u32x2_t Ph = {ph[0] | (ph[1] << 16), ph[2] | (ph[3] << 16)};
        const u32x2_t Pl = {pl[0] | (pl[1] << 16), pl[2] | (pl[3] << 16)};
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          u32x2_t B;
          if constexpr (BITS == 8) {
            B = codes_to_f16(vc[u][n / 4][n % 4]);
          } else {  // word n/2 holds tiles n & ~1 (values 0, 1) and n | 1 (values 2, 3)
            const u32x4_t f = nibbles_to_f16(vc[u][0][n / 2]);
            B = (n & 1) ? u32x2_t{f[2], f[3]} : u32x2_t{f[0], f[1]};
          }
          accb[n] = mfma_f16_k16(Ph, B, accb[n]);
          if constexpr (TWO) accb[n] = mfma_f16_k16(Pl, B, accb[n]);
        }
        pbias = mfma_f16_k16(Ph, c1152x4, pbias);
        if constexpr (TWO) pbias = mfma_f16_k16(Pl, c1152x4, pbias);
        __builtin_amdgcn_sched_barrier(0);
      }
      }
      // end of block: fold in the V scales
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const float sv = half_lo(svraw[n]);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) lds[(4 * n + rr) * 64 + lane] += sv * (accb[n][rr] - pbias[rr]);
      }
    }
  }

  const float l_tot = xor32_sum(xor16_sum(l_run));
  TG_GLOBAL float* acc_out = a.ws_acc + static_cast<int64_t>(slot) * G * D;
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int g = 4 * lj + rr;
    if (g < G) {
#pragma unroll
      for (int n = 0; n < NT; ++n) acc_out[g * D + 16 * n + lg] = lds[(4 * n + rr) * 64 + lane];
    }
  }
  if (lj == 0 && has) {
    a.ws_ml[(static_cast<int64_t>(slot) * G + lg) * 2 + 0] = m_ref * kLn2;
    a.ws_ml[(static_cast<int64_t>(slot) * G + lg) * 2 + 1] = l_tot;
  }
}

// Floats of LDS accumulator one wavefront needs for an INT8 item.
template <int D>
constexpr int kI8LdsFloats = (D / 16) * 4 * 64;

// Runs plan item `w` (an INT8-tier item) with `lds` as the wave's
// accumulator (kI8LdsFloats<D> floats).
template <int D, int G, bool QF32, int DEPTH, int BITS = 8>
__device__ __forceinline__ void i8_dispatch(const SplitArgs& a, const TG_GLOBAL int32_t* w, float* lds) {
  const int r = uniform(w[0]), h = uniform(w[1]);
  const int t0 = uniform(w[3]), slot = uniform(w[5]);
  // plans built for growth cover the reserved capacity: clip to the live rows
  const int t1 = min(uniform(w[4]), uniform(a.len[2 * (r * a.n_kv_heads + h)]));
  if (t0 >= t1) {
    write_empty_partial<D, G>(a, slot);
    return;
  }
  const int cl = uniform(a.cluster_of_head[h]);
  const int hs = uniform(a.slot_in_cluster[h]);
  const int64_t head_off = static_cast<int64_t>(hs) * a.head_stride[cl][TG_TIER_I8];
  const TG_GLOBAL int32_t* bt_row =
      a.bt[cl][TG_TIER_I8] != nullptr ? a.bt[cl][TG_TIER_I8] + static_cast<int64_t>(r) * a.stride[cl][TG_TIER_I8]
                                      : nullptr;
  gptr pool = a.pool[cl][TG_TIER_I8];
  const int64_t pbytes = a.page_bytes[cl][TG_TIER_I8];
  bool shared = false;  // an item that starts on the shared radix path reads through the caches
  if (a.n_fixed) shared = t0 + kQBlock <= uniform(a.n_fixed[r]);
  if (shared)
    i8_item<D, G, QF32, DEPTH, false, BITS>(a, r, h, t0, t1, slot, head_off, bt_row, pool, pbytes, lds);
  else
    i8_item<D, G, QF32, DEPTH, true, BITS>(a, r, h, t0, t1, slot, head_off, bt_row, pool, pbytes, lds);
}

}  // namespace tg_dev

#endif  // TG_ITEM_I8_H_
