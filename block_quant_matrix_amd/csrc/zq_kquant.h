// zq_kquant.h -- device pieces of the K-quant super-block kernels (gfx950):
// the format traits, one lane's weight-unit loads, and its unit dot
// product against an int8 activation held in registers (the layouts and the
// lane mapping are described in dmmv_k.hip).  Shared by the K-quant DMMV and
// the K-quant MoE gate/up pass.  Nothing here is shared with the CPU oracle.
#pragma once

#include "zq_common.h"

namespace zq {

template <int WT> struct KQ;
// NWD: dwords of one unit's weights held between load and arithmetic
template <> struct KQ<ZQ_Q4_K> { static constexpr int BYTES = 144; static constexpr int NWD = 12; };
template <> struct KQ<ZQ_Q5_K> { static constexpr int BYTES = 176; static constexpr int NWD = 20; };
// Q6_K: three 5-dword windows, a 3-dword scale window, d, the window offset
template <> struct KQ<ZQ_Q6_K> { static constexpr int BYTES = 210; static constexpr int NWD = 20; };

// Activation of one unit.  Q4_K / Q5_K: codes of blocks 2u (q[0..7]) and
// 2u+1 (q[8..15]), their scales d[0..1] and code sums fs[0..1].  Q6_K: for
// c = 0..3 the 16 codes q[4c..4c+3] of the unit's run in quarter c, that
// block's scale d[c] and minus 32 times the run's code sum, m32[c].
// load_unit_act only issues the loads (raw block sums in sraw); finish_act
// derives the sums once the wave's weight loads are in flight, so a wave
// never waits on the activation before its weights are requested.
struct KUnitAct {
  uint32_t q[16];
  float d[4];
  int32_t sraw[2];
  float fs[2];
  int32_t m32[4];
};

__device__ __forceinline__ int32_t code_sum(const uint32_t *q, int n) {
  int32_t s = 0;
  for (int k = 0; k < n; ++k) s = __builtin_amdgcn_sdot4(static_cast<int>(q[k]), 0x01010101, s, false);
  return s;
}

// 5 dwords starting at p rounded down to 4 (p is 2-byte aligned).
__device__ __forceinline__ void load5(const uint8_t *p, uint32_t *w) {
  const g_u32 *pw = (const g_u32 *)(reinterpret_cast<uintptr_t>(p) & ~uintptr_t(3));
  const u32x4a4 v = *(const g_u32x4a4 *)pw;
  w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  w[4] = pw[4];
}

// Issue the loads of one unit of super-block sb for a lane at position p.
template <int WT>
__device__ __forceinline__ void load_unit_w(const uint8_t *sb, int p, uint32_t (&v)[KQ<WT>::NWD]) {
  if constexpr (WT == ZQ_Q6_K) {
    const int h = p >> 1, t = p & 1;
    const uint8_t *ql = sb + 64 * h + 16 * t;
    load5(ql, &v[0]);                           // low bits, quarters 0 and 2
    load5(ql + 32, &v[5]);                      // low bits, quarters 1 and 3
    load5(sb + 128 + 32 * h + 16 * t, &v[10]);  // high bits
    // scales 8h..8h+7 live at sb+192+8h; the 3-dword window from
    // (sb+190+8h) rounded down to 4 ends at or before sb+210
    const g_u32 *ps = (const g_u32 *)(reinterpret_cast<uintptr_t>(sb + 190 + 8 * h) & ~uintptr_t(3));
    v[15] = ps[0]; v[16] = ps[1]; v[17] = ps[2];
    v[18] = *(const __attribute__((address_space(1))) uint16_t *)(sb + 208);
    v[19] = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(sb) & 3u);  // 0 or 2
  } else {
    constexpr int QS = WT == ZQ_Q4_K ? 16 : 48;
    const u32x4 h = *reinterpret_cast<const u32x4 *>(sb);
    const u32x4 q0 = *reinterpret_cast<const u32x4 *>(sb + QS + 32 * p);
    const u32x4 q1 = *reinterpret_cast<const u32x4 *>(sb + QS + 16 + 32 * p);
    v[0] = h.x; v[1] = h.y; v[2] = h.z; v[3] = h.w;
    v[4] = q0.x; v[5] = q0.y; v[6] = q0.z; v[7] = q0.w;
    v[8] = q1.x; v[9] = q1.y; v[10] = q1.z; v[11] = q1.w;
    if constexpr (WT == ZQ_Q5_K) {
      const u32x4 e0 = *reinterpret_cast<const u32x4 *>(sb + 16);
      const u32x4 e1 = *reinterpret_cast<const u32x4 *>(sb + 32);
      v[12] = e0.x; v[13] = e0.y; v[14] = e0.z; v[15] = e0.w;
      v[16] = e1.x; v[17] = e1.y; v[18] = e1.z; v[19] = e1.w;
    }
  }
}

// The 6-bit scale and min of sub-block j (0..7) from the scale bytes held in
// the dwords s0 (bytes 0-3), s1 (4-7), s2 (8-11): sub-blocks 0-3 keep scale
// and min in the low 6 bits of byte j and j+4; sub-blocks 4-7 keep their low
// 4 bits in the nibbles of byte j+4 and their top 2 bits in the top bits of
// bytes j-4 (scale) and j (min).
__device__ __forceinline__ void k4_scale_min(uint32_t s0, uint32_t s1, uint32_t s2, int j,
                                             float &sc, float &mn) {
  const uint32_t sh = 8u * static_cast<uint32_t>(j & 3);
  const uint32_t b0 = (s0 >> sh) & 0xFFu;
  const uint32_t b1 = (s1 >> sh) & 0xFFu;
  const uint32_t b2 = (s2 >> sh) & 0xFFu;
  uint32_t c, m;
  if (j < 4) {
    c = b0 & 63u;
    m = b1 & 63u;
  } else {
    c = (b2 & 15u) | ((b0 >> 6) << 4);
    m = (b2 >> 4) | ((b1 >> 6) << 4);
  }
  sc = static_cast<float>(c);
  mn = static_cast<float>(m);
}

// The unit's contribution to its row, and its integer sums: Q4_K / Q5_K
// is[0..1] = isum of blocks 2u, 2u+1; Q6_K is[c] = sc*sum (q-32)*qx over the
// lane's 16 elements of quarter c.
template <int WT>
__device__ __forceinline__ float unit_dot(const uint32_t (&v)[KQ<WT>::NWD], int p,
                                          const KUnitAct &A, int32_t (&is)[4]) {
  if constexpr (WT == ZQ_Q6_K) {
    const uint32_t o = v[19];
    const uint32_t sel = 0x03020100u + o * 0x01010101u;         // bytes o..o+3
    const uint32_t sels = 0x03020100u + (4u - o) * 0x01010101u;  // scale window offset 4-o
    uint32_t l0[4], l1[4], hb[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      l0[k] = __builtin_amdgcn_perm(v[k + 1], v[k], sel);
      l1[k] = __builtin_amdgcn_perm(v[k + 6], v[k + 5], sel);
      hb[k] = __builtin_amdgcn_perm(v[k + 11], v[k + 10], sel);
    }
    const uint32_t s01 = __builtin_amdgcn_perm(v[16], v[15], sels);  // scales 8h..8h+3
    const uint32_t s23 = __builtin_amdgcn_perm(v[17], v[16], sels);  // scales 8h+4..8h+7
    const int t8 = 8 * (p & 1);
    const int sc[4] = {static_cast<int8_t>(s01 >> t8), static_cast<int8_t>(s01 >> (t8 + 16)),
                       static_cast<int8_t>(s23 >> t8), static_cast<int8_t>(s23 >> (t8 + 16))};
    float part = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      // sum (q - 32) * qx over the run: the dot chain starts at -32 * sum qx
      int32_t s = A.m32[c];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t lw = (c & 1) ? l1[k] : l0[k];
        const uint32_t lo = (c < 2 ? lw : lw >> 4) & 0x0F0F0F0Fu;
        const uint32_t hi = c < 3 ? (hb[k] << (4 - 2 * c)) & 0x30303030u : (hb[k] >> 2) & 0x30303030u;
        s = __builtin_amdgcn_sdot4(static_cast<int>(lo | hi), static_cast<int>(A.q[4 * c + k]), s, false);
      }
      is[c] = __mul24(sc[c], s);  // |.| <= 128*32*127*16 < 2^24: exact in 24-bit
      part = __builtin_fmaf(A.d[c], static_cast<float>(is[c]), part);
    }
    return f16_to_f32(v[18]) * part;
  } else {
    const float d = f16_to_f32(v[0] & 0xFFFFu);
    const float dmin = f16_to_f32(v[0] >> 16);
    float sc0, mn0, sc1, mn1;
    k4_scale_min(v[1], v[2], v[3], 2 * p, sc0, mn0);
    k4_scale_min(v[1], v[2], v[3], 2 * p + 1, sc1, mn1);
    int32_t is0 = 0, is1 = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      uint32_t lo = v[4 + k] & 0x0F0F0F0Fu;
      uint32_t hi = (v[4 + k] >> 4) & 0x0F0F0F0Fu;
      if constexpr (WT == ZQ_Q5_K) {
        const uint32_t e = v[12 + k] >> (2 * p);
        lo |= (e << 4) & 0x10101010u;
        hi |= (e << 3) & 0x10101010u;
      }
      is0 = __builtin_amdgcn_sdot4(static_cast<int>(lo), static_cast<int>(A.q[k]), is0, false);
      is1 = __builtin_amdgcn_sdot4(static_cast<int>(hi), static_cast<int>(A.q[8 + k]), is1, false);
    }
    is[0] = is0;
    is[1] = is1;
    const float a0 = (d * sc0) * static_cast<float>(is0);
    const float b0 = (dmin * mn0) * A.fs[0];
    const float a1 = (d * sc1) * static_cast<float>(is1);
    const float b1 = (dmin * mn1) * A.fs[1];
    return __builtin_fmaf(A.d[1], a1 - b1, A.d[0] * (a0 - b0));
  }
}

}  // namespace zq
