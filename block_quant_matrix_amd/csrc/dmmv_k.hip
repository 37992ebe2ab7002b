// dmmv_k.hip -- DMMV over Q4_K super-blocks (gfx950, wave64).
//
// Q4_K is GGML's 256-element super-block, bit for bit (144 bytes): fp16 d,
// fp16 dmin, twelve bytes of 6-bit sub-block scales and mins, and 128 bytes
// of nibbles in four 64-element groups; within group g, byte l holds element
// l of sub-block 2g in its low nibble and element l of sub-block 2g+1 in its
// high nibble.  An element is d*sc*q - dmin*m with q in 0..15.
//
// Against the int8 activation blocks of 32 (which line up with the 32-element
// sub-blocks), a sub-block j with activation block b contributes
//   dx_b * (d*sc_j * isum - dmin*m_j * s_b),   isum = sum q*qx,  s_b = sum qx,
// two exact integers and the block's sum of codes.
//
// Mapping: one lane per 64-element group (a "unit", two sub-blocks and two
// activation blocks).  The lane loads the 16-byte super-block header (d, dmin,
// scales: one 16-byte load, shared by the four lanes of the super-block
// through the cache) and its 32 bytes of nibbles (two 16-byte loads; every
// super-block is 16-byte aligned because 144 = 9*16).  A row slot of LPR
// lanes walks the row as in the Q4_0/Q8_0 DMMV (dmmv.hip): the lane keeps its
// units' activation codes, scales and sums in registers, issues the loads of
// RB row steps before any arithmetic, and the row partials are folded across
// lanes by RowReduce.
#include "zq_common.h"
#include "zq_internal.h"

namespace zq {

namespace {

constexpr int K4_BYTES = 144;

// activation of one unit: codes of blocks 2u and 2u+1, their scales and sums
struct KUnitAct {
  uint32_t q[2][8];
  float d[2];
  float s[2];
};

template <int LPR, int BPL>
__device__ __forceinline__ void load_unit_act(KUnitAct (&act)[BPL], const DmmvArgs &a, int pass,
                                              int j, int nu) {
#pragma unroll
  for (int i = 0; i < BPL; ++i) {
    const int u = pass * LPR * BPL + j + LPR * i;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (u < nu) {
        const int b = 2 * u + h;
        const u32x4 v0 = *reinterpret_cast<const u32x4 *>(a.qx + 32 * b);
        const u32x4 v1 = *reinterpret_cast<const u32x4 *>(a.qx + 32 * b + 16);
        act[i].q[h][0] = v0.x; act[i].q[h][1] = v0.y; act[i].q[h][2] = v0.z; act[i].q[h][3] = v0.w;
        act[i].q[h][4] = v1.x; act[i].q[h][5] = v1.y; act[i].q[h][6] = v1.z; act[i].q[h][7] = v1.w;
        act[i].d[h] = a.dx[b];
        int32_t sum;
        if (a.sx) {
          sum = a.sx[b];
        } else {
          sum = 0;
#pragma unroll
          for (int k = 0; k < 8; ++k)
            sum = __builtin_amdgcn_sdot4(static_cast<int>(act[i].q[h][k]), 0x01010101, sum, false);
        }
        act[i].s[h] = static_cast<float>(sum);  // |sum| <= 32*127: exact
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) act[i].q[h][k] = 0;
        act[i].d[h] = 0.0f;
        act[i].s[h] = 0.0f;
      }
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

template <int LPR, int BPL, int RB, bool ISUMS>
__global__ __launch_bounds__(256) void dmmv_q4k_kernel(const DmmvArgs a) {
  constexpr int S = 64 / LPR;
  const int lane = static_cast<int>(threadIdx.x & 63);
  const int j = lane & (LPR - 1);
  const int slot = lane / LPR;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t n_waves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
  const int nu = a.nb / 2;  // 64-element units per row
  const int n_pass = (nu + LPR * BPL - 1) / (LPR * BPL);
  // every unit of this lane has the same group inside its super-block
  const int grp = j & 3;

  KUnitAct act[BPL];
  if (n_pass == 1) load_unit_act<LPR, BPL>(act, a, 0, j, nu);

  for (int64_t gi = wave; gi < a.n_groups; gi += n_waves) {
    const int64_t row0 = gi * (RB * S);
    float acc[RB];
#pragma unroll
    for (int t = 0; t < RB; ++t) acc[t] = 0.0f;
    for (int pass = 0; pass < n_pass; ++pass) {
      if (n_pass > 1) load_unit_act<LPR, BPL>(act, a, pass, j, nu);
      u32x4 hdr[RB][BPL], qa[RB][BPL], qb[RB][BPL];
#pragma unroll
      for (int t = 0; t < RB; ++t) {
        int64_t row = row0 + t * S + slot;
        row = row < a.rows ? row : a.rows - 1;
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
          int u = pass * LPR * BPL + j + LPR * i;
          u = u < nu ? u : nu - 1;
          const uint8_t *sb = a.w + row * a.row_bytes + static_cast<int64_t>(u >> 2) * K4_BYTES;
          hdr[t][i] = *reinterpret_cast<const u32x4 *>(sb);
          qa[t][i] = *reinterpret_cast<const u32x4 *>(sb + 16 + 32 * (u & 3));
          qb[t][i] = *reinterpret_cast<const u32x4 *>(sb + 32 + 32 * (u & 3));
        }
      }
#pragma unroll
      for (int t = 0; t < RB; ++t) {
        float p = 0.0f;
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
          const u32x4 h = hdr[t][i];
          const float d = f16_to_f32(h.x & 0xFFFFu);
          const float dmin = f16_to_f32(h.x >> 16);
          float sc0, mn0, sc1, mn1;
          k4_scale_min(h.y, h.z, h.w, 2 * grp, sc0, mn0);
          k4_scale_min(h.y, h.z, h.w, 2 * grp + 1, sc1, mn1);
          const uint32_t w[8] = {qa[t][i].x, qa[t][i].y, qa[t][i].z, qa[t][i].w,
                                 qb[t][i].x, qb[t][i].y, qb[t][i].z, qb[t][i].w};
          int32_t is0 = 0, is1 = 0;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const uint32_t lo = w[k] & 0x0F0F0F0Fu;
            const uint32_t hi = (w[k] >> 4) & 0x0F0F0F0Fu;
            is0 = __builtin_amdgcn_sdot4(static_cast<int>(lo), static_cast<int>(act[i].q[0][k]), is0, false);
            is1 = __builtin_amdgcn_sdot4(static_cast<int>(hi), static_cast<int>(act[i].q[1][k]), is1, false);
          }
          if constexpr (ISUMS) {
            const int64_t row = row0 + t * S + slot;
            const int u = pass * LPR * BPL + j + LPR * i;
            if (row < a.rows && u < nu) {
              a.isums[row * a.nb + 2 * u] = is0;
              a.isums[row * a.nb + 2 * u + 1] = is1;
            }
          }
          const float a0 = (d * sc0) * static_cast<float>(is0);
          const float b0 = (dmin * mn0) * act[i].s[0];
          const float a1 = (d * sc1) * static_cast<float>(is1);
          const float b1 = (dmin * mn1) * act[i].s[1];
          p = __builtin_fmaf(act[i].d[0], a0 - b0, p);
          p = __builtin_fmaf(act[i].d[1], a1 - b1, p);
        }
        acc[t] += p;
      }
    }
    if constexpr (!ISUMS) {
      using R = RowReduce<LPR, RB>;
      float out[R::NOUT];
      R::run(acc, out);
      if (R::writer(lane)) {
#pragma unroll
        for (int m = 0; m < R::NOUT; ++m) {
          const int64_t row = row0 + static_cast<int64_t>(R::rowstep(m, lane)) * S + slot;
          if (row < a.rows) {
            float *yp = a.y + row;
            *yp = (a.flags & ZQ_ACCUMULATE) ? *yp + out[m] : out[m];
          }
        }
      }
    }
  }
}

struct KShape {
  int lpr, bpl;
};
// (LPR, BPL) layouts over units; any row length is served, further passes
// take the units beyond LPR*BPL.  LPR is a multiple of 4, so a lane's units
// all sit at the same group of their super-blocks.
constexpr KShape kKShapes[] = {{8, 1}, {16, 1}, {32, 1}, {64, 1}, {64, 2}, {64, 4}, {16, 5}};

KShape choose_kshape(int nu) {
  KShape best = kKShapes[0];
  int64_t best_waste = -1, best_pass = 0;
  for (const KShape &s : kKShapes) {
    const int64_t per = static_cast<int64_t>(s.lpr) * s.bpl;
    const int64_t passes = (nu + per - 1) / per;
    const int64_t waste = passes * per - nu;
    const bool better = best_waste < 0 || passes < best_pass ||
                        (passes == best_pass && waste < best_waste) ||
                        (passes == best_pass && waste == best_waste && s.lpr > best.lpr);
    if (better) {
      best = s;
      best_waste = waste;
      best_pass = passes;
    }
  }
  return best;
}

// Rows per wave group = RB * (64/LPR): the largest RB (three 16-byte loads
// per unit held per lane, RB*BPL <= 8) that still leaves >= 2048 waves.
int choose_krb(const KShape &sh, int64_t rows, bool isums) {
  if (isums) return 1;
  const int S = 64 / sh.lpr;
  const int cap = 8 / sh.bpl;
  for (int rb : {8, 4, 2, 1}) {
    if (rb > cap) continue;
    if ((rows + rb * S - 1) / (rb * S) >= 2048) return rb;
  }
  return 1;
}

template <int LPR, int BPL, int RB, bool ISUMS>
int launch_k1(DmmvArgs a, hipStream_t stream) {
  constexpr int S = 64 / LPR;
  a.n_groups = (a.rows + RB * S - 1) / (RB * S);
  const int64_t blocks = (a.n_groups + 3) / 4;
  const unsigned grid = static_cast<unsigned>(blocks < 1048576 ? blocks : 1048576);
  hipLaunchKernelGGL((dmmv_q4k_kernel<LPR, BPL, RB, ISUMS>), dim3(grid), dim3(256), 0, stream, a);
  ZQ_LAUNCH_CHECK();
  return ZQ_OK;
}

template <int LPR, int BPL, bool ISUMS>
int launch_krb(int rb, const DmmvArgs &a, hipStream_t stream) {
  if constexpr (ISUMS) return launch_k1<LPR, BPL, 1, true>(a, stream);
  switch (rb) {
    case 1: return launch_k1<LPR, BPL, 1, ISUMS>(a, stream);
    case 2: return launch_k1<LPR, BPL, 2, ISUMS>(a, stream);
    case 4: return launch_k1<LPR, BPL, 4, ISUMS>(a, stream);
    default:
      if constexpr (BPL == 1) return launch_k1<LPR, BPL, 8, ISUMS>(a, stream);
      return launch_k1<LPR, BPL, 4, ISUMS>(a, stream);
  }
}

template <bool ISUMS>
int launch_kshape(const KShape &sh, int rb, const DmmvArgs &a, hipStream_t stream) {
  if (sh.lpr == 8) return launch_krb<8, 1, ISUMS>(rb, a, stream);
  if (sh.lpr == 16 && sh.bpl == 1) return launch_krb<16, 1, ISUMS>(rb, a, stream);
  if (sh.lpr == 16) return launch_krb<16, 5, ISUMS>(rb, a, stream);
  if (sh.lpr == 32) return launch_krb<32, 1, ISUMS>(rb, a, stream);
  if (sh.bpl == 1) return launch_krb<64, 1, ISUMS>(rb, a, stream);
  if (sh.bpl == 2) return launch_krb<64, 2, ISUMS>(rb, a, stream);
  return launch_krb<64, 4, ISUMS>(rb, a, stream);
}

}  // namespace

int launch_dmmv_q4k(DmmvArgs a, bool isums, hipStream_t stream) {
  if (a.rows == 0) return ZQ_OK;
  a.row_bytes = static_cast<int64_t>(a.nb / 8) * K4_BYTES;
  const KShape sh = choose_kshape(a.nb / 2);
  const int rb = choose_krb(sh, a.rows, isums);
  if (isums) return launch_kshape<true>(sh, rb, a, stream);
  return launch_kshape<false>(sh, rb, a, stream);
}

}  // namespace zq
