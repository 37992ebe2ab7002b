// dmmv_k.hip -- DMMV over GGML K-quant super-blocks: Q4_K, Q5_K, Q6_K
// (gfx950, wave64).
//
// The three formats hold 256 elements per super-block, bit for bit as GGML
// stores them:
//   Q4_K (144 B): fp16 d, fp16 dmin, twelve bytes of 6-bit sub-block scales
//     and mins, then 128 bytes of nibbles in four 64-element groups; within
//     group g, byte l holds element l of sub-block 2g in its low nibble and
//     element l of sub-block 2g+1 in its high nibble.  Element: d*sc*q -
//     dmin*m, q in 0..15.
//   Q5_K (176 B): as Q4_K with 32 bytes of fifth bits between the scales and
//     the nibbles: bit 2g (2g+1) of byte l is the fifth bit of element l of
//     sub-block 2g (2g+1).  q in 0..31.
//   Q6_K (210 B): 128 bytes of low nibbles, 64 bytes of 2-bit highs, sixteen
//     int8 scales of 16-element sub-blocks, fp16 d last.  In half h (128
//     elements), element 32c+l (c = 0..3, l = 0..31) takes its low 4 bits
//     from byte 64h+32(c&1)+l (low nibble for c < 2, high for c >= 2) and its
//     top 2 bits from bits 2c..2c+1 of high byte 32h+l.  Element:
//     d*sc*(q-32), q in 0..63.
//
// Against the int8 activation blocks of 32 (aligned with the sub-blocks):
//   Q4_K / Q5_K: block b (sub-block j) adds dx_b*(d*sc_j*isum - dmin*m_j*s_b),
//     isum = sum q*qx and s_b = sum qx, both exact integers;
//   Q6_K: block b (two 16-element sub-blocks) adds dx_b*d*isum_b with
//     isum_b = sum sc*(q-32)*qx over its 32 elements, an exact integer.
//
// Mapping: one lane per "unit" of 64 elements, four units per super-block;
// a lane's position p = 0..3 inside its super-blocks is fixed (LPR is a
// multiple of 4).  Q4_K / Q5_K unit p is group p (sub-blocks 2p, 2p+1: one
// 16-byte header load shared by the super-block's four lanes through the
// cache, 32 bytes of nibbles, and for Q5_K the 32 bytes of fifth bits).
// Q6_K unit p is half h = p>>1, elements l in [16t, 16t+16) with t = p&1, of
// all four quarters c: its low bits are two 16-byte runs, its high bits one,
// all disjoint between the four lanes; since 210-byte super-blocks are only
// 2-byte aligned, each run is read as a 5-dword window and realigned with
// v_perm_b32, and no window reaches past its super-block's own 210 bytes.
// A row slot of LPR lanes walks the row as in the Q4_0 / Q8_0 DMMV
// (dmmv.hip): activation codes, scales and sums of the lane's units stay in
// registers, the loads of RB row steps are issued before any arithmetic, and
// row partials are folded across lanes by RowReduce.
#include "zq_common.h"
#include "zq_f32in.h"
#include "zq_internal.h"
#include "zq_kquant.h"

namespace zq {

namespace {

// Loads only.  Units past the row end load the row's last unit; their
// scales are zeroed in finish_act.
template <int WT, int LPR, int BPL>
__device__ __forceinline__ void load_unit_act(KUnitAct (&act)[BPL], const DmmvArgs &a, int s,
                                              int pass, int j, int nu) {
  // slot s's activation; block sums come from sx when given, otherwise the
  // loads read dx (any valid address) and finish_act sums the codes
  const int8_t *qx = a.qx + static_cast<int64_t>(s) * a.x_stride;
  const float *dx = a.dx + static_cast<int64_t>(s) * (a.x_stride / 32);
  const int32_t *sxp = a.sx ? a.sx + static_cast<int64_t>(s) * (a.x_stride / 32)
                            : reinterpret_cast<const int32_t *>(dx);
#pragma unroll
  for (int i = 0; i < BPL; ++i) {
    int u = pass * LPR * BPL + j + LPR * i;
    u = u < nu ? u : nu - 1;
    KUnitAct &A = act[i];
    if constexpr (WT == ZQ_Q6_K) {
      const int base = 256 * (u >> 2) + 128 * ((u >> 1) & 1) + 16 * (u & 1);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int e0 = base + 32 * c;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(qx + e0);
        A.q[4 * c] = v.x; A.q[4 * c + 1] = v.y; A.q[4 * c + 2] = v.z; A.q[4 * c + 3] = v.w;
        A.d[c] = dx[e0 >> 5];
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int b = 2 * u + h;
        const u32x4 v0 = *reinterpret_cast<const u32x4 *>(qx + 32 * b);
        const u32x4 v1 = *reinterpret_cast<const u32x4 *>(qx + 32 * b + 16);
        uint32_t *q = &A.q[8 * h];
        q[0] = v0.x; q[1] = v0.y; q[2] = v0.z; q[3] = v0.w;
        q[4] = v1.x; q[5] = v1.y; q[6] = v1.z; q[7] = v1.w;
        A.d[h] = dx[b];
        A.sraw[h] = sxp[b];
      }
    }
  }
}

// The arithmetic half of the activation set-up (no loads, so the counters
// of outstanding loads are the same on every path).
template <int WT, int LPR, int BPL>
__device__ __forceinline__ void finish_act(KUnitAct (&act)[BPL], const DmmvArgs &a, int pass,
                                           int j, int nu) {
#pragma unroll
  for (int i = 0; i < BPL; ++i) {
    const bool ok = pass * LPR * BPL + j + LPR * i < nu;
    KUnitAct &A = act[i];
    if constexpr (WT == ZQ_Q6_K) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        A.m32[c] = -32 * code_sum(&A.q[4 * c], 4);
        A.d[c] = ok ? A.d[c] : 0.0f;
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int32_t sum = a.sx ? A.sraw[h] : code_sum(&A.q[8 * h], 8);
        A.fs[h] = static_cast<float>(sum);  // |sum| <= 32*127: exact
        A.d[h] = ok ? A.d[h] : 0.0f;
      }
    }
  }
}

// The occupancy target is capped at 2 waves per SIMD: aiming higher, the
// scheduler trades the loads of later row steps (issued together, so a wave
// has all its bytes in flight at once) for registers and serialises them.
//
// MODE: MODE_PLAIN / MODE_ISUMS (one matrix), MODE_GATHER (grid.y = slot s:
// y[s] = W[e_s] . x_s), MODE_WEIGHTED (every slot: y = sum_s wts[s] W[e_s]
// . x_s, folded into the row partials before the lane reduction); expert
// e_s = ids[s] - id_base, skipped (and reported) outside [0, n_experts).
template <int WT, int LPR, int BPL, int RB, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void dmmv_k_kernel(
    const uint8_t *w, const int8_t *qx, const float *dx, int64_t rows, int64_t row_bytes,
    int64_t n_groups, int32_t nb, int32_t id_base, const DmmvArgs a_in) {
  DmmvArgs a = a_in;
  dmmv_hot(a, w, qx, dx, rows, row_bytes, n_groups, nb, id_base);
  constexpr bool ISUMS = MODE == MODE_ISUMS;
  constexpr int S = 64 / LPR;
  constexpr int NWD = KQ<WT>::NWD;
  const int lane = static_cast<int>(threadIdx.x & 63);
  const int j = lane & (LPR - 1);
  const int slot = lane / LPR;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t n_waves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
  const int nu = a.nb / 2;  // 64-element units per row
  const int n_pass = (nu + LPR * BPL - 1) / (LPR * BPL);
  const int p = j & 3;      // the lane's unit position in every super-block it visits

  int s0 = 0, s1 = 1;
  if constexpr (MODE == MODE_GATHER) {
    s0 = static_cast<int>(blockIdx.y);
    s1 = s0 + 1;
    const int e = a.ids[s0] - a.id_base;
    if (e < 0 || e >= a.n_experts) {  // uniform over the workgroup
      if (a.status) *a.status = ZQ_ERANGE;
      return;
    }
  } else if constexpr (MODE == MODE_WEIGHTED) {
    s1 = a.n_sel;
  }

  KUnitAct act[BPL];
  const bool hoist = (n_pass == 1) && (MODE != MODE_WEIGHTED);
  if (hoist) load_unit_act<WT, LPR, BPL>(act, a, s0, 0, j, nu);

  for (int64_t gi = wave; gi < a.n_groups; gi += n_waves) {
    const int64_t row0 = gi * (RB * S);
    float acc[RB];
#pragma unroll
    for (int t = 0; t < RB; ++t) acc[t] = 0.0f;
    for (int s = s0; s < s1; ++s) {
      const uint8_t *wb = a.w;
      float ws = 1.0f;
      if constexpr (MODE == MODE_GATHER || MODE == MODE_WEIGHTED) {
        const int e = a.ids[s] - a.id_base;
        if (e < 0 || e >= a.n_experts) {
          if (a.status) *a.status = ZQ_ERANGE;
          continue;
        }
        wb = a.w + static_cast<int64_t>(e) * a.expert_stride;
        if constexpr (MODE == MODE_WEIGHTED) ws = a.wts[s];
      }
      for (int pass = 0; pass < n_pass; ++pass) {
        if (!hoist) load_unit_act<WT, LPR, BPL>(act, a, s, pass, j, nu);
        uint32_t v[RB][BPL][NWD];
#pragma unroll
        for (int t = 0; t < RB; ++t) {
          int64_t row = row0 + t * S + slot;
          row = row < a.rows ? row : a.rows - 1;
#pragma unroll
          for (int i = 0; i < BPL; ++i) {
            int u = pass * LPR * BPL + j + LPR * i;
            u = u < nu ? u : nu - 1;
            const uint8_t *sb = wb + row * a.row_bytes + static_cast<int64_t>(u >> 2) * KQ<WT>::BYTES;
            load_unit_w<WT>(sb, p, v[t][i]);
          }
        }
        // re-derived every group: a few dot4 per unit, no loads
        finish_act<WT, LPR, BPL>(act, a, pass, j, nu);
#pragma unroll
        for (int t = 0; t < RB; ++t) {
          float part = 0.0f;
#pragma unroll
          for (int i = 0; i < BPL; ++i) {
            int32_t is[4];
            part += unit_dot<WT>(v[t][i], p, act[i], is);
            if constexpr (ISUMS) {
              const int64_t row = row0 + t * S + slot;
              const int u = pass * LPR * BPL + j + LPR * i;
              if constexpr (WT == ZQ_Q6_K) {
                // a block's two 16-element runs sit in lanes p and p^1
                int32_t blk[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) blk[c] = is[c] + __shfl_xor(is[c], 1);
                if (row < a.rows && u < nu && (p & 1) == 0) {
                  int32_t *dst = a.isums + row * a.nb + 8 * (u >> 2) + 4 * (p >> 1);
#pragma unroll
                  for (int c = 0; c < 4; ++c) dst[c] = blk[c];
                }
              } else {
                if (row < a.rows && u < nu) {
                  a.isums[row * a.nb + 2 * u] = is[0];
                  a.isums[row * a.nb + 2 * u + 1] = is[1];
                }
              }
            }
          }
          if constexpr (MODE == MODE_WEIGHTED) {
            acc[t] = __builtin_fmaf(ws, part, acc[t]);
          } else {
            acc[t] += part;
          }
        }
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
            if constexpr (MODE == MODE_GATHER) yp += static_cast<int64_t>(s0) * a.rows;
            *yp = (a.flags & ZQ_ACCUMULATE) ? *yp + out[m] : out[m];
          }
        }
      }
    }
  }
}

// The weighted sum over experts with the experts spread over the lanes:
// for rows of LPR units (k = 64 * LPR, one pass), a wave holds 64 / LPR
// slots side by side, lane = (slot, unit), and reduces over all 64 lanes,
// so the selected experts' rows are requested together instead of one
// expert after another.  Slots beyond 64 / LPR take further rounds.  Each
// lane folds its slot's weight into its partial; a lane whose expert id is
// out of range contributes nothing and reports ZQ_ERANGE.
//
// SWT (ZQ_Q4_0 / ZQ_Q8_0, or 0 for none): the shared expert a.w2 in a
// block format joins the same reduction: for each row step t, 64 / RB lanes
// take the row's k / 32 blocks against slot n_sel's activation, weighted by
// wts[n_sel].
template <int WT, int LPR, int RB, int SWT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void dmmv_k_wsum_kernel(
    const int32_t *ids, const float *wts, const int8_t *qx, const float *dx, int64_t n_groups,
    int32_t n_sel, int32_t nb, int32_t id_base, const DmmvArgs a_in) {
  // leading scalars: preloaded kernel arguments (as dmmv_hot)
  DmmvArgs a = a_in;
  a.ids = ids;
  a.wts = wts;
  a.qx = qx;
  a.dx = dx;
  a.n_groups = n_groups;
  a.n_sel = n_sel;
  a.nb = nb;
  a.id_base = id_base;
  constexpr int SL = 64 / LPR;
  constexpr int NWD = KQ<WT>::NWD;
  constexpr int LS = 64 / RB;                       // shared: lanes per row step
  constexpr int NBK = 2 * LPR;                      // blocks per row
  constexpr int BS = (NBK + LS - 1) / LS;           // shared: blocks per lane
  const int lane = static_cast<int>(threadIdx.x & 63);
  const int j = lane & (LPR - 1);
  const int sl = lane / LPR;
  const int p = j & 3;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t n_waves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
  const int n_rounds = (a.n_sel + SL - 1) / SL;

  KUnitAct act[1];
  const bool hoist = n_rounds == 1;
  if (hoist && a.n_sel > 0) {
    load_unit_act<WT, LPR, 1>(act, a, sl < a.n_sel ? sl : a.n_sel - 1, 0, j, LPR);
  }
  for (int64_t gi = wave; gi < a.n_groups; gi += n_waves) {
    const int64_t row0 = gi * RB;
    float acc[RB];
#pragma unroll
    for (int t = 0; t < RB; ++t) acc[t] = 0.0f;
    for (int r = 0; r < n_rounds; ++r) {
      const int s = r * SL + sl;
      const bool in = s < a.n_sel;
      const int sc = in ? s : a.n_sel - 1;
      const int e = a.ids[sc] - a.id_base;
      const bool ok = in && e >= 0 && e < a.n_experts;
      if (in && !ok && a.status) *a.status = ZQ_ERANGE;
      const float ws = a.wts[sc];
      const uint8_t *wb = a.w + static_cast<int64_t>(ok ? e : 0) * a.expert_stride;
      if (!hoist) load_unit_act<WT, LPR, 1>(act, a, sc, 0, j, LPR);
      uint32_t v[RB][NWD];
#pragma unroll
      for (int t = 0; t < RB; ++t) {
        int64_t row = row0 + t;
        row = row < a.rows ? row : a.rows - 1;
        load_unit_w<WT>(wb + row * a.row_bytes + static_cast<int64_t>(j >> 2) * KQ<WT>::BYTES, p,
                        v[t]);
      }
      finish_act<WT, LPR, 1>(act, a, 0, j, LPR);
#pragma unroll
      for (int t = 0; t < RB; ++t) {
        int32_t is[4];
        const float part = unit_dot<WT>(v[t], p, act[0], is);
        acc[t] = ok ? __builtin_fmaf(ws, part, acc[t]) : acc[t];
      }
    }
    if constexpr (SWT != 0) {
      constexpr int NW = Blk<SWT>::NW;
      const int st = lane / LS;  // the lane's row step
      const int c = lane % LS;
      int64_t row = row0 + st;
      row = row < a.rows ? row : a.rows - 1;
      uint32_t win[BS][NW];
      uint32_t off[BS];
#pragma unroll
      for (int i = 0; i < BS; ++i) {
        int b = c + LS * i;
        b = b < NBK ? b : NBK - 1;
        off[i] = load_window<SWT>(a.w2 + row * a.row_bytes2 + static_cast<int64_t>(b) * Blk<SWT>::BYTES,
                                  win[i]);
      }
      const int8_t *qx = a.qx + static_cast<int64_t>(a.n_sel) * a.x_stride;
      const float *dx = a.dx + static_cast<int64_t>(a.n_sel) * (a.x_stride / 32);
      const int32_t *sx = a.sx ? a.sx + static_cast<int64_t>(a.n_sel) * (a.x_stride / 32) : nullptr;
      const float wsh = a.wts[a.n_sel];
      float part = 0.0f;
#pragma unroll
      for (int i = 0; i < BS; ++i) {
        const int b = c + LS * i;
        if (b < NBK) {
          uint32_t xq[8];
          const u32x4 v0 = *reinterpret_cast<const u32x4 *>(qx + 32 * b);
          const u32x4 v1 = *reinterpret_cast<const u32x4 *>(qx + 32 * b + 16);
          xq[0] = v0.x; xq[1] = v0.y; xq[2] = v0.z; xq[3] = v0.w;
          xq[4] = v1.x; xq[5] = v1.y; xq[6] = v1.z; xq[7] = v1.w;
          const float dw = window_scale(win[i][0], off[i]);
          const uint32_t sel = quant_selector(off[i]);
          int32_t isum;
          if constexpr (SWT == ZQ_Q4_0) {
            const int32_t sum = sx ? sx[b] : code_sum(xq, 8);
            isum = q4_raw_dot(win[i], sel, xq) - 8 * sum;
          } else {
            isum = q8_dot(win[i], sel, xq);
          }
          part = __builtin_fmaf(dw * dx[b], static_cast<float>(isum), part);
        }
      }
#pragma unroll
      for (int t = 0; t < RB; ++t) acc[t] = t == st ? __builtin_fmaf(wsh, part, acc[t]) : acc[t];
    }
    using R = RowReduce<64, RB>;
    float out[R::NOUT];
    R::run(acc, out);
    if (R::writer(lane)) {
#pragma unroll
      for (int m = 0; m < R::NOUT; ++m) {
        const int64_t row = row0 + R::rowstep(m, lane);
        if (row < a.rows) {
          float *yp = a.y + row;
          *yp = (a.flags & ZQ_ACCUMULATE) ? *yp + out[m] : out[m];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32-input form: y (+)= W . Q(x) in one launch, Q the activation quantizer
// of quantize.hip.  Each workgroup (WPB waves) issues its loads of x (two lanes
// per 32-element block), then every lane issues its first row group's weight
// units, then x is quantized into LDS (codes, scales, code sums) while the
// weights stream in; after one barrier each lane takes its units' codes from
// LDS and the row groups proceed as in dmmv_k_kernel (one pass over the
// units: k <= 64 * LPR * BPL).  Workgroup 0 can also store the quantized
// activation.  PIPE: the grid is persistent and each wave walks many groups,
// requesting the next group's units before the current group's arithmetic.
template <int WT, int LPR, int BPL, int RB, int WPB, bool PIPE>
__global__ __launch_bounds__(64 * WPB) __attribute__((amdgpu_waves_per_eu(1, 2))) void dmmv_k_f32_kernel(
    const uint8_t *w, const float *x, int64_t rows, int64_t row_bytes, int64_t n_groups,
    int32_t k, int32_t nb, const DmmvKF32Args a_in) {
  // leading scalars: preloaded kernel arguments (as dmmv_hot)
  DmmvKF32Args a = a_in;
  a.w = w;
  a.x = x;
  a.rows = rows;
  a.row_bytes = row_bytes;
  a.n_groups = n_groups;
  a.k = k;
  a.nb = nb;
  constexpr int S = 64 / LPR;
  constexpr int NWD = KQ<WT>::NWD;
  constexpr int T = 64 * WPB;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int8_t *lq = reinterpret_cast<int8_t *>(smem);                       // [k]
  float *ld = reinterpret_cast<float *>(smem + a.k);                   // [nb]
  int32_t *ls = reinterpret_cast<int32_t *>(smem + a.k + 4 * a.nb);    // [nb]
  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & 63;
  const int j = lane & (LPR - 1);
  const int slot = lane / LPR;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * T + tid) >> 6;
  const int64_t n_waves = (static_cast<int64_t>(gridDim.x) * T) >> 6;
  const int nu = a.nb / 2;  // 64-element units per row
  const int p = j & 3;

  // 1. x: this thread's first block half (16 elements)
  const int g = tid & 1;
  int qb = tid >> 1;
  float xv[16];
  if (qb < a.nb) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float4 f = *reinterpret_cast<const float4 *>(a.x + qb * 32 + g * 16 + 4 * u);
      xv[4 * u] = f.x; xv[4 * u + 1] = f.y; xv[4 * u + 2] = f.z; xv[4 * u + 3] = f.w;
    }
  }

  // 2. the first row group's weight units
  uint32_t v[RB][BPL][NWD];
  auto load_group_into = [&](uint32_t (&v)[RB][BPL][NWD], int64_t gi) {
    const int64_t row0 = gi * (RB * S);
#pragma unroll
    for (int t = 0; t < RB; ++t) {
      int64_t row = row0 + t * S + slot;
      row = row < a.rows ? row : a.rows - 1;
#pragma unroll
      for (int i = 0; i < BPL; ++i) {
        int u = j + LPR * i;
        u = u < nu ? u : nu - 1;
        load_unit_w<WT>(a.w + row * a.row_bytes + static_cast<int64_t>(u >> 2) * KQ<WT>::BYTES, p,
                        v[t][i]);
      }
    }
  };
  // (unconditional, past the last group the last one again: a load under a
  // branch would make the activation's quantization below wait for every
  // weight load, the wait counts being merged over both paths)
  int64_t gi = wave;
  load_group_into(v, gi < a.n_groups ? gi : a.n_groups - 1);

  // 3. quantize x into LDS
  const bool out = blockIdx.x == 0 && a.qx_out != nullptr;
  for (; qb < a.nb; qb += T / 2) {
    if (qb != (tid >> 1)) {  // further blocks when k > 16 * T
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4 f = *reinterpret_cast<const float4 *>(a.x + qb * 32 + g * 16 + 4 * u);
        xv[4 * u] = f.x; xv[4 * u + 1] = f.y; xv[4 * u + 2] = f.z; xv[4 * u + 3] = f.w;
      }
    }
    uint32_t pk[4];
    float d;
    int32_t sum;
    quantize_block<2>(xv, pk, d, sum);
    *reinterpret_cast<u32x4 *>(lq + qb * 32 + g * 16) = u32x4{pk[0], pk[1], pk[2], pk[3]};
    if (g == 0) {
      ld[qb] = d;
      ls[qb] = sum;
    }
    if (out) {
      uint32_t *qo = reinterpret_cast<uint32_t *>(a.qx_out + qb * 32 + g * 16);
      qo[0] = pk[0]; qo[1] = pk[1]; qo[2] = pk[2]; qo[3] = pk[3];
      if (g == 0) {
        if (a.dx_out) a.dx_out[qb] = d;
        if (a.sx_out) a.sx_out[qb] = sum;
      }
    }
  }
  __syncthreads();

  // 4. this lane's units' activation; units past the row end take the last
  //    unit's codes and zero scales
  KUnitAct act[BPL];
#pragma unroll
  for (int i = 0; i < BPL; ++i) {
    const int u0 = j + LPR * i;
    const bool ok = u0 < nu;
    const int u = ok ? u0 : nu - 1;
    KUnitAct &A = act[i];
    if constexpr (WT == ZQ_Q6_K) {
      const int base = 256 * (u >> 2) + 128 * ((u >> 1) & 1) + 16 * (u & 1);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int e0 = base + 32 * c;
        const u32x4 q = *reinterpret_cast<const u32x4 *>(lq + e0);
        A.q[4 * c] = q.x; A.q[4 * c + 1] = q.y; A.q[4 * c + 2] = q.z; A.q[4 * c + 3] = q.w;
        A.d[c] = ok ? ld[e0 >> 5] : 0.0f;
        A.m32[c] = -32 * code_sum(&A.q[4 * c], 4);
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int b = 2 * u + h;
        const u32x4 q0 = *reinterpret_cast<const u32x4 *>(lq + 32 * b);
        const u32x4 q1 = *reinterpret_cast<const u32x4 *>(lq + 32 * b + 16);
        uint32_t *q = &A.q[8 * h];
        q[0] = q0.x; q[1] = q0.y; q[2] = q0.z; q[3] = q0.w;
        q[4] = q1.x; q[5] = q1.y; q[6] = q1.z; q[7] = q1.w;
        A.d[h] = ok ? ld[b] : 0.0f;
        A.fs[h] = static_cast<float>(ls[b]);  // |sum| <= 32*127: exact
      }
    }
  }

  // 5. the row groups: dots, reduction, store
  auto run_group = [&](const uint32_t (&v)[RB][BPL][NWD], int64_t gi) {
    const int64_t row0 = gi * (RB * S);
    float acc[RB];
#pragma unroll
    for (int t = 0; t < RB; ++t) {
      float part = 0.0f;
#pragma unroll
      for (int i = 0; i < BPL; ++i) {
        int32_t is[4];
        part += unit_dot<WT>(v[t][i], p, act[i], is);
      }
      acc[t] = part;
    }
    using R = RowReduce<LPR, RB>;
    float res[R::NOUT];
    R::run(acc, res);
    if (R::writer(lane)) {
#pragma unroll
      for (int m = 0; m < R::NOUT; ++m) {
        const int64_t row = row0 + static_cast<int64_t>(R::rowstep(m, lane)) * S + slot;
        if (row < a.rows) {
          float *yp = a.y + row;
          *yp = (a.flags & ZQ_ACCUMULATE) ? *yp + res[m] : res[m];
        }
      }
    }
  };
  if constexpr (PIPE) {
    // A wave that walks several groups requests the next group's units
    // before it computes the current one, in a second register set; the
    // last group is peeled off so that every load sits on a straight path
    // (a load under a branch would merge the wait counts of both paths).
    uint32_t v2[RB][BPL][NWD];
    while (gi < a.n_groups) {
      const int64_t g1 = gi + n_waves;
      if (g1 >= a.n_groups) {
        run_group(v, gi);
        break;
      }
      load_group_into(v2, g1);
      run_group(v, gi);
      gi = g1;
      const int64_t g2 = gi + n_waves;
      if (g2 >= a.n_groups) {
        run_group(v2, gi);
        break;
      }
      load_group_into(v, g2);
      run_group(v2, gi);
      gi = g2;
    }
  } else {
    // then the next group's units, after this one's arithmetic
    while (gi < a.n_groups) {
      run_group(v, gi);
      gi += n_waves;
      if (gi < a.n_groups) load_group_into(v, gi);
    }
  }
}

template <int WT, int LPR, int RB, int SWT>
int launch_wsum1(DmmvArgs a, hipStream_t stream) {
  a.n_groups = (a.rows + RB - 1) / RB;
  const int64_t blocks = (a.n_groups + 3) / 4;
  const unsigned grid = static_cast<unsigned>(blocks < 1048576 ? blocks : 1048576);
  hipLaunchKernelGGL((dmmv_k_wsum_kernel<WT, LPR, RB, SWT>), dim3(grid), dim3(256), 0, stream, a.ids,
                     a.wts, a.qx, a.dx, a.n_groups, a.n_sel, a.nb, a.id_base, a);
  ZQ_LAUNCH_CHECK();
  return ZQ_OK;
}

// Row steps per wave: the largest of 4, 2, 1 that keeps >= 1024 waves.
template <int WT, int LPR, int SWT>
int launch_wsum_rb(const DmmvArgs &a, hipStream_t stream) {
  if ((a.rows + 3) / 4 >= 1024) return launch_wsum1<WT, LPR, 4, SWT>(a, stream);
  if ((a.rows + 1) / 2 >= 1024) return launch_wsum1<WT, LPR, 2, SWT>(a, stream);
  return launch_wsum1<WT, LPR, 1, SWT>(a, stream);
}

// nu = k / 64 of 4, 8, 16 or 32 (wsum_fits).
template <int WT, int SWT = 0>
int launch_wsum(int nu, const DmmvArgs &a, hipStream_t stream) {
  if (nu == 4) return launch_wsum_rb<WT, 4, SWT>(a, stream);
  if (nu == 8) return launch_wsum_rb<WT, 8, SWT>(a, stream);
  if (nu == 16) return launch_wsum_rb<WT, 16, SWT>(a, stream);
  return launch_wsum_rb<WT, 32, SWT>(a, stream);
}

template <int WT>
int launch_wsum_shared(int sh_wtype, int nu, DmmvArgs a, hipStream_t stream) {
  a.row_bytes = static_cast<int64_t>(a.nb / 8) * KQ<WT>::BYTES;
  a.row_bytes2 = static_cast<int64_t>(a.nb) * (sh_wtype == ZQ_Q4_0 ? 18 : 34);
  if (sh_wtype == ZQ_Q4_0) return launch_wsum<WT, ZQ_Q4_0>(nu, a, stream);
  return launch_wsum<WT, ZQ_Q8_0>(nu, a, stream);
}

bool wsum_fits(int nu) { return nu == 4 || nu == 8 || nu == 16 || nu == 32; }

struct KShape {
  int lpr, bpl;
};
// (LPR, BPL) layouts over units; any row length is served, further passes
// take the units beyond LPR*BPL.  LPR is a multiple of 4, so a lane's units
// all sit at the same position of their super-blocks.
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

// Largest row steps per group RB whose weight registers (RB*BPL units of
// NWD dwords) stay within 96 dwords and that still leaves >= 2048 waves
// (counting every gathered slot); the MoE modes keep RB <= 4.
template <int WT>
int choose_krb(const KShape &sh, int64_t rows, int mode, int64_t slots) {
  if (mode == MODE_ISUMS) return 1;
  const int S = 64 / sh.lpr;
  const int cap = 96 / (KQ<WT>::NWD * sh.bpl);
  for (int rb : {8, 4, 2, 1}) {
    if (rb > cap && rb > 1) continue;
    if (rb > 4 && mode != MODE_PLAIN) continue;
    if (rb == 1 || (rows + rb * S - 1) / (rb * S) * slots >= 2048) return rb;
  }
  return 1;
}

template <int WT, int LPR, int BPL, int RB, int MODE>
int launch_k1(DmmvArgs a, hipStream_t stream) {
  constexpr int S = 64 / LPR;
  a.n_groups = (a.rows + RB * S - 1) / (RB * S);
  const int64_t blocks = (a.n_groups + 3) / 4;
  const unsigned grid = static_cast<unsigned>(blocks < 1048576 ? blocks : 1048576);
  const unsigned gy = MODE == MODE_GATHER ? static_cast<unsigned>(a.n_sel) : 1u;
  hipLaunchKernelGGL((dmmv_k_kernel<WT, LPR, BPL, RB, MODE>), dim3(grid, gy), dim3(256), 0, stream,
                     ZQ_DMMV_HOT(a), a);
  ZQ_LAUNCH_CHECK();
  return ZQ_OK;
}

// RB values instantiated per (type, BPL, mode): those choose_krb can return.
template <int WT, int LPR, int BPL, int MODE>
int launch_krb(int rb, const DmmvArgs &a, hipStream_t stream) {
  constexpr int CAP0 = 96 / (KQ<WT>::NWD * BPL);
  constexpr int CAP = MODE == MODE_PLAIN ? CAP0 : (CAP0 < 4 ? CAP0 : 4);
  if constexpr (MODE == MODE_ISUMS) {
    return launch_k1<WT, LPR, BPL, 1, MODE>(a, stream);
  } else {
    if constexpr (CAP >= 8) {
      if (rb >= 8) return launch_k1<WT, LPR, BPL, 8, MODE>(a, stream);
    }
    if constexpr (CAP >= 4) {
      if (rb >= 4) return launch_k1<WT, LPR, BPL, 4, MODE>(a, stream);
    }
    if constexpr (CAP >= 2) {
      if (rb >= 2) return launch_k1<WT, LPR, BPL, 2, MODE>(a, stream);
    }
    return launch_k1<WT, LPR, BPL, 1, MODE>(a, stream);
  }
}

template <int WT, int MODE>
int launch_kshape(const KShape &sh, int rb, const DmmvArgs &a, hipStream_t stream) {
  if (sh.lpr == 8) return launch_krb<WT, 8, 1, MODE>(rb, a, stream);
  if (sh.lpr == 16 && sh.bpl == 1) return launch_krb<WT, 16, 1, MODE>(rb, a, stream);
  if (sh.lpr == 16) return launch_krb<WT, 16, 5, MODE>(rb, a, stream);
  if (sh.lpr == 32) return launch_krb<WT, 32, 1, MODE>(rb, a, stream);
  if (sh.bpl == 1) return launch_krb<WT, 64, 1, MODE>(rb, a, stream);
  if (sh.bpl == 2) return launch_krb<WT, 64, 2, MODE>(rb, a, stream);
  return launch_krb<WT, 64, 4, MODE>(rb, a, stream);
}

template <int WT>
int launch_type(int mode, DmmvArgs a, hipStream_t stream) {
  a.row_bytes = static_cast<int64_t>(a.nb / 8) * KQ<WT>::BYTES;
  if (mode == MODE_WEIGHTED && wsum_fits(a.nb / 2)) return launch_wsum<WT>(a.nb / 2, a, stream);
  const KShape sh = choose_kshape(a.nb / 2);
  const int64_t slots = mode == MODE_GATHER ? a.n_sel : 1;
  const int rb = choose_krb<WT>(sh, a.rows, mode, slots);
  switch (mode) {
    case MODE_PLAIN: return launch_kshape<WT, MODE_PLAIN>(sh, rb, a, stream);
    case MODE_ISUMS: return launch_kshape<WT, MODE_ISUMS>(sh, rb, a, stream);
    case MODE_GATHER: return launch_kshape<WT, MODE_GATHER>(sh, rb, a, stream);
    default: return launch_kshape<WT, MODE_WEIGHTED>(sh, rb, a, stream);
  }
}

// The fp32-input form: the plain layout and row steps, a workgroup's
// activation staged once, one row group per wave.  Row groups beyond what kKF32Walk workgroups take in one pass (the LM-head
// shapes) go to a persistent grid of one workgroup per CU whose waves walk
// the groups, each requesting the next group's units before it computes the
// current one.  Q6_K LM head (248 320 x 2048), one box, alternating: 72.3-
// 72.7 us with 256 such workgroups, against 81.3-81.9 us for a grid capped
// at 4096 workgroups that walked without the second register set
// (1024: 74.5-75.0 us, 512: 73.4-73.5 us; the second register set at 512
// workgroups, two waves per SIMD: 74.8-75.2 us).
constexpr int64_t kKF32Walk = 4096;
constexpr int kKF32WalkGrid = 256;
constexpr int kKF32WalkWpb = 4;

inline bool kf_walks(int64_t n_groups) { return n_groups > 4 * kKF32Walk; }

template <int WT, int LPR, int BPL, int RB, int WPB = 4>
int launch_kf1(DmmvKF32Args a, hipStream_t stream) {
  constexpr int S = 64 / LPR;
  a.n_groups = (a.rows + RB * S - 1) / (RB * S);
  const int64_t blocks = (a.n_groups + WPB - 1) / WPB;
  const size_t lds = static_cast<size_t>(a.k) + 8 * static_cast<size_t>(a.nb);
  if constexpr (WPB == kKF32WalkWpb) {
    if (kf_walks(a.n_groups)) {
      hipLaunchKernelGGL((dmmv_k_f32_kernel<WT, LPR, BPL, RB, WPB, true>), dim3(kKF32WalkGrid),
                         dim3(64 * WPB), lds, stream, a.w, a.x, a.rows, a.row_bytes, a.n_groups, a.k,
                         a.nb, a);
      ZQ_LAUNCH_CHECK();
      return ZQ_OK;
    }
  }
  {
    hipLaunchKernelGGL((dmmv_k_f32_kernel<WT, LPR, BPL, RB, WPB, false>), dim3(static_cast<unsigned>(blocks)),
                       dim3(64 * WPB), lds, stream, a.w, a.x, a.rows, a.row_bytes, a.n_groups, a.k,
                       a.nb, a);
  }
  ZQ_LAUNCH_CHECK();
  return ZQ_OK;
}

template <int WT, int LPR, int BPL, int WPB>
int launch_kfrb(int rb, const DmmvKF32Args &a, hipStream_t stream) {
  constexpr int CAP = 96 / (KQ<WT>::NWD * BPL);
  if constexpr (CAP >= 8) {
    if (rb >= 8) return launch_kf1<WT, LPR, BPL, 8, WPB>(a, stream);
  }
  if constexpr (CAP >= 4) {
    if (rb >= 4) return launch_kf1<WT, LPR, BPL, 4, WPB>(a, stream);
  }
  if constexpr (CAP >= 2) {
    if (rb >= 2) return launch_kf1<WT, LPR, BPL, 2, WPB>(a, stream);
  }
  return launch_kf1<WT, LPR, BPL, 1, WPB>(a, stream);
}

template <int WT, int WPB>
int launch_kf_shape(const KShape &sh, int rb, const DmmvKF32Args &a, hipStream_t stream) {
  if (sh.lpr == 8) return launch_kfrb<WT, 8, 1, WPB>(rb, a, stream);
  if (sh.lpr == 16 && sh.bpl == 1) return launch_kfrb<WT, 16, 1, WPB>(rb, a, stream);
  if (sh.lpr == 16) return launch_kfrb<WT, 16, 5, WPB>(rb, a, stream);
  if (sh.lpr == 32) return launch_kfrb<WT, 32, 1, WPB>(rb, a, stream);
  if (sh.bpl == 1) return launch_kfrb<WT, 64, 1, WPB>(rb, a, stream);
  if (sh.bpl == 2) return launch_kfrb<WT, 64, 2, WPB>(rb, a, stream);
  return launch_kfrb<WT, 64, 4, WPB>(rb, a, stream);
}

template <int WT>
int launch_kf_type(DmmvKF32Args a, hipStream_t stream) {
  a.row_bytes = static_cast<int64_t>(a.nb / 8) * KQ<WT>::BYTES;
  const int nu = a.nb / 2;
  const KShape sh = choose_kshape(nu);
  if (static_cast<int64_t>(sh.lpr) * sh.bpl < nu) return ZQ_EINVAL;  // one pass only
  const int rb = choose_krb<WT>(sh, a.rows, MODE_PLAIN, 1);
  // 8 waves per workgroup where the row groups still fill 256 workgroups
  // (fewer workgroups quantize x, each stages it for twice the rows):
  // 4096 x 4096 Q4_K / Q5_K / Q6_K 3.57 / 4.30 / 5.01 us against 4.08 /
  // 4.51 / 5.44 with 4 waves, 4096 x 14336 Q4_K 11.1 against 12.9;
  // below that (2048 x 2048: 128 workgroups) 4 waves (2.41 against 2.64).
  // The LM-head shapes keep 4.
  const int64_t groups = (a.rows + static_cast<int64_t>(rb) * (64 / sh.lpr) - 1) /
                         (static_cast<int64_t>(rb) * (64 / sh.lpr));
  if (kf_walks(groups)) return launch_kf_shape<WT, kKF32WalkWpb>(sh, rb, a, stream);
  if (a.rows <= 16384 && groups >= 8 * 256) return launch_kf_shape<WT, 8>(sh, rb, a, stream);
  return launch_kf_shape<WT, 4>(sh, rb, a, stream);
}

}  // namespace

int launch_dmmv_k_f32(int wtype, DmmvKF32Args a, hipStream_t stream) {
  if (a.rows == 0) return ZQ_OK;
  switch (wtype) {
    case ZQ_Q4_K: return launch_kf_type<ZQ_Q4_K>(a, stream);
    case ZQ_Q5_K: return launch_kf_type<ZQ_Q5_K>(a, stream);
    case ZQ_Q6_K: return launch_kf_type<ZQ_Q6_K>(a, stream);
    default: return ZQ_EINVAL;
  }
}

bool dmmv_k_wsum_shared_fits(int wtype, int sh_wtype, int64_t k) {
  return (wtype == ZQ_Q4_K || wtype == ZQ_Q5_K || wtype == ZQ_Q6_K) &&
         (sh_wtype == ZQ_Q4_0 || sh_wtype == ZQ_Q8_0) && k % 64 == 0 &&
         wsum_fits(static_cast<int>(k / 64));
}

int launch_dmmv_k_wsum_shared(int wtype, int sh_wtype, DmmvArgs a, hipStream_t stream) {
  if (a.rows == 0) return ZQ_OK;
  if (!a.w2 || !dmmv_k_wsum_shared_fits(wtype, sh_wtype, static_cast<int64_t>(a.nb) * 32))
    return ZQ_EINVAL;
  const int nu = a.nb / 2;
  switch (wtype) {
    case ZQ_Q4_K: return launch_wsum_shared<ZQ_Q4_K>(sh_wtype, nu, a, stream);
    case ZQ_Q5_K: return launch_wsum_shared<ZQ_Q5_K>(sh_wtype, nu, a, stream);
    default: return launch_wsum_shared<ZQ_Q6_K>(sh_wtype, nu, a, stream);
  }
}

int launch_dmmv_k(int wtype, int mode, DmmvArgs a, hipStream_t stream) {
  if (a.rows == 0) return ZQ_OK;
  if (mode == MODE_GATHER && a.n_sel == 0) return ZQ_OK;
  switch (wtype) {
    case ZQ_Q4_K: return launch_type<ZQ_Q4_K>(mode, a, stream);
    case ZQ_Q5_K: return launch_type<ZQ_Q5_K>(mode, a, stream);
    case ZQ_Q6_K: return launch_type<ZQ_Q6_K>(mode, a, stream);
    default: return ZQ_EINVAL;
  }
}

}  // namespace zq
