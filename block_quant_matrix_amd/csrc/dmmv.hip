// dmmv.hip -- dequantizing matrix-vector products over Q4_0 / Q8_0 blocks
// (gfx950, wave64).
//
// Mapping: one lane per weight block.  A row slot of LPR consecutive lanes
// (LPR in {8,16,32,64}) walks one row; lane j of the slot owns blocks
// j, j+LPR, ..., j+(BPL-1)*LPR of every row it visits, so its activation
// blocks (8 dwords of codes, the scale and 8*sum) stay in registers for the
// whole wave lifetime.  One load instruction of the wave therefore covers
// LPR*block_bytes contiguous bytes per slot (1152 B for Q4_0 with LPR = 64):
// fully coalesced HBM reads.  Because 18- and 34-byte blocks are only 2-byte
// aligned, each lane loads a dword-aligned window (5 or 9 dwords) and picks
// its bytes out with v_perm_b32.
//
// Each wave handles RB row steps per group (S = 64/LPR rows per step), with
// all RB*BPL block windows issued before any arithmetic so the wave keeps
// RB*BPL*block_bytes per lane in flight.  Per block: 8 packed int8 dot
// products (v_dot4), the exact int32 block sum, one fp32 scale product and
// one FMA into the row partial.  Row partials are folded across lanes with
// v_permlane32/16_swap halving steps plus DPP sums.
//
// The same inner loop serves four modes: plain (y = / += W.x), isums (the
// integer block sums, for tests), MoE gather (one expert per grid.y slot)
// and MoE weighted sum (all selected experts accumulated per row before the
// lane reduction, so the weighting costs one FMA per row partial).
#include "zq_common.h"
#include "zq_internal.h"

namespace zq {

template <int BPL> struct ActRegs {
  uint32_t q[BPL][8];
  float d[BPL];
  int32_t sraw[BPL];
  int32_t s8[BPL];
};

// Issue the loads of the lane's activation blocks (codes, scale, block sum
// when sx is given).  Blocks past the row end load the last block; finish_act
// zeroes their scales.  No arithmetic on the loaded values here, so the wave
// requests its weight windows before it waits on any of them.
template <int WT, int LPR, int BPL>
__device__ __forceinline__ void load_act(ActRegs<BPL> &act, const DmmvArgs &a, int s, int pass,
                                         int j) {
  const int8_t *qx = a.qx + static_cast<int64_t>(s) * a.x_stride;
  const float *dx = a.dx + static_cast<int64_t>(s) * (a.x_stride / 32);
  // with no sx the sum loads read dx (a valid address) and are not used
  const int32_t *sx = a.sx ? a.sx + static_cast<int64_t>(s) * (a.x_stride / 32)
                           : reinterpret_cast<const int32_t *>(dx);
#pragma unroll
  for (int i = 0; i < BPL; ++i) {
    int b = pass * LPR * BPL + j + LPR * i;
    b = b < a.nb ? b : a.nb - 1;
    const u32x4 v0 = *reinterpret_cast<const u32x4 *>(qx + 32 * b);
    const u32x4 v1 = *reinterpret_cast<const u32x4 *>(qx + 32 * b + 16);
    act.q[i][0] = v0.x; act.q[i][1] = v0.y; act.q[i][2] = v0.z; act.q[i][3] = v0.w;
    act.q[i][4] = v1.x; act.q[i][5] = v1.y; act.q[i][6] = v1.z; act.q[i][7] = v1.w;
    act.d[i] = dx[b];
    if constexpr (WT == ZQ_Q4_0) act.sraw[i] = sx[b];
  }
}

// The arithmetic half: 8 * block sum for the Q4_0 offset, and zero scales
// for the blocks past the row end.  No loads, so the outstanding-load
// counters agree on every path.
template <int WT, int LPR, int BPL>
__device__ __forceinline__ void finish_act(ActRegs<BPL> &act, const DmmvArgs &a, int pass, int j) {
#pragma unroll
  for (int i = 0; i < BPL; ++i) {
    const bool ok = pass * LPR * BPL + j + LPR * i < a.nb;
    act.d[i] = ok ? act.d[i] : 0.0f;
    if constexpr (WT == ZQ_Q4_0) {
      int32_t sum = act.sraw[i];
      if (!a.sx) {
        sum = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k)
          sum = __builtin_amdgcn_sdot4(static_cast<int>(act.q[i][k]), 0x01010101, sum, false);
      }
      act.s8[i] = 8 * sum;
    } else {
      act.s8[i] = 0;
    }
  }
}

// Load and reduce one pass (BPL blocks per lane) of RB row steps.
template <int WT, int LPR, int BPL, int RB, int MODE>
__device__ __forceinline__ void block_pass(const DmmvArgs &a, const uint8_t *wb, int64_t row0,
                                           int pass, int j, int slot, ActRegs<BPL> &act,
                                           float (&part)[RB]) {
  constexpr int NW = Blk<WT>::NW;
  constexpr int BB = Blk<WT>::BYTES;
  constexpr int S = 64 / LPR;
  uint32_t win[RB][BPL][NW];
  uint32_t off[RB][BPL];
#pragma unroll
  for (int t = 0; t < RB; ++t) {
    int64_t row = row0 + t * S + slot;
    row = row < a.rows ? row : a.rows - 1;
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      int b = pass * LPR * BPL + j + LPR * i;
      b = b < a.nb ? b : a.nb - 1;
      off[t][i] = load_window<WT>(wb + row * a.row_bytes + static_cast<int64_t>(b) * BB, win[t][i]);
    }
  }
  // re-derived on every pass: one multiply (or 8 dot4) per block, no loads
  finish_act<WT, LPR, BPL>(act, a, pass, j);
#pragma unroll
  for (int t = 0; t < RB; ++t) {
    float p = 0.0f;
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      const float dw = window_scale(win[t][i][0], off[t][i]);
      const uint32_t sel = quant_selector(off[t][i]);
      int32_t isum;
      if constexpr (WT == ZQ_Q4_0) {
        isum = q4_raw_dot(win[t][i], sel, act.q[i]) - act.s8[i];
      } else {
        isum = q8_dot(win[t][i], sel, act.q[i]);
      }
      if constexpr (MODE == MODE_ISUMS) {
        const int64_t row = row0 + t * S + slot;
        const int b = pass * LPR * BPL + j + LPR * i;
        if (row < a.rows && b < a.nb) a.isums[row * a.nb + b] = isum;
      }
      p = __builtin_fmaf(dw * act.d[i], static_cast<float>(isum), p);
    }
    part[t] = p;
  }
}

template <int WT, int LPR, int BPL, int RB, int MODE>
__global__ __launch_bounds__(256) void dmmv_kernel(const uint8_t *w, const int8_t *qx,
                                                   const float *dx, int64_t rows,
                                                   int64_t row_bytes, int64_t n_groups, int32_t nb,
                                                   int32_t id_base, const DmmvArgs a_in) {
  DmmvArgs a = a_in;
  dmmv_hot(a, w, qx, dx, rows, row_bytes, n_groups, nb, id_base);
  constexpr int S = 64 / LPR;
  const int lane = static_cast<int>(threadIdx.x & 63);
  const int j = lane & (LPR - 1);
  const int slot = lane / LPR;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t n_waves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
  const int n_pass = (a.nb + LPR * BPL - 1) / (LPR * BPL);

  int s0 = 0, s1 = 1;
  if constexpr (MODE == MODE_GATHER) {
    s0 = static_cast<int>(blockIdx.y);
    s1 = s0 + 1;
    const int e = a.ids[s0] - a.id_base;
    if (e < 0 || e >= a.n_experts) {  // uniform over the block
      if (a.status) *a.status = ZQ_ERANGE;
      return;
    }
  } else if constexpr (MODE == MODE_WEIGHTED) {
    s1 = a.n_sel;
  }

  ActRegs<BPL> act;
  const bool hoist = (n_pass == 1) && (MODE != MODE_WEIGHTED);
  if (hoist) load_act<WT, LPR, BPL>(act, a, s0, 0, j);

  for (int64_t g = wave; g < a.n_groups; g += n_waves) {
    const int64_t row0 = g * (RB * S);
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
        if (!hoist) load_act<WT, LPR, BPL>(act, a, s, pass, j);
        float part[RB];
        block_pass<WT, LPR, BPL, RB, MODE>(a, wb, row0, pass, j, slot, act, part);
#pragma unroll
        for (int t = 0; t < RB; ++t) {
          if constexpr (MODE == MODE_WEIGHTED) {
            acc[t] = __builtin_fmaf(ws, part[t], acc[t]);
          } else {
            acc[t] += part[t];
          }
        }
      }
    }
    if constexpr (MODE != MODE_ISUMS) {
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

// ------------------------------------------------------------ dispatch ----

namespace {

struct Shape {
  int lpr, bpl;
};
// (LPR, BPL) layouts that are compiled.  Any nb is served: blocks beyond
// LPR*BPL are handled in further passes.
constexpr Shape kShapes[] = {{8, 1}, {16, 1}, {32, 1}, {64, 1}, {64, 2}, {64, 4}, {32, 5}};

Shape choose_shape(int32_t nb) {
  Shape best = kShapes[0];
  int64_t best_waste = -1, best_pass = 0;
  for (const Shape &s : kShapes) {
    const int64_t per = static_cast<int64_t>(s.lpr) * s.bpl;
    const int64_t passes = (nb + per - 1) / per;
    const int64_t waste = passes * per - nb;
    bool better = best_waste < 0 || waste < best_waste ||
                  (waste == best_waste && passes < best_pass) ||
                  (waste == best_waste && passes == best_pass && s.lpr > best.lpr);
    if (better) {
      best = s;
      best_waste = waste;
      best_pass = passes;
    }
  }
  return best;
}

// Rows per wave group = RB * (64 / LPR).  Prefer the largest RB that still
// leaves >= 2048 waves (8 per CU) to keep HBM busy; windows held per lane
// are capped (RB * BPL <= 16 for Q4_0, 8 for Q8_0).
int choose_rb(int wtype, int mode, const Shape &sh, int64_t rows) {
  if (mode == MODE_ISUMS) return 1;
  const int S = 64 / sh.lpr;
  const int cap = (wtype == ZQ_Q4_0 ? 16 : 8) / sh.bpl;
  const int cands[] = {8, 4, 2, 1};
  for (int rb : cands) {
    if (rb > cap) continue;
    if (mode == MODE_GATHER || mode == MODE_WEIGHTED) {
      if (rb > 4) continue;
    }
    const int64_t groups = (rows + rb * S - 1) / (rb * S);
    if (groups >= 2048) return rb;
  }
  return 1;
}

template <int WT, int LPR, int BPL, int RB, int MODE>
int launch_one(const DmmvArgs &a, hipStream_t stream, unsigned grid_y) {
  constexpr int S = 64 / LPR;
  DmmvArgs b = a;
  b.n_groups = (a.rows + RB * S - 1) / (RB * S);
  const int64_t blocks = (b.n_groups + 3) / 4;  // 4 waves per 256-thread block
  const unsigned grid_x = static_cast<unsigned>(blocks < 1048576 ? blocks : 1048576);
  hipLaunchKernelGGL((dmmv_kernel<WT, LPR, BPL, RB, MODE>), dim3(grid_x, grid_y), dim3(256), 0,
                     stream, ZQ_DMMV_HOT(b), b);
  ZQ_LAUNCH_CHECK();
  return ZQ_OK;
}

template <int WT, int LPR, int BPL, int MODE>
int launch_rb(int rb, const DmmvArgs &a, hipStream_t stream, unsigned gy) {
  switch (rb) {
    case 1: return launch_one<WT, LPR, BPL, 1, MODE>(a, stream, gy);
    case 2: return launch_one<WT, LPR, BPL, 2, MODE>(a, stream, gy);
    case 4: return launch_one<WT, LPR, BPL, 4, MODE>(a, stream, gy);
    default:
      if constexpr (MODE == MODE_PLAIN && (WT == ZQ_Q4_0 ? BPL * 8 <= 16 : BPL * 8 <= 8))
        return launch_one<WT, LPR, BPL, 8, MODE>(a, stream, gy);
      return launch_one<WT, LPR, BPL, 4, MODE>(a, stream, gy);
  }
}

template <int WT, int MODE>
int launch_shape(const Shape &sh, int rb, const DmmvArgs &a, hipStream_t stream, unsigned gy) {
  if (sh.lpr == 8) return launch_rb<WT, 8, 1, MODE>(rb, a, stream, gy);
  if (sh.lpr == 16) return launch_rb<WT, 16, 1, MODE>(rb, a, stream, gy);
  if (sh.lpr == 32 && sh.bpl == 1) return launch_rb<WT, 32, 1, MODE>(rb, a, stream, gy);
  if (sh.lpr == 32 && sh.bpl == 5) return launch_rb<WT, 32, 5, MODE>(rb, a, stream, gy);
  if (sh.lpr == 64 && sh.bpl == 1) return launch_rb<WT, 64, 1, MODE>(rb, a, stream, gy);
  if (sh.lpr == 64 && sh.bpl == 2) return launch_rb<WT, 64, 2, MODE>(rb, a, stream, gy);
  return launch_rb<WT, 64, 4, MODE>(rb, a, stream, gy);
}

template <int WT>
int launch_mode(int mode, const Shape &sh, int rb, const DmmvArgs &a, hipStream_t stream) {
  switch (mode) {
    case MODE_PLAIN: return launch_shape<WT, MODE_PLAIN>(sh, rb, a, stream, 1);
    case MODE_ISUMS: return launch_shape<WT, MODE_ISUMS>(sh, rb, a, stream, 1);
    case MODE_GATHER:
      return launch_shape<WT, MODE_GATHER>(sh, rb, a, stream, static_cast<unsigned>(a.n_sel));
    default: return launch_shape<WT, MODE_WEIGHTED>(sh, rb, a, stream, 1);
  }
}

}  // namespace

int launch_dmmv(int wtype, int mode, DmmvArgs a, hipStream_t stream) {
  if (a.rows == 0) return ZQ_OK;
  if (mode == MODE_GATHER && a.n_sel == 0) return ZQ_OK;
  const int bb = wtype == ZQ_Q4_0 ? 18 : 34;
  a.row_bytes = static_cast<int64_t>(a.nb) * bb;
  const Shape sh = choose_shape(a.nb);
  const int rb = choose_rb(wtype, mode, sh, a.rows);
  if (wtype == ZQ_Q4_0) return launch_mode<ZQ_Q4_0>(mode, sh, rb, a, stream);
  return launch_mode<ZQ_Q8_0>(mode, sh, rb, a, stream);
}

}  // namespace zq
