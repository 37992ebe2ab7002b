// dmmv_tok.hip -- multi-token DMMV over Q4_0 / Q8_0 blocks (gfx950, wave64):
// y[t][r] = sum_b d_w[r][b] * dx[t][b] * isum_t[r][b] for 2..8 tokens decoded
// together, in one pass over the weights.
//
// Mapping: as the single-token DMMV (dmmv.hip): a row slot of LPR lanes walks
// one row, lane j owns blocks j, j+LPR, ... (BPL of them per pass), and each
// wave issues the windows of RB row steps before any arithmetic.  The lane
// holds the codes, scales and sums of its blocks for all T tokens (T*BPL <= 8
// blocks of activation), so each weight block is unpacked once and dotted
// with T activation blocks.  The RB*T row partials per lane are folded by
// one RowReduce.  Tokens past n_tok load the last token and get zero scales;
// their rows are not written.
#include "zq_common.h"
#include "zq_internal.h"

namespace zq {

namespace {

template <int T, int BPL> struct TokAct {
  uint32_t q[T][BPL][8];
  float d[T][BPL];
  int32_t sraw[T][BPL];
  int32_t s8[T][BPL];
};

// Loads only (the sums are derived once the weight windows are in flight).
template <int WT, int LPR, int BPL, int T>
__device__ __forceinline__ void tok_load_act(TokAct<T, BPL> &A, const DmmvTokArgs &a, int pass,
                                             int j) {
  const int32_t *sxb = a.sx ? a.sx : reinterpret_cast<const int32_t *>(a.dx);
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int tt = t < a.n_tok ? t : a.n_tok - 1;
    const int8_t *qx = a.qx + static_cast<int64_t>(tt) * a.k;
    const float *dx = a.dx + static_cast<int64_t>(tt) * a.nb;
    const int32_t *sx = sxb + static_cast<int64_t>(tt) * a.nb;
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      int b = pass * LPR * BPL + j + LPR * i;
      b = b < a.nb ? b : a.nb - 1;
      const u32x4 v0 = *reinterpret_cast<const u32x4 *>(qx + 32 * b);
      const u32x4 v1 = *reinterpret_cast<const u32x4 *>(qx + 32 * b + 16);
      A.q[t][i][0] = v0.x; A.q[t][i][1] = v0.y; A.q[t][i][2] = v0.z; A.q[t][i][3] = v0.w;
      A.q[t][i][4] = v1.x; A.q[t][i][5] = v1.y; A.q[t][i][6] = v1.z; A.q[t][i][7] = v1.w;
      A.d[t][i] = dx[b];
      if constexpr (WT == ZQ_Q4_0) A.sraw[t][i] = sx[b];
    }
  }
}

template <int WT, int LPR, int BPL, int T>
__device__ __forceinline__ void tok_finish_act(TokAct<T, BPL> &A, const DmmvTokArgs &a, int pass,
                                               int j) {
#pragma unroll
  for (int t = 0; t < T; ++t) {
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      const bool ok = t < a.n_tok && pass * LPR * BPL + j + LPR * i < a.nb;
      A.d[t][i] = ok ? A.d[t][i] : 0.0f;
      if constexpr (WT == ZQ_Q4_0) {
        int32_t sum = A.sraw[t][i];
        if (!a.sx) {
          sum = 0;
#pragma unroll
          for (int k = 0; k < 8; ++k)
            sum = __builtin_amdgcn_sdot4(static_cast<int>(A.q[t][i][k]), 0x01010101, sum, false);
        }
        A.s8[t][i] = 8 * sum;
      } else {
        A.s8[t][i] = 0;
      }
    }
  }
}

template <int WT, int LPR, int BPL, int RB, int T>
__global__ __launch_bounds__(256) void dmmv_tok_kernel(const DmmvTokArgs a) {
  constexpr int S = 64 / LPR;
  constexpr int NW = Blk<WT>::NW;
  constexpr int BB = Blk<WT>::BYTES;
  const int lane = static_cast<int>(threadIdx.x & 63);
  const int j = lane & (LPR - 1);
  const int slot = lane / LPR;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t n_waves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
  const int n_pass = (a.nb + LPR * BPL - 1) / (LPR * BPL);

  TokAct<T, BPL> act;
  if (n_pass == 1) tok_load_act<WT, LPR, BPL, T>(act, a, 0, j);

  for (int64_t g = wave; g < a.n_groups; g += n_waves) {
    const int64_t row0 = g * (RB * S);
    float acc[RB * T];
#pragma unroll
    for (int f = 0; f < RB * T; ++f) acc[f] = 0.0f;
    for (int pass = 0; pass < n_pass; ++pass) {
      if (n_pass > 1) tok_load_act<WT, LPR, BPL, T>(act, a, pass, j);
      uint32_t win[RB][BPL][NW];
      uint32_t off[RB][BPL];
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        int64_t row = row0 + r * S + slot;
        row = row < a.rows ? row : a.rows - 1;
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
          int b = pass * LPR * BPL + j + LPR * i;
          b = b < a.nb ? b : a.nb - 1;
          off[r][i] = load_window<WT>(a.w + row * a.row_bytes + static_cast<int64_t>(b) * BB, win[r][i]);
        }
      }
      tok_finish_act<WT, LPR, BPL, T>(act, a, pass, j);
#pragma unroll
      for (int r = 0; r < RB; ++r) {
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
          const float dw = window_scale(win[r][i][0], off[r][i]);
          const uint32_t sel = quant_selector(off[r][i]);
          // the block's codes, unpacked once for all tokens
          uint32_t c[8];
          if constexpr (WT == ZQ_Q4_0) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const uint32_t q = __builtin_amdgcn_perm(win[r][i][k + 1], win[r][i][k], sel);
              c[k] = q & 0x0F0F0F0Fu;             // elements 4k..4k+3
              c[4 + k] = (q >> 4) & 0x0F0F0F0Fu;  // elements 16+4k..16+4k+3
            }
          } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) c[k] = __builtin_amdgcn_perm(win[r][i][k + 1], win[r][i][k], sel);
          }
#pragma unroll
          for (int t = 0; t < T; ++t) {
            int32_t s = -act.s8[t][i];
#pragma unroll
            for (int k = 0; k < 8; ++k)
              s = __builtin_amdgcn_sdot4(static_cast<int>(c[k]), static_cast<int>(act.q[t][i][k]), s, false);
            acc[r * T + t] = __builtin_fmaf(dw * act.d[t][i], static_cast<float>(s), acc[r * T + t]);
          }
        }
      }
    }
    using R = RowReduce<LPR, RB * T>;
    float out[R::NOUT];
    R::run(acc, out);
    if (R::writer(lane)) {
#pragma unroll
      for (int m = 0; m < R::NOUT; ++m) {
        const int f = R::rowstep(m, lane);
        const int t = f % T;
        const int64_t row = row0 + static_cast<int64_t>(f / T) * S + slot;
        if (row < a.rows && t < a.n_tok) {
          float *yp = a.y + static_cast<int64_t>(t) * a.rows + row;
          *yp = (a.flags & ZQ_ACCUMULATE) ? *yp + out[m] : out[m];
        }
      }
    }
  }
}

struct TShape {
  int lpr, bpl;
};

// The layout with fewest passes, then least idle lanes, among LPR in
// {8,16,32,64} and BPL up to 8/T.
TShape choose_tshape(int32_t nb, int T) {
  TShape best{8, 1};
  int64_t best_pass = -1, best_waste = 0;
  for (int lpr : {8, 16, 32, 64}) {
    for (int bpl : {1, 2, 4}) {
      if (bpl * T > 8) continue;
      const int64_t per = static_cast<int64_t>(lpr) * bpl;
      const int64_t passes = (nb + per - 1) / per;
      const int64_t waste = passes * per - nb;
      if (best_pass < 0 || passes < best_pass || (passes == best_pass && waste < best_waste) ||
          (passes == best_pass && waste == best_waste && lpr > best.lpr)) {
        best = TShape{lpr, bpl};
        best_pass = passes;
        best_waste = waste;
      }
    }
  }
  return best;
}

template <int WT, int LPR, int BPL, int RB, int T>
int launch_t1(DmmvTokArgs a, hipStream_t stream) {
  constexpr int S = 64 / LPR;
  a.n_groups = (a.rows + RB * S - 1) / (RB * S);
  const int64_t blocks = (a.n_groups + 3) / 4;
  const unsigned grid = static_cast<unsigned>(blocks < 1048576 ? blocks : 1048576);
  hipLaunchKernelGGL((dmmv_tok_kernel<WT, LPR, BPL, RB, T>), dim3(grid), dim3(256), 0, stream, a);
  ZQ_LAUNCH_CHECK();
  return ZQ_OK;
}

// Row steps per group: 4 while that leaves >= 2048 waves, else 2, else 1;
// with T = 8 and BPL = 1 at most 2 (registers).
template <int WT, int LPR, int BPL, int T>
int launch_trb(const DmmvTokArgs &a, hipStream_t stream) {
  constexpr int S = 64 / LPR;
  const auto groups = [&](int rb) { return (a.rows + rb * S - 1) / (rb * S); };
  if constexpr (T * BPL <= 4) {
    if (groups(4) >= 2048) return launch_t1<WT, LPR, BPL, 4, T>(a, stream);
  }
  if (groups(2) >= 2048) return launch_t1<WT, LPR, BPL, 2, T>(a, stream);
  return launch_t1<WT, LPR, BPL, 1, T>(a, stream);
}

template <int WT, int T>
int launch_tshape(const TShape &s, const DmmvTokArgs &a, hipStream_t stream) {
  if constexpr (T <= 2) {
    if (s.bpl == 4) {
      if (s.lpr == 8) return launch_trb<WT, 8, 4, T>(a, stream);
      if (s.lpr == 16) return launch_trb<WT, 16, 4, T>(a, stream);
      if (s.lpr == 32) return launch_trb<WT, 32, 4, T>(a, stream);
      return launch_trb<WT, 64, 4, T>(a, stream);
    }
  }
  if constexpr (T <= 4) {
    if (s.bpl == 2) {
      if (s.lpr == 8) return launch_trb<WT, 8, 2, T>(a, stream);
      if (s.lpr == 16) return launch_trb<WT, 16, 2, T>(a, stream);
      if (s.lpr == 32) return launch_trb<WT, 32, 2, T>(a, stream);
      return launch_trb<WT, 64, 2, T>(a, stream);
    }
  }
  if (s.lpr == 8) return launch_trb<WT, 8, 1, T>(a, stream);
  if (s.lpr == 16) return launch_trb<WT, 16, 1, T>(a, stream);
  if (s.lpr == 32) return launch_trb<WT, 32, 1, T>(a, stream);
  return launch_trb<WT, 64, 1, T>(a, stream);
}

template <int WT>
int launch_tw(DmmvTokArgs a, hipStream_t stream) {
  const int T = a.n_tok <= 2 ? 2 : (a.n_tok <= 4 ? 4 : 8);
  const TShape s = choose_tshape(a.nb, T);
  if (T == 2) return launch_tshape<WT, 2>(s, a, stream);
  if (T == 4) return launch_tshape<WT, 4>(s, a, stream);
  return launch_tshape<WT, 8>(s, a, stream);
}

}  // namespace

int launch_dmmv_tok(int wtype, DmmvTokArgs a, hipStream_t stream) {
  if (a.rows == 0 || a.n_tok == 0) return ZQ_OK;
  a.row_bytes = static_cast<int64_t>(a.nb) * (wtype == ZQ_Q4_0 ? 18 : 34);
  if (wtype == ZQ_Q4_0) return launch_tw<ZQ_Q4_0>(a, stream);
  return launch_tw<ZQ_Q8_0>(a, stream);
}

}  // namespace zq
