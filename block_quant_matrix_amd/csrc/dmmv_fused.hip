// dmmv_fused.hip -- activation quantization fused into the DMMV (gfx950).
//
//   y (+)= W . Q(x)      Q = the activation block quantizer of quantize.hip
//
// One launch per matrix-vector product.  Each workgroup (WPB waves) owns
// WPB*RB*(64/LPR) consecutive rows.  Order of work inside a workgroup:
//   1. every thread issues its load of the fp32 activation (two lanes per
//      32-element block, four float4 each),
//   2. every lane issues all of its weight-block windows (the DMMV mapping of
//      dmmv.hip: one lane per block, RB row steps x BPL blocks),
//   3. the activation (which returns first) is quantized by 2-lane groups
//      into LDS -- codes, scale and 8*sum -- while the weights stream in,
//   4. barrier; each lane reads its blocks' codes from LDS (the activation is
//      staged in LDS once per workgroup and shared by all its waves),
//   5. packed int8 dots per block, fp32 scaling, lane reduction, store.
// The quantized activation can also be written out (by workgroup 0) so that
// later products against the same input need not quantize again.
//
// Each wave walks row groups with a grid stride.  The decode shapes launch
// one group per wave; the LM head (hundreds of thousands of rows) launches a
// bounded grid so that every workgroup quantizes the activation once and then
// streams several groups, and with ARGMAX every workgroup also keeps the best
// (logit, row) pair of the rows it wrote and leaves it for the one-block
// final argmax.
#include "zq_common.h"
#include "zq_internal.h"

namespace zq {

// w, x, rows, row_bytes, k and nb (the fields the first loads need) arrive
// as leading scalars, preloaded into SGPRs (dmmv_hot in zq_internal.h); a
// holds the rest.
template <int WT, int LPR, int BPL, int RB, int WPB, bool ARGMAX, bool NORM>
__global__ __launch_bounds__(64 * WPB) void dmmv_f32x_kernel(const uint8_t *__restrict__ w,
                                                             const float *__restrict__ x,
                                                             int64_t rows, int64_t row_bytes,
                                                             int32_t k, int32_t nb,
                                                             const DmmvF32Args a) {
  constexpr int S = 64 / LPR;
  constexpr int NW = Blk<WT>::NW;
  constexpr int BB = Blk<WT>::BYTES;
  constexpr int T = 64 * WPB;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int8_t *lq = reinterpret_cast<int8_t *>(smem);                  // [k]
  float *ld = reinterpret_cast<float *>(smem + k);                // [nb]
  int32_t *ls8 = reinterpret_cast<int32_t *>(smem + k + 4 * nb);  // [nb]

  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int j = lane & (LPR - 1);
  const int slot = lane / LPR;
  const int64_t n_groups = (rows + RB * S - 1) / (RB * S);
  const int64_t gstride = static_cast<int64_t>(gridDim.x) * WPB;
  int64_t grp = static_cast<int64_t>(blockIdx.x) * WPB + wv;   // first row group of this wave
  int64_t row0 = grp * (RB * S);

  // 1. activation loads for this thread's first block: two lanes per block,
  //    16 elements (four float4) each
  const int g = tid & 1;
  int qb = tid >> 1;
  float xv[16];
  float nw[16];  // the norm weights of the same elements (NORM)
  if (qb < nb) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float4 v = *reinterpret_cast<const float4 *>(x + qb * 32 + g * 16 + 4 * u);
      xv[4 * u] = v.x; xv[4 * u + 1] = v.y; xv[4 * u + 2] = v.z; xv[4 * u + 3] = v.w;
      if constexpr (NORM) {
        const float4 q = *reinterpret_cast<const float4 *>(a.norm_w + qb * 32 + g * 16 + 4 * u);
        nw[4 * u] = q.x; nw[4 * u + 1] = q.y; nw[4 * u + 2] = q.z; nw[4 * u + 3] = q.w;
      }
    }
  }

  // 2. weight windows
  uint32_t win[RB][BPL][NW];
  uint32_t off[RB][BPL];
#pragma unroll
  for (int t = 0; t < RB; ++t) {
    int64_t row = row0 + t * S + slot;
    row = row < rows ? row : rows - 1;
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      int b = j + LPR * i;
      b = b < nb ? b : nb - 1;
      off[t][i] = load_window<WT>(w + row * row_bytes + static_cast<int64_t>(b) * BB, win[t][i]);
    }
  }

  // 2b. NORM: the sum of squares of x over the workgroup (fused
  //     multiply-adds per thread, then block_sum_all), and the factor
  float inv = 1.0f;
  if constexpr (NORM) {
    float ss = 0.0f;
    for (int b = tid >> 1; b < nb; b += T / 2) {
      if (b == (tid >> 1)) {
#pragma unroll
        for (int e = 0; e < 16; ++e) ss = __builtin_fmaf(xv[e], xv[e], ss);
      } else {  // further blocks when k > 16*T
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float4 v = *reinterpret_cast<const float4 *>(x + b * 32 + g * 16 + 4 * u);
          ss = __builtin_fmaf(v.x, v.x, ss);
          ss = __builtin_fmaf(v.y, v.y, ss);
          ss = __builtin_fmaf(v.z, v.z, ss);
          ss = __builtin_fmaf(v.w, v.w, ss);
        }
      }
    }
    ss = block_sum_all<WPB>(ss);
    inv = rms_inv(ss, k, a.eps);
  }

  // 3. quantize the activation into LDS.  Two lanes per block keep the
  //    per-block work (the two IEEE divisions) on as few waves as possible.
  const bool out = (blockIdx.x == 0) && (a.qx_out != nullptr);
  const bool xn_out = NORM && (blockIdx.x == 0) && (a.xn_out != nullptr);
  for (; qb < nb; qb += T / 2) {
    if (qb != (tid >> 1)) {  // further blocks when k > 16*T (not for k <= 16384)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4 v = *reinterpret_cast<const float4 *>(x + qb * 32 + g * 16 + 4 * u);
        xv[4 * u] = v.x; xv[4 * u + 1] = v.y; xv[4 * u + 2] = v.z; xv[4 * u + 3] = v.w;
        if constexpr (NORM) {
          const float4 q = *reinterpret_cast<const float4 *>(a.norm_w + qb * 32 + g * 16 + 4 * u);
          nw[4 * u] = q.x; nw[4 * u + 1] = q.y; nw[4 * u + 2] = q.z; nw[4 * u + 3] = q.w;
        }
      }
    }
    if constexpr (NORM) {
#pragma clang fp contract(off)
#pragma unroll
      for (int e = 0; e < 16; ++e) xv[e] = (xv[e] * inv) * nw[e];
      if (xn_out) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          *reinterpret_cast<float4 *>(a.xn_out + qb * 32 + g * 16 + 4 * u) =
              make_float4(xv[4 * u], xv[4 * u + 1], xv[4 * u + 2], xv[4 * u + 3]);
      }
    }
    uint32_t pk[4];
    float d;
    int32_t s;
    quantize_block<2>(xv, pk, d, s);
    *reinterpret_cast<u32x4 *>(lq + qb * 32 + g * 16) = u32x4{pk[0], pk[1], pk[2], pk[3]};
    if (g == 0) {
      ld[qb] = d;
      ls8[qb] = 8 * s;
    }
    if (out) {
      uint32_t *qo = reinterpret_cast<uint32_t *>(a.qx_out + qb * 32 + g * 16);
      qo[0] = pk[0]; qo[1] = pk[1]; qo[2] = pk[2]; qo[3] = pk[3];
      if (g == 0) {
        if (a.dx_out) a.dx_out[qb] = d;
        if (a.sx_out) a.sx_out[qb] = s;
      }
    }
  }
  __syncthreads();

  // 4. this lane's activation blocks from LDS
  uint32_t xq[BPL][8];
  float xd[BPL];
  int32_t xs8[BPL];
#pragma unroll
  for (int i = 0; i < BPL; ++i) {
    const int b = j + LPR * i;
    if (b < nb) {
      const u32x4 v0 = *reinterpret_cast<const u32x4 *>(lq + 32 * b);
      const u32x4 v1 = *reinterpret_cast<const u32x4 *>(lq + 32 * b + 16);
      xq[i][0] = v0.x; xq[i][1] = v0.y; xq[i][2] = v0.z; xq[i][3] = v0.w;
      xq[i][4] = v1.x; xq[i][5] = v1.y; xq[i][6] = v1.z; xq[i][7] = v1.w;
      xd[i] = ld[b];
      xs8[i] = WT == ZQ_Q4_0 ? ls8[b] : 0;
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) xq[i][k] = 0;
      xd[i] = 0.0f;
      xs8[i] = 0;
    }
  }

  // 5. dots, scaling, reduction, store; then the next row group
  float best_v = -__builtin_inff();
  int32_t best_i = 0x7fffffff;
  for (;;) {
    float acc[RB];
#pragma unroll
    for (int t = 0; t < RB; ++t) {
      float p = 0.0f;
#pragma unroll
      for (int i = 0; i < BPL; ++i) {
        const float dw = window_scale(win[t][i][0], off[t][i]);
        const uint32_t sel = quant_selector(off[t][i]);
        int32_t isum;
        if constexpr (WT == ZQ_Q4_0) {
          isum = q4_raw_dot(win[t][i], sel, xq[i]) - xs8[i];
        } else {
          isum = q8_dot(win[t][i], sel, xq[i]);
        }
        p = __builtin_fmaf(dw * xd[i], static_cast<float>(isum), p);
      }
      acc[t] = p;
    }
    using R = RowReduce<LPR, RB>;
    float res[R::NOUT];
    R::run(acc, res);
    if (R::writer(lane)) {
#pragma unroll
      for (int m = 0; m < R::NOUT; ++m) {
        const int64_t row = row0 + static_cast<int64_t>(R::rowstep(m, lane)) * S + slot;
        if (row < rows) {
          float *yp = a.y + row;
          const float v = (a.flags & ZQ_ACCUMULATE) ? *yp + res[m] : res[m];
          *yp = v;
          if constexpr (ARGMAX) {
            if (beats(v, static_cast<int32_t>(row), best_v, best_i)) {
              best_v = v;
              best_i = static_cast<int32_t>(row);
            }
          }
        }
      }
    }
    grp += gstride;
    if (grp >= n_groups) break;
    row0 = grp * (RB * S);
#pragma unroll
    for (int t = 0; t < RB; ++t) {
      int64_t row = row0 + t * S + slot;
      row = row < rows ? row : rows - 1;
#pragma unroll
      for (int i = 0; i < BPL; ++i) {
        int b = j + LPR * i;
        b = b < nb ? b : nb - 1;
        off[t][i] = load_window<WT>(w + row * row_bytes + static_cast<int64_t>(b) * BB, win[t][i]);
      }
    }
  }
  if constexpr (ARGMAX) {
    block_best<WPB>(best_v, best_i);
    if (threadIdx.x == 0) static_cast<ValIdx *>(a.part)[blockIdx.x] = ValIdx{best_v, best_i};
  }
}

namespace {

struct FShape {
  int lpr, bpl;
};
// Single-pass layouts: nb <= LPR * BPL.
constexpr FShape kFShapes[] = {{8, 1}, {16, 1}, {32, 1}, {64, 1}, {64, 2}, {32, 5}, {64, 4}, {64, 8}};

template <int WT, int LPR, int BPL, int RB, int WPB>
int launch_f(const DmmvF32Args &a, hipStream_t stream) {
  constexpr int S = 64 / LPR;
  const int64_t rows_per_wg = static_cast<int64_t>(WPB) * RB * S;
  int64_t grid = (a.rows + rows_per_wg - 1) / rows_per_wg;
  const size_t lds = static_cast<size_t>(a.k) + 8 * static_cast<size_t>(a.nb);
  const dim3 gd(static_cast<unsigned>(a.part && grid > kArgmaxMaxParts ? kArgmaxMaxParts : grid));
  if (a.part) {
    if (a.norm_w)
      hipLaunchKernelGGL((dmmv_f32x_kernel<WT, LPR, BPL, RB, WPB, true, true>), gd, dim3(64 * WPB),
                         lds, stream, a.w, a.x, a.rows, a.row_bytes, a.k, a.nb, a);
    else
      hipLaunchKernelGGL((dmmv_f32x_kernel<WT, LPR, BPL, RB, WPB, true, false>), gd, dim3(64 * WPB),
                         lds, stream, a.w, a.x, a.rows, a.row_bytes, a.k, a.nb, a);
    ZQ_LAUNCH_CHECK();
    if (a.out_idx) return launch_argmax_final(a.part, static_cast<int>(gd.x), a.out_idx, stream);
    return ZQ_OK;
  }
  if (a.norm_w)
    hipLaunchKernelGGL((dmmv_f32x_kernel<WT, LPR, BPL, RB, WPB, false, true>), gd, dim3(64 * WPB),
                       lds, stream, a.w, a.x, a.rows, a.row_bytes, a.k, a.nb, a);
  else
    hipLaunchKernelGGL((dmmv_f32x_kernel<WT, LPR, BPL, RB, WPB, false, false>), gd, dim3(64 * WPB),
                       lds, stream, a.w, a.x, a.rows, a.row_bytes, a.k, a.nb, a);
  ZQ_LAUNCH_CHECK();
  return ZQ_OK;
}

// Small matrices (decode, up to 256 workgroups): one workgroup quantizes the
// activation for all of its rows.  With one or two blocks per lane, 8 waves
// of two row steps each (16 rows of 4096, 3.33 us against 3.40 for 16 waves
// of one row and 3.47 for 4 waves of four; 2048 x 2048: 2.38 against 2.56),
// except for a few hundred rows without the norm, which keep 16 waves of one
// row step (64 x 2048 Q8_0: 2.28 against 2.37 us), and with the norm, whose
// sum of squares is reduced over the workgroup, fewer waves (below).
// With more blocks per lane, 8 waves of one row step (2048 x 8192: 4.28
// against 4.83 for two).
template <int WT, int LPR, int BPL>
int launch_fs(const DmmvF32Args &a, hipStream_t stream) {
  constexpr int S = 64 / LPR;
  constexpr int RBS = BPL <= 2 ? 2 : 1;
  if constexpr (BPL <= 2) {
    if (a.rows <= 256 && a.norm_w == nullptr) return launch_f<WT, LPR, BPL, 1, 16>(a, stream);
  }
  // A few hundred rows with the norm: 4 waves of one row step.  The 128-row
  // router of a 40-layer chain (32 workgroups), alternating on one box:
  // 673-674 us per token against 689-690 with 8 waves of two row steps
  // (4 x 2: 675; 2 x 2: 672-674; 2 x 1: 676; 1 x 2: 732).
  if (a.norm_w && a.rows <= 256) return launch_f<WT, LPR, BPL, 1, 4>(a, stream);
  if (a.rows <= static_cast<int64_t>(256) * 8 * RBS * S)
    return launch_f<WT, LPR, BPL, RBS, 8>(a, stream);
  if (a.rows <= 16384) {
    // Mid-size matrices: 8 waves per workgroup, row steps by blocks per lane
    // (a sweep of 1/2/4/8 row steps x 4/8 waves; us per launch):
    //   one block per lane, 4 row steps: 6144 x 2048 3.01 (4 waves of 8
    //     steps: 3.35), 16384 x 2048 4.79 (5.05), 11008 x 2048 4.53 (4.78);
    //   two blocks, 2 row steps up to 8192 rows, else 4: 8192 x 4096 4.94
    //     (4 waves of 4: 5.14), 14336 x 4096 7.36 (8.16);
    //   four or more, 2 row steps: 4096 x 8192 5.66 (4 waves: 6.82),
    //     5120 x 5120 5.47 (6.78), 4096 x 14336 10.64 (12.46).
    if constexpr (BPL == 1) return launch_f<WT, LPR, BPL, 4, 8>(a, stream);
    if constexpr (BPL == 2) {
      if (a.rows <= static_cast<int64_t>(8192) * S) return launch_f<WT, LPR, BPL, 2, 8>(a, stream);
      return launch_f<WT, LPR, BPL, 4, 8>(a, stream);
    }
    return launch_f<WT, LPR, BPL, 2, 8>(a, stream);
  }
  // Large matrices (the LM head), windows held per lane RB * BPL.  One
  // block per lane: 8 waves of 4 row steps (the 248 320 x 2048 LM head with
  // argmax, Q4_0 50.3 us against 50.9 for 4 waves of 8, Q8_0 89.3 against
  // 93.0); otherwise four waves of several row steps.
  if constexpr (BPL == 1) return launch_f<WT, LPR, BPL, 4, 8>(a, stream);
  if constexpr (BPL == 2) return launch_f<WT, LPR, BPL, 4, 4>(a, stream);
  return launch_f<WT, LPR, BPL, 2, 4>(a, stream);
}

template <int WT>
int launch_fw(const FShape &s, const DmmvF32Args &a, hipStream_t stream) {
  if (s.lpr == 8) return launch_fs<WT, 8, 1>(a, stream);
  if (s.lpr == 16) return launch_fs<WT, 16, 1>(a, stream);
  if (s.lpr == 32 && s.bpl == 1) return launch_fs<WT, 32, 1>(a, stream);
  if (s.lpr == 32 && s.bpl == 5) return launch_fs<WT, 32, 5>(a, stream);
  if (s.lpr == 64 && s.bpl == 1) return launch_fs<WT, 64, 1>(a, stream);
  if (s.lpr == 64 && s.bpl == 2) return launch_fs<WT, 64, 2>(a, stream);
  if (s.lpr == 64 && s.bpl == 4) return launch_fs<WT, 64, 4>(a, stream);
  return launch_fs<WT, 64, 8>(a, stream);
}

}  // namespace

int launch_dmmv_f32x(int wtype, DmmvF32Args a, hipStream_t stream) {
  if (a.rows == 0) return ZQ_OK;
  a.row_bytes = static_cast<int64_t>(a.nb) * (wtype == ZQ_Q4_0 ? 18 : 34);
  // the single-pass layout with the least idle lanes
  FShape best = kFShapes[0];
  int64_t waste = -1;
  for (const FShape &s : kFShapes) {
    const int64_t cap = static_cast<int64_t>(s.lpr) * s.bpl;
    if (cap < a.nb) continue;
    const int64_t w = cap - a.nb;
    if (waste < 0 || w < waste || (w == waste && s.lpr > best.lpr)) {
      best = s;
      waste = w;
    }
  }
  if (waste < 0) return ZQ_EINVAL;
  if (wtype == ZQ_Q4_0) return launch_fw<ZQ_Q4_0>(best, a, stream);
  return launch_fw<ZQ_Q8_0>(best, a, stream);
}

}  // namespace zq
