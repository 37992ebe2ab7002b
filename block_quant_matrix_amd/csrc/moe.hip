// moe.hip -- the MoE expert FFN of one token in two launches (gfx950).
//
// gate/up pass (moe_gate_up_kernel): one workgroup of 16 waves per
// (selected expert, 32-wide block of the FFN width).  It quantizes the fp32
// activation into LDS (two lanes per 32-element block), computes the 32 gate
// rows and the 32 matching up rows of that expert with the lane-per-block
// DMMV mapping, and finishes in its epilogue with SwiGLU
// h = silu(g) * u (fp64, one rounding to fp32) and the re-quantization of
// that 32-element block of h: codes, scale and block sum go straight to the
// down pass's input.  The swiglu + quantize step never round-trips through
// a separate launch.
//
// down pass (moe_down_kernel): every lane owns one (row, block) of the down
// matrices and issues the windows of ALL selected experts before any
// arithmetic (up to 16 per chunk), with the selected experts' quantized
// activations staged in LDS.  The per-expert weight multiplies each expert's
// partial before the single lane reduction, so the weighted accumulate costs
// one FMA per expert and lane.
#include <type_traits>

#include "zq_common.h"
#include "zq_internal.h"
#include "zq_kquant.h"
#include "zq_moe_tok.h"

namespace zq {

// ------------------------------------------------------------- gate/up ----
// Pieces shared by the block-format and K-quant gate/up kernels: one
// workgroup of T threads per (selected expert, 32-wide block of the FFN
// width), computing 32 gate rows and the 32 matching up rows.

// The gate/up kernels' leading scalars: the fields their first loads need,
// as preloaded kernel arguments (see dmmv_hot in zq_internal.h).
__device__ __forceinline__ void gu_hot(MoeGateUpArgs &a, const float *x, const float *logits,
                                       const int32_t *ids, int32_t nb, int32_t k, int32_t n_routed,
                                       int32_t top_k, int32_t id_base) {
  a.x = x;
  a.logits = logits;
  a.ids = ids;
  a.nb = nb;
  a.k = k;
  a.n_routed = n_routed;
  a.top_k = top_k;
  a.id_base = id_base;
}

// Loads of the fp32 activation for this thread's first 32-element block (two
// lanes per block, 16 elements each); issued before anything is waited on.
__device__ __forceinline__ void gu_load_x(const MoeGateUpArgs &a, int nb, int tid,
                                          float (&xv)[16]) {
  const int g = tid & 1;
  const int qb = tid >> 1;
  if (qb < nb) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float4 v = *reinterpret_cast<const float4 *>(a.x + qb * 32 + g * 16 + 4 * u);
      xv[4 * u] = v.x; xv[4 * u + 1] = v.y; xv[4 * u + 2] = v.z; xv[4 * u + 3] = v.w;
    }
  }
}

// The expert of slot s: ranked from the logits by the workgroup itself
// (ROUTED: slot s < top_k takes rank s, slot top_k the shared expert, id
// n_routed) or read from ids, less id_base.  rsel / rselv (LDS, 64) keep the
// ranked selection for the publication at the end.  Every thread calls it.
template <bool ROUTED, int T>
__device__ __forceinline__ int gu_expert(const MoeGateUpArgs &a, int tid, int s, int32_t *rsel,
                                         float *rselv) {
  if constexpr (ROUTED) {
    // the shared slot's workgroups need no ranking (the publication is
    // slot 0's)
    if (s >= a.top_k) return a.n_routed;  // uniform over the workgroup
    __shared__ __attribute__((aligned(16))) float rlv[1024];
    const int n_pad = route_stage<8, T>(rlv, a.logits, a.n_routed);
    __syncthreads();
    route_rank<8, T>(rlv, a.n_routed, n_pad, a.top_k, rsel, rselv);
    __syncthreads();
    return s < a.top_k ? rsel[s] : a.n_routed;
  } else {
    return a.ids[s] - a.id_base;
  }
}

// Quantize x into LDS (two lanes per block, the first block already in xv):
// codes, scales and the block sums times SUMX.
template <int T, int SUMX>
__device__ __forceinline__ void gu_quantize_x(const MoeGateUpArgs &a, int nb, int tid,
                                              float (&xv)[16], int8_t *lq, float *ld,
                                              int32_t *ls) {
  const int g = tid & 1;
  for (int qb = tid >> 1; qb < nb; qb += T / 2) {
    if (qb != (tid >> 1)) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4 v = *reinterpret_cast<const float4 *>(a.x + qb * 32 + g * 16 + 4 * u);
        xv[4 * u] = v.x; xv[4 * u + 1] = v.y; xv[4 * u + 2] = v.z; xv[4 * u + 3] = v.w;
      }
    }
    uint32_t pk[4];
    float d;
    int32_t sum;
    quantize_block<2>(xv, pk, d, sum);
    *reinterpret_cast<u32x4 *>(lq + qb * 32 + g * 16) = u32x4{pk[0], pk[1], pk[2], pk[3]};
    if (g == 0) {
      ld[qb] = d;
      ls[qb] = SUMX * sum;
    }
  }
}

// Gate row lr (0..31) or up row lr (32..63) of FFN block hb, as a matrix row.
__device__ __forceinline__ int64_t gu_row(const MoeGateUpArgs &a, int hb, int lr) {
  return (lr < 32) ? (32 * hb + lr) : (a.d_ff + 32 * hb + (lr - 32));
}

// Epilogue, after the 64 row results are in lrow: SwiGLU over the 32
// outputs (fp64, one rounding; one output per lane of wave 0, so the 32
// exponentials run side by side) and their quantization (8 lanes, four
// elements each, gathered by shuffles), then the router's publication
// (ROUTED, one workgroup).
template <bool ROUTED>
__device__ __forceinline__ void gu_epilogue(const MoeGateUpArgs &a, int tid, int s, int hb,
                                            const float *lrow, const int32_t *rsel,
                                            const float *rselv) {
  float h = 0.0f;
  if (tid < 64) {
    const int i = tid & 31;
    const double gd = static_cast<double>(lrow[i]);
    const double silu = gd / (1.0 + exp(-gd));
    h = static_cast<float>(silu * static_cast<double>(lrow[32 + i]));
  }
  float hv[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) hv[q] = __shfl(h, 4 * (tid & 7) + q);
  if (tid < 8) {
    const int i0 = 4 * tid;
    uint32_t packed[1];
    float d;
    int32_t sum;
    quantize_block<8>(hv, packed, d, sum);
    const int64_t hoff = static_cast<int64_t>(s) * a.d_ff + 32 * hb + i0;
    *reinterpret_cast<uint32_t *>(a.qh + hoff) = packed[0];
    if (tid == 0) {
      a.dh[static_cast<int64_t>(s) * (a.d_ff / 32) + hb] = d;
      if (a.sh) a.sh[static_cast<int64_t>(s) * (a.d_ff / 32) + hb] = sum;
    }
    if (a.h_out) *reinterpret_cast<float4 *>(a.h_out + hoff) = make_float4(hv[0], hv[1], hv[2], hv[3]);
    if (a.gu_out) {
      float *gp = a.gu_out + static_cast<int64_t>(s) * 2 * a.d_ff;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        gp[32 * hb + i0 + q] = lrow[i0 + q];
        gp[a.d_ff + 32 * hb + i0 + q] = lrow[32 + i0 + q];
      }
    }
  }
  // one workgroup publishes the expert list and weights for the down pass,
  // last, so that the fp64 softmax delays none of its loads
  if constexpr (ROUTED) {
    if (blockIdx.x == 0 && blockIdx.y == 0) {  // uniform over the workgroup
      __shared__ double rsele[64];
      route_weights(rsel, rselv, rsele, a.n_routed, a.top_k, a.shared_gate, a.ids_out, a.wts_out);
    }
  }
}

// The 64 rows of one gate/up workgroup in the block formats (Q4_0 / Q8_0):
// LPR lanes per row, BPL blocks per lane, RB row steps per wave, 16 waves.
// load() issues the weight windows; rows() takes the activation from LDS
// (codes, scales and SUMX times the block sums) and leaves the 64 row
// results in lrow.
template <int WT, int LPR, int BPL, int RB>
struct GuBlockRows {
  static constexpr int S = 64 / LPR;
  static constexpr int NW = Blk<WT>::NW;
  static constexpr int BB = Blk<WT>::BYTES;
  static constexpr int SUMX = 8;  // the Q4_0 dot subtracts 8 times the code sum
  static_assert(RB * S * 16 == 64, "a workgroup computes 32 gate + 32 up rows");
  static constexpr int64_t row_bytes_for(int nb) { return static_cast<int64_t>(nb) * BB; }
  uint32_t win[RB][BPL][NW];
  uint32_t off[RB][BPL];

  __device__ __forceinline__ void load(const MoeGateUpArgs &a, int nb, const uint8_t *wb,
                                       int64_t row_bytes, int hb, int tid) {
    const int lane = tid & 63, wv = tid >> 6;
    const int j = lane & (LPR - 1), slot = lane / LPR;
#pragma unroll
    for (int t = 0; t < RB; ++t) {
      const int64_t row = gu_row(a, hb, wv * (RB * S) + t * S + slot);
#pragma unroll
      for (int i = 0; i < BPL; ++i) {
        int b = j + LPR * i;
        b = b < nb ? b : nb - 1;
        off[t][i] = load_window<WT>(wb + row * row_bytes + static_cast<int64_t>(b) * BB, win[t][i]);
      }
    }
  }

  __device__ __forceinline__ void rows(int nb, const int8_t *lq, const float *ld,
                                       const int32_t *ls, float *lrow, int tid) {
    const int lane = tid & 63, wv = tid >> 6;
    const int j = lane & (LPR - 1), slot = lane / LPR;
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
        xs8[i] = WT == ZQ_Q4_0 ? ls[b] : 0;
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) xq[i][k] = 0;
        xd[i] = 0.0f;
        xs8[i] = 0;
      }
    }
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
      for (int m = 0; m < R::NOUT; ++m) lrow[wv * (RB * S) + R::rowstep(m, lane) * S + slot] = res[m];
    }
  }
};

// The same for the K-quants: one lane per 64-element unit, the row in one
// pass (k = 64 * LPR), against the activation staged in LDS with plain code
// sums.
template <int WT, int LPR, int RB>
struct GuKRows {
  static constexpr int S = 64 / LPR;
  static constexpr int NWD = KQ<WT>::NWD;
  static constexpr int SUMX = 1;
  static_assert(RB * S * 16 == 64, "a workgroup computes 32 gate + 32 up rows");
  static constexpr int64_t row_bytes_for(int nb) {
    return static_cast<int64_t>(nb / 8) * KQ<WT>::BYTES;
  }
  uint32_t v[RB][NWD];

  __device__ __forceinline__ void load(const MoeGateUpArgs &a, int nb, const uint8_t *wb,
                                       int64_t row_bytes, int hb, int tid) {
    (void)nb;
    const int lane = tid & 63, wv = tid >> 6;
    const int j = lane & (LPR - 1), slot = lane / LPR;
#pragma unroll
    for (int t = 0; t < RB; ++t) {
      const int64_t row = gu_row(a, hb, wv * (RB * S) + t * S + slot);
      load_unit_w<WT>(wb + row * row_bytes + static_cast<int64_t>(j >> 2) * KQ<WT>::BYTES, j & 3,
                      v[t]);
    }
  }

  __device__ __forceinline__ void rows(int nb, const int8_t *lq, const float *ld,
                                       const int32_t *ls, float *lrow, int tid) {
    (void)nb;
    const int lane = tid & 63, wv = tid >> 6;
    const int j = lane & (LPR - 1), slot = lane / LPR;
    KUnitAct act;
    if constexpr (WT == ZQ_Q6_K) {
      const int base = 256 * (j >> 2) + 128 * ((j >> 1) & 1) + 16 * (j & 1);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 q = *reinterpret_cast<const u32x4 *>(lq + base + 32 * c);
        act.q[4 * c] = q.x; act.q[4 * c + 1] = q.y; act.q[4 * c + 2] = q.z; act.q[4 * c + 3] = q.w;
        act.d[c] = ld[(base + 32 * c) >> 5];
        act.m32[c] = -32 * code_sum(&act.q[4 * c], 4);
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 q = *reinterpret_cast<const u32x4 *>(lq + 64 * j + 16 * c);
        act.q[4 * c] = q.x; act.q[4 * c + 1] = q.y; act.q[4 * c + 2] = q.z; act.q[4 * c + 3] = q.w;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        act.d[h] = ld[2 * j + h];
        act.fs[h] = static_cast<float>(ls[2 * j + h]);
      }
    }
    float acc[RB];
#pragma unroll
    for (int t = 0; t < RB; ++t) {
      int32_t is[4];
      acc[t] = unit_dot<WT>(v[t], j & 3, act, is);
    }
    using R = RowReduce<LPR, RB>;
    float res[R::NOUT];
    R::run(acc, res);
    if (R::writer(lane)) {
#pragma unroll
      for (int m = 0; m < R::NOUT; ++m) lrow[wv * (RB * S) + R::rowstep(m, lane) * S + slot] = res[m];
    }
  }
};

// The row layouts per d_model: 64 rows per 16-wave workgroup, one pass.
template <int WT, int NB> struct GuRowsFor;
template <int WT> struct GuRowsFor<WT, 16> { using type = GuBlockRows<WT, 16, 1, 1>; };
template <int WT> struct GuRowsFor<WT, 32> { using type = GuBlockRows<WT, 32, 1, 2>; };
template <int WT> struct GuRowsFor<WT, 64> { using type = GuBlockRows<WT, 64, 1, 4>; };
template <int WT> struct GuRowsFor<WT, 128> { using type = GuBlockRows<WT, 64, 2, 4>; };
template <int WT, int NB> struct GuKRowsFor;
template <int WT> struct GuKRowsFor<WT, 32> { using type = GuKRows<WT, 16, 1>; };
template <int WT> struct GuKRowsFor<WT, 64> { using type = GuKRows<WT, 32, 2>; };
template <int WT> struct GuKRowsFor<WT, 128> { using type = GuKRows<WT, 64, 4>; };

// LDS of a gate/up workgroup: x codes [k], scales [nb], sums [nb], then the
// 64 row results.
struct GuLds {
  int8_t *lq;
  float *ld;
  int32_t *ls;
  float *lrow;
  __device__ __forceinline__ GuLds(uint8_t *smem, int k, int nb)
      : lq(reinterpret_cast<int8_t *>(smem)),
        ld(reinterpret_cast<float *>(smem + k)),
        ls(reinterpret_cast<int32_t *>(smem + k + 4 * nb)),
        lrow(reinterpret_cast<float *>(smem + k + 8 * nb)) {}
};

// One workgroup of the gate/up pass after its expert is known: issue the
// weights, quantize x into LDS meanwhile, the 64 rows, the epilogue.
template <class Rows, bool ROUTED>
__device__ __forceinline__ void gu_run(const MoeGateUpArgs &a, int nb, const uint8_t *wb,
                                       int64_t row_bytes, float (&xv)[16], const GuLds &L,
                                       int tid, int s, int hb, const int32_t *rsel,
                                       const float *rselv) {
  constexpr int T = 1024;
  Rows r;
  r.load(a, nb, wb, row_bytes, hb, tid);
  gu_quantize_x<T, Rows::SUMX>(a, nb, tid, xv, L.lq, L.ld, L.ls);
  __syncthreads();
  r.rows(nb, L.lq, L.ld, L.ls, L.lrow, tid);
  __syncthreads();
  gu_epilogue<ROUTED>(a, tid, s, hb, L.lrow, rsel, rselv);
}

// The gate/up pass over one bank (Rows: GuBlockRows or GuKRows): grid
// (d_ff / 32, n_sel), 1024 threads.
template <class Rows, bool ROUTED>
__global__ __launch_bounds__(1024) void moe_gate_up_kernel(const float *x, const float *logits,
                                                           const int32_t *ids, int32_t nb, int32_t k,
                                                           int32_t n_routed, int32_t top_k,
                                                           int32_t id_base, const MoeGateUpArgs a_in) {
  MoeGateUpArgs a = a_in;
  gu_hot(a, x, logits, ids, nb, k, n_routed, top_k, id_base);
  constexpr int T = 1024;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const GuLds L(smem, a.k, a.nb);
  const int tid = static_cast<int>(threadIdx.x);
  const int hb = static_cast<int>(blockIdx.x);  // 32-wide block of the FFN width
  const int s = static_cast<int>(blockIdx.y);   // selected-expert slot
  // activation loads, issued before the expert id so that they share its
  // round trip
  float xv[16];
  gu_load_x(a, a.nb, tid, xv);
  __shared__ int32_t rsel[64];
  __shared__ float rselv[64];
  const int e = gu_expert<ROUTED, T>(a, tid, s, rsel, rselv);
  if (e < 0 || e >= a.n_experts) {  // uniform over the workgroup
    if (a.status && tid == 0) *a.status = ZQ_ERANGE;
    return;
  }
  gu_run<Rows, ROUTED>(a, a.nb, a.bank + static_cast<int64_t>(e) * a.expert_stride, a.row_bytes,
                       xv, L, tid, s, hb, rsel, rselv);
}

// Routed experts and a shared expert of another format in one launch, the
// router folded in: slots 0..top_k-1 (Rows over a.bank) take the experts
// the workgroups rank; slot top_k (SRows over a.bank2, one matrix) is the
// shared expert.  grid (d_ff / 32, top_k + 1).  The row width (NB blocks)
// is a compile-time constant here, which keeps the scalar registers of the
// two layouts within bounds.
template <class Rows, class SRows, int NB>
__global__ __launch_bounds__(1024) void moe_gate_up_mix_kernel(const float *x, const float *logits,
                                                               const int32_t *ids, int32_t nb,
                                                               int32_t k, int32_t n_routed,
                                                               int32_t top_k, int32_t id_base,
                                                               const MoeGateUpArgs a_in) {
  MoeGateUpArgs a = a_in;
  gu_hot(a, x, logits, ids, nb, k, n_routed, top_k, id_base);
  constexpr int T = 1024;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const GuLds L(smem, 32 * NB, NB);
  const int tid = static_cast<int>(threadIdx.x);
  const int hb = static_cast<int>(blockIdx.x);
  const int s = static_cast<int>(blockIdx.y);
  float xv[16];
  gu_load_x(a, NB, tid, xv);
  __shared__ int32_t rsel[64];
  __shared__ float rselv[64];
  if (s < a.top_k) {  // uniform over the workgroup
    const int e = gu_expert<true, T>(a, tid, s, rsel, rselv);  // in [0, n_routed)
    gu_run<Rows, true>(a, NB, a.bank + static_cast<int64_t>(e) * a.expert_stride,
                       Rows::row_bytes_for(NB), xv, L, tid, s, hb, rsel, rselv);
  } else {
    // (the publication is slot 0's, never this slot's)
    gu_run<SRows, false>(a, NB, a.bank2, SRows::row_bytes_for(NB), xv, L, tid, s, hb, rsel, rselv);
  }
}

// ---------------------------------------------------------------- down -----

// The down kernels' leading scalars (preloaded kernel arguments, as dmmv_hot).
__device__ __forceinline__ void dn_hot(MoeDownArgs &a, const int32_t *ids, const int8_t *qx,
                                       const float *dx, int64_t x_stride, int64_t rows,
                                       int32_t n_sel, int32_t nb, int32_t id_base) {
  a.ids = ids;
  a.qx = qx;
  a.dx = dx;
  a.x_stride = x_stride;
  a.rows = rows;
  a.n_sel = n_sel;
  a.nb = nb;
  a.id_base = id_base;
}

// The weighted sum over experts with the experts spread over the lanes (as
// the K-quant form in dmmv_k.hip): lane = (slot, part), LPS lanes per slot
// and BPL blocks per lane (k = 32 * nb <= 32 * LPS * BPL), 64 / LPS slots
// side by side, the partials reduced over the whole wave.  A wave takes RB
// consecutive rows; every selected expert's windows for them are requested
// at once.  Slots beyond 64 / LPS take further rounds.  A lane whose expert
// id is out of range contributes nothing and reports ZQ_ERANGE.
template <int WT, int LPS, int BPL, int RB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void moe_down_wsum_kernel(
    const int32_t *ids, const int8_t *qx, const float *dx, int64_t x_stride, int64_t rows,
    int32_t n_sel, int32_t nb, int32_t id_base, const MoeDownArgs a_in) {
  MoeDownArgs a = a_in;
  dn_hot(a, ids, qx, dx, x_stride, rows, n_sel, nb, id_base);
  constexpr int SL = 64 / LPS;
  constexpr int NW = Blk<WT>::NW;
  constexpr int BB = Blk<WT>::BYTES;
  const int lane = static_cast<int>(threadIdx.x & 63);
  const int j = lane & (LPS - 1);
  const int sl = lane / LPS;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t n_waves = static_cast<int64_t>(gridDim.x) * 4;
  const int64_t n_groups = (a.rows + RB - 1) / RB;
  const int n_rounds = (a.n_sel + SL - 1) / SL;
  const int64_t xs32 = a.x_stride / 32;

  uint32_t xq[BPL][8];
  float xd[BPL];
  int32_t xsr[BPL];  // Q4_0: the blocks' code sums as given (sx), else unused
  // the lane's slot's activation blocks (scale 0 past the row end); loads
  // only, the sums of a missing sx are taken once the weights are requested
  auto load_act = [&](int sc) {
    const int8_t *qx = a.qx + static_cast<int64_t>(sc) * a.x_stride;
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      int b = j + LPS * i;
      const bool bok = b < a.nb;
      b = bok ? b : a.nb - 1;
      const u32x4 v0 = *reinterpret_cast<const u32x4 *>(qx + 32 * b);
      const u32x4 v1 = *reinterpret_cast<const u32x4 *>(qx + 32 * b + 16);
      xq[i][0] = v0.x; xq[i][1] = v0.y; xq[i][2] = v0.z; xq[i][3] = v0.w;
      xq[i][4] = v1.x; xq[i][5] = v1.y; xq[i][6] = v1.z; xq[i][7] = v1.w;
      const float d = a.dx[sc * xs32 + b];
      xd[i] = bok ? d : 0.0f;
      xsr[i] = (WT == ZQ_Q4_0 && a.sx) ? a.sx[sc * xs32 + b] : 0;
    }
  };
  const bool hoist = n_rounds == 1;
  if (hoist && a.n_sel > 0) load_act(sl < a.n_sel ? sl : a.n_sel - 1);

  for (int64_t gi = wave; gi < n_groups; gi += n_waves) {
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
      const uint8_t *wb = a.bank + static_cast<int64_t>(ok ? e : 0) * a.expert_stride;
      if (!hoist) load_act(sc);
      uint32_t win[RB][BPL][NW];
      uint32_t off[RB][BPL];
#pragma unroll
      for (int t = 0; t < RB; ++t) {
        int64_t row = row0 + t;
        row = row < a.rows ? row : a.rows - 1;
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
          int b = j + LPS * i;
          b = b < a.nb ? b : a.nb - 1;
          off[t][i] = load_window<WT>(wb + row * a.row_bytes + static_cast<int64_t>(b) * BB, win[t][i]);
        }
      }
      int32_t xsum[BPL];
#pragma unroll
      for (int i = 0; i < BPL; ++i) {
        xsum[i] = 0;
        if constexpr (WT == ZQ_Q4_0) xsum[i] = a.sx ? xsr[i] : code_sum(xq[i], 8);
      }
#pragma unroll
      for (int t = 0; t < RB; ++t) {
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
          const float dw = window_scale(win[t][i][0], off[t][i]);
          const uint32_t sel = quant_selector(off[t][i]);
          int32_t isum;
          if constexpr (WT == ZQ_Q4_0) {
            isum = q4_raw_dot(win[t][i], sel, xq[i]) - 8 * xsum[i];
          } else {
            isum = q8_dot(win[t][i], sel, xq[i]);
          }
          part = __builtin_fmaf(dw * xd[i], static_cast<float>(isum), part);
        }
        acc[t] = ok ? __builtin_fmaf(ws, part, acc[t]) : acc[t];
      }
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

constexpr int kDownMaxSel = 16;  // experts whose windows are in flight at once

template <int WT, int LPR, int BPL, int WPB>
__global__ __launch_bounds__(64 * WPB) void moe_down_kernel(const int32_t *ids, const int8_t *qx,
                                                           const float *dx, int64_t x_stride,
                                                           int64_t rows, int32_t n_sel, int32_t nb,
                                                           int32_t id_base, const MoeDownArgs a_in) {
  MoeDownArgs a = a_in;
  dn_hot(a, ids, qx, dx, x_stride, rows, n_sel, nb, id_base);
  constexpr int S = 64 / LPR;
  constexpr int NW = Blk<WT>::NW;
  constexpr int BB = Blk<WT>::BYTES;
  constexpr int T = 64 * WPB;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // per slot: codes [k], then scales [nb] and 8*sums [nb] after all codes
  int8_t *lq = reinterpret_cast<int8_t *>(smem);
  float *ld = reinterpret_cast<float *>(smem + static_cast<int64_t>(a.n_sel) * a.k);
  int32_t *ls8 = reinterpret_cast<int32_t *>(ld + static_cast<int64_t>(a.n_sel) * a.nb);

  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int j = lane & (LPR - 1);
  const int slot = lane / LPR;
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * WPB + wv) * S;
  int64_t row = row0 + slot;
  const bool row_ok = row < a.rows;
  row = row_ok ? row : a.rows - 1;

  float acc = 0.0f;
  bool first = true;
  for (int s0 = 0; s0 < a.n_sel; s0 += kDownMaxSel) {
    // All of the chunk's expert ids first: a window address depends on its
    // id, and the loads' counter is in order, so waiting for an id issued
    // after other windows would wait for those windows too.
    // One vector load brings the chunk's ids (lane c holds id c), then
    // v_readlane makes each one uniform; the weights come the same way.
    const int cl = lane & (kDownMaxSel - 1);
    const bool cok = s0 + cl < a.n_sel;
    const int my_id = cok ? a.ids[s0 + cl] - a.id_base : -1;
    const float my_w = cok ? a.wts[s0 + cl] : 0.0f;
    int eid[kDownMaxSel];
#pragma unroll
    for (int c = 0; c < kDownMaxSel; ++c) eid[c] = __builtin_amdgcn_readlane(my_id, c);
    uint32_t win[kDownMaxSel][BPL][NW];
    uint32_t off[kDownMaxSel][BPL];
#pragma unroll
    for (int c = 0; c < kDownMaxSel; ++c) {
      const int s = s0 + c;
      if (s < a.n_sel) {
        const int e = eid[c];
        const bool eok = e >= 0 && e < a.n_experts;
        const uint8_t *wb = a.bank + static_cast<int64_t>(eok ? e : 0) * a.expert_stride;
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
          int b = j + LPR * i;
          b = b < a.nb ? b : a.nb - 1;
          off[c][i] = load_window<WT>(wb + row * a.row_bytes + static_cast<int64_t>(b) * BB, win[c][i]);
        }
      }
    }
    if (first) {
      // The first chunk's windows are in flight: stage every slot's
      // activation (codes in 16-byte pieces, scales, 8*sums) in LDS meanwhile.
      // Each thread issues up to kStage loads of each kind before it stores
      // any, so a pass costs one cache latency rather than one per item.
      constexpr int kStage = 4;
      const int64_t nq = static_cast<int64_t>(a.n_sel) * a.k / 16;
      const int64_t nsc = static_cast<int64_t>(a.n_sel) * a.nb;
      const int64_t nmax = nq > nsc ? nq : nsc;
      for (int64_t base = tid; base < nmax; base += kStage * T) {
        u32x4 cv[kStage];
        float dv[kStage];
        int32_t sv[kStage];
#pragma unroll
        for (int u = 0; u < kStage; ++u) {
          const int64_t q = base + u * T;
          if (q < nq) {
            const int64_t sl = q * 16 / a.k, in = q * 16 - sl * a.k;
            cv[u] = *reinterpret_cast<const u32x4 *>(a.qx + sl * a.x_stride + in);
          }
          if (q < nsc) {
            const int64_t sl = q / a.nb, b = q - sl * a.nb;
            dv[u] = a.dx[sl * (a.x_stride / 32) + b];
            if constexpr (WT == ZQ_Q4_0) {
              if (a.sx) {
                sv[u] = a.sx[sl * (a.x_stride / 32) + b];
              } else {
                int32_t sum = 0;
                const uint32_t *cq = reinterpret_cast<const uint32_t *>(a.qx + sl * a.x_stride + 32 * b);
#pragma unroll
                for (int k = 0; k < 8; ++k)
                  sum = __builtin_amdgcn_sdot4(static_cast<int>(cq[k]), 0x01010101, sum, false);
                sv[u] = sum;
              }
            }
          }
        }
#pragma unroll
        for (int u = 0; u < kStage; ++u) {
          const int64_t q = base + u * T;
          if (q < nq) *reinterpret_cast<u32x4 *>(lq + q * 16) = cv[u];
          if (q < nsc) {
            ld[q] = dv[u];
            if constexpr (WT == ZQ_Q4_0) ls8[q] = 8 * sv[u];
          }
        }
      }
      __syncthreads();  // the staged activations are visible
      first = false;
    }
#pragma unroll
    for (int c = 0; c < kDownMaxSel; ++c) {
      const int s = s0 + c;
      if (s < a.n_sel) {
        const int e = eid[c];
        if (e < 0 || e >= a.n_experts) {
          if (a.status) *a.status = ZQ_ERANGE;
          continue;
        }
        const float ws = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_w), c));
        float p = 0.0f;
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
          const int b = j + LPR * i;
          const bool bok = b < a.nb;
          const int bc = bok ? b : 0;
          const int8_t *cq = lq + static_cast<int64_t>(s) * a.k + 32 * bc;
          const u32x4 v0 = *reinterpret_cast<const u32x4 *>(cq);
          const u32x4 v1 = *reinterpret_cast<const u32x4 *>(cq + 16);
          const uint32_t xq[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
          const float xd = bok ? ld[static_cast<int64_t>(s) * a.nb + bc] : 0.0f;
          const float dw = window_scale(win[c][i][0], off[c][i]);
          const uint32_t sel = quant_selector(off[c][i]);
          int32_t isum;
          if constexpr (WT == ZQ_Q4_0) {
            isum = q4_raw_dot(win[c][i], sel, xq) - ls8[static_cast<int64_t>(s) * a.nb + bc];
          } else {
            isum = q8_dot(win[c][i], sel, xq);
          }
          p = __builtin_fmaf(dw * xd, static_cast<float>(isum), p);
        }
        acc = __builtin_fmaf(ws, p, acc);
      }
    }
  }
  if (first) __syncthreads();  // (n_sel == 0) keep the barrier count uniform

  using R = RowReduce<LPR, 1>;
  float v[1] = {acc};
  float res[1];
  R::run(v, res);
  if (R::writer(lane) && row_ok) {
    float *yp = a.y + row0 + slot;
    *yp = (a.flags & ZQ_ACCUMULATE) ? *yp + res[0] : res[0];
  }
}

// ------------------------------------------------------------ dispatch -----

namespace {

size_t gu_lds(const MoeGateUpArgs &a) {
  return static_cast<size_t>(a.k) + 8 * static_cast<size_t>(a.nb) + 64 * 4;
}

template <class Rows>
int launch_gu(const MoeGateUpArgs &a, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(a.d_ff / 32), static_cast<unsigned>(a.n_sel));
  if (a.logits)
    hipLaunchKernelGGL((moe_gate_up_kernel<Rows, true>), grid, dim3(1024), gu_lds(a), stream,
                       a.x, a.logits, a.ids, a.nb, a.k, a.n_routed, a.top_k, a.id_base, a);
  else
    hipLaunchKernelGGL((moe_gate_up_kernel<Rows, false>), grid, dim3(1024), gu_lds(a), stream,
                       a.x, a.logits, a.ids, a.nb, a.k, a.n_routed, a.top_k, a.id_base, a);
  ZQ_LAUNCH_CHECK();
  return ZQ_OK;
}

template <int WT>
int launch_gu_w(const MoeGateUpArgs &a, hipStream_t stream) {
  // single-pass layouts with 64 rows per 16-wave workgroup
  if (a.nb <= 16) return launch_gu<GuBlockRows<WT, 16, 1, 1>>(a, stream);
  if (a.nb <= 32) return launch_gu<GuBlockRows<WT, 32, 1, 2>>(a, stream);
  if (a.nb <= 64) return launch_gu<GuBlockRows<WT, 64, 1, 4>>(a, stream);
  return launch_gu<GuBlockRows<WT, 64, 2, 4>>(a, stream);  // nb <= 128 (moe_gate_up_fits)
}

template <int WT>
int launch_gu_k_w(const MoeGateUpArgs &a, hipStream_t stream) {
  // one 64-element unit per lane, the row in one pass (k = 64 * LPR)
  if (a.k == 1024) return launch_gu<GuKRows<WT, 16, 1>>(a, stream);
  if (a.k == 2048) return launch_gu<GuKRows<WT, 32, 2>>(a, stream);
  return launch_gu<GuKRows<WT, 64, 4>>(a, stream);  // k == 4096 (moe_gate_up_k_fits)
}

// The mixed launch: the row layouts of both formats at this d_model.
template <int WT, int NB>
using GuAnyRows = typename std::conditional<(WT == ZQ_Q4_0 || WT == ZQ_Q8_0), GuRowsFor<WT, NB>,
                                            GuKRowsFor<WT, NB>>::type::type;

template <class Rows, class SRows, int NB>
int launch_gu_mix(const MoeGateUpArgs &a, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(a.d_ff / 32), static_cast<unsigned>(a.top_k + 1));
  hipLaunchKernelGGL((moe_gate_up_mix_kernel<Rows, SRows, NB>), grid, dim3(1024), gu_lds(a), stream,
                     a.x, a.logits, a.ids, a.nb, a.k, a.n_routed, a.top_k, a.id_base, a);
  ZQ_LAUNCH_CHECK();
  return ZQ_OK;
}

template <int NB, int WT>
int gu_mix_shared(int sh_wtype, const MoeGateUpArgs &a, hipStream_t stream) {
  using R = GuAnyRows<WT, NB>;
  switch (sh_wtype) {
    case ZQ_Q4_0: return launch_gu_mix<R, GuAnyRows<ZQ_Q4_0, NB>, NB>(a, stream);
    case ZQ_Q8_0: return launch_gu_mix<R, GuAnyRows<ZQ_Q8_0, NB>, NB>(a, stream);
    case ZQ_Q4_K: return launch_gu_mix<R, GuAnyRows<ZQ_Q4_K, NB>, NB>(a, stream);
    case ZQ_Q5_K: return launch_gu_mix<R, GuAnyRows<ZQ_Q5_K, NB>, NB>(a, stream);
    case ZQ_Q6_K: return launch_gu_mix<R, GuAnyRows<ZQ_Q6_K, NB>, NB>(a, stream);
    default: return ZQ_EINVAL;
  }
}

template <int NB>
int gu_mix_routed(int wtype, int sh_wtype, const MoeGateUpArgs &a, hipStream_t stream) {
  switch (wtype) {
    case ZQ_Q4_0: return gu_mix_shared<NB, ZQ_Q4_0>(sh_wtype, a, stream);
    case ZQ_Q8_0: return gu_mix_shared<NB, ZQ_Q8_0>(sh_wtype, a, stream);
    case ZQ_Q4_K: return gu_mix_shared<NB, ZQ_Q4_K>(sh_wtype, a, stream);
    case ZQ_Q5_K: return gu_mix_shared<NB, ZQ_Q5_K>(sh_wtype, a, stream);
    case ZQ_Q6_K: return gu_mix_shared<NB, ZQ_Q6_K>(sh_wtype, a, stream);
    default: return ZQ_EINVAL;
  }
}

// Bytes of one row of k elements in wtype.
int64_t gu_row_bytes(int wtype, int64_t k) {
  switch (wtype) {
    case ZQ_Q4_0: return (k / 32) * 18;
    case ZQ_Q8_0: return (k / 32) * 34;
    case ZQ_Q4_K: return (k / 256) * KQ<ZQ_Q4_K>::BYTES;
    case ZQ_Q5_K: return (k / 256) * KQ<ZQ_Q5_K>::BYTES;
    case ZQ_Q6_K: return (k / 256) * KQ<ZQ_Q6_K>::BYTES;
    default: return -1;
  }
}

template <int WT, int LPR, int BPL>
int launch_dn(const MoeDownArgs &a, hipStream_t stream) {
  constexpr int WPB = 2;
  constexpr int S = 64 / LPR;
  const int64_t rows_per_wg = WPB * S;
  const unsigned grid = static_cast<unsigned>((a.rows + rows_per_wg - 1) / rows_per_wg);
  hipLaunchKernelGGL((moe_down_kernel<WT, LPR, BPL, WPB>), dim3(grid), dim3(64 * WPB),
                     moe_down_lds_bytes(a.n_sel, a.k), stream, a.ids, a.qx, a.dx, a.x_stride, a.rows,
                     a.n_sel, a.nb, a.id_base, a);
  ZQ_LAUNCH_CHECK();
  return ZQ_OK;
}

template <int WT, int LPS, int BPL, int RB>
int launch_dn_wsum1(const MoeDownArgs &a, hipStream_t stream) {
  const int64_t n_groups = (a.rows + RB - 1) / RB;
  const int64_t blocks = (n_groups + 3) / 4;
  const unsigned grid = static_cast<unsigned>(blocks < 1048576 ? blocks : 1048576);
  hipLaunchKernelGGL((moe_down_wsum_kernel<WT, LPS, BPL, RB>), dim3(grid), dim3(256), 0, stream,
                     a.ids, a.qx, a.dx, a.x_stride, a.rows, a.n_sel, a.nb, a.id_base, a);
  ZQ_LAUNCH_CHECK();
  return ZQ_OK;
}

// Row steps per wave: the largest of 4, 2, 1 that keeps >= 1024 waves.
template <int WT, int LPS, int BPL>
int launch_dn_wsum_rb(const MoeDownArgs &a, hipStream_t stream) {
  if ((a.rows + 3) / 4 >= 1024) return launch_dn_wsum1<WT, LPS, BPL, 4>(a, stream);
  if ((a.rows + 1) / 2 >= 1024) return launch_dn_wsum1<WT, LPS, BPL, 2>(a, stream);
  return launch_dn_wsum1<WT, LPS, BPL, 1>(a, stream);
}

// Slots in lanes while one or two rounds take every slot: 4 lanes per slot
// (16 slots a round) up to 16 blocks per row, 8 lanes (8 slots) up to 32.
bool down_wsum_fits(int nb, int n_sel) { return nb <= 16 ? n_sel <= 32 : (nb <= 32 && n_sel <= 16); }

template <int WT>
int launch_dn_wsum(const MoeDownArgs &a, hipStream_t stream) {
  if (a.nb <= 4) return launch_dn_wsum_rb<WT, 4, 1>(a, stream);
  if (a.nb <= 8) return launch_dn_wsum_rb<WT, 4, 2>(a, stream);
  if (a.nb <= 12) return launch_dn_wsum_rb<WT, 4, 3>(a, stream);
  if (a.nb <= 16) return launch_dn_wsum_rb<WT, 4, 4>(a, stream);
  if (a.nb <= 24) return launch_dn_wsum_rb<WT, 8, 3>(a, stream);
  return launch_dn_wsum_rb<WT, 8, 4>(a, stream);  // nb <= 32 (down_wsum_fits)
}

template <int WT>
int launch_dn_w(const MoeDownArgs &a, hipStream_t stream) {
  if (down_wsum_fits(a.nb, a.n_sel)) return launch_dn_wsum<WT>(a, stream);
  if (a.nb <= 8) return launch_dn<WT, 8, 1>(a, stream);
  if (a.nb <= 16) return launch_dn<WT, 16, 1>(a, stream);
  if (a.nb <= 32) return launch_dn<WT, 32, 1>(a, stream);
  if (a.nb <= 64) return launch_dn<WT, 64, 1>(a, stream);
  return launch_dn<WT, 64, 2>(a, stream);
}

}  // namespace

size_t moe_down_lds_bytes(int64_t n_sel, int64_t k) {
  return static_cast<size_t>(n_sel) * (static_cast<size_t>(k) + 8 * static_cast<size_t>(k / 32));
}

// 1024-thread workgroups leave 128 VGPRs per wave: two blocks per lane at most.
bool moe_gate_up_fits(int64_t d_model) { return d_model <= 4096; }
bool moe_down_fits(int64_t n_sel, int64_t k) {
  return k <= 4096 && moe_down_lds_bytes(n_sel, k) <= 64 * 1024;
}

int launch_moe_gate_up(int wtype, MoeGateUpArgs a, hipStream_t stream) {
  if (a.n_sel == 0 || a.d_ff == 0) return ZQ_OK;
  a.nb = static_cast<int32_t>(a.k / 32);
  a.row_bytes = static_cast<int64_t>(a.nb) * (wtype == ZQ_Q4_0 ? 18 : 34);
  return wtype == ZQ_Q4_0 ? launch_gu_w<ZQ_Q4_0>(a, stream) : launch_gu_w<ZQ_Q8_0>(a, stream);
}

bool moe_gate_up_k_fits(int64_t d_model) {
  return d_model == 1024 || d_model == 2048 || d_model == 4096;
}

int launch_moe_gate_up_k(int wtype, MoeGateUpArgs a, hipStream_t stream) {
  if (a.n_sel == 0 || a.d_ff == 0) return ZQ_OK;
  a.nb = static_cast<int32_t>(a.k / 32);
  a.row_bytes = gu_row_bytes(wtype, a.k);
  switch (wtype) {
    case ZQ_Q4_K: return launch_gu_k_w<ZQ_Q4_K>(a, stream);
    case ZQ_Q5_K: return launch_gu_k_w<ZQ_Q5_K>(a, stream);
    case ZQ_Q6_K: return launch_gu_k_w<ZQ_Q6_K>(a, stream);
    default: return ZQ_EINVAL;
  }
}

// (at d_model 4096 the two layouts together would spill registers)
bool moe_gate_up_mix_fits(int64_t d_model) { return d_model == 1024 || d_model == 2048; }

int launch_moe_gate_up_mix(int wtype, int sh_wtype, MoeGateUpArgs a, hipStream_t stream) {
  if (a.d_ff == 0) return ZQ_OK;
  a.nb = static_cast<int32_t>(a.k / 32);
  a.n_sel = a.top_k + 1;
  a.row_bytes = gu_row_bytes(wtype, a.k);
  a.row_bytes2 = gu_row_bytes(sh_wtype, a.k);
  if (a.row_bytes < 0 || a.row_bytes2 < 0 || !a.logits || !a.bank2) return ZQ_EINVAL;
  if (a.nb == 32) return gu_mix_routed<32>(wtype, sh_wtype, a, stream);
  return gu_mix_routed<64>(wtype, sh_wtype, a, stream);  // nb == 64 (moe_gate_up_mix_fits)
}

int launch_moe_down(int wtype, MoeDownArgs a, hipStream_t stream) {
  if (a.rows == 0) return ZQ_OK;
  a.nb = static_cast<int32_t>(a.k / 32);
  a.row_bytes = static_cast<int64_t>(a.nb) * (wtype == ZQ_Q4_0 ? 18 : 34);
  return wtype == ZQ_Q4_0 ? launch_dn_w<ZQ_Q4_0>(a, stream) : launch_dn_w<ZQ_Q8_0>(a, stream);
}

// ------------------------------------------------------- several tokens ---
// Up to kTokMax tokens, each with its own router logits (top_k routed
// experts and an optional shared expert), through one pass over the union of
// the experts they touch, in three launches:
//   route: a workgroup per token runs the single-token router on its logits
//     (rank selection and fp64 softmax, so ids and weights are those of
//     zq_moe_route bit for bit), and another per token quantizes its
//     activation (the codes of zq_quantize_act);
//   gate/up: a workgroup per (flattened slot j = t * n_sel + s, 32-wide block
//     of the FFN width) reads every token's expert ids; unless an earlier
//     slot holds the same expert it loads the expert's 64 gate/up rows once,
//     stages the codes of every token that selected that expert (its
//     members) in LDS, runs the 64 rows for each member, and finishes each
//     member's SwiGLU + re-quantization on a wave of its own (the
//     single-token stage's codes, bit for bit).  The workgroups of block 0
//     record every slot's members for the down pass (none for a slot whose
//     expert an earlier slot holds);
//   down: a workgroup per 8 output rows lists the first-use slots (the
//     distinct experts), requests the first ones' down rows, stages every
//     slot's hidden codes in LDS (when they fit), and its 16 waves take the
//     experts (the first 16 in order, the rest claimed from an LDS counter
//     so that a wave slowed by an expert with many members takes fewer),
//     each reading its experts' down rows once (the next one's requested
//     before the current one's members are computed) and leaving every
//     member slot's row value in LDS; then
//     y[t] (+)= sum_s wts[t][s] * rows[t * n_sel + s], the slots in order.

// Route (blockIdx.y 0) and quantize (blockIdx.y 1) token blockIdx.x.
template <int P>
__global__ __launch_bounds__(1024) void moe_tok_route_kernel(const float *logits, const float *x,
                                                             const float *shared_gate, int8_t *qx,
                                                             float *dx, int32_t n_routed,
                                                             int32_t top_k, int32_t d_model,
                                                             const MoeTokArgs a_in) {
  // leading scalars: preloaded kernel arguments (as dmmv_hot)
  MoeTokArgs a = a_in;
  a.logits = logits;
  a.x = x;
  a.shared_gate = shared_gate;
  a.qx = qx;
  a.dx = dx;
  a.n_routed = n_routed;
  a.top_k = top_k;
  a.d_model = d_model;
  const int t = static_cast<int>(blockIdx.x);
  const int tid = static_cast<int>(threadIdx.x);
  if (blockIdx.y == 1) {
    // 8 lanes per 32-element block (d_model <= 4096: one pass)
    const int nbx = a.d_model / 32;
    const int b = tid >> 3, g = tid & 7;
    if (b < nbx) {  // whole 8-lane groups
      const int64_t o = static_cast<int64_t>(t) * a.d_model + b * 32 + g * 4;
      const float4 v = *reinterpret_cast<const float4 *>(a.x + o);
      const float xv[4] = {v.x, v.y, v.z, v.w};
      float d;
      int32_t sum;
      const uint32_t packed = quantize_block8(xv, d, sum);
      *reinterpret_cast<uint32_t *>(a.qx + o) = packed;
      if (g == 0) {
        a.dx[t * nbx + b] = d;
        a.sx[t * nbx + b] = sum;
      }
    }
    return;
  }
  __shared__ __attribute__((aligned(16))) float lv[1024];
  __shared__ int32_t sel_id[64];
  __shared__ float sel_v[64];
  __shared__ double sel_e[64];
  const int n = a.n_routed;
  const int n_sel = a.top_k + (a.shared_gate ? 1 : 0);
  const int n_pad = route_stage<P, 1024>(lv, a.logits + static_cast<int64_t>(t) * n, n);
  __syncthreads();
  route_rank<P, 1024>(lv, n, n_pad, a.top_k, sel_id, sel_v);
  __syncthreads();
  route_weights(sel_id, sel_v, sel_e, n, a.top_k, a.shared_gate ? a.shared_gate + t : nullptr,
                a.ids + t * n_sel, a.wts + t * n_sel);
}

// gate/up: grid (d_ff / 32, J).  a.ids: every token's expert ids [J];
// mem: the member table [J][kTokMax] (written by the workgroups of block
// 0): the member slots of first-use slot j in token order, then -1; all -1
// for a slot that is not a first use.
template <class Rows>
__global__ __launch_bounds__(1024) void moe_gate_up_tok_kernel(const int32_t *ids, int32_t *mem,
                                                               const int8_t *qx, const float *dx,
                                                               int32_t n_sel, int32_t k_in,
                                                               int32_t nb_in, int n_tok,
                                                               int n_sel_tok,
                                                               const MoeGateUpArgs a_in,
                                                               const int32_t *sx) {
  // leading scalars: preloaded kernel arguments (as dmmv_hot)
  MoeGateUpArgs a = a_in;
  a.ids = ids;
  a.n_sel = n_sel;
  a.k = k_in;
  a.nb = nb_in;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int32_t lid[kTokMax * 65];
  __shared__ int32_t mslot[kTokMax];
  __shared__ int32_t mt[kTokMax], mj[kTokMax];   // member token and slot, compacted
  __shared__ int32_t dup, n_mem;
  const int tid = static_cast<int>(threadIdx.x);
  const int hb = static_cast<int>(blockIdx.x);
  const int j = static_cast<int>(blockIdx.y);
  const int J = a.n_sel;  // <= kTokMax * 65 < 1024
  const int k = a.k, nb = a.nb;
  if (tid < J) lid[tid] = a.ids[tid];
  if (tid < kTokMax) mslot[tid] = -1;
  if (tid == 0) dup = 0;
  __syncthreads();
  const int e = lid[j];
  // an earlier slot with the same expert makes this one a duplicate; a token
  // selects distinct experts, so each token holds e in at most one slot
  if (tid < J && lid[tid] == e) {
    if (tid < j) dup = 1;
    mslot[tid / n_sel_tok] = tid;
  }
  __syncthreads();
  const bool bad = e < 0 || e >= a.n_experts;
  if (tid < 64) {  // the members in token order; block 0 records them for the down pass
    const int v = tid < kTokMax && !dup && !bad ? mslot[tid] : -1;
    const uint64_t m = __ballot(v >= 0);
    const int cnt = __popcll(m);
    if (v >= 0) {
      const int pos = __popcll(m & ((uint64_t(1) << tid) - 1));
      mt[pos] = tid;
      mj[pos] = v;
      if (hb == 0) mem[kTokMax * j + pos] = v;
    }
    if (hb == 0 && tid >= cnt && tid < kTokMax) mem[kTokMax * j + tid] = -1;
    if (tid == 0) n_mem = cnt;
  }
  if (dup) return;  // uniform over the workgroup
  if (bad) {
    if (a.status && tid == 0) *a.status = ZQ_ERANGE;
    return;
  }
  Rows r;
  r.load(a, nb, a.bank + static_cast<int64_t>(e) * a.expert_stride, a.row_bytes, hb, tid);
  __syncthreads();
  const int c = n_mem;
  // LDS: member codes [c][k], scales [c][nb], SUMX * sums [c][nb], rows [c][64]
  int8_t *lq = reinterpret_cast<int8_t *>(smem);
  float *ld = reinterpret_cast<float *>(smem + c * k);
  int32_t *ls = reinterpret_cast<int32_t *>(smem + c * k + 4 * c * nb);
  float *lrow = reinterpret_cast<float *>(smem + c * k + 8 * c * nb);
  const int cpm = k / 16;  // 16-byte pieces of codes per member
  for (int idx = tid; idx < c * cpm; idx += 1024) {
    const int m = idx / cpm, p = idx - m * cpm;
    reinterpret_cast<u32x4 *>(lq)[idx] =
        *reinterpret_cast<const u32x4 *>(qx + static_cast<int64_t>(mt[m]) * k + 16 * p);
  }
  for (int idx = tid; idx < c * nb; idx += 1024) {
    const int m = idx / nb, b = idx - m * nb;
    ld[idx] = dx[mt[m] * nb + b];
    ls[idx] = Rows::SUMX * sx[mt[m] * nb + b];
  }
  __syncthreads();
  for (int m = 0; m < c; ++m) r.rows(nb, lq + m * k, ld + m * nb, ls + m * nb, lrow + 64 * m, tid);
  __syncthreads();
  const int wave = tid >> 6;
  if (wave < c) gu_epilogue<false>(a, tid - 64 * wave, mj[wave], hb, lrow + 64 * wave, nullptr,
                                   nullptr);
}

// The LDS of a down workgroup (byte offsets), with the hidden codes staged
// when STAGE.
struct DnTokLds {
  int part, mem, ent, lid, wts, q, d, s, total;
  __host__ __device__ DnTokLds(int J, int k, int rows, bool stage) {
    const int nb = k / 32;
    part = 0;
    mem = part + 4 * J * rows;
    ent = mem + 4 * kTokMax * J;
    lid = ent + 4 * J;
    wts = lid + 4 * J;
    q = (wts + 4 * J + 15) / 16 * 16;
    d = q + (stage ? J * k : 0);
    s = d + (stage ? 4 * J * nb : 0);
    total = s + (stage ? 4 * J * nb : 0);
  }
};

constexpr int kDnTokLdsMax = 60 * 1024;

// down: LPR = k / 32 lanes per row (one block each), RB row steps of 64 /
// LPR rows: 8 rows per workgroup of 16 waves.  grid (rows / 8).
template <int WT, int LPR, int RB, bool STAGE>
__global__ __launch_bounds__(1024) void moe_down_tok_kernel(int32_t *mem_in, const int32_t *ids,
                                                            const float *wts, int64_t rows,
                                                            int32_t n_sel, int32_t k_in,
                                                            int32_t nb_in,
                                                            const MoeDownTokArgs a_in) {
  // leading scalars: preloaded kernel arguments (as dmmv_hot)
  MoeDownTokArgs a = a_in;
  a.mem = mem_in;
  a.ids = ids;
  a.wts = wts;
  a.rows = rows;
  a.n_sel = n_sel;
  a.k = k_in;
  a.nb = nb_in;
  constexpr int S = 64 / LPR;
  constexpr int ROWS = RB * S;
  constexpr int NW = Blk<WT>::NW;
  constexpr int BB = Blk<WT>::BYTES;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int32_t n_ent, dctr;
  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & 63, wv = tid >> 6;
  const int jl = lane & (LPR - 1), slot = lane / LPR;
  const int J = a.n_sel, k = a.k, nb = a.nb;
  const DnTokLds L(J, k, ROWS, STAGE);
  float *part = reinterpret_cast<float *>(smem + L.part);
  int32_t *mem = reinterpret_cast<int32_t *>(smem + L.mem);
  int32_t *ent = reinterpret_cast<int32_t *>(smem + L.ent);
  int32_t *lid = reinterpret_cast<int32_t *>(smem + L.lid);
  float *lw = reinterpret_cast<float *>(smem + L.wts);
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * ROWS;
  for (int i = tid; i < kTokMax * J; i += 1024) mem[i] = a.mem[i];
  for (int i = tid; i < J; i += 1024) {
    lid[i] = a.ids[i];
    lw[i] = a.wts[i];
  }
  for (int i = tid; i < J * ROWS; i += 1024) part[i] = 0.0f;
  if (tid == 0) dctr = 0;
  __syncthreads();
  // the first-use slots in order: the slots whose member row is not empty
  if (tid < 64) {
    int before = 0;
    for (int j0 = 0; j0 < J; j0 += 64) {
      const int j = j0 + tid;
      const bool f = j < J && mem[kTokMax * j] >= 0;
      const uint64_t m = __ballot(f);
      if (f) ent[before + __popcll(m & ((uint64_t(1) << tid) - 1))] = j;
      before += __popcll(m);
    }
    if (tid == 0) n_ent = before;
  }
  __syncthreads();
  const int ne = n_ent;

  constexpr int NBUF = RB > 4 ? 1 : 2;
  uint32_t win[NBUF][RB][NW];
  uint32_t off[NBUF][RB];
  auto load = [&](int u, int buf) {
    u = u < ne ? u : ne - 1;  // past the last entry: the last one again
    int e = lid[ent[u]];
    e = e < 0 ? 0 : (e >= a.n_experts ? a.n_experts - 1 : e);  // reported below
    const uint8_t *wb = a.bank + static_cast<int64_t>(e) * a.expert_stride;
#pragma unroll
    for (int t2 = 0; t2 < RB; ++t2) {
      int64_t row = row0 + t2 * S + slot;
      row = row < a.rows ? row : a.rows - 1;
      off[buf][t2] = load_window<WT>(wb + row * a.row_bytes + static_cast<int64_t>(jl) * BB,
                                     win[buf][t2]);
    }
  };
  auto run = [&](int u, int buf) {
    const int j = ent[u];
    const int e = lid[j];
    if (e < 0 || e >= a.n_experts) {  // uniform
      if (a.status && lane == 0) *a.status = ZQ_ERANGE;
      return;
    }
    for (int m = 0; m < kTokMax; ++m) {
      const int js = mem[kTokMax * j + m];
      if (js < 0) break;  // uniform
      const int hb = js * nb + jl;
      u32x4 v0, v1;
      float hd;
      int32_t hsum;
      if constexpr (STAGE) {
        v0 = *reinterpret_cast<const u32x4 *>(smem + L.q + 32 * hb);
        v1 = *reinterpret_cast<const u32x4 *>(smem + L.q + 32 * hb + 16);
        hd = reinterpret_cast<const float *>(smem + L.d)[hb];
        hsum = reinterpret_cast<const int32_t *>(smem + L.s)[hb];
      } else {
        v0 = *reinterpret_cast<const u32x4 *>(a.qh + 32 * static_cast<int64_t>(hb));
        v1 = *reinterpret_cast<const u32x4 *>(a.qh + 32 * static_cast<int64_t>(hb) + 16);
        hd = a.dh[hb];
        hsum = a.sh[hb];
      }
      const uint32_t xq[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      const int32_t hs8 = WT == ZQ_Q4_0 ? 8 * hsum : 0;
      float p[RB];
#pragma unroll
      for (int t2 = 0; t2 < RB; ++t2) {
        const float dw = window_scale(win[buf][t2][0], off[buf][t2]);
        const uint32_t sel = quant_selector(off[buf][t2]);
        int32_t isum;
        if constexpr (WT == ZQ_Q4_0) {
          isum = q4_raw_dot(win[buf][t2], sel, xq) - hs8;
        } else {
          isum = q8_dot(win[buf][t2], sel, xq);
        }
        p[t2] = dw * hd * static_cast<float>(isum);
      }
      using R = RowReduce<LPR, RB>;
      float res[R::NOUT];
      R::run(p, res);
      if (R::writer(lane)) {
#pragma unroll
        for (int m = 0; m < R::NOUT; ++m) part[js * ROWS + R::rowstep(m, lane) * S + slot] = res[m];
      }
    }
  };
  // the first entries' rows are requested before the hidden codes are
  // staged (with two window sets)
  // entries past a wave's first are claimed from an LDS counter, so that a
  // wave slowed by an expert with many members takes fewer entries
  auto claim = [&]() {
    int c = 0;
    if (lane == 0) c = atomicAdd(&dctr, 1);
    return 16 + __shfl(c, 0);
  };
  int u = wv, un = 0;
  if constexpr (NBUF == 2) {
    if (wv < ne) {
      un = claim();
      load(u, 0);
      load(un, 1);
    }
  }
  if constexpr (STAGE) {
    const int pieces = J * k / 16;
    for (int i = tid; i < pieces; i += 1024)
      reinterpret_cast<u32x4 *>(smem + L.q)[i] = reinterpret_cast<const u32x4 *>(a.qh)[i];
    for (int i = tid; i < J * nb; i += 1024) {
      reinterpret_cast<float *>(smem + L.d)[i] = a.dh[i];
      reinterpret_cast<int32_t *>(smem + L.s)[i] = a.sh[i];
    }
    __syncthreads();
  }
  // two window sets (up to 4 row steps): entry u + 16 is requested before
  // entry u is computed; 8 row steps keep one set, within the registers
  if constexpr (RB > 4) {
    while (u < ne) {
      load(u, 0);
      run(u, 0);
      u = claim();
    }
  } else if (wv < ne) {
    // buffer 0 holds entry u, buffer 1 entry un
    for (;;) {
      run(u, 0);
      if (un >= ne) break;
      u = claim();
      load(u, 0);
      run(un, 1);
      if (u >= ne) break;
      un = claim();
      load(un, 1);
    }
  }
  __syncthreads();
  const int ns = a.n_sel_tok;
  for (int idx = tid; idx < a.n_tok * ROWS; idx += 1024) {
    const int t = idx / ROWS, rr = idx - t * ROWS;
    const int64_t row = row0 + rr;
    if (row >= a.rows) continue;
    float acc = 0.0f;
    for (int s = 0; s < ns; ++s) acc = __builtin_fmaf(lw[t * ns + s], part[(t * ns + s) * ROWS + rr], acc);
    float *yp = a.y + static_cast<int64_t>(t) * a.rows + row;
    *yp = (a.flags & ZQ_ACCUMULATE) ? *yp + acc : acc;
  }
}

namespace {

template <int P>
void launch_tok_route(const MoeTokArgs &p, hipStream_t stream) {
  hipLaunchKernelGGL((moe_tok_route_kernel<P>), dim3(static_cast<unsigned>(p.n_tok), 2),
                     dim3(1024), 0, stream, p.logits, p.x, p.shared_gate, p.qx, p.dx, p.n_routed,
                     p.top_k, p.d_model, p);
}

template <class Rows>
int launch_gu_tok(const MoeGateUpArgs &a, int32_t *mem, const MoeTokArgs &p, int n_sel_tok,
                  hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(a.d_ff / 32), static_cast<unsigned>(a.n_sel));
  const int c = p.n_tok;  // at most this many members per expert
  const size_t lds = static_cast<size_t>(c) * (a.k + 8 * a.nb + 64 * 4);
  hipLaunchKernelGGL((moe_gate_up_tok_kernel<Rows>), grid, dim3(1024), lds, stream, a.ids, mem,
                     p.qx, p.dx, a.n_sel, a.k, a.nb, p.n_tok, n_sel_tok, a, p.sx);
  ZQ_LAUNCH_CHECK();
  return ZQ_OK;
}

template <int WT>
int launch_gu_tok_w(const MoeGateUpArgs &a, int32_t *mem, const MoeTokArgs &p, int n_sel_tok,
                    hipStream_t stream) {
  if (a.nb <= 16) return launch_gu_tok<GuBlockRows<WT, 16, 1, 1>>(a, mem, p, n_sel_tok, stream);
  if (a.nb <= 32) return launch_gu_tok<GuBlockRows<WT, 32, 1, 2>>(a, mem, p, n_sel_tok, stream);
  if (a.nb <= 64) return launch_gu_tok<GuBlockRows<WT, 64, 1, 4>>(a, mem, p, n_sel_tok, stream);
  return launch_gu_tok<GuBlockRows<WT, 64, 2, 4>>(a, mem, p, n_sel_tok, stream);
}

template <int WT, int LPR, int RB>
int launch_dn_tok(const MoeDownTokArgs &a, hipStream_t stream) {
  constexpr int ROWS = RB * (64 / LPR);
  const dim3 grid(static_cast<unsigned>((a.rows + ROWS - 1) / ROWS));
  const DnTokLds staged(a.n_sel, a.k, ROWS, true);
  if (staged.total <= kDnTokLdsMax) {
    hipLaunchKernelGGL((moe_down_tok_kernel<WT, LPR, RB, true>), grid, dim3(1024),
                       static_cast<size_t>(staged.total), stream, a.mem, a.ids, a.wts, a.rows,
                       a.n_sel, a.k, a.nb, a);
  } else {
    const DnTokLds plain(a.n_sel, a.k, ROWS, false);
    hipLaunchKernelGGL((moe_down_tok_kernel<WT, LPR, RB, false>), grid, dim3(1024),
                       static_cast<size_t>(plain.total), stream, a.mem, a.ids, a.wts, a.rows,
                       a.n_sel, a.k, a.nb, a);
  }
  ZQ_LAUNCH_CHECK();
  return ZQ_OK;
}

// d_ff of 256 (8 lanes per row), 512 (16), 1024 (32) or 2048 (64 lanes): 8
// rows per workgroup
template <int WT>
int launch_dn_tok_w(const MoeDownTokArgs &a, hipStream_t stream) {
  if (a.nb == 8) return launch_dn_tok<WT, 8, 1>(a, stream);
  if (a.nb == 16) return launch_dn_tok<WT, 16, 2>(a, stream);
  if (a.nb == 32) return launch_dn_tok<WT, 32, 4>(a, stream);
  return launch_dn_tok<WT, 64, 8>(a, stream);
}

}  // namespace

bool moe_tok_fits(int64_t d_model, int64_t d_ff) {
  return moe_gate_up_fits(d_model) && (d_ff == 256 || d_ff == 512 || d_ff == 1024 || d_ff == 2048);
}

int launch_moe_ffn_tok(int wtype, const MoeTokArgs &p, MoeGateUpArgs g, MoeDownTokArgs d,
                       hipStream_t stream) {
  // P threads per logit while n_routed * P fits the 1024 threads (P <= 16),
  // as the single-token router
  int pp = 1;
  while (pp < 16 && p.n_routed * (pp * 2) <= 1024) pp *= 2;
  switch (pp) {
    case 16: launch_tok_route<16>(p, stream); break;
    case 8: launch_tok_route<8>(p, stream); break;
    case 4: launch_tok_route<4>(p, stream); break;
    case 2: launch_tok_route<2>(p, stream); break;
    default: launch_tok_route<1>(p, stream); break;
  }
  ZQ_LAUNCH_CHECK();
  const int n_sel_tok = d.n_sel_tok;
  g.ids = p.ids;
  g.nb = static_cast<int32_t>(g.k / 32);
  g.row_bytes = static_cast<int64_t>(g.nb) * (wtype == ZQ_Q4_0 ? 18 : 34);
  int rc = wtype == ZQ_Q4_0 ? launch_gu_tok_w<ZQ_Q4_0>(g, d.mem, p, n_sel_tok, stream)
                            : launch_gu_tok_w<ZQ_Q8_0>(g, d.mem, p, n_sel_tok, stream);
  if (rc != ZQ_OK) return rc;
  d.ids = p.ids;
  d.nb = static_cast<int32_t>(d.k / 32);
  d.row_bytes = static_cast<int64_t>(d.nb) * (wtype == ZQ_Q4_0 ? 18 : 34);
  return wtype == ZQ_Q4_0 ? launch_dn_tok_w<ZQ_Q4_0>(d, stream) : launch_dn_tok_w<ZQ_Q8_0>(d, stream);
}

}  // namespace zq
