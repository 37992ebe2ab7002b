// zq_common.h -- device helpers shared by the libzq HIP kernels (gfx950 only).
//
// Wave64 throughout.  Nothing here is shared with the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/zq.h"

namespace zq {

// ------------------------------------------------------------ block types --

template <int WT> struct Blk;
// Q4_0: fp16 d + 16 bytes of nibbles = 18 bytes.  A 4-byte-aligned window of
// 5 dwords starting at (block address rounded down to 4) covers the block.
template <> struct Blk<ZQ_Q4_0> { static constexpr int BYTES = 18; static constexpr int NW = 5; };
// Q8_0: fp16 d + 32 int8 = 34 bytes; a 9-dword window covers it.
template <> struct Blk<ZQ_Q8_0> { static constexpr int BYTES = 34; static constexpr int NW = 9; };

typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// Global-address-space views: loads through these are global_load (vmcnt
// only).  A generic pointer would become flat_load, which also counts in
// lgkmcnt and makes the compiler wait for every load before touching LDS.
typedef __attribute__((address_space(1))) const uint32_t g_u32;
typedef __attribute__((address_space(1))) const u32x4a4 g_u32x4a4;

// Load the NW-dword window holding the block at byte address p (p is 2-byte
// aligned; the window starts at p rounded down to 4).  Returns the byte
// offset o in {0, 2} of the block inside the window.
template <int WT>
__device__ __forceinline__ uint32_t load_window(const uint8_t *p, uint32_t (&w)[Blk<WT>::NW]) {
  const uint32_t o = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p) & 3u);
  const g_u32 *pw = (const g_u32 *)(p - o);
  const u32x4a4 v0 = *(const g_u32x4a4 *)pw;
  w[0] = v0.x; w[1] = v0.y; w[2] = v0.z; w[3] = v0.w;
  if constexpr (WT == ZQ_Q4_0) {
    w[4] = pw[4];
  } else {
    const u32x4a4 v1 = *(const g_u32x4a4 *)(pw + 4);
    w[4] = v1.x; w[5] = v1.y; w[6] = v1.z; w[7] = v1.w;
    w[8] = pw[8];
  }
  return o;
}

// fp16 bits (low 16 bits of h) -> fp32, exact for every finite value
// including subnormals.
__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

// The block's fp16 scale, at byte o of the window.
__device__ __forceinline__ float window_scale(uint32_t w0, uint32_t o) {
  return f16_to_f32(__builtin_amdgcn_ubfe(w0, o * 8u, 16u));
}

// Byte selector that extracts window bytes [o+2, o+6) from the dword pair
// (w[k+1]:w[k]) with v_perm_b32.
__device__ __forceinline__ uint32_t quant_selector(uint32_t o) {
  return 0x05040302u + o * 0x01010101u;
}

// sum_i nib_i * xq_i over one Q4_0 block (nibbles 0..15 taken as they are):
// the caller subtracts 8 * sum(xq) to get sum (nib-8)*xq.  xq[0..3] hold
// activation elements 0..15, xq[4..7] elements 16..31 (4 int8 per dword).
__device__ __forceinline__ int32_t q4_raw_dot(const uint32_t (&w)[5], uint32_t sel,
                                              const uint32_t (&xq)[8]) {
  int32_t s = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t q = __builtin_amdgcn_perm(w[k + 1], w[k], sel);
    const uint32_t lo = q & 0x0F0F0F0Fu;
    const uint32_t hi = (q >> 4) & 0x0F0F0F0Fu;
    s = __builtin_amdgcn_sdot4(static_cast<int>(lo), static_cast<int>(xq[k]), s, false);
    s = __builtin_amdgcn_sdot4(static_cast<int>(hi), static_cast<int>(xq[4 + k]), s, false);
  }
  return s;
}

// sum_i q_i * xq_i over one Q8_0 block.
__device__ __forceinline__ int32_t q8_dot(const uint32_t (&w)[9], uint32_t sel,
                                          const uint32_t (&xq)[8]) {
  int32_t s = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t q = __builtin_amdgcn_perm(w[k + 1], w[k], sel);
    s = __builtin_amdgcn_sdot4(static_cast<int>(q), static_cast<int>(xq[k]), s, false);
  }
  return s;
}

// ----------------------------------------------------------- reductions ---

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// DPP controls (gfx9 encoding).
constexpr int DPP_QUAD_XOR1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

// Sum over each aligned group of G lanes (G in {1,2,4,8,16}); every lane of
// the group receives the total.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 2) v += dpp<DPP_QUAD_XOR1>(v);
  if constexpr (G >= 4) v += dpp<DPP_QUAD_XOR2>(v);
  if constexpr (G >= 8) v += dpp<DPP_ROW_HALF_MIRROR>(v);
  if constexpr (G >= 16) v += dpp<DPP_ROW_MIRROR>(v);
  return v;
}

// v_permlane32_swap / v_permlane16_swap: exchange the odd 32-lane (16-lane)
// rows of a with the even rows of b.
__device__ __forceinline__ void swap32(float &a, float &b) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, a),
                                            __builtin_bit_cast(uint32_t, b), false, false);
  a = __builtin_bit_cast(float, static_cast<uint32_t>(r[0]));
  b = __builtin_bit_cast(float, static_cast<uint32_t>(r[1]));
}
__device__ __forceinline__ void swap16(float &a, float &b) {
  auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, a),
                                            __builtin_bit_cast(uint32_t, b), false, false);
  a = __builtin_bit_cast(float, static_cast<uint32_t>(r[0]));
  b = __builtin_bit_cast(float, static_cast<uint32_t>(r[1]));
}

// Row reduction of a wave holding RB partial sums per lane, where each row
// slot is LPR consecutive lanes (LPR in {8,16,32,64}).  Halving steps with
// the permlane swaps fold pairs of partials while summing across 32- and
// 16-lane halves; the rest is a DPP sum inside 16 (or 8) lanes.
// On return, out[m] (m < RB >> halvings()) holds in every lane of its
// sub-group the full sum of row-step rowstep(m, lane).
template <int LPR, int RB>
struct RowReduce {
  static constexpr bool H32 = (LPR == 64) && (RB >= 2);
  static constexpr bool H16 = (LPR >= 32) && ((H32 ? RB / 2 : RB) >= 2);
  static constexpr int NH = (H32 ? 1 : 0) + (H16 ? 1 : 0);
  static constexpr int NOUT = RB >> NH;
  static constexpr int G = LPR < 16 ? LPR : 16;

  __device__ __forceinline__ static void run(float (&v)[RB], float (&out)[NOUT]) {
    constexpr int N1 = H32 ? RB / 2 : RB;
    float u[N1];
    if constexpr (H32) {
#pragma unroll
      for (int m = 0; m < N1; ++m) {
        float a = v[2 * m], b = v[2 * m + 1];
        swap32(a, b);
        u[m] = a + b;
      }
    } else {
#pragma unroll
      for (int m = 0; m < N1; ++m) u[m] = v[m];
    }
    if constexpr (H16) {
#pragma unroll
      for (int m = 0; m < NOUT; ++m) {
        float a = u[2 * m], b = u[2 * m + 1];
        swap16(a, b);
        out[m] = a + b;
      }
    } else {
#pragma unroll
      for (int m = 0; m < NOUT; ++m) out[m] = u[m];
    }
#pragma unroll
    for (int m = 0; m < NOUT; ++m) {
      float t = group_sum<G>(out[m]);
      if constexpr (LPR >= 32 && !H16) {
        float a = t, b = t;
        swap16(a, b);
        t = a + b;
      }
      if constexpr (LPR == 64 && !H32) {
        float a = t, b = t;
        swap32(a, b);
        t = a + b;
      }
      out[m] = t;
    }
  }
  // Row step of output m held by `lane`.
  __device__ __forceinline__ static int rowstep(int m, int lane) {
    const int A = (lane >> 5) & 1;
    const int B = (lane >> 4) & 1;
    int t = m << NH;
    if constexpr (H16) t |= B << (H32 ? 1 : 0);
    if constexpr (H32) t |= A;
    return t;
  }
  // Exactly one lane per (output, row slot) writes it: the outputs repeat
  // with a period of LPR >> NH lanes inside a slot.
  __device__ __forceinline__ static bool writer(int lane) {
    return (lane & ((LPR >> NH) - 1)) == 0;
  }
};

// --------------------------------------------------------- quantization ---

// Round half away from zero, for |v| < 2^23.  v must already be a rounded
// fp32 value: the callers keep FMA contraction off so that v - trunc(v) is
// not fused with the multiply that produced v.
__device__ __forceinline__ float round_half_away(float v) {
#pragma clang fp contract(off)
  const float t = __builtin_truncf(v);
  const float f = v - t;  // exact
  return (__builtin_fabsf(f) >= 0.5f) ? t + __builtin_copysignf(1.0f, v) : t;
}

// Quantize one 32-element block held by G consecutive lanes (G in {2,4,8}),
// lane g of the group holding elements g*E .. g*E+E-1 with E = 32/G.  The
// codes come back packed little-endian, four per dword; d and s (the block
// scale and code sum) are valid in every lane of the group.  The result does
// not depend on G: max is exact, the scale is one IEEE division, and every
// element is rounded on its own.
template <int G>
__device__ __forceinline__ void quantize_block(const float (&x)[32 / G], uint32_t (&packed)[8 / G],
                                               float &d_out, int32_t &s_out) {
  // Every step below is one IEEE fp32 operation, rounded on its own: x*id
  // must be rounded before its fractional part decides the code.
#pragma clang fp contract(off)
  constexpr int E = 32 / G;
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < E; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[i]));
  if constexpr (G >= 2) amax = __builtin_fmaxf(amax, dpp<DPP_QUAD_XOR1>(amax));
  if constexpr (G >= 4) amax = __builtin_fmaxf(amax, dpp<DPP_QUAD_XOR2>(amax));
  if constexpr (G >= 8) amax = __builtin_fmaxf(amax, dpp<DPP_ROW_HALF_MIRROR>(amax));
  const float d = amax / 127.0f;              // IEEE division (no fast-math)
  const float id = (d != 0.0f) ? 1.0f / d : 0.0f;
  int32_t s = 0;
#pragma unroll
  for (int w = 0; w < E / 4; ++w) {
    uint32_t p = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int q = static_cast<int>(round_half_away(x[4 * w + i] * id));
      q = q > 127 ? 127 : (q < -127 ? -127 : q);
      s += q;
      p |= (static_cast<uint32_t>(q) & 0xFFu) << (8 * i);
    }
    packed[w] = p;
  }
  float sf = static_cast<float>(s);  // |s| <= 32*127: exact in fp32
  if constexpr (G >= 2) sf += dpp<DPP_QUAD_XOR1>(sf);
  if constexpr (G >= 4) sf += dpp<DPP_QUAD_XOR2>(sf);
  if constexpr (G >= 8) sf += dpp<DPP_ROW_HALF_MIRROR>(sf);
  d_out = d;
  s_out = static_cast<int32_t>(sf);
}

// The 8-lane form (four elements per lane) used by the standalone kernels.
__device__ __forceinline__ uint32_t quantize_block8(const float (&x)[4], float &d_out,
                                                   int32_t &s_out) {
  uint32_t packed[1];
  quantize_block<8>(x, packed, d_out, s_out);
  return packed[0];
}


// ------------------------------------------------------------- rms norm --
// 1 / sqrt(ss / k + eps), the RMS normalization factor: the mean is one IEEE
// division, and the root and the reciprocal are correctly rounded (no
// fast-math), each step rounded on its own.
__device__ __forceinline__ float rms_inv(float ss, int k, float eps) {
#pragma clang fp contract(off)
  const float ms = ss / static_cast<float>(k) + eps;
  return 1.0f / __builtin_sqrtf(ms);
}

// Sum of v over a workgroup of NWAVES waves, returned to every thread.
// Every thread must call it (it synchronizes twice).
template <int NWAVES>
__device__ __forceinline__ float block_sum_all(float v) {
  __shared__ float part[NWAVES];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  const int w = static_cast<int>(threadIdx.x >> 6);
  if ((threadIdx.x & 63) == 0) part[w] = v;
  __syncthreads();
  float t = 0.0f;
#pragma unroll
  for (int i = 0; i < NWAVES; ++i) t += part[i];
  __syncthreads();
  return t;
}

// ---------------------------------------------------------------- argmax --
// A (value, index) pair; a beats b when its value is larger, or equal at a
// lower index (ties go to the lowest index).
struct ValIdx {
  float v;
  int32_t i;
};

__device__ __forceinline__ bool beats(float av, int32_t ai, float bv, int32_t bi) {
  return av > bv || (av == bv && ai < bi);
}

template <int CTRL>
__device__ __forceinline__ int32_t dpp_i(int32_t v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ void take_best(float &v, int32_t &i, float ov, int32_t oi) {
  if (beats(ov, oi, v, i)) {
    v = ov;
    i = oi;
  }
}

// The best pair of the wave, in every lane: DPP moves inside 16-lane rows,
// then the permlane swaps across rows (a few cycles each; lane shuffles
// would cost a round trip through LDS per step).  "beats" is a total order
// on the pairs (ties go to the lower index), so the order of the steps does
// not change the result.
__device__ __forceinline__ void wave_best(float &v, int32_t &i) {
  take_best(v, i, dpp<DPP_QUAD_XOR1>(v), dpp_i<DPP_QUAD_XOR1>(i));
  take_best(v, i, dpp<DPP_QUAD_XOR2>(v), dpp_i<DPP_QUAD_XOR2>(i));
  take_best(v, i, dpp<DPP_ROW_HALF_MIRROR>(v), dpp_i<DPP_ROW_HALF_MIRROR>(i));
  take_best(v, i, dpp<DPP_ROW_MIRROR>(v), dpp_i<DPP_ROW_MIRROR>(i));
  // rows 0/1 and 2/3: each lane sees both rows of its 32-lane half
  {
    float a = v, b = v;
    swap16(a, b);
    float ai = __builtin_bit_cast(float, i), bi = ai;
    swap16(ai, bi);
    take_best(v, i, a, __builtin_bit_cast(int32_t, ai));
    take_best(v, i, b, __builtin_bit_cast(int32_t, bi));
  }
  // the two halves
  {
    float a = v, b = v;
    swap32(a, b);
    float ai = __builtin_bit_cast(float, i), bi = ai;
    swap32(ai, bi);
    take_best(v, i, a, __builtin_bit_cast(int32_t, ai));
    take_best(v, i, b, __builtin_bit_cast(int32_t, bi));
  }
}

// Best pair of a workgroup of NWAVES waves, valid in thread 0.  Every thread
// of the workgroup must call it.
template <int NWAVES>
__device__ __forceinline__ void block_best(float &v, int32_t &i) {
  __shared__ float sv[NWAVES];
  __shared__ int32_t si[NWAVES];
  wave_best(v, i);
  const int w = static_cast<int>(threadIdx.x >> 6);
  if ((threadIdx.x & 63) == 0) {
    sv[w] = v;
    si[w] = i;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < NWAVES; ++k)
      if (beats(sv[k], si[k], v, i)) {
        v = sv[k];
        i = si[k];
      }
  }
}


// ---------------------------------------------------------------- router --
// A logit as staged for ranking: NaN becomes -inf, so that "beats" is a total
// order on the staged values and every rank 0..n-1 is taken exactly once (a
// NaN logit could otherwise leave a rank, and with it an expert slot, empty).
__device__ __forceinline__ float route_key(float v) { return v != v ? -__builtin_inff() : v; }

// The logits staged for ranking: lv[i] = route_key(logits[i]) for i < n,
// -inf for n <= i < n_pad, n_pad = n rounded up to 16 * P (lv holds at
// least that many).  Every one of the NT threads of the workgroup calls it
// (NT a compile-time constant: reading the workgroup size would cost a
// memory round trip before the first logit load); the caller synchronizes
// before ranking.  Returns n_pad.
template <int P, int NT>
__device__ __forceinline__ int route_stage(float *lv, const float *logits, int n) {
  const int n_pad = (n + 16 * P - 1) / (16 * P) * (16 * P);
  for (int i = static_cast<int>(threadIdx.x); i < n_pad; i += NT)
    lv[i] = i < n ? route_key(logits[i]) : -__builtin_inff();
  return n_pad;
}

// Rank selection over n logits staged by route_stage (lv, 16-byte aligned,
// n_pad entries) by the whole workgroup, P threads per logit: a logit's
// rank is the number of logits that beat it (larger, or equal at a lower
// id), and the logits of rank < top_k are stored at their rank (sel_id,
// sel_v), largest first with ties to the lower id.  The -inf padding
// beats nothing: it is not larger than any staged value, and an equal one
// has a higher id.  Each of the P threads scans a contiguous n_pad / P
// run, 16 values per step from four 16-byte LDS reads.  Counts are small
// integers, exact in fp32.  Every one of the NT threads of the workgroup
// must call it; the caller synchronizes before reading sel_*.
template <int P, int NT>
__device__ __forceinline__ void route_rank(const float *lv, int n, int n_pad, int top_k,
                                           int32_t *sel_id, float *sel_v) {
  const int t = static_cast<int>(threadIdx.x);
  constexpr int n_groups = NT / P;
  const int part = t & (P - 1);
  const int chunk = n_pad / P;  // a multiple of 16
  for (int e0 = 0; e0 < n; e0 += n_groups) {  // uniform trip count
    const int e = e0 + t / P;
    const bool ok = e < n;
    const float v = ok ? lv[e] : 0.0f;
    int cnt = 0;
    if (ok) {
      const int j0 = part * chunk;
      for (int c = 0; c < chunk; c += 16) {
        float u[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 f = *reinterpret_cast<const float4 *>(lv + j0 + c + 4 * q);
          u[4 * q] = f.x; u[4 * q + 1] = f.y; u[4 * q + 2] = f.z; u[4 * q + 3] = f.w;
        }
        // four compares at a time: each leaves a lane mask in scalar
        // registers, and sixteen in flight would exhaust them
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int m = 4 * g; m < 4 * g + 4; ++m) {
            const int j = j0 + c + m;
            cnt += (u[m] > v || (u[m] == v && j < e)) ? 1 : 0;
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const float total = group_sum<P>(static_cast<float>(cnt));
    if (ok && part == 0) {
      const int rank = static_cast<int>(total);
      if (rank < top_k) {
        sel_id[rank] = e;
        sel_v[rank] = v;
      }
    }
  }
}

// Expert list and weights from the ranked selection: ids[r] = sel_id[r] and
// wts = softmax over the selected logits, each exponential evaluated in fp64
// by its own thread and the normalizer summed in rank order; with a shared
// gate, the shared expert (id n) follows with weight sigmoid(g) in fp64.
// sel_e: LDS scratch of top_k doubles.  Every thread of the workgroup must
// call it (it synchronizes).
__device__ __forceinline__ void route_weights(const int32_t *sel_id, const float *sel_v,
                                              double *sel_e, int n, int top_k,
                                              const float *shared_gate, int32_t *ids,
                                              float *wts) {
  const int t = static_cast<int>(threadIdx.x);
  if (t < top_k) sel_e[t] = exp(static_cast<double>(sel_v[t]) - static_cast<double>(sel_v[0]));
  __syncthreads();
  if (t < top_k) {
    double z = 0.0;
    for (int r = 0; r < top_k; ++r) z += sel_e[r];
    ids[t] = sel_id[t];
    wts[t] = static_cast<float>(sel_e[t] / z);
  }
  if (t == top_k && shared_gate) {
    ids[top_k] = n;
    wts[top_k] = static_cast<float>(1.0 / (1.0 + exp(-static_cast<double>(*shared_gate))));
  }
}

}  // namespace zq

// Host-side launch helpers.
#define ZQ_LAUNCH_CHECK()                                   \
  do {                                                      \
    if (hipGetLastError() != hipSuccess) return ZQ_ELAUNCH; \
  } while (0)
