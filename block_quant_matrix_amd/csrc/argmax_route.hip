// argmax_route.hip -- LM-head argmax and the MoE softmax_topk router (gfx950).
#include "zq_common.h"
#include "zq_internal.h"

namespace zq {

namespace {

constexpr int kArgmaxThreads = 256;
constexpr int kArgmaxMaxBlocks = 1024;

struct ValIdx {
  float v;
  int32_t i;
};

// a beats b: larger value, or equal value at a lower index.
__device__ __forceinline__ bool beats(float av, int32_t ai, float bv, int32_t bi) {
  return av > bv || (av == bv && ai < bi);
}

__device__ __forceinline__ void wave_best(float &v, int32_t &i) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(v, m);
    const int32_t oi = __shfl_xor(i, m);
    if (beats(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
}

// Best (value, index) of the 256-thread block, valid in thread 0.
__device__ __forceinline__ void block_best(float &v, int32_t &i) {
  __shared__ float sv[kArgmaxThreads / 64];
  __shared__ int32_t si[kArgmaxThreads / 64];
  wave_best(v, i);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sv[w] = v;
    si[w] = i;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < kArgmaxThreads / 64; ++k)
      if (beats(sv[k], si[k], v, i)) {
        v = sv[k];
        i = si[k];
      }
  }
}

}  // namespace

// Stage 1: each block scans a contiguous chunk and writes its best pair.
__global__ __launch_bounds__(kArgmaxThreads) void argmax_partial_kernel(const float *__restrict__ y,
                                                                        int64_t n, int64_t chunk,
                                                                        ValIdx *__restrict__ part) {
  const int64_t lo = static_cast<int64_t>(blockIdx.x) * chunk;
  const int64_t hi = lo + chunk < n ? lo + chunk : n;
  float v = -__builtin_inff();
  int32_t i = 0x7fffffff;
  for (int64_t k = lo + threadIdx.x; k < hi; k += kArgmaxThreads) {
    const float yk = y[k];
    if (beats(yk, static_cast<int32_t>(k), v, i)) {
      v = yk;
      i = static_cast<int32_t>(k);
    }
  }
  block_best(v, i);
  if (threadIdx.x == 0) part[blockIdx.x] = ValIdx{v, i};
}

// Stage 2: one block reduces the partial pairs.
__global__ __launch_bounds__(kArgmaxThreads) void argmax_final_kernel(const ValIdx *__restrict__ part,
                                                                      int nparts,
                                                                      int32_t *__restrict__ out) {
  float v = -__builtin_inff();
  int32_t i = 0x7fffffff;
  for (int k = threadIdx.x; k < nparts; k += kArgmaxThreads) {
    const ValIdx p = part[k];
    if (beats(p.v, p.i, v, i)) {
      v = p.v;
      i = p.i;
    }
  }
  block_best(v, i);
  if (threadIdx.x == 0) *out = i;
}

static int argmax_blocks(int64_t n) {
  int64_t b = (n + 4 * kArgmaxThreads - 1) / (4 * kArgmaxThreads);
  if (b < 1) b = 1;
  if (b > kArgmaxMaxBlocks) b = kArgmaxMaxBlocks;
  return static_cast<int>(b);
}

size_t argmax_workspace(int64_t n) { return sizeof(ValIdx) * static_cast<size_t>(argmax_blocks(n)); }

int launch_argmax(const float *y, int64_t n, int32_t *out_idx, void *ws, hipStream_t stream) {
  const int nb = argmax_blocks(n);
  const int64_t chunk = (n + nb - 1) / nb;
  ValIdx *part = static_cast<ValIdx *>(ws);
  hipLaunchKernelGGL(argmax_partial_kernel, dim3(nb), dim3(kArgmaxThreads), 0, stream, y, n, chunk,
                     part);
  ZQ_LAUNCH_CHECK();
  hipLaunchKernelGGL(argmax_final_kernel, dim3(1), dim3(kArgmaxThreads), 0, stream, part, nb,
                     out_idx);
  ZQ_LAUNCH_CHECK();
  return ZQ_OK;
}

// ------------------------------------------------------------- router -----

// One wave.  Lane l holds logits l, l+64, ... (up to 16 per lane).  top_k
// rounds of a wave-wide (value, id) maximum pick the experts largest first,
// ties to the lower id.  The softmax over the selected logits and the
// shared-expert sigmoid are evaluated in fp64 by lane 0, in selection order.
__global__ __launch_bounds__(64) void moe_route_kernel(const float *__restrict__ logits,
                                                       int32_t n_routed, int32_t top_k,
                                                       const float *__restrict__ shared_gate,
                                                       int32_t *__restrict__ ids,
                                                       float *__restrict__ wts) {
  constexpr int PER = 16;
  const int lane = static_cast<int>(threadIdx.x);
  float v[PER];
  bool taken[PER];
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int e = lane + 64 * r;
    v[r] = e < n_routed ? logits[e] : -__builtin_inff();
    taken[r] = e >= n_routed;
  }
  __shared__ int32_t sel_id[64];
  __shared__ float sel_v[64];
  for (int s = 0; s < top_k; ++s) {
    float bv = -__builtin_inff();
    int32_t bi = 0x7fffffff;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int e = lane + 64 * r;
      if (!taken[r] && beats(v[r], e, bv, bi)) {
        bv = v[r];
        bi = e;
      }
    }
    wave_best(bv, bi);
#pragma unroll
    for (int r = 0; r < PER; ++r)
      if (lane + 64 * r == bi) taken[r] = true;
    if (lane == 0) {
      sel_id[s] = bi;
      sel_v[s] = bv;
    }
  }
  __syncthreads();
  if (lane == 0) {
    const double m = static_cast<double>(sel_v[0]);
    double z = 0.0;
    for (int s = 0; s < top_k; ++s) z += exp(static_cast<double>(sel_v[s]) - m);
    for (int s = 0; s < top_k; ++s) {
      ids[s] = sel_id[s];
      wts[s] = static_cast<float>(exp(static_cast<double>(sel_v[s]) - m) / z);
    }
    if (shared_gate) {
      ids[top_k] = n_routed;
      wts[top_k] = static_cast<float>(1.0 / (1.0 + exp(-static_cast<double>(*shared_gate))));
    }
  }
}

int launch_moe_route(const float *logits, int32_t n_routed, int32_t top_k, const float *shared_gate,
                     int32_t *ids, float *wts, hipStream_t stream) {
  hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(64), 0, stream, logits, n_routed, top_k,
                     shared_gate, ids, wts);
  ZQ_LAUNCH_CHECK();
  return ZQ_OK;
}

}  // namespace zq
