// argmax_route.hip -- LM-head argmax and the MoE softmax_topk router (gfx950).
#include "zq_common.h"
#include "zq_internal.h"

namespace zq {

namespace {

constexpr int kArgmaxThreads = 256;
constexpr int kArgmaxMaxBlocks = 1024;

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
  block_best<kArgmaxThreads / 64>(v, i);
  if (threadIdx.x == 0) part[blockIdx.x] = ValIdx{v, i};
}

// Stage 2: one workgroup of 1024 threads reduces the partial pairs.  Each
// thread requests its pairs (two per round, 2048 per round over the
// workgroup) before comparing any, so a round costs one memory latency; the
// pairs meet within each wave through DPP moves inside 16-lane rows and the
// permlane swaps across rows (a few cycles each, against a round trip
// through LDS per step for lane shuffles), then across the 16 waves through
// LDS and the same wave reduction once more.
constexpr int kFinalThreads = 1024;

__global__ __launch_bounds__(kFinalThreads) void argmax_final_kernel(const ValIdx *__restrict__ part,
                                                                     int nparts,
                                                                     int32_t *__restrict__ out) {
  __shared__ float sv[kFinalThreads / 64];
  __shared__ int32_t si[kFinalThreads / 64];
  const int tid = static_cast<int>(threadIdx.x);
  float v = -__builtin_inff();
  int32_t i = 0x7fffffff;
  for (int base = 0; base < nparts; base += 2 * kFinalThreads) {
    const int k0 = base + tid, k1 = base + kFinalThreads + tid;
    const ValIdx p0 = k0 < nparts ? part[k0] : ValIdx{-__builtin_inff(), 0x7fffffff};
    const ValIdx p1 = k1 < nparts ? part[k1] : ValIdx{-__builtin_inff(), 0x7fffffff};
    take_best(v, i, p0.v, p0.i);
    take_best(v, i, p1.v, p1.i);
  }
  wave_best(v, i);
  const int w = tid >> 6;
  if ((tid & 63) == 0) {
    sv[w] = v;
    si[w] = i;
  }
  __syncthreads();
  if (tid < 64) {
    v = tid < kFinalThreads / 64 ? sv[tid] : -__builtin_inff();
    i = tid < kFinalThreads / 64 ? si[tid] : 0x7fffffff;
    wave_best(v, i);
    if (tid == 0) *out = i;
  }
}

static int argmax_blocks(int64_t n) {
  int64_t b = (n + 4 * kArgmaxThreads - 1) / (4 * kArgmaxThreads);
  if (b < 1) b = 1;
  if (b > kArgmaxMaxBlocks) b = kArgmaxMaxBlocks;
  return static_cast<int>(b);
}

size_t argmax_workspace(int64_t n) { return sizeof(ValIdx) * static_cast<size_t>(argmax_blocks(n)); }

int launch_argmax_final(const void *part, int nparts, int32_t *out_idx, hipStream_t stream) {
  hipLaunchKernelGGL(argmax_final_kernel, dim3(1), dim3(kFinalThreads), 0, stream,
                     static_cast<const ValIdx *>(part), nparts, out_idx);
  ZQ_LAUNCH_CHECK();
  return ZQ_OK;
}

int launch_argmax(const float *y, int64_t n, int32_t *out_idx, void *ws, hipStream_t stream) {
  const int nb = argmax_blocks(n);
  const int64_t chunk = (n + nb - 1) / nb;
  ValIdx *part = static_cast<ValIdx *>(ws);
  hipLaunchKernelGGL(argmax_partial_kernel, dim3(nb), dim3(kArgmaxThreads), 0, stream, y, n, chunk,
                     part);
  ZQ_LAUNCH_CHECK();
  hipLaunchKernelGGL(argmax_final_kernel, dim3(1), dim3(kFinalThreads), 0, stream, part, nb,
                     out_idx);
  ZQ_LAUNCH_CHECK();
  return ZQ_OK;
}

// ------------------------------------------------------------- router -----

// The router: rank selection and fp64 softmax (route_rank, route_weights in
// zq_common.h) in one workgroup.
template <int P>
__global__ __launch_bounds__(1024) void moe_route_kernel(const float *__restrict__ logits,
                                                         int32_t n_routed, int32_t top_k,
                                                         const float *__restrict__ shared_gate,
                                                         int32_t *__restrict__ ids,
                                                         float *__restrict__ wts) {
  __shared__ __attribute__((aligned(16))) float lv[1024];
  __shared__ int32_t sel_id[64];
  __shared__ float sel_v[64];
  __shared__ double sel_e[64];
  const int n_pad = route_stage<P, 1024>(lv, logits, n_routed);
  __syncthreads();
  route_rank<P, 1024>(lv, n_routed, n_pad, top_k, sel_id, sel_v);
  __syncthreads();
  route_weights(sel_id, sel_v, sel_e, n_routed, top_k, shared_gate, ids, wts);
}

int launch_moe_route(const float *logits, int32_t n_routed, int32_t top_k, const float *shared_gate,
                     int32_t *ids, float *wts, hipStream_t stream) {
  // 1024 threads; P threads per logit while n_routed * P fits (P <= 16)
  int p = 1;
  while (p < 16 && n_routed * (p * 2) <= 1024) p *= 2;
  switch (p) {
    case 16: hipLaunchKernelGGL(moe_route_kernel<16>, dim3(1), dim3(1024), 0, stream, logits, n_routed, top_k, shared_gate, ids, wts); break;
    case 8: hipLaunchKernelGGL(moe_route_kernel<8>, dim3(1), dim3(1024), 0, stream, logits, n_routed, top_k, shared_gate, ids, wts); break;
    case 4: hipLaunchKernelGGL(moe_route_kernel<4>, dim3(1), dim3(1024), 0, stream, logits, n_routed, top_k, shared_gate, ids, wts); break;
    case 2: hipLaunchKernelGGL(moe_route_kernel<2>, dim3(1), dim3(1024), 0, stream, logits, n_routed, top_k, shared_gate, ids, wts); break;
    default: hipLaunchKernelGGL(moe_route_kernel<1>, dim3(1), dim3(1024), 0, stream, logits, n_routed, top_k, shared_gate, ids, wts); break;
  }
  ZQ_LAUNCH_CHECK();
  return ZQ_OK;
}

}  // namespace zq
