// probe.hip -- a measurement hook: a plain streaming read of a device
// buffer, the ceiling the weight-streaming kernels are compared with.
#include "zq_common.h"
#include "zq_internal.h"

namespace zq {

int launch_read_probe(const void *buf, int64_t bytes, uint32_t *sink, hipStream_t stream);

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;  // 16-byte loads in flight per lane
constexpr int kProbeMaxBlocks = 8192;
// Large buffers (the streaming-read ceiling): 1024-thread workgroups and up
// to 32768 of them.  Over 1 GiB: 6.56-6.59 TB/s, against 6.2 for 256
// threads and 8192 workgroups (a sweep of 256/512/1024 threads x 4/8/16
// loads x 4K-32K workgroups).
constexpr int kProbeBigThreads = 1024;
constexpr int kProbeBigMaxBlocks = 32768;
constexpr int64_t kProbeBigBytes = static_cast<int64_t>(256) << 20;

}  // namespace

// Each workgroup reads one contiguous chunk with 16-byte loads (kProbeUnroll
// per lane in flight on large buffers) and folds them with XOR.  The one store is taken only
// when the fold equals a fixed word, which the compiler cannot rule out, so
// every load stays and (almost) nothing is written.
template <int T>
__global__ __launch_bounds__(T) void read_probe_kernel(const uint4 *__restrict__ p, int64_t n16,
                                                       int64_t chunk, uint32_t *__restrict__ sink) {
  const int64_t lo = static_cast<int64_t>(blockIdx.x) * chunk;
  const int64_t hi = lo + chunk < n16 ? lo + chunk : n16;
  uint32_t acc = 0;
  constexpr int64_t step = static_cast<int64_t>(T) * kProbeUnroll;
  int64_t i = lo + threadIdx.x;
  for (; i + (kProbeUnroll - 1) * T < hi; i += step) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = p[i + u * T];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < hi; i += T) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x5a17c0deu) *sink = acc;
}

int launch_read_probe(const void *buf, int64_t bytes, uint32_t *sink, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  if (n16 == 0) return ZQ_OK;
  if (bytes >= kProbeBigBytes) {
    int64_t blocks = (n16 + kProbeBigThreads - 1) / kProbeBigThreads;
    if (blocks > kProbeBigMaxBlocks) blocks = kProbeBigMaxBlocks;
    const int64_t chunk = (n16 + blocks - 1) / blocks;
    blocks = (n16 + chunk - 1) / chunk;
    hipLaunchKernelGGL(read_probe_kernel<kProbeBigThreads>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kProbeBigThreads), 0, stream, static_cast<const uint4 *>(buf), n16, chunk,
                       sink);
    ZQ_LAUNCH_CHECK();
    return ZQ_OK;
  }
  // a load per lane per workgroup where that keeps the grid within
  // kProbeMaxBlocks (small buffers: as many waves as the DMMV launches
  // over the same bytes), else kProbeUnroll loads per lane in flight
  int64_t blocks = (n16 + kProbeThreads - 1) / kProbeThreads;
  if (blocks > kProbeMaxBlocks) blocks = kProbeMaxBlocks;
  const int64_t chunk = (n16 + blocks - 1) / blocks;
  blocks = (n16 + chunk - 1) / chunk;
  hipLaunchKernelGGL(read_probe_kernel<kProbeThreads>, dim3(static_cast<unsigned>(blocks)),
                     dim3(kProbeThreads), 0, stream, static_cast<const uint4 *>(buf), n16, chunk, sink);
  ZQ_LAUNCH_CHECK();
  return ZQ_OK;
}

}  // namespace zq
