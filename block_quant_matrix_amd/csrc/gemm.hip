// gemm.hip -- batched prefill GEMM over Q4_0 / Q8_0 weights on int8 matrix
// cores (gfx950).
//
//   Y[m][n] (+)= sum_b dx[m][b] * d_w[n][b] * isum(m, n, b)
//
// Each workgroup (4 waves) owns a 64 (tokens) x 64 (weight rows) tile; each
// wave a 32 x 32 quarter = 2 x 2 tiles of v_mfma_i32_16x16x32_i8.  The K
// step of that instruction is exactly one 32-element block, so every block's
// integer sum comes out of the matrix core on its own and is rescaled in fp32
// (convert, d_x*d_w, FMA) before the next block: a K=64 form would add two
// blocks with different scales.
//
// K is staged through LDS four blocks at a time, double-buffered: activation
// codes are copied as they are; weight blocks are unpacked once per tile to
// signed int8 (Q4_0: nib - 8 via (nib + 0x78) ^ 0x80 per byte) so the unpack
// is amortized over the 64 tokens of the tile.  Tiles are assigned so that
// consecutive workgroups on one XCD walk all token tiles of the same weight
// rows (L2 reuse of the weight slice).
#include "zq_common.h"
#include "zq_internal.h"

namespace zq {

namespace {

constexpr int BM = 64;
constexpr int BN = 64;
constexpr int KB = 4;                       // blocks per stage
constexpr int ROWB = KB * 32 + 16;          // LDS row stride (bytes), padded
constexpr int A_BYTES = BM * ROWB;
constexpr int B_BYTES = BN * ROWB;

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

struct GemmArgs {
  const uint8_t *w;
  const int8_t *qx;
  const float *dx;
  float *y;
  int32_t *isums;
  int64_t n, k, m;
  int64_t m_begin, m_end, n_begin, n_end;
  int64_t row_bytes;
  int32_t nb;
  int32_t tiles_m, tiles_n;
  uint32_t flags;
};

struct StageRegs {
  u32x4 a0, a1;     // 32 activation bytes
  float dxv;        // activation scale of (row, block)
  uint32_t wq[8];   // 32 unpacked weight bytes (signed int8)
  float dwv;        // weight scale of (row, block)
};

template <int WT>
__device__ __forceinline__ void load_stage(const GemmArgs &g, int64_t m0, int64_t n0, int kb0,
                                           StageRegs &r) {
  const int t = static_cast<int>(threadIdx.x);
  const int row = t >> 2;     // 0..63
  const int blk = t & 3;      // 0..3
  const int b = kb0 + blk;
  const bool bok = b < g.nb;
  const int bc = bok ? b : g.nb - 1;
  // activation: token row m0+row, block b
  int64_t mr = m0 + row;
  mr = mr < g.m_end ? mr : g.m_end - 1;
  const int8_t *ap = g.qx + mr * g.k + static_cast<int64_t>(bc) * 32;
  r.a0 = *reinterpret_cast<const u32x4 *>(ap);
  r.a1 = *reinterpret_cast<const u32x4 *>(ap + 16);
  r.dxv = bok ? g.dx[mr * g.nb + bc] : 0.0f;
  // weight: row n0+row, block b
  int64_t nr = n0 + row;
  nr = nr < g.n_end ? nr : g.n_end - 1;
  uint32_t w[Blk<WT>::NW];
  const uint32_t o = load_window<WT>(g.w + nr * g.row_bytes + static_cast<int64_t>(bc) * Blk<WT>::BYTES, w);
  const uint32_t sel = quant_selector(o);
  r.dwv = bok ? window_scale(w[0], o) : 0.0f;
  if constexpr (WT == ZQ_Q4_0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t p = __builtin_amdgcn_perm(w[q + 1], w[q], sel);
      r.wq[q] = ((p & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u;
      r.wq[4 + q] = (((p >> 4) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u;
    }
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) r.wq[q] = __builtin_amdgcn_perm(w[q + 1], w[q], sel);
  }
  if (!bok) {
    r.a0 = u32x4{0, 0, 0, 0};
    r.a1 = u32x4{0, 0, 0, 0};
#pragma unroll
    for (int q = 0; q < 8; ++q) r.wq[q] = 0;
  }
}

__device__ __forceinline__ void store_stage(uint8_t *lds, const StageRegs &r) {
  const int t = static_cast<int>(threadIdx.x);
  const int row = t >> 2;
  const int blk = t & 3;
  uint8_t *A = lds;
  uint8_t *B = lds + A_BYTES;
  float *DX = reinterpret_cast<float *>(lds + A_BYTES + B_BYTES);
  float *DW = DX + KB * BM;
  *reinterpret_cast<u32x4 *>(A + row * ROWB + blk * 32) = r.a0;
  *reinterpret_cast<u32x4 *>(A + row * ROWB + blk * 32 + 16) = r.a1;
  *reinterpret_cast<u32x4 *>(B + row * ROWB + blk * 32) = u32x4{r.wq[0], r.wq[1], r.wq[2], r.wq[3]};
  *reinterpret_cast<u32x4 *>(B + row * ROWB + blk * 32 + 16) =
      u32x4{r.wq[4], r.wq[5], r.wq[6], r.wq[7]};
  DX[blk * BM + row] = r.dxv;
  DW[blk * BN + row] = r.dwv;
}

constexpr int STAGE_BYTES = A_BYTES + B_BYTES + 2 * KB * 64 * 4;

template <int WT, bool ISUMS>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][STAGE_BYTES];
  // XCD-aware tile order: workgroup ids go round-robin over the 8 XCDs; give
  // each XCD a contiguous run of tiles that share weight rows.
  const int64_t tiles = static_cast<int64_t>(g.tiles_m) * g.tiles_n;
  int64_t id = blockIdx.x;
  if (tiles % 8 == 0) id = (id % 8) * (tiles / 8) + id / 8;
  const int tm = static_cast<int>(id % g.tiles_m);
  const int tn = static_cast<int>(id / g.tiles_m);
  const int64_t m0 = g.m_begin + static_cast<int64_t>(tm) * BM;
  const int64_t n0 = g.n_begin + static_cast<int64_t>(tn) * BN;

  const int lane = static_cast<int>(threadIdx.x & 63);
  const int wv = static_cast<int>(threadIdx.x >> 6);
  const int wm = wv & 1, wn = wv >> 1;
  const int l16 = lane & 15, lg = lane >> 4;

  float acc[2][2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[a][b][r] = 0.0f;

  const int n_stages = (g.nb + KB - 1) / KB;
  StageRegs sr;
  load_stage<WT>(g, m0, n0, 0, sr);
  store_stage(lds[0], sr);
  __syncthreads();

  for (int st = 0; st < n_stages; ++st) {
    const int cur = st & 1;
    if (st + 1 < n_stages) load_stage<WT>(g, m0, n0, (st + 1) * KB, sr);
    const uint8_t *A = lds[cur];
    const uint8_t *B = lds[cur] + A_BYTES;
    const float *DX = reinterpret_cast<const float *>(lds[cur] + A_BYTES + B_BYTES);
    const float *DW = DX + KB * BM;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      int64_t af[2], bf[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        af[t] = *reinterpret_cast<const int64_t *>(A + (wm * 32 + t * 16 + l16) * ROWB + kb * 32 + lg * 8);
        bf[t] = *reinterpret_cast<const int64_t *>(B + (wn * 32 + t * 16 + l16) * ROWB + kb * 32 + lg * 8);
      }
      float4 dxa[2];
      float dwb[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        dxa[t] = *reinterpret_cast<const float4 *>(DX + kb * BM + wm * 32 + t * 16 + lg * 4);
        dwb[t] = DW[kb * BN + wn * 32 + t * 16 + l16];
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const i32x4 z = {0, 0, 0, 0};
          const i32x4 is = __builtin_amdgcn_mfma_i32_16x16x32_i8(af[mt], bf[nt], z, 0, 0, 0);
          if constexpr (ISUMS) {
            const int b = st * KB + kb;
            const int64_t n = n0 + wn * 32 + nt * 16 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int64_t m = m0 + wm * 32 + mt * 16 + lg * 4 + r;
              if (b < g.nb && m < g.m_end && n < g.n_end)
                g.isums[((m - g.m_begin) * (g.n_end - g.n_begin) + (n - g.n_begin)) * g.nb + b] = is[r];
            }
          } else {
            const float dxs[4] = {dxa[mt].x, dxa[mt].y, dxa[mt].z, dxa[mt].w};
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[mt][nt][r] =
                  __builtin_fmaf(dxs[r] * dwb[nt], static_cast<float>(is[r]), acc[mt][nt][r]);
          }
        }
      }
    }
    if (st + 1 < n_stages) store_stage(lds[cur ^ 1], sr);
    __syncthreads();
  }

  if constexpr (!ISUMS) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int64_t n = n0 + wn * 32 + nt * 16 + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t m = m0 + wm * 32 + mt * 16 + lg * 4 + r;
          if (m < g.m_end && n < g.n_end) {
            float *yp = g.y + m * g.n + n;
            *yp = (g.flags & ZQ_ACCUMULATE) ? *yp + acc[mt][nt][r] : acc[mt][nt][r];
          }
        }
      }
  }
}

}  // namespace

int launch_gemm(int wtype, const void *w, int64_t n, int64_t k, const int8_t *qx, const float *dx,
                int64_t m, float *y, uint32_t flags, int32_t *isums, int64_t m0, int64_t m1,
                int64_t n0, int64_t n1, hipStream_t stream) {
  if (m1 <= m0 || n1 <= n0) return ZQ_OK;
  GemmArgs g;
  g.w = static_cast<const uint8_t *>(w);
  g.qx = qx;
  g.dx = dx;
  g.y = y;
  g.isums = isums;
  g.n = n;
  g.k = k;
  g.m = m;
  g.m_begin = m0;
  g.m_end = m1;
  g.n_begin = n0;
  g.n_end = n1;
  g.nb = static_cast<int32_t>(k / 32);
  g.row_bytes = static_cast<int64_t>(g.nb) * (wtype == ZQ_Q4_0 ? 18 : 34);
  g.tiles_m = static_cast<int32_t>((m1 - m0 + BM - 1) / BM);
  g.tiles_n = static_cast<int32_t>((n1 - n0 + BN - 1) / BN);
  g.flags = flags;
  const unsigned grid = static_cast<unsigned>(static_cast<int64_t>(g.tiles_m) * g.tiles_n);
  if (wtype == ZQ_Q4_0) {
    if (isums)
      hipLaunchKernelGGL((gemm_kernel<ZQ_Q4_0, true>), dim3(grid), dim3(256), 0, stream, g);
    else
      hipLaunchKernelGGL((gemm_kernel<ZQ_Q4_0, false>), dim3(grid), dim3(256), 0, stream, g);
  } else {
    if (isums)
      hipLaunchKernelGGL((gemm_kernel<ZQ_Q8_0, true>), dim3(grid), dim3(256), 0, stream, g);
    else
      hipLaunchKernelGGL((gemm_kernel<ZQ_Q8_0, false>), dim3(grid), dim3(256), 0, stream, g);
  }
  ZQ_LAUNCH_CHECK();
  return ZQ_OK;
}

}  // namespace zq
