// gemm.hip -- batched prefill GEMM over Q4_0 / Q8_0 weights on int8 matrix
// cores (gfx950).
//
//   Y[m][n] (+)= sum_b dx[m][b] * d_w[n][b] * isum(m, n, b)
//
// One v_mfma_i32_16x16x32_i8 covers exactly one 32-element block of one
// 16 (tokens) x 16 (weight rows) tile, so every block's integer sum leaves
// the matrix core on its own and is rescaled in fp32 (convert, d_x*d_w,
// FMA) before the next block; a K=64 form would add two blocks with
// different scales.  The matrix cores finish a tile's block in 16 cycles,
// the 12 VALU operations of its rescale take 48: the epilogue, not the
// MFMA, bounds this kernel, so the layout below is chosen to keep every
// other cost (LDS traffic, staging, idle CUs) under it.
//
// Workgroup tile: 128 tokens x 80 weight rows, 8 waves.  For the prefill
// shape (512 x 5120) that is 4 x 64 = 256 tiles, one per CU of the chip, so
// no CU runs a second tile while others idle.  The waves split K: waves 0-3
// take blocks 0-1 of every 4-block stage, waves 4-7 blocks 2-3; each wave
// owns 32 tokens x 80 rows (2 x 5 MFMA tiles).  The two K halves are added
// through LDS at the end.
//
// Staging: every stage (4 blocks) is loaded from global memory into
// registers two stages ahead and written to LDS double-buffered.  Activation
// codes are copied as they are; weight blocks are unpacked once per tile to
// signed int8 (Q4_0: nib - 8 via (nib + 0x78) ^ 0x80 per byte).  In LDS a
// row is laid out [lane group g][block][8 bytes], so one 16-byte read gives
// a lane its MFMA fragment (k = 8g..8g+7) for two consecutive blocks.
// Tiles are ordered so that each XCD walks all token tiles of a contiguous
// range of weight rows (L2 reuse of that weight slice).
#include "zq_common.h"
#include "zq_internal.h"

namespace zq {

namespace {

constexpr int BM = 128;                 // tokens per tile
constexpr int BN = 80;                  // weight rows per tile
constexpr int KB = 4;                   // blocks per stage
constexpr int NT = 512;                 // threads (8 waves)
constexpr int MS = 2;                   // 16-token subtiles per wave
constexpr int NS = BN / 16;             // 16-row subtiles per wave (5)
constexpr int ROWB = KB * 32 + 16;      // LDS bytes per row: [g][kb][8] + pad
constexpr int A_OFF = 0;
constexpr int B_OFF = A_OFF + BM * ROWB;
// The weight region has BM rows although only BN are read: threads of rows
// BN..BM-1 store their (clamped, unused) copy there, which keeps the staging
// code free of divergent branches.
constexpr int DX_OFF = B_OFF + BM * ROWB;      // float [KB][BM]
constexpr int DW_OFF = DX_OFF + KB * BM * 4;   // float [BM][KB]
constexpr int STAGE_BYTES = DW_OFF + BM * KB * 4;
static_assert(BM * KB == NT, "one activation (row, block) per thread");
static_assert(BN <= BM, "weight rows fit the staging grid");
constexpr int RING = 2;                 // stages of global loads in flight
static_assert(RING % 2 == 0, "the LDS double buffer alternates with the unrolled ring");
// More than half of the CU's 160 KB, so a CU never holds two tiles while
// another CU idles.
constexpr int LDS_BYTES = 2 * STAGE_BYTES > 82 * 1024 ? 2 * STAGE_BYTES : 82 * 1024;
static_assert(4 * MS * NS * 4 * 64 * 4 <= 2 * STAGE_BYTES, "K-split exchange fits in LDS");

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

template <int WT>
struct StageRegs {
  u32x4 a0, a1;                // 32 activation bytes of (row, block)
  float dxv;                   // its scale
  uint32_t w[Blk<WT>::NW];     // weight window of (row, block), raw
  uint32_t o;                  // byte offset of the block inside the window
  bool a_ok, b_ok;             // block index < nb
};

// Every thread issues the same loads for every stage (rows and blocks past
// the end are clamped to valid addresses and zeroed at the LDS store), so the
// number of loads in flight is the same on every path and the compiler can
// wait for the oldest stage only.
template <int WT>
__device__ __forceinline__ void load_stage(const GemmArgs &g, int64_t m0, int64_t n0, int kb0,
                                           StageRegs<WT> &r) {
  const int t = static_cast<int>(threadIdx.x);
  const int row = t >> 2;
  const int blk = t & 3;
  const int b = kb0 + blk;
  const bool bok = b < g.nb;
  const int bc = bok ? b : g.nb - 1;
  int64_t mr = m0 + row;
  mr = mr < g.m_end ? mr : g.m_end - 1;
  const int8_t *ap = g.qx + mr * g.k + static_cast<int64_t>(bc) * 32;
  r.a0 = *reinterpret_cast<const u32x4 *>(ap);
  r.a1 = *reinterpret_cast<const u32x4 *>(ap + 16);
  r.dxv = g.dx[mr * g.nb + bc];
  r.a_ok = bok;
  int64_t nr = n0 + (row < BN ? row : BN - 1);
  nr = nr < g.n_end ? nr : g.n_end - 1;
  r.o = load_window<WT>(g.w + nr * g.row_bytes + static_cast<int64_t>(bc) * Blk<WT>::BYTES, r.w);
  r.b_ok = bok;
}

// Blocks past nb (ragged K, padded stages) keep the clamped codes that were
// loaded and get zero scales: d_x * d_w = 0 times a finite integer sum adds
// an exact zero, so their codes need not be cleared.
template <int WT>
__device__ __forceinline__ void store_stage(uint8_t *lds, const StageRegs<WT> &r) {
  const int t = static_cast<int>(threadIdx.x);
  const int row = t >> 2;
  const int blk = t & 3;
  {
    uint8_t *p = lds + A_OFF + row * ROWB + blk * 8;
    *reinterpret_cast<u32x2 *>(p + 0) = u32x2{r.a0.x, r.a0.y};
    *reinterpret_cast<u32x2 *>(p + 32) = u32x2{r.a0.z, r.a0.w};
    *reinterpret_cast<u32x2 *>(p + 64) = u32x2{r.a1.x, r.a1.y};
    *reinterpret_cast<u32x2 *>(p + 96) = u32x2{r.a1.z, r.a1.w};
    reinterpret_cast<float *>(lds + DX_OFF)[blk * BM + row] = r.a_ok ? r.dxv : 0.0f;
  }
  {
    uint32_t wq[8];
    const uint32_t sel = quant_selector(r.o);
    if constexpr (WT == ZQ_Q4_0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t p = __builtin_amdgcn_perm(r.w[q + 1], r.w[q], sel);
        wq[q] = ((p & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u;
        wq[4 + q] = (((p >> 4) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) wq[q] = __builtin_amdgcn_perm(r.w[q + 1], r.w[q], sel);
    }
    uint8_t *p = lds + B_OFF + row * ROWB + blk * 8;
#pragma unroll
    for (int gi = 0; gi < 4; ++gi)
      *reinterpret_cast<u32x2 *>(p + 32 * gi) = u32x2{wq[2 * gi], wq[2 * gi + 1]};
    reinterpret_cast<float *>(lds + DW_OFF)[row * KB + blk] =
        r.b_ok ? window_scale(r.w[0], r.o) : 0.0f;
  }
}

__device__ __forceinline__ int64_t as_i64(uint32_t lo, uint32_t hi) {
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

template <int WT, bool ISUMS>
__device__ __forceinline__ void compute_stage(const GemmArgs &g, const uint8_t *S, int st, int64_t m0,
                                              int64_t n0, int mp, int kb0, int lane,
                                              float (&acc)[MS][NS][4]) {
  const int l16 = lane & 15, lg = lane >> 4;
  u32x4 af[MS], bf[NS];
  float4 dxa[MS][2];
  float2 dwb[NS];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) {
    const int row = mp * 32 + ms * 16;
    af[ms] = *reinterpret_cast<const u32x4 *>(S + A_OFF + (row + l16) * ROWB + lg * 32 + kb0 * 8);
#pragma unroll
    for (int q = 0; q < 2; ++q)
      dxa[ms][q] = *reinterpret_cast<const float4 *>(S + DX_OFF + ((kb0 + q) * BM + row + 4 * lg) * 4);
  }
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    bf[j] = *reinterpret_cast<const u32x4 *>(S + B_OFF + (j * 16 + l16) * ROWB + lg * 32 + kb0 * 8);
    dwb[j] = *reinterpret_cast<const float2 *>(S + DW_OFF + ((j * 16 + l16) * KB + kb0) * 4);
  }
  constexpr int NTILE = 2 * MS * NS;   // (block, token subtile, row subtile)
  i32x4 is[NTILE];
#pragma unroll
  for (int t = 0; t < NTILE; ++t) {
    const int q = t / (MS * NS), ms = (t / NS) % MS, j = t % NS;
    const int64_t a = q == 0 ? as_i64(af[ms].x, af[ms].y) : as_i64(af[ms].z, af[ms].w);
    const int64_t b = q == 0 ? as_i64(bf[j].x, bf[j].y) : as_i64(bf[j].z, bf[j].w);
    const i32x4 z = {0, 0, 0, 0};
    is[t] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, z, 0, 0, 0);
  }
#pragma unroll
  for (int t = 0; t < NTILE; ++t) {
    const int q = t / (MS * NS), ms = (t / NS) % MS, j = t % NS;
    if constexpr (ISUMS) {
      const int blk = st * KB + kb0 + q;
      const int64_t n = n0 + j * 16 + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + mp * 32 + ms * 16 + lg * 4 + r;
        if (blk < g.nb && m < g.m_end && n < g.n_end)
          g.isums[((m - g.m_begin) * (g.n_end - g.n_begin) + (n - g.n_begin)) * g.nb + blk] = is[t][r];
      }
    } else {
      const float dxs[4] = {dxa[ms][q].x, dxa[ms][q].y, dxa[ms][q].z, dxa[ms][q].w};
      const float dw = q == 0 ? dwb[j].x : dwb[j].y;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        acc[ms][j][r] = __builtin_fmaf(dxs[r] * dw, static_cast<float>(is[t][r]), acc[ms][j][r]);
    }
  }
}

template <int WT, bool ISUMS>
__global__ __launch_bounds__(NT) void gemm_kernel(const GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
  const int64_t tiles = static_cast<int64_t>(g.tiles_m) * g.tiles_n;
  int64_t id = blockIdx.x;
  if (tiles % 8 == 0) id = (id % 8) * (tiles / 8) + id / 8;
  const int tm = static_cast<int>(id % g.tiles_m);
  const int tn = static_cast<int>(id / g.tiles_m);
  const int64_t m0 = g.m_begin + static_cast<int64_t>(tm) * BM;
  const int64_t n0 = g.n_begin + static_cast<int64_t>(tn) * BN;

  const int lane = static_cast<int>(threadIdx.x & 63);
  const int wv = static_cast<int>(threadIdx.x >> 6);
  const int kh = wv >> 2;           // K half: blocks 2kh, 2kh+1 of each stage
  const int mp = wv & 3;            // tokens mp*32 .. mp*32+31 of the tile
  const int l16 = lane & 15, lg = lane >> 4;
  const int kb0 = 2 * kh;

  float acc[MS][NS][4];
#pragma unroll
  for (int a = 0; a < MS; ++a)
#pragma unroll
    for (int b = 0; b < NS; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[a][b][r] = 0.0f;

  // Stage s is loaded into register slot s % RING, RING stages ahead of the
  // compute that consumes it, so RING stages of compute cover the latency of
  // its global loads.
  // The stage count is padded to a multiple of RING so that the unrolled
  // loop body has no branch.  A stage past the end has all its blocks past
  // nb: its loads are clamped to valid addresses and store_stage zeroes its
  // codes and scales, so computing it adds exact zeros.
  const int n_stages = (g.nb + KB - 1) / KB;
  const int n_pad = (n_stages + RING - 1) / RING * RING;
  StageRegs<WT> sr[RING];
#pragma unroll
  for (int p = 0; p < RING; ++p) load_stage<WT>(g, m0, n0, p * KB, sr[p]);
  store_stage<WT>(lds, sr[0]);
  load_stage<WT>(g, m0, n0, RING * KB, sr[0]);
  __syncthreads();

  for (int st0 = 0; st0 < n_pad; st0 += RING) {
#pragma unroll
    for (int p = 0; p < RING; ++p) {
      const int st = st0 + p;
      compute_stage<WT, ISUMS>(g, lds + (p & 1) * STAGE_BYTES, st, m0, n0, mp, kb0, lane, acc);
      const int slot = (p + 1) % RING;
      store_stage<WT>(lds + ((p + 1) & 1) * STAGE_BYTES, sr[slot]);
      load_stage<WT>(g, m0, n0, (st + 1 + RING) * KB, sr[slot]);
      __syncthreads();
    }
  }

  if constexpr (!ISUMS) {
    // Add the two K halves: the wave of half kh keeps token subtile ms = kh
    // and hands the other one to its partner through LDS.
    float *red = reinterpret_cast<float *>(lds);   // [mp][ms][NS*4][64]
    auto slot = [&](int ms, int v) { return ((mp * MS + ms) * (NS * 4) + v) * 64 + lane; };
    const int give = 1 - kh;
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[slot(give, j * 4 + r)] = give == 0 ? acc[0][j][r] : acc[1][j][r];
    __syncthreads();
    const int keep = kh;
    const int64_t mbase = m0 + mp * 32 + keep * 16 + lg * 4;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int64_t n = n0 + j * 16 + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = (keep == 0 ? acc[0][j][r] : acc[1][j][r]) + red[slot(keep, j * 4 + r)];
        const int64_t m = mbase + r;
        if (m < g.m_end && n < g.n_end) {
          float *yp = g.y + m * g.n + n;
          *yp = (g.flags & ZQ_ACCUMULATE) ? *yp + v : v;
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
      hipLaunchKernelGGL((gemm_kernel<ZQ_Q4_0, true>), dim3(grid), dim3(NT), 0, stream, g);
    else
      hipLaunchKernelGGL((gemm_kernel<ZQ_Q4_0, false>), dim3(grid), dim3(NT), 0, stream, g);
  } else {
    if (isums)
      hipLaunchKernelGGL((gemm_kernel<ZQ_Q8_0, true>), dim3(grid), dim3(NT), 0, stream, g);
    else
      hipLaunchKernelGGL((gemm_kernel<ZQ_Q8_0, false>), dim3(grid), dim3(NT), 0, stream, g);
  }
  ZQ_LAUNCH_CHECK();
  return ZQ_OK;
}

}  // namespace zq
