// dmmv_tok.hip -- multi-token DMMV over Q4_0 / Q8_0 blocks (gfx950, wave64):
// y[t][r] = sum_b d_w[r][b] * dx[t][b] * isum_t[r][b] for 2..8 tokens decoded
// together, in one pass over the weights.  Three forms: the vector form
// below (packed dot4 per token), and two on the int8 matrix cores further
// down -- the tall form for 65 536 rows and more, the tile form for shorter
// matrices with 5..8 tokens.  launch_dmmv_tok picks one.
//
// Vector form.  Mapping: as the single-token DMMV (dmmv.hip): a row slot of
// LPR lanes walks one row, lane j owns blocks j, j+LPR, ... (BPL of them per
// pass), and each wave issues the windows of RB row steps before any
// arithmetic.  The lane holds the codes, scales and sums of its blocks for
// all T tokens (T*BPL <= 8 blocks of activation), so each weight block is
// unpacked once and dotted with T activation blocks.  The RB*T row partials
// per lane are folded by one RowReduce.  Tokens past n_tok load the last
// token and get zero scales; their rows are not written.
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
__global__ __launch_bounds__(256) void dmmv_tok_kernel(const uint8_t *w, const int8_t *qx,
                                                       const float *dx, int64_t rows,
                                                       int64_t row_bytes, int64_t n_groups,
                                                       int32_t k, int32_t nb,
                                                       const DmmvTokArgs a_in) {
  // leading scalars: preloaded kernel arguments (as dmmv_hot in zq_internal.h)
  DmmvTokArgs a = a_in;
  a.w = w;
  a.qx = qx;
  a.dx = dx;
  a.rows = rows;
  a.row_bytes = row_bytes;
  a.n_groups = n_groups;
  a.k = k;
  a.nb = nb;
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

// ---------------------------------------------------------------------------
// Matrix-core form for tall matrices (the LM head): one
// v_mfma_i32_16x16x32_i8 per (16 weight rows, block) gives the block's int32
// sums for all tokens at once (tokens past n_tok read token 0's codes and
// take zero scales), instead of 8 packed dot4 per (row, block, token) on the
// vector units.
//
// Each wave owns 16 consecutive rows and walks k in chunks of KC blocks.
// Staging: the wave reads its 16 rows' chunk with the lanes on consecutive
// blocks of a row (64/KC rows per load instruction, as the single-token
// DMMV reads), and writes each block's codes and scale (fp32) to its own LDS
// region; the next chunk's windows are requested before this chunk's
// arithmetic.  Compute: lane (n = lane % 16, g = lane / 16) takes 8 of row
// n's codes and token n's codes for the same 8 k from LDS, and receives the
// sums of tokens 4g..4g+3 against row n.  Q8_0: k = 8g..8g+7.
//
// Q4_0: a lane's 8 codes are the nibbles of one dword of the block's 16 code
// bytes, dword g: its low nibbles (k = 4g..4g+3), then its high nibbles
// (k = 16+4g..16+4g+3); the tokens' codes are staged in that k order.  The
// codes are staged with every nibble's top bit flipped (q ^ 8), so a nibble
// in the high half of its byte reads as the int8 16 * (q - 8): the low
// nibbles shift left by 4, and one AND each clears the rest.  The sums come
// out 16 times too large, exactly; the staged scale carries the 1/16.
//
// With at most 8 tokens only the lanes g = 0, 1 hold real tokens.  Blocks
// are taken in pairs: v_permlane32_swap moves the second block's real half
// into the first block's lanes 32..63, so one convert / scale / FMA pass
// rescales both blocks (lanes 0..31 accumulate the even blocks, 32..63 the
// odd ones), and the halves are added once at the end.
constexpr int kTmWaves = 8;   // waves (16 rows each) per workgroup

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

template <int WT> struct Tm;
// KC blocks per chunk: small chunks keep a workgroup's LDS small, and the
// occupancy that buys hides more latency than longer chunks would (8 vs 32
// blocks: 69 vs 101 us for 8 tokens through the Q4_0 LM head).  KC is even:
// blocks are rescaled in pairs.
template <> struct Tm<ZQ_Q4_0> { static constexpr int KC = 8; static constexpr int QB = 16; };
template <> struct Tm<ZQ_Q8_0> { static constexpr int KC = 8; static constexpr int QB = 32; };

// LDS row padding.  A staged weight row (KC*QB + 8 bytes, 34 dwords for
// Q4_0) puts the 16 rows a wave reads at once 2 banks apart; a token's row
// (k + 32 bytes, 8 banks apart for k a multiple of 256) does the same for
// the 8 tokens x 4 k-groups of one read.  At 8 tokens and k = 2048 a Q4_0
// launch then needs 39.1 KB, so 4 workgroups (32 waves) fit in a CU.
constexpr int kTmPad = 8;
constexpr int kTmXPad = 32;

// LDS bytes of one launch: tokens' codes [n_tok][k + xpad], their scales
// [nb_pad][8], and per wave a chunk of codes [16][KC*QB + pad] and scales
// [KC][16].
size_t tm_lds_bytes(int wtype, int32_t n_tok, int32_t k) {
  const int kc = wtype == ZQ_Q4_0 ? Tm<ZQ_Q4_0>::KC : Tm<ZQ_Q8_0>::KC;
  const int qb = wtype == ZQ_Q4_0 ? Tm<ZQ_Q4_0>::QB : Tm<ZQ_Q8_0>::QB;
  const int64_t nb = k / 32, nb_pad = (nb + kc - 1) / kc * kc;
  return static_cast<size_t>(n_tok) * (k + kTmXPad) + static_cast<size_t>(nb_pad) * 32 +
         static_cast<size_t>(kTmWaves) * (16 * (kc * qb + kTmPad) + kc * 64);
}

__device__ __forceinline__ void swap32_i(int32_t &a, int32_t &b) {
  auto r = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(a), static_cast<uint32_t>(b),
                                            false, false);
  a = static_cast<int32_t>(r[0]);
  b = static_cast<int32_t>(r[1]);
}

// The matrix-core and tile kernels' leading scalars: preloaded kernel
// arguments (as dmmv_hot in zq_internal.h).
__device__ __forceinline__ void tok_tile_hot(DmmvTokArgs &a, const uint8_t *w, const int8_t *qx,
                                             const float *dx, int64_t rows, int64_t row_bytes,
                                             int32_t k, int32_t nb, int32_t n_tok) {
  a.w = w;
  a.qx = qx;
  a.dx = dx;
  a.rows = rows;
  a.row_bytes = row_bytes;
  a.k = k;
  a.nb = nb;
  a.n_tok = n_tok;
}

template <int WT>
__global__ __launch_bounds__(64 * kTmWaves) void dmmv_tok_mfma_kernel(const uint8_t *w,
                                                                     const int8_t *qx,
                                                                     const float *dx, int64_t rows,
                                                                     int64_t row_bytes, int32_t k,
                                                                     int32_t nb, int32_t n_tok,
                                                                     const DmmvTokArgs a_in) {
  DmmvTokArgs a = a_in;
  tok_tile_hot(a, w, qx, dx, rows, row_bytes, k, nb, n_tok);
  constexpr int NW = Blk<WT>::NW;
  constexpr int BB = Blk<WT>::BYTES;
  constexpr int KC = Tm<WT>::KC;
  constexpr int QB = Tm<WT>::QB;
  constexpr int RPI = 64 / KC;       // rows per staging load instruction
  constexpr int NL = 16 / RPI;       // staging loads per lane per chunk
  constexpr int WROW = KC * QB + kTmPad;   // LDS bytes per staged weight row
  static_assert(KC % 2 == 0, "blocks are rescaled in pairs");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int nb_pad = (a.nb + KC - 1) / KC * KC;
  const int xrowb = a.k + kTmXPad;         // LDS bytes per staged token
  int8_t *lq = reinterpret_cast<int8_t *>(smem);                                        // [n_tok][k + xpad]
  float *ldx = reinterpret_cast<float *>(smem + static_cast<int64_t>(a.n_tok) * xrowb);  // [nb_pad][8]
  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & 63;
  const int wv = tid >> 6;
  uint8_t *wq = smem + static_cast<int64_t>(a.n_tok) * xrowb + static_cast<int64_t>(nb_pad) * 32 +
                wv * (16 * WROW + KC * 64);                                            // [16][WROW]
  float *wd = reinterpret_cast<float *>(wq + 16 * WROW);                               // [KC][16]

  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * kTmWaves + wv) * 16;
  // staging: lane -> (row row0 + RPI*l + lane / KC, block c0 + lane % KC)
  const int sb = lane % KC;
  const int sr = lane / KC;
  const uint8_t *wrow[NL];
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    int64_t row = row0 + RPI * l + sr;
    row = row < a.rows ? row : a.rows - 1;
    wrow[l] = a.w + row * a.row_bytes;
  }
  uint32_t win[NL][NW];
  uint32_t off[NL];
  auto load_chunk = [&](int c0) {
    int b = c0 + sb;
    b = b < a.nb ? b : a.nb - 1;
#pragma unroll
    for (int l = 0; l < NL; ++l) off[l] = load_window<WT>(wrow[l] + b * BB, win[l]);
  };
  load_chunk(0);

  // the tokens' codes (16-byte pieces; n_tok * k / 16 < 2^32, so the
  // piece -> token division is a 32-bit one) and scales
  if constexpr (WT == ZQ_Q4_0) {
    // Q4_0 takes k in the order of the codes' dwords: a lane's 8 codes are
    // the low nibbles of one dword of a block (k = 4j..4j+3) and then its
    // high nibbles (k = 16+4j..16+4j+3), so each token block is staged with
    // its dwords in the order 0 4 1 5 2 6 3 7.  The int32 sum of the block
    // is the same in any k order.
    const uint32_t nbq = static_cast<uint32_t>(a.n_tok) * static_cast<uint32_t>(a.nb);
    const uint32_t bpr = static_cast<uint32_t>(a.nb);     // blocks per token
    for (uint32_t q = tid; q < nbq; q += 64 * kTmWaves) {
      const uint32_t t = q / bpr, in = q - t * bpr;
      const u32x4 lo = *reinterpret_cast<const u32x4 *>(a.qx + 32 * static_cast<int64_t>(q));
      const u32x4 hi = *reinterpret_cast<const u32x4 *>(a.qx + 32 * static_cast<int64_t>(q) + 16);
      int8_t *dst = lq + t * xrowb + 32 * in;
      *reinterpret_cast<u32x4 *>(dst) = u32x4{lo.x, hi.x, lo.y, hi.y};
      *reinterpret_cast<u32x4 *>(dst + 16) = u32x4{lo.z, hi.z, lo.w, hi.w};
    }
  } else {
    const uint32_t nq = static_cast<uint32_t>(a.n_tok) * static_cast<uint32_t>(a.k / 16);
    const uint32_t qpr = static_cast<uint32_t>(a.k / 16);  // 16-byte pieces per token
    for (uint32_t q = tid; q < nq; q += 64 * kTmWaves) {
      const uint32_t t = q / qpr, in = q - t * qpr;
      *reinterpret_cast<u32x4 *>(lq + t * xrowb + 16 * in) =
          *reinterpret_cast<const u32x4 *>(a.qx + 16 * static_cast<int64_t>(q));
    }
  }
  for (int q = tid; q < nb_pad * 8; q += 64 * kTmWaves) {
    const int b = q >> 3, t = q & 7;
    ldx[q] = (t < a.n_tok && b < a.nb) ? a.dx[static_cast<int64_t>(t) * a.nb + b] : 0.0f;
  }
  __syncthreads();

  const int n = lane & 15;
  const int g = lane >> 4;
  const int hb = g >> 1;   // after the swap: 0 = the pair's first block, 1 = its second
  const int tg = g & 1;    // tokens 4*tg .. 4*tg+3 of that block
  // Token n's row (token 0's for n >= n_tok: those sums are never used).
  // Blocks past nb read up to 32 * (nb_pad - nb) - 32 bytes past the last
  // token's codes, into the scale table that follows; their scales are zero.
  const int8_t *xrow = lq + static_cast<int64_t>(n < a.n_tok ? n : 0) * xrowb + 8 * g;
  // this lane's weight codes inside a staged block: Q8_0 8 bytes, Q4_0 one
  // dword (its low nibbles, then its high nibbles)
  const uint8_t *wl = wq + n * WROW + (WT == ZQ_Q4_0 ? 4 * g : 8 * g);
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int c0 = 0; c0 < a.nb; c0 += KC) {
    // the chunk's blocks into the wave's LDS region: codes (Q4_0: nibbles
    // with the top bit flipped), scale as fp32 (Q4_0: / 16; 0 for the
    // clamped blocks past nb)
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      const uint32_t sel = quant_selector(off[l]);
      uint8_t *dst = wq + (RPI * l + sr) * WROW + sb * QB;
#pragma unroll
      for (int q = 0; q < QB / 16; ++q) {
        u32x4 v;
        v.x = __builtin_amdgcn_perm(win[l][4 * q + 1], win[l][4 * q], sel);
        v.y = __builtin_amdgcn_perm(win[l][4 * q + 2], win[l][4 * q + 1], sel);
        v.z = __builtin_amdgcn_perm(win[l][4 * q + 3], win[l][4 * q + 2], sel);
        v.w = __builtin_amdgcn_perm(win[l][4 * q + 4], win[l][4 * q + 3], sel);
        if constexpr (WT == ZQ_Q4_0) v ^= 0x88888888u;
        // rows are 8-byte aligned (WROW = 8 mod 16)
        *reinterpret_cast<uint2 *>(dst + 16 * q) = uint2{v.x, v.y};
        *reinterpret_cast<uint2 *>(dst + 16 * q + 8) = uint2{v.z, v.w};
      }
      const float d = window_scale(win[l][0], off[l]);
      wd[sb * 16 + RPI * l + sr] = c0 + sb >= a.nb ? 0.0f : WT == ZQ_Q4_0 ? d * 0.0625f : d;
    }
    // the next chunk's windows, in flight during this chunk's arithmetic
    if (c0 + KC < a.nb) load_chunk(c0 + KC);  // uniform
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int bi = 0; bi < KC; bi += 2) {
      const int b = c0 + bi;
      uint2 wa, wb;
      if constexpr (WT == ZQ_Q4_0) {
        const uint32_t da = *reinterpret_cast<const uint32_t *>(wl + bi * QB);
        const uint32_t db = *reinterpret_cast<const uint32_t *>(wl + (bi + 1) * QB);
        wa = uint2{(da << 4) & 0xF0F0F0F0u, da & 0xF0F0F0F0u};
        wb = uint2{(db << 4) & 0xF0F0F0F0u, db & 0xF0F0F0F0u};
      } else {
        wa = *reinterpret_cast<const uint2 *>(wl + bi * QB);
        wb = *reinterpret_cast<const uint2 *>(wl + (bi + 1) * QB);
      }
      const uint2 xa = *reinterpret_cast<const uint2 *>(xrow + 32 * b);
      const uint2 xb = *reinterpret_cast<const uint2 *>(xrow + 32 * (b + 1));
      const float4 dx4 = *reinterpret_cast<const float4 *>(ldx + 8 * (b + hb) + 4 * tg);
      const float dw = wd[(bi + hb) * 16 + n];
      const i32x4 z = {0, 0, 0, 0};
      i32x4 sa = __builtin_amdgcn_mfma_i32_16x16x32_i8(
          static_cast<int64_t>((static_cast<uint64_t>(xa.y) << 32) | xa.x),
          static_cast<int64_t>((static_cast<uint64_t>(wa.y) << 32) | wa.x), z, 0, 0, 0);
      i32x4 sb2 = __builtin_amdgcn_mfma_i32_16x16x32_i8(
          static_cast<int64_t>((static_cast<uint64_t>(xb.y) << 32) | xb.x),
          static_cast<int64_t>((static_cast<uint64_t>(wb.y) << 32) | wb.x), z, 0, 0, 0);
      int32_t s[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int32_t u = sa[r], v = sb2[r];
        swap32_i(u, v);   // u: lanes 0..31 block b, lanes 32..63 block b + 1
        s[r] = u;
      }
      acc[0] = __builtin_fmaf(dx4.x * dw, static_cast<float>(s[0]), acc[0]);
      acc[1] = __builtin_fmaf(dx4.y * dw, static_cast<float>(s[1]), acc[1]);
      acc[2] = __builtin_fmaf(dx4.z * dw, static_cast<float>(s[2]), acc[2]);
      acc[3] = __builtin_fmaf(dx4.w * dw, static_cast<float>(s[3]), acc[3]);
    }
    __builtin_amdgcn_wave_barrier();
  }
  // lanes 0..31 add the odd blocks' sums held by lanes 32..63
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float u = acc[r], v = acc[r];
    swap32(u, v);   // v: lanes 0..31 hold lanes 32..63 of acc
    acc[r] += v;
  }
  if (g < 2 && row0 + n < a.rows) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * g + r;
      if (t < a.n_tok) {
        float *yp = a.y + static_cast<int64_t>(t) * a.rows + row0 + n;
        *yp = (a.flags & ZQ_ACCUMULATE) ? *yp + acc[r] : acc[r];
      }
    }
  }
}

template <int WT>
int launch_tm(const DmmvTokArgs &a, hipStream_t stream) {
  const int64_t rows_per_wg = 16 * kTmWaves;
  const unsigned grid = static_cast<unsigned>((a.rows + rows_per_wg - 1) / rows_per_wg);
  hipLaunchKernelGGL((dmmv_tok_mfma_kernel<WT>), dim3(grid), dim3(64 * kTmWaves),
                     tm_lds_bytes(WT, a.n_tok, a.k), stream, a.w, a.qx, a.dx, a.rows, a.row_bytes,
                     a.k, a.nb, a.n_tok, a);
  ZQ_LAUNCH_CHECK();
  return ZQ_OK;
}

// ---------------------------------------------------------------------------
// Tile form on the matrix cores for matrices too short for the tall form
// (fewer than 65 536 rows, e.g. 4096 x 4096): one workgroup of 16 waves per
// 16 rows and rows of up to 128 blocks.  Wave w reads row w whole (the
// lanes on consecutive blocks, as the single-token DMMV reads a row: split
// over several waves, a row reads far slower) into the workgroup's LDS tile,
// and with it the tokens' codes of its chunk (8 bytes per lane and block,
// straight from global memory); after one barrier wave w takes KC-block
// chunk w of all 16 rows on the matrix cores.  The waves' partial sums meet
// in LDS and 128 threads add them in wave order and store.
constexpr int kTtWaves = 16;

typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) const u32x2v g_u32x2;

// Tile geometry: codes [16][nb_pad*QB + 16] (a row stride of an odd number
// of 16-byte units puts the 16 rows of a read in different banks), scales
// [16][nb_pad + 1] fp32, the tokens' scales [nb_pad][8], partials
// [16][32][4].
struct TtLayout {
  int64_t nb_pad, crow, srow, scales, ldx, red, bytes;
  __host__ __device__ TtLayout(int wtype, int32_t nb) {
    const int qb = wtype == ZQ_Q4_0 ? Tm<ZQ_Q4_0>::QB : Tm<ZQ_Q8_0>::QB;
    const int kc = Tm<ZQ_Q4_0>::KC;
    nb_pad = (nb + kc - 1) / kc * kc;
    crow = nb_pad * qb + 16;
    srow = nb_pad + 1;
    scales = 16 * crow;
    ldx = scales + 16 * srow * 4;
    red = ldx + nb_pad * 32;
    bytes = red + kTtWaves * 32 * 4 * 4;
  }
};

template <int WT, int BPL>
__global__ __launch_bounds__(64 * kTtWaves) void dmmv_tok_tile_kernel(const uint8_t *w,
                                                                     const int8_t *qx,
                                                                     const float *dx, int64_t rows,
                                                                     int64_t row_bytes, int32_t k,
                                                                     int32_t nb, int32_t n_tok,
                                                                     const DmmvTokArgs a_in) {
  DmmvTokArgs a = a_in;
  tok_tile_hot(a, w, qx, dx, rows, row_bytes, k, nb, n_tok);
  constexpr int NW = Blk<WT>::NW;
  constexpr int BB = Blk<WT>::BYTES;
  constexpr int KC = Tm<WT>::KC;
  constexpr int QB = Tm<WT>::QB;
  static_assert(KC % 2 == 0, "blocks are rescaled in pairs");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const TtLayout T(WT, a.nb);
  const int nb_pad = static_cast<int>(T.nb_pad);
  const int n_chunks = nb_pad / KC;
  const int W = n_chunks < kTtWaves ? n_chunks : kTtWaves;   // waves with a chunk
  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & 63;
  const int wv = tid >> 6;
  uint8_t *tq = smem;                                               // [16][crow]
  float *ts = reinterpret_cast<float *>(smem + T.scales);           // [16][srow]
  float *ldx = reinterpret_cast<float *>(smem + T.ldx);             // [nb_pad][8]
  float *red = reinterpret_cast<float *>(smem + T.red);             // [16][32][4]
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * 16;
  // (nb <= 128: at most 16 chunks, so wave wv has chunk wv or none)
  const int c0 = wv * KC;
  const bool has_chunk = wv < n_chunks;   // uniform over the wave
  const int n = lane & 15;
  const int g = lane >> 4;
  const int hb = g >> 1;
  const int tg = g & 1;
  // this wave's tokens' codes (token n's for k = 8g..8g+7 of each block of
  // its chunk; token 0's for n >= n_tok, whose sums take zero scales),
  // requested with the weights
  const int8_t *xg = a.qx + static_cast<int64_t>(n < a.n_tok ? n : 0) * a.k + 8 * g;
  u32x2v x[KC];
  if (has_chunk) {
#pragma unroll
    for (int bi = 0; bi < KC; ++bi) {
      const int bx = c0 + bi < a.nb ? c0 + bi : a.nb - 1;
      x[bi] = *(const g_u32x2 *)(xg + 32 * bx);
    }
  }

  // 1. wave wv reads row row0 + wv: lane j takes blocks j, j + 64, ...
  {
    int64_t row = row0 + wv;
    row = row < a.rows ? row : a.rows - 1;
    const uint8_t *wr = a.w + row * a.row_bytes;
    uint32_t win[BPL][NW];
    uint32_t off[BPL];
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      int b = lane + 64 * i;
      b = b < a.nb ? b : a.nb - 1;
      off[i] = load_window<WT>(wr + b * BB, win[i]);
    }
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      const int b = lane + 64 * i;
      if (b < nb_pad) {
        const uint32_t sel = quant_selector(off[i]);
        uint8_t *dst = tq + wv * T.crow + b * QB;
#pragma unroll
        for (int q = 0; q < QB / 16; ++q) {
          u32x4 v;
          v.x = __builtin_amdgcn_perm(win[i][4 * q + 1], win[i][4 * q], sel);
          v.y = __builtin_amdgcn_perm(win[i][4 * q + 2], win[i][4 * q + 1], sel);
          v.z = __builtin_amdgcn_perm(win[i][4 * q + 3], win[i][4 * q + 2], sel);
          v.w = __builtin_amdgcn_perm(win[i][4 * q + 4], win[i][4 * q + 3], sel);
          if constexpr (WT == ZQ_Q4_0) v ^= 0x88888888u;
          *reinterpret_cast<u32x4 *>(dst + 16 * q) = v;
        }
        const float d = window_scale(win[i][0], off[i]);
        ts[wv * T.srow + b] = b >= a.nb ? 0.0f : WT == ZQ_Q4_0 ? d * 0.0625f : d;
      }
    }
  }
  for (int q = tid; q < nb_pad * 8; q += 64 * kTtWaves) {
    const int b = q >> 3, t = q & 7;
    ldx[q] = (t < a.n_tok && b < a.nb) ? a.dx[static_cast<int64_t>(t) * a.nb + b] : 0.0f;
  }
  __syncthreads();

  // 2. wave wv: chunk wv of all 16 rows
  const int qoff = WT == ZQ_Q4_0 ? 8 * (g & 1) : 8 * g;
  const int shl = WT == ZQ_Q4_0 ? (1 - (g >> 1)) * 4 : 0;
  const uint8_t *wl = tq + n * T.crow + qoff;
  const float *wsl = ts + n * T.srow;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (has_chunk) {
#pragma unroll
    for (int bi = 0; bi < KC; bi += 2) {
      const int b = c0 + bi;
      uint2 wa = *reinterpret_cast<const uint2 *>(wl + b * QB);
      uint2 wb = *reinterpret_cast<const uint2 *>(wl + (b + 1) * QB);
      if constexpr (WT == ZQ_Q4_0) {
        wa.x = (wa.x << shl) & 0xF0F0F0F0u;
        wa.y = (wa.y << shl) & 0xF0F0F0F0u;
        wb.x = (wb.x << shl) & 0xF0F0F0F0u;
        wb.y = (wb.y << shl) & 0xF0F0F0F0u;
      }
      const float4 dx4 = *reinterpret_cast<const float4 *>(ldx + 8 * (b + hb) + 4 * tg);
      const float dw = wsl[b + hb];
      const i32x4 z = {0, 0, 0, 0};
      i32x4 sa = __builtin_amdgcn_mfma_i32_16x16x32_i8(
          static_cast<int64_t>((static_cast<uint64_t>(x[bi].y) << 32) | x[bi].x),
          static_cast<int64_t>((static_cast<uint64_t>(wa.y) << 32) | wa.x), z, 0, 0, 0);
      i32x4 sb2 = __builtin_amdgcn_mfma_i32_16x16x32_i8(
          static_cast<int64_t>((static_cast<uint64_t>(x[bi + 1].y) << 32) | x[bi + 1].x),
          static_cast<int64_t>((static_cast<uint64_t>(wb.y) << 32) | wb.x), z, 0, 0, 0);
      int32_t s4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int32_t u = sa[r], v = sb2[r];
        swap32_i(u, v);   // u: lanes 0..31 block b, lanes 32..63 block b + 1
        s4[r] = u;
      }
      acc[0] = __builtin_fmaf(dx4.x * dw, static_cast<float>(s4[0]), acc[0]);
      acc[1] = __builtin_fmaf(dx4.y * dw, static_cast<float>(s4[1]), acc[1]);
      acc[2] = __builtin_fmaf(dx4.z * dw, static_cast<float>(s4[2]), acc[2]);
      acc[3] = __builtin_fmaf(dx4.w * dw, static_cast<float>(s4[3]), acc[3]);
    }
  }
  // 3. this wave's partials: lanes 0..31 add the odd blocks' sums of lanes
  // 32..63 and leave (token 4g + r, row n) in LDS; then the sum over the
  // waves that had a chunk
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float u = acc[r], v = acc[r];
    swap32(u, v);
    acc[r] += v;
  }
  if (wv < W && lane < 32) {
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(wv * 32 + lane) * 4 + r] = acc[r];
  }
  __syncthreads();
  if (tid < 128) {
    const int L = tid & 31, r = tid >> 5;
    const int t = 4 * (L >> 4) + r;
    const int64_t row = row0 + (L & 15);
    float sum = 0.0f;
    for (int w = 0; w < W; ++w) sum += red[(w * 32 + L) * 4 + r];
    if (t < a.n_tok && row < a.rows) {
      float *yp = a.y + static_cast<int64_t>(t) * a.rows + row;
      *yp = (a.flags & ZQ_ACCUMULATE) ? *yp + sum : sum;
    }
  }
}

template <int WT>
int launch_tt(const DmmvTokArgs &a, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>((a.rows + 15) / 16);
  const size_t lds = static_cast<size_t>(TtLayout(WT, a.nb).bytes);
  if (a.nb <= 64)
    hipLaunchKernelGGL((dmmv_tok_tile_kernel<WT, 1>), dim3(grid), dim3(64 * kTtWaves), lds, stream,
                       a.w, a.qx, a.dx, a.rows, a.row_bytes, a.k, a.nb, a.n_tok, a);
  else
    hipLaunchKernelGGL((dmmv_tok_tile_kernel<WT, 2>), dim3(grid), dim3(64 * kTtWaves), lds, stream,
                       a.w, a.qx, a.dx, a.rows, a.row_bytes, a.k, a.nb, a.n_tok, a);
  ZQ_LAUNCH_CHECK();
  return ZQ_OK;
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
  hipLaunchKernelGGL((dmmv_tok_kernel<WT, LPR, BPL, RB, T>), dim3(grid), dim3(256), 0, stream, a.w,
                     a.qx, a.dx, a.rows, a.row_bytes, a.n_groups, a.k, a.nb, a);
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

bool dmmv_tok_mfma_fits(int wtype, int64_t rows, int32_t k, int32_t n_tok) {
  // tall matrices with three to eight tokens (at two the vector units'
  // dot products are faster; the kernel keeps real tokens in lanes 0..31),
  // the LDS of a launch within 64 KB
  return n_tok >= 3 && n_tok <= 8 && rows >= 65536 && tm_lds_bytes(wtype, n_tok, k) <= 64 * 1024;
}

// Shorter matrices: the tile form where it measured faster than the vector
// form -- five to eight tokens, rows of 64 to 128 blocks, at least 8 M
// weights (4096 x 4096 at 8 tokens: 6.8 against 7.4 us; at 3 tokens, or
// 1024 x 2048, or 20000 x 1024, the vector form is faster) -- with its LDS
// within 64 KB.
bool dmmv_tok_tile_fits(int wtype, int64_t rows, int32_t k, int32_t n_tok) {
  const int32_t nb = k / 32;
  return n_tok >= 5 && n_tok <= 8 && rows < 65536 && nb >= 64 && nb <= 128 &&
         rows * k >= (int64_t(8) << 20) && TtLayout(wtype, nb).bytes <= 64 * 1024;
}

int launch_dmmv_tok(int wtype, DmmvTokArgs a, hipStream_t stream) {
  if (a.rows == 0 || a.n_tok == 0) return ZQ_OK;
  a.row_bytes = static_cast<int64_t>(a.nb) * (wtype == ZQ_Q4_0 ? 18 : 34);
  if (dmmv_tok_mfma_fits(wtype, a.rows, a.k, a.n_tok)) {
    return wtype == ZQ_Q4_0 ? launch_tm<ZQ_Q4_0>(a, stream) : launch_tm<ZQ_Q8_0>(a, stream);
  }
  if (dmmv_tok_tile_fits(wtype, a.rows, a.k, a.n_tok)) {
    return wtype == ZQ_Q4_0 ? launch_tt<ZQ_Q4_0>(a, stream) : launch_tt<ZQ_Q8_0>(a, stream);
  }
  if (wtype == ZQ_Q4_0) return launch_tw<ZQ_Q4_0>(a, stream);
  return launch_tw<ZQ_Q8_0>(a, stream);
}

}  // namespace zq
