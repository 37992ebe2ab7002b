// zq_api.hip -- the extern "C" boundary of libzq: argument checks, then
// launches on the caller's stream.  Every check runs before any launch, so a
// rejected call writes nothing.
#include <atomic>
#include <cstring>

#include "zq_common.h"
#include "zq_f32in.h"
#include "zq_float.h"
#include "zq_internal.h"
#include "zq_moe_tok.h"

namespace {

constexpr int kMaxDevices = 64;
// Per-device capability cache: 0 unknown, 1 gfx950, -1 other.
std::atomic<int> g_dev_ok[kMaxDevices];

int check_device(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return ZQ_EDEVICE;
  int v = g_dev_ok[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ZQ_EDEVICE;
    v = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    g_dev_ok[dev].store(v, std::memory_order_relaxed);
  }
  return v == 1 ? ZQ_OK : ZQ_EDEVICE;
}

int check_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return ZQ_EDEVICE;
  return check_device(dev);
}

inline bool al(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline bool k_ok(int64_t k) { return k > 0 && k % 32 == 0 && k / 32 <= (int64_t(1) << 30); }
inline hipStream_t S(void *s) { return static_cast<hipStream_t>(s); }
inline int64_t block_bytes(int wtype) { return wtype == ZQ_Q4_0 ? 18 : (wtype == ZQ_Q8_0 ? 34 : -1); }
inline bool is_k(int wtype) { return wtype == ZQ_Q4_K || wtype == ZQ_Q5_K || wtype == ZQ_Q6_K; }

// Bytes of one rows x k matrix in wtype, or -1 for an unknown type.
inline int64_t matrix_bytes(int wtype, int64_t rows, int64_t k) {
  if (wtype == ZQ_Q4_0 || wtype == ZQ_Q8_0) return rows * (k / 32) * block_bytes(wtype);
  if (!is_k(wtype)) return -1;
  const int64_t sbb = wtype == ZQ_Q4_K ? 144 : (wtype == ZQ_Q5_K ? 176 : 210);
  return rows * (k / 256) * sbb;
}

// An expert bank's alignment: K-quant units are read with 16-byte loads.
inline bool bank_al(int wtype, const void *p, int64_t stride) {
  return is_k(wtype) ? (al(p, 16) && stride % 16 == 0) : (al(p, 4) && stride % 2 == 0);
}

// The fused gate/up pass (both formats) and the d_model it serves.
inline bool gate_up_fits(int wtype, int64_t d_model) {
  return is_k(wtype) ? zq::moe_gate_up_k_fits(d_model) : zq::moe_gate_up_fits(d_model);
}
inline int launch_gate_up(int wtype, const zq::MoeGateUpArgs &a, hipStream_t s) {
  return is_k(wtype) ? zq::launch_moe_gate_up_k(wtype, a, s) : zq::launch_moe_gate_up(wtype, a, s);
}

#define ZQ_REQUIRE(cond, code) \
  do {                         \
    if (!(cond)) return (code); \
  } while (0)

constexpr size_t kAlign = 256;
inline size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct MoeWorkspace {
  size_t qx, dx, sx, gu, qh, dh, sh, total;
};

MoeWorkspace moe_layout(int64_t d_model, int64_t d_ff, int32_t n_sel) {
  MoeWorkspace w;
  size_t off = 0;
  w.qx = off; off += round_up(static_cast<size_t>(d_model));
  w.dx = off; off += round_up(static_cast<size_t>(d_model / 32) * 4);
  w.sx = off; off += round_up(static_cast<size_t>(d_model / 32) * 4);
  w.gu = off; off += round_up(static_cast<size_t>(n_sel) * 2 * d_ff * 4);
  w.qh = off; off += round_up(static_cast<size_t>(n_sel) * d_ff);
  w.dh = off; off += round_up(static_cast<size_t>(n_sel) * (d_ff / 32) * 4);
  w.sh = off; off += round_up(static_cast<size_t>(n_sel) * (d_ff / 32) * 4);
  w.total = off;
  return w;
}

int dmmv_common(int wtype, const void *w, int64_t rows, int64_t k, const int8_t *qx,
                const float *dx, const int32_t *sx, float *y, uint32_t flags, void *stream) {
  ZQ_REQUIRE(w && qx && dx && y, ZQ_ENULL);
  ZQ_REQUIRE(rows >= 0 && k_ok(k), ZQ_EINVAL);
  ZQ_REQUIRE((flags & ~uint32_t(ZQ_ACCUMULATE)) == 0, ZQ_EINVAL);
  ZQ_REQUIRE(al(w, 4) && al(qx, 16) && al(dx, 4) && al(y, 4) && al(sx, 4), ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  zq::DmmvArgs a{};
  a.w = static_cast<const uint8_t *>(w);
  a.qx = qx;
  a.dx = dx;
  a.sx = wtype == ZQ_Q4_0 ? sx : nullptr;
  a.y = y;
  a.rows = rows;
  a.nb = static_cast<int32_t>(k / 32);
  a.flags = flags;
  return zq::launch_dmmv(wtype, zq::MODE_PLAIN, a, S(stream));
}

// The K-quant DMMV and its isums hook share the checks: k a multiple of
// 256, w 16-byte aligned (super-blocks of 144 and 176 bytes stay 16-byte
// aligned; the 210-byte Q6_K ones are read through dword windows).
int dmmv_k_common(int wtype, const void *w, int64_t rows, int64_t k, const int8_t *qx,
                  const float *dx, const int32_t *sx, float *y, int32_t *isums, uint32_t flags,
                  void *stream) {
  ZQ_REQUIRE(wtype == ZQ_Q4_K || wtype == ZQ_Q5_K || wtype == ZQ_Q6_K, ZQ_EINVAL);
  ZQ_REQUIRE(w && qx && (isums || (dx && y)), ZQ_ENULL);
  ZQ_REQUIRE(rows >= 0 && k_ok(k) && k % 256 == 0, ZQ_EINVAL);
  ZQ_REQUIRE((flags & ~uint32_t(ZQ_ACCUMULATE)) == 0, ZQ_EINVAL);
  ZQ_REQUIRE(al(w, 16) && al(qx, 16) && al(dx, 4) && al(y, 4) && al(sx, 4) && al(isums, 4),
             ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  zq::DmmvArgs a{};
  a.w = static_cast<const uint8_t *>(w);
  a.qx = qx;
  // the isums hook has no scales: qx's bytes stand in for dx (k bytes cover
  // the k/32 fp32 values), their values only feed the unused row partials
  a.dx = isums ? reinterpret_cast<const float *>(qx) : dx;
  a.sx = wtype == ZQ_Q6_K ? nullptr : sx;
  a.y = y;
  a.isums = isums;
  a.rows = rows;
  a.nb = static_cast<int32_t>(k / 32);
  a.flags = flags;
  return zq::launch_dmmv_k(wtype, isums ? zq::MODE_ISUMS : zq::MODE_PLAIN, a, S(stream));
}

// Expert-indexed K-quant DMMV (gather / weighted sum); id_base is
// subtracted from every id (a bank that holds experts id_base.. only).
int dmmv_moe_k(int wtype, const void *bank, int64_t n_experts, int64_t expert_stride_bytes,
               int64_t rows, int64_t k, const int32_t *ids, const float *wts, int32_t n_sel,
               const int8_t *qx, const float *dx, const int32_t *sx, int64_t x_stride, int mode,
               float *y, uint32_t flags, int32_t *dev_status, int32_t id_base, hipStream_t stream) {
  const int64_t sbb = wtype == ZQ_Q4_K ? 144 : (wtype == ZQ_Q5_K ? 176 : 210);
  ZQ_REQUIRE(mode == ZQ_MOE_GATHER || mode == ZQ_MOE_WEIGHTED_SUM, ZQ_EINVAL);
  ZQ_REQUIRE(bank && ids && qx && dx && y, ZQ_ENULL);
  ZQ_REQUIRE(mode == ZQ_MOE_GATHER || wts, ZQ_ENULL);
  ZQ_REQUIRE(n_experts >= 1 && n_experts <= INT32_MAX && rows >= 0 && k_ok(k) && k % 256 == 0,
             ZQ_EINVAL);
  ZQ_REQUIRE(n_sel >= 0 && n_sel <= 65535, ZQ_EINVAL);
  ZQ_REQUIRE(x_stride >= 0 && x_stride % 32 == 0 && (x_stride == 0 || x_stride >= k), ZQ_EINVAL);
  ZQ_REQUIRE(expert_stride_bytes >= rows * (k / 256) * sbb, ZQ_EINVAL);
  if (mode == ZQ_MOE_GATHER) {
    ZQ_REQUIRE(flags == 0, ZQ_EINVAL);
  } else {
    ZQ_REQUIRE((flags & ~uint32_t(ZQ_ACCUMULATE)) == 0, ZQ_EINVAL);
  }
  ZQ_REQUIRE(al(bank, 16) && expert_stride_bytes % 16 == 0 && al(ids, 4) && al(wts, 4) &&
                 al(qx, 16) && al(dx, 4) && al(sx, 4) && al(y, 4) && al(dev_status, 4),
             ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  zq::DmmvArgs a{};
  a.w = static_cast<const uint8_t *>(bank);
  a.qx = qx;
  a.dx = dx;
  a.sx = wtype == ZQ_Q6_K ? nullptr : sx;
  a.y = y;
  a.ids = ids;
  a.wts = wts;
  a.status = dev_status;
  a.rows = rows;
  a.expert_stride = expert_stride_bytes;
  a.x_stride = x_stride;
  a.nb = static_cast<int32_t>(k / 32);
  a.n_experts = static_cast<int32_t>(n_experts);
  a.n_sel = n_sel;
  a.flags = flags;
  a.id_base = id_base;
  return zq::launch_dmmv_k(wtype, mode == ZQ_MOE_GATHER ? zq::MODE_GATHER : zq::MODE_WEIGHTED, a,
                           stream);
}

}  // namespace

extern "C" {

int zq_version(void) { return 1; }

const char *zq_strerror(int status) {
  switch (status) {
    case ZQ_OK: return "ok";
    case ZQ_EINVAL: return "invalid argument (size, k % 32, flags, type, mode or range)";
    case ZQ_ENULL: return "a required pointer is NULL";
    case ZQ_EALIGN: return "misaligned pointer or stride";
    case ZQ_ERANGE: return "expert id out of range";
    case ZQ_EDEVICE: return "current device is not a gfx950 GPU";
    case ZQ_ELAUNCH: return "kernel launch failed";
    default: return "unknown zq status";
  }
}

int zq_device_check(int device) { return check_device(device); }

int zq_quantize_act(const float *x, int64_t n_tok, int64_t k, int64_t x_stride, int8_t *qx,
                    float *dx, int32_t *sx, void *stream) {
  ZQ_REQUIRE(x && qx && dx, ZQ_ENULL);
  ZQ_REQUIRE(n_tok >= 0 && k_ok(k) && x_stride >= k, ZQ_EINVAL);
  ZQ_REQUIRE(n_tok * (k / 32) <= (int64_t(1) << 31), ZQ_EINVAL);
  ZQ_REQUIRE(al(x, 16) && x_stride % 4 == 0 && al(qx, 16) && al(dx, 4) && al(sx, 4), ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  return zq::launch_quantize_act(x, n_tok, k, x_stride, qx, dx, sx, S(stream));
}

int zq_dmmv_q8_0(const void *w, int64_t rows, int64_t k, const int8_t *qx, const float *dx,
                 float *y, uint32_t flags, void *stream) {
  return dmmv_common(ZQ_Q8_0, w, rows, k, qx, dx, nullptr, y, flags, stream);
}

int zq_dmmv_q4_0(const void *w, int64_t rows, int64_t k, const int8_t *qx, const float *dx,
                 const int32_t *sx, float *y, uint32_t flags, void *stream) {
  return dmmv_common(ZQ_Q4_0, w, rows, k, qx, dx, sx, y, flags, stream);
}

int zq_dmmv_q4_k(const void *w, int64_t rows, int64_t k, const int8_t *qx, const float *dx,
                 const int32_t *sx, float *y, uint32_t flags, void *stream) {
  return dmmv_k_common(ZQ_Q4_K, w, rows, k, qx, dx, sx, y, nullptr, flags, stream);
}

int zq_dmmv_q5_k(const void *w, int64_t rows, int64_t k, const int8_t *qx, const float *dx,
                 const int32_t *sx, float *y, uint32_t flags, void *stream) {
  return dmmv_k_common(ZQ_Q5_K, w, rows, k, qx, dx, sx, y, nullptr, flags, stream);
}

int zq_dmmv_q6_k(const void *w, int64_t rows, int64_t k, const int8_t *qx, const float *dx,
                 float *y, uint32_t flags, void *stream) {
  return dmmv_k_common(ZQ_Q6_K, w, rows, k, qx, dx, nullptr, y, nullptr, flags, stream);
}

int zq_dmmv_tokens(int wtype, const void *w, int64_t rows, int64_t k, const int8_t *qx,
                   const float *dx, const int32_t *sx, int32_t n_tok, float *y, uint32_t flags,
                   void *stream) {
  ZQ_REQUIRE(block_bytes(wtype) > 0, ZQ_EINVAL);
  ZQ_REQUIRE(w && qx && dx && y, ZQ_ENULL);
  ZQ_REQUIRE(rows >= 0 && k_ok(k) && k <= (int64_t(1) << 30), ZQ_EINVAL);
  ZQ_REQUIRE(n_tok >= 1 && n_tok <= 8, ZQ_EINVAL);
  ZQ_REQUIRE((flags & ~uint32_t(ZQ_ACCUMULATE)) == 0, ZQ_EINVAL);
  ZQ_REQUIRE(al(w, 4) && al(qx, 16) && al(dx, 4) && al(y, 4) && al(sx, 4), ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  zq::DmmvTokArgs a{};
  a.w = static_cast<const uint8_t *>(w);
  a.qx = qx;
  a.dx = dx;
  a.sx = wtype == ZQ_Q4_0 ? sx : nullptr;
  a.y = y;
  a.rows = rows;
  a.k = static_cast<int32_t>(k);
  a.nb = static_cast<int32_t>(k / 32);
  a.n_tok = n_tok;
  a.flags = flags;
  return zq::launch_dmmv_tok(wtype, a, S(stream));
}

int zq_dmmv_f32(int wtype, const void *w, int64_t rows, int64_t k, const float *x, float *y,
                uint32_t flags, int8_t *qx_out, float *dx_out, int32_t *sx_out, void *stream) {
  ZQ_REQUIRE(block_bytes(wtype) > 0, ZQ_EINVAL);
  ZQ_REQUIRE(w && x && y, ZQ_ENULL);
  ZQ_REQUIRE(rows >= 0 && k_ok(k) && k <= 16384, ZQ_EINVAL);
  ZQ_REQUIRE((flags & ~uint32_t(ZQ_ACCUMULATE)) == 0, ZQ_EINVAL);
  ZQ_REQUIRE(al(w, 4) && al(x, 16) && al(y, 4) && al(qx_out, 4) && al(dx_out, 4) && al(sx_out, 4),
             ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  zq::DmmvF32Args a{};
  a.w = static_cast<const uint8_t *>(w);
  a.x = x;
  a.y = y;
  a.qx_out = qx_out;
  a.dx_out = dx_out;
  a.sx_out = sx_out;
  a.rows = rows;
  a.k = static_cast<int32_t>(k);
  a.nb = static_cast<int32_t>(k / 32);
  a.flags = flags;
  return zq::launch_dmmv_f32x(wtype, a, S(stream));
}

int zq_dmmv_k_f32(int wtype, const void *w, int64_t rows, int64_t k, const float *x, float *y,
                  uint32_t flags, int8_t *qx_out, float *dx_out, int32_t *sx_out, void *stream) {
  ZQ_REQUIRE(is_k(wtype), ZQ_EINVAL);
  ZQ_REQUIRE(w && x && y, ZQ_ENULL);
  ZQ_REQUIRE(rows >= 0 && k >= 256 && k % 256 == 0 && k <= 16384, ZQ_EINVAL);
  ZQ_REQUIRE((flags & ~uint32_t(ZQ_ACCUMULATE)) == 0, ZQ_EINVAL);
  ZQ_REQUIRE(al(w, 16) && al(x, 16) && al(y, 4) && al(qx_out, 4) && al(dx_out, 4) &&
                 al(sx_out, 4),
             ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  zq::DmmvKF32Args a{};
  a.w = static_cast<const uint8_t *>(w);
  a.x = x;
  a.y = y;
  a.qx_out = qx_out;
  a.dx_out = dx_out;
  a.sx_out = sx_out;
  a.rows = rows;
  a.k = static_cast<int32_t>(k);
  a.nb = static_cast<int32_t>(k / 32);
  a.flags = flags;
  return zq::launch_dmmv_k_f32(wtype, a, S(stream));
}

int zq_dmmv_tokens_f32(int wtype, const void *w, int64_t rows, int64_t k, const float *x,
                       int32_t n_tok, int8_t *qx, float *dx, int32_t *sx, float *y, uint32_t flags,
                       void *stream) {
  ZQ_REQUIRE(block_bytes(wtype) > 0, ZQ_EINVAL);
  ZQ_REQUIRE(w && x && qx && dx && sx && y, ZQ_ENULL);
  ZQ_REQUIRE(rows >= 0 && k_ok(k) && k <= (int64_t(1) << 30), ZQ_EINVAL);
  ZQ_REQUIRE(n_tok >= 1 && n_tok <= 8, ZQ_EINVAL);
  ZQ_REQUIRE(int64_t(n_tok) * (k / 32) <= (int64_t(1) << 31), ZQ_EINVAL);
  ZQ_REQUIRE((flags & ~uint32_t(ZQ_ACCUMULATE)) == 0, ZQ_EINVAL);
  ZQ_REQUIRE(al(w, 4) && al(x, 16) && al(qx, 16) && al(dx, 4) && al(sx, 4) && al(y, 4),
             ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  // every workgroup of every multi-token form needs all the tokens' codes:
  // quantizing inside the product's launch would redo the whole
  // quantization in each workgroup, so the quantizer runs first
  const int rc = zq::launch_quantize_act(x, n_tok, k, k, qx, dx, sx, S(stream));
  if (rc != ZQ_OK) return rc;
  zq::DmmvTokArgs a{};
  a.w = static_cast<const uint8_t *>(w);
  a.qx = qx;
  a.dx = dx;
  a.sx = wtype == ZQ_Q4_0 ? sx : nullptr;
  a.y = y;
  a.rows = rows;
  a.k = static_cast<int32_t>(k);
  a.nb = static_cast<int32_t>(k / 32);
  a.n_tok = n_tok;
  a.flags = flags;
  return zq::launch_dmmv_tok(wtype, a, S(stream));
}

int zq_dmmv_isums(int wtype, const void *w, int64_t rows, int64_t k, const int8_t *qx,
                  const int32_t *sx, int32_t *isums, void *stream) {
  if (wtype == ZQ_Q4_K || wtype == ZQ_Q5_K || wtype == ZQ_Q6_K)
    return dmmv_k_common(wtype, w, rows, k, qx, nullptr, sx, nullptr, isums, 0, stream);
  ZQ_REQUIRE(block_bytes(wtype) > 0, ZQ_EINVAL);
  ZQ_REQUIRE(w && qx && isums, ZQ_ENULL);
  ZQ_REQUIRE(rows >= 0 && k_ok(k), ZQ_EINVAL);
  ZQ_REQUIRE(al(w, 4) && al(qx, 16) && al(sx, 4) && al(isums, 4), ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  zq::DmmvArgs a{};
  a.w = static_cast<const uint8_t *>(w);
  a.qx = qx;
  a.sx = wtype == ZQ_Q4_0 ? sx : nullptr;
  a.isums = isums;
  a.rows = rows;
  a.nb = static_cast<int32_t>(k / 32);
  // dx must be readable by the shared inner loop: point it at qx's bytes,
  // which span k bytes >= (k/32)*4 bytes; the value only feeds the unused
  // fp32 partial.
  a.dx = reinterpret_cast<const float *>(qx);
  return zq::launch_dmmv(wtype, zq::MODE_ISUMS, a, S(stream));
}

int zq_dmmv_float(int wtype, const void *w, int64_t rows, int64_t k, const float *x, float *y,
                  uint32_t flags, void *stream) {
  ZQ_REQUIRE(wtype == ZQ_F16 || wtype == ZQ_F32, ZQ_EINVAL);
  ZQ_REQUIRE(w && x && y, ZQ_ENULL);
  ZQ_REQUIRE(rows >= 0 && k > 0 && k % 8 == 0 && k <= 16384, ZQ_EINVAL);
  ZQ_REQUIRE((flags & ~uint32_t(ZQ_ACCUMULATE)) == 0, ZQ_EINVAL);
  ZQ_REQUIRE(al(w, 16) && al(x, 16) && al(y, 4), ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  zq::FloatDmmvArgs a{};
  a.w = static_cast<const uint8_t *>(w);
  a.x = x;
  a.y = y;
  a.rows = rows;
  a.k = static_cast<int32_t>(k);
  a.flags = flags;
  return zq::launch_dmmv_float(wtype, a, S(stream));
}

size_t zq_argmax_workspace_bytes(int64_t n) { return zq::argmax_workspace(n); }

int zq_argmax_f32(const float *y, int64_t n, int32_t *out_idx, void *workspace,
                  size_t workspace_bytes, void *stream) {
  ZQ_REQUIRE(y && out_idx && workspace, ZQ_ENULL);
  ZQ_REQUIRE(n >= 1 && n <= INT32_MAX, ZQ_EINVAL);
  ZQ_REQUIRE(workspace_bytes >= zq::argmax_workspace(n), ZQ_EINVAL);
  ZQ_REQUIRE(al(y, 4) && al(out_idx, 4) && al(workspace, 8), ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  return zq::launch_argmax(y, n, out_idx, workspace, S(stream));
}

size_t zq_dmmv_f32_argmax_workspace_bytes(void) {
  return sizeof(zq::ValIdx) * static_cast<size_t>(zq::kArgmaxMaxParts);
}

int zq_dmmv_f32_argmax(int wtype, const void *w, int64_t rows, int64_t k, const float *x, float *y,
                       int32_t *out_idx, void *workspace, size_t workspace_bytes, void *stream) {
  ZQ_REQUIRE(block_bytes(wtype) > 0, ZQ_EINVAL);
  ZQ_REQUIRE(w && x && y && workspace, ZQ_ENULL);
  ZQ_REQUIRE(rows >= 1 && rows <= INT32_MAX && k_ok(k) && k <= 16384, ZQ_EINVAL);
  ZQ_REQUIRE(workspace_bytes >= zq_dmmv_f32_argmax_workspace_bytes(), ZQ_EINVAL);
  ZQ_REQUIRE(al(w, 4) && al(x, 16) && al(y, 4) && al(out_idx, 4) && al(workspace, 8), ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  zq::DmmvF32Args a{};
  a.w = static_cast<const uint8_t *>(w);
  a.x = x;
  a.y = y;
  a.part = workspace;
  a.out_idx = out_idx;
  a.rows = rows;
  a.k = static_cast<int32_t>(k);
  a.nb = static_cast<int32_t>(k / 32);
  return zq::launch_dmmv_f32x(wtype, a, S(stream));
}

namespace {

// The allocation-free LM-head step keeps its argmax partials (one (logit,
// row) pair per workgroup of the persistent DMMV launch) in this array.  Each
// GPU the library runs on holds its own copy until the process ends.  In host
// code `scratch` names a host-side stand-in, never the device memory: the
// launches take the address hipGetSymbolAddress returns on each device.
constexpr size_t kScratchBytes = sizeof(zq::ValIdx) * static_cast<size_t>(zq::kArgmaxMaxParts);
__device__ __align__(256) unsigned char scratch[kScratchBytes];
std::atomic<void *> g_scratch[kMaxDevices];

// The device address of `scratch` on the current device, looked up once per
// device with that device current (two threads racing here store the same
// address).  nullptr if the runtime cannot resolve it.
void *scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void *p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();  // leave no error behind for the next launch check
      return nullptr;
    }
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

int zq_dmmv_f32_argmax_noalloc(int wtype, const void *w, int64_t rows, int64_t k, const float *x,
                               float *y, int32_t *out_idx, void *stream) {
  static_assert(sizeof(zq::ValIdx) * zq::kArgmaxMaxParts <= kScratchBytes,
                "every partial of the persistent launch fits the scratch array");
  ZQ_REQUIRE(block_bytes(wtype) > 0, ZQ_EINVAL);
  ZQ_REQUIRE(w && x && y && out_idx, ZQ_ENULL);
  ZQ_REQUIRE(rows >= 1 && rows <= INT32_MAX && k_ok(k) && k <= 16384, ZQ_EINVAL);
  ZQ_REQUIRE(al(w, 4) && al(x, 16) && al(y, 4) && al(out_idx, 4), ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  void *part = scratch_on_current_device();
  if (part == nullptr) return ZQ_ELAUNCH;
  zq::DmmvF32Args a{};
  a.w = static_cast<const uint8_t *>(w);
  a.x = x;
  a.y = y;
  a.part = part;  // every slot the final pass reads is written by this call's DMMV launch
  a.out_idx = out_idx;
  a.rows = rows;
  a.k = static_cast<int32_t>(k);
  a.nb = static_cast<int32_t>(k / 32);
  return zq::launch_dmmv_f32x(wtype, a, S(stream));
}

inline bool eps_ok(float eps) { return eps >= 0.0f && eps <= 3.0e38f; }  // finite, not NaN

int zq_rms_norm_quantize(const float *x, const float *norm_w, float eps, int64_t n_tok, int64_t k,
                         int64_t x_stride, int8_t *qx, float *dx, int32_t *sx, float *xn_out,
                         void *stream) {
  ZQ_REQUIRE(x && norm_w && qx && dx, ZQ_ENULL);
  ZQ_REQUIRE(n_tok >= 0 && n_tok <= INT32_MAX && k_ok(k) && k <= (int64_t(1) << 30) &&
                 x_stride >= k && eps_ok(eps),
             ZQ_EINVAL);
  ZQ_REQUIRE(al(x, 16) && x_stride % 4 == 0 && al(norm_w, 16) && al(qx, 16) && al(dx, 4) &&
                 al(sx, 4) && al(xn_out, 16),
             ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  zq::RmsNormArgs a{};
  a.x = x;
  a.w = norm_w;
  a.qx = qx;
  a.dx = dx;
  a.sx = sx;
  a.xn_out = xn_out;
  a.n_tok = n_tok;
  a.x_stride = x_stride;
  a.k = static_cast<int32_t>(k);
  a.eps = eps;
  return zq::launch_rms_norm_quantize(a, S(stream));
}

int zq_rms_norm_dmmv_f32(int wtype, const void *w, int64_t rows, int64_t k, const float *x,
                         const float *norm_w, float eps, float *y, uint32_t flags, int8_t *qx_out,
                         float *dx_out, int32_t *sx_out, float *xn_out, void *stream) {
  ZQ_REQUIRE(block_bytes(wtype) > 0, ZQ_EINVAL);
  ZQ_REQUIRE(w && x && norm_w && y, ZQ_ENULL);
  ZQ_REQUIRE(rows >= 0 && k_ok(k) && k <= 16384 && eps_ok(eps), ZQ_EINVAL);
  ZQ_REQUIRE((flags & ~uint32_t(ZQ_ACCUMULATE)) == 0, ZQ_EINVAL);
  ZQ_REQUIRE(al(w, 4) && al(x, 16) && al(norm_w, 16) && al(y, 4) && al(qx_out, 4) &&
                 al(dx_out, 4) && al(sx_out, 4) && al(xn_out, 16),
             ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  zq::DmmvF32Args a{};
  a.w = static_cast<const uint8_t *>(w);
  a.x = x;
  a.y = y;
  a.qx_out = qx_out;
  a.dx_out = dx_out;
  a.sx_out = sx_out;
  a.norm_w = norm_w;
  a.eps = eps;
  a.xn_out = xn_out;
  a.rows = rows;
  a.k = static_cast<int32_t>(k);
  a.nb = static_cast<int32_t>(k / 32);
  a.flags = flags;
  return zq::launch_dmmv_f32x(wtype, a, S(stream));
}

int zq_rms_norm_dmmv_f32_argmax(int wtype, const void *w, int64_t rows, int64_t k, const float *x,
                                const float *norm_w, float eps, float *y, int32_t *out_idx,
                                void *workspace, size_t workspace_bytes, void *stream) {
  ZQ_REQUIRE(block_bytes(wtype) > 0, ZQ_EINVAL);
  ZQ_REQUIRE(w && x && norm_w && y && workspace, ZQ_ENULL);
  ZQ_REQUIRE(rows >= 1 && rows <= INT32_MAX && k_ok(k) && k <= 16384 && eps_ok(eps), ZQ_EINVAL);
  ZQ_REQUIRE(workspace_bytes >= zq_dmmv_f32_argmax_workspace_bytes(), ZQ_EINVAL);
  ZQ_REQUIRE(al(w, 4) && al(x, 16) && al(norm_w, 16) && al(y, 4) && al(out_idx, 4) &&
                 al(workspace, 8),
             ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  zq::DmmvF32Args a{};
  a.w = static_cast<const uint8_t *>(w);
  a.x = x;
  a.y = y;
  a.part = workspace;
  a.out_idx = out_idx;
  a.norm_w = norm_w;
  a.eps = eps;
  a.rows = rows;
  a.k = static_cast<int32_t>(k);
  a.nb = static_cast<int32_t>(k / 32);
  return zq::launch_dmmv_f32x(wtype, a, S(stream));
}

int zq_moe_route(const float *logits, int32_t n_routed, int32_t top_k, const float *shared_gate,
                 int32_t *ids, float *wts, void *stream) {
  ZQ_REQUIRE(logits && ids && wts, ZQ_ENULL);
  ZQ_REQUIRE(top_k >= 1 && top_k <= 64 && n_routed >= top_k && n_routed <= 1024, ZQ_EINVAL);
  ZQ_REQUIRE(al(logits, 4) && al(ids, 4) && al(wts, 4) && al(shared_gate, 4), ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  return zq::launch_moe_route(logits, n_routed, top_k, shared_gate, ids, wts, S(stream));
}

int zq_dmmv_moe(int wtype, const void *bank, int64_t n_experts, int64_t expert_stride_bytes,
                int64_t rows, int64_t k, const int32_t *ids, const float *wts, int32_t n_sel,
                const int8_t *qx, const float *dx, const int32_t *sx, int64_t x_stride, int mode,
                float *y, uint32_t flags, int32_t *dev_status, void *stream) {
  if (wtype == ZQ_Q4_K || wtype == ZQ_Q5_K || wtype == ZQ_Q6_K)
    return dmmv_moe_k(wtype, bank, n_experts, expert_stride_bytes, rows, k, ids, wts, n_sel, qx,
                      dx, sx, x_stride, mode, y, flags, dev_status, 0, S(stream));
  const int64_t bb = block_bytes(wtype);
  ZQ_REQUIRE(bb > 0, ZQ_EINVAL);
  ZQ_REQUIRE(mode == ZQ_MOE_GATHER || mode == ZQ_MOE_WEIGHTED_SUM, ZQ_EINVAL);
  ZQ_REQUIRE(bank && ids && qx && dx && y, ZQ_ENULL);
  ZQ_REQUIRE(mode == ZQ_MOE_GATHER || wts, ZQ_ENULL);
  ZQ_REQUIRE(n_experts >= 1 && n_experts <= INT32_MAX && rows >= 0 && k_ok(k), ZQ_EINVAL);
  ZQ_REQUIRE(n_sel >= 0 && n_sel <= 65535, ZQ_EINVAL);
  ZQ_REQUIRE(x_stride >= 0 && x_stride % 32 == 0 && (x_stride == 0 || x_stride >= k), ZQ_EINVAL);
  ZQ_REQUIRE(expert_stride_bytes >= rows * (k / 32) * bb && expert_stride_bytes % 2 == 0,
             ZQ_EINVAL);
  if (mode == ZQ_MOE_GATHER) {
    ZQ_REQUIRE(flags == 0, ZQ_EINVAL);
  } else {
    ZQ_REQUIRE((flags & ~uint32_t(ZQ_ACCUMULATE)) == 0, ZQ_EINVAL);
  }
  ZQ_REQUIRE(al(bank, 4) && al(ids, 4) && al(wts, 4) && al(qx, 16) && al(dx, 4) && al(sx, 4) &&
                 al(y, 4) && al(dev_status, 4),
             ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  zq::DmmvArgs a{};
  a.w = static_cast<const uint8_t *>(bank);
  a.qx = qx;
  a.dx = dx;
  a.sx = wtype == ZQ_Q4_0 ? sx : nullptr;
  a.y = y;
  a.ids = ids;
  a.wts = wts;
  a.status = dev_status;
  a.rows = rows;
  a.expert_stride = expert_stride_bytes;
  a.x_stride = x_stride;
  a.nb = static_cast<int32_t>(k / 32);
  a.n_experts = static_cast<int32_t>(n_experts);
  a.n_sel = n_sel;
  a.flags = flags;
  if (mode == ZQ_MOE_WEIGHTED_SUM && x_stride % 32 == 0 && zq::moe_down_fits(n_sel, k)) {
    zq::MoeDownArgs b{};
    b.bank = static_cast<const uint8_t *>(bank);
    b.expert_stride = expert_stride_bytes;
    b.n_experts = static_cast<int32_t>(n_experts);
    b.ids = ids;
    b.wts = wts;
    b.n_sel = n_sel;
    b.qx = qx;
    b.dx = dx;
    b.sx = wtype == ZQ_Q4_0 ? sx : nullptr;
    b.x_stride = x_stride;
    b.k = static_cast<int32_t>(k);
    b.rows = rows;
    b.y = y;
    b.flags = flags;
    b.status = dev_status;
    return zq::launch_moe_down(wtype, b, S(stream));
  }
  return zq::launch_dmmv(wtype, mode == ZQ_MOE_GATHER ? zq::MODE_GATHER : zq::MODE_WEIGHTED, a,
                         S(stream));
}

int zq_moe_gate_up(int wtype, const void *gu_bank, int64_t gu_stride_bytes, int64_t n_experts,
                   int64_t d_model, int64_t d_ff, const int32_t *ids, int32_t n_sel,
                   const float *x, int8_t *qh, float *dh, int32_t *sh, float *h_out,
                   float *gu_out, int32_t *dev_status, void *stream) {
  ZQ_REQUIRE(matrix_bytes(wtype, 1, 256) > 0, ZQ_EINVAL);
  ZQ_REQUIRE(gu_bank && ids && x && qh && dh, ZQ_ENULL);
  ZQ_REQUIRE(n_experts >= 1 && n_experts <= INT32_MAX && k_ok(d_model) && k_ok(d_ff), ZQ_EINVAL);
  ZQ_REQUIRE(gate_up_fits(wtype, d_model) && d_ff <= (int64_t(1) << 30), ZQ_EINVAL);
  ZQ_REQUIRE(n_sel >= 0 && n_sel <= 65535, ZQ_EINVAL);
  ZQ_REQUIRE(gu_stride_bytes >= matrix_bytes(wtype, 2 * d_ff, d_model), ZQ_EINVAL);
  ZQ_REQUIRE(bank_al(wtype, gu_bank, gu_stride_bytes) && al(ids, 4) && al(x, 16) && al(qh, 16) &&
                 al(dh, 4) && al(sh, 4) && al(h_out, 16) && al(gu_out, 4) && al(dev_status, 4),
             ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  zq::MoeGateUpArgs a{};
  a.bank = static_cast<const uint8_t *>(gu_bank);
  a.expert_stride = gu_stride_bytes;
  a.n_experts = static_cast<int32_t>(n_experts);
  a.ids = ids;
  a.n_sel = n_sel;
  a.x = x;
  a.k = static_cast<int32_t>(d_model);
  a.d_ff = static_cast<int32_t>(d_ff);
  a.qh = qh;
  a.dh = dh;
  a.sh = sh;
  a.h_out = h_out;
  a.gu_out = gu_out;
  a.status = dev_status;
  return launch_gate_up(wtype, a, S(stream));
}

int zq_moe_gate_up_route(int wtype, const void *gu_bank, int64_t gu_stride_bytes,
                         int64_t n_experts, int64_t d_model, int64_t d_ff, const float *logits,
                         int32_t n_routed, int32_t top_k, const float *shared_gate,
                         const float *x, int32_t *ids, float *wts, int8_t *qh, float *dh,
                         int32_t *sh, float *h_out, float *gu_out, void *stream) {
  ZQ_REQUIRE(matrix_bytes(wtype, 1, 256) > 0, ZQ_EINVAL);
  ZQ_REQUIRE(gu_bank && logits && ids && wts && x && qh && dh, ZQ_ENULL);
  ZQ_REQUIRE(top_k >= 1 && top_k <= 64 && n_routed >= top_k && n_routed <= 1024, ZQ_EINVAL);
  const int32_t n_sel = top_k + (shared_gate ? 1 : 0);
  ZQ_REQUIRE(n_experts >= n_sel - top_k + n_routed && n_experts <= INT32_MAX && k_ok(d_model) &&
                 k_ok(d_ff),
             ZQ_EINVAL);
  ZQ_REQUIRE(gate_up_fits(wtype, d_model) && d_ff <= (int64_t(1) << 30), ZQ_EINVAL);
  ZQ_REQUIRE(gu_stride_bytes >= matrix_bytes(wtype, 2 * d_ff, d_model), ZQ_EINVAL);
  ZQ_REQUIRE(bank_al(wtype, gu_bank, gu_stride_bytes) && al(logits, 4) && al(shared_gate, 4) &&
                 al(ids, 4) && al(wts, 4) && al(x, 16) && al(qh, 16) && al(dh, 4) && al(sh, 4) &&
                 al(h_out, 16) && al(gu_out, 4),
             ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  zq::MoeGateUpArgs a{};
  a.bank = static_cast<const uint8_t *>(gu_bank);
  a.expert_stride = gu_stride_bytes;
  a.n_experts = static_cast<int32_t>(n_experts);
  a.ids = ids;
  a.n_sel = n_sel;
  a.x = x;
  a.k = static_cast<int32_t>(d_model);
  a.d_ff = static_cast<int32_t>(d_ff);
  a.qh = qh;
  a.dh = dh;
  a.sh = sh;
  a.h_out = h_out;
  a.gu_out = gu_out;
  a.logits = logits;
  a.n_routed = n_routed;
  a.top_k = top_k;
  a.shared_gate = shared_gate;
  a.ids_out = ids;
  a.wts_out = wts;
  return launch_gate_up(wtype, a, S(stream));
}

int zq_moe_gate_up_mixed(int gu_wtype, const void *gu_bank, int64_t gu_stride_bytes,
                         int sh_wtype, const void *sh_gu, int64_t d_model, int64_t d_ff,
                         const float *logits, int32_t n_routed, int32_t top_k,
                         const float *shared_gate, const float *x, int32_t *ids, float *wts,
                         int8_t *qh, float *dh, int32_t *sh, void *stream) {
  ZQ_REQUIRE(matrix_bytes(gu_wtype, 1, 256) > 0 && matrix_bytes(sh_wtype, 1, 256) > 0, ZQ_EINVAL);
  ZQ_REQUIRE(gu_bank && sh_gu && logits && shared_gate && x && ids && wts && qh && dh, ZQ_ENULL);
  ZQ_REQUIRE(top_k >= 1 && top_k <= 64 && n_routed >= top_k && n_routed <= 1024, ZQ_EINVAL);
  ZQ_REQUIRE(zq::moe_gate_up_mix_fits(d_model) && k_ok(d_ff) && d_ff <= (int64_t(1) << 24),
             ZQ_EINVAL);
  ZQ_REQUIRE(gu_stride_bytes >= matrix_bytes(gu_wtype, 2 * d_ff, d_model), ZQ_EINVAL);
  ZQ_REQUIRE(bank_al(gu_wtype, gu_bank, gu_stride_bytes) && bank_al(sh_wtype, sh_gu, 0) &&
                 al(logits, 4) && al(shared_gate, 4) && al(x, 16) && al(ids, 4) && al(wts, 4) &&
                 al(qh, 16) && al(dh, 4) && al(sh, 4),
             ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  zq::MoeGateUpArgs a{};
  a.bank = static_cast<const uint8_t *>(gu_bank);
  a.expert_stride = gu_stride_bytes;
  a.n_experts = n_routed;
  a.ids = ids;
  a.x = x;
  a.k = static_cast<int32_t>(d_model);
  a.d_ff = static_cast<int32_t>(d_ff);
  a.qh = qh;
  a.dh = dh;
  a.sh = sh;
  a.logits = logits;
  a.n_routed = n_routed;
  a.top_k = top_k;
  a.shared_gate = shared_gate;
  a.ids_out = ids;
  a.wts_out = wts;
  a.bank2 = static_cast<const uint8_t *>(sh_gu);
  return zq::launch_moe_gate_up_mix(gu_wtype, sh_wtype, a, S(stream));
}

int zq_swiglu_quantize(const float *gu, int64_t n, int64_t f, int8_t *qh, float *dh, int32_t *sh,
                       float *h_out, void *stream) {
  ZQ_REQUIRE(gu && qh && dh, ZQ_ENULL);
  ZQ_REQUIRE(n >= 0 && k_ok(f) && n * (f / 32) <= (int64_t(1) << 31), ZQ_EINVAL);
  ZQ_REQUIRE(al(gu, 16) && al(qh, 16) && al(dh, 4) && al(sh, 4) && al(h_out, 16), ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  return zq::launch_swiglu_quantize(gu, n, f, qh, dh, sh, h_out, S(stream));
}

size_t zq_moe_ffn_workspace_bytes(int64_t d_model, int64_t d_ff, int32_t n_sel) {
  if (d_model <= 0 || d_ff <= 0 || n_sel < 0) return 0;
  return moe_layout(d_model, d_ff, n_sel).total;
}

namespace {

// The router's arguments when the expert list is computed on the GPU.
struct MoeRoute {
  const float *logits;
  int32_t n_routed;
  int32_t top_k;
  const float *shared_gate;
};

// One token through the selected experts, arguments already checked.  With
// route set, ids / wts are written (by the gate/up pass, or by the router
// launch on the wide-model path) before the down pass reads them.
int moe_ffn_run(int wtype, const void *gu_bank, int64_t gu_stride_bytes, const void *down_bank,
                int64_t down_stride_bytes, int64_t n_experts, int64_t d_model, int64_t d_ff,
                int32_t *ids, float *wts, int32_t n_sel, const float *x, void *workspace,
                float *y, uint32_t flags, int32_t *dev_status, const MoeRoute *route,
                hipStream_t s) {
  const MoeWorkspace L = moe_layout(d_model, d_ff, n_sel);
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  int8_t *qh = reinterpret_cast<int8_t *>(ws + L.qh);
  float *dh = reinterpret_cast<float *>(ws + L.dh);
  int32_t *sh = reinterpret_cast<int32_t *>(ws + L.sh);
  int rc;
  if (zq::moe_gate_up_fits(d_model)) {
    zq::MoeGateUpArgs a{};
    a.bank = static_cast<const uint8_t *>(gu_bank);
    a.expert_stride = gu_stride_bytes;
    a.n_experts = static_cast<int32_t>(n_experts);
    a.ids = ids;
    if (route) {
      a.logits = route->logits;
      a.n_routed = route->n_routed;
      a.top_k = route->top_k;
      a.shared_gate = route->shared_gate;
      a.ids_out = ids;
      a.wts_out = wts;
    }
    a.n_sel = n_sel;
    a.x = x;
    a.k = static_cast<int32_t>(d_model);
    a.d_ff = static_cast<int32_t>(d_ff);
    a.qh = qh;
    a.dh = dh;
    a.sh = sh;
    a.status = dev_status;
    rc = zq::launch_moe_gate_up(wtype, a, s);
    if (rc != ZQ_OK) return rc;
  } else if (n_sel > 0) {
    // wide models: the router (if asked), quantize x, gather gate||up rows,
    // then swiglu + quantize
    if (route) {
      rc = zq::launch_moe_route(route->logits, route->n_routed, route->top_k, route->shared_gate,
                                ids, wts, s);
      if (rc != ZQ_OK) return rc;
    }
    int8_t *qx = reinterpret_cast<int8_t *>(ws + L.qx);
    float *dx = reinterpret_cast<float *>(ws + L.dx);
    int32_t *sx = reinterpret_cast<int32_t *>(ws + L.sx);
    float *gu = reinterpret_cast<float *>(ws + L.gu);
    rc = zq::launch_quantize_act(x, 1, d_model, d_model, qx, dx, sx, s);
    if (rc != ZQ_OK) return rc;
    zq::DmmvArgs a{};
    a.w = static_cast<const uint8_t *>(gu_bank);
    a.qx = qx;
    a.dx = dx;
    a.sx = wtype == ZQ_Q4_0 ? sx : nullptr;
    a.y = gu;
    a.ids = ids;
    a.status = dev_status;
    a.rows = 2 * d_ff;
    a.expert_stride = gu_stride_bytes;
    a.x_stride = 0;
    a.nb = static_cast<int32_t>(d_model / 32);
    a.n_experts = static_cast<int32_t>(n_experts);
    a.n_sel = n_sel;
    rc = zq::launch_dmmv(wtype, zq::MODE_GATHER, a, s);
    if (rc != ZQ_OK) return rc;
    rc = zq::launch_swiglu_quantize(gu, n_sel, d_ff, qh, dh, sh, nullptr, s);
    if (rc != ZQ_OK) return rc;
  }
  // With no selected expert the down pass writes y = 0 (or leaves y as it
  // is with ZQ_ACCUMULATE) and reads no activation.
  if (zq::moe_down_fits(n_sel, d_ff)) {
    zq::MoeDownArgs b{};
    b.bank = static_cast<const uint8_t *>(down_bank);
    b.expert_stride = down_stride_bytes;
    b.n_experts = static_cast<int32_t>(n_experts);
    b.ids = ids;
    b.wts = wts;
    b.n_sel = n_sel;
    b.qx = qh;
    b.dx = dh;
    b.sx = wtype == ZQ_Q4_0 ? sh : nullptr;
    b.x_stride = d_ff;
    b.k = static_cast<int32_t>(d_ff);
    b.rows = d_model;
    b.y = y;
    b.flags = flags;
    b.status = dev_status;
    return zq::launch_moe_down(wtype, b, s);
  }
  zq::DmmvArgs b{};
  b.w = static_cast<const uint8_t *>(down_bank);
  b.qx = qh;
  b.dx = dh;
  b.sx = wtype == ZQ_Q4_0 ? sh : nullptr;
  b.y = y;
  b.ids = ids;
  b.wts = wts;
  b.status = dev_status;
  b.rows = d_model;
  b.expert_stride = down_stride_bytes;
  b.x_stride = d_ff;
  b.nb = static_cast<int32_t>(d_ff / 32);
  b.n_experts = static_cast<int32_t>(n_experts);
  b.n_sel = n_sel;
  b.flags = flags;
  return zq::launch_dmmv(wtype, zq::MODE_WEIGHTED, b, s);
}


}  // namespace

int zq_moe_ffn(int wtype, const void *gu_bank, int64_t gu_stride_bytes, const void *down_bank,
               int64_t down_stride_bytes, int64_t n_experts, int64_t d_model, int64_t d_ff,
               const int32_t *ids, const float *wts, int32_t n_sel, const float *x,
               void *workspace, size_t workspace_bytes, float *y, uint32_t flags,
               int32_t *dev_status, void *stream) {
  const int64_t bb = block_bytes(wtype);
  ZQ_REQUIRE(bb > 0, ZQ_EINVAL);
  ZQ_REQUIRE(gu_bank && down_bank && ids && wts && x && workspace && y, ZQ_ENULL);
  ZQ_REQUIRE(n_experts >= 1 && n_experts <= INT32_MAX && k_ok(d_model) && k_ok(d_ff), ZQ_EINVAL);
  ZQ_REQUIRE(n_sel >= 0 && n_sel <= 65535, ZQ_EINVAL);
  ZQ_REQUIRE(gu_stride_bytes >= 2 * d_ff * (d_model / 32) * bb && gu_stride_bytes % 2 == 0,
             ZQ_EINVAL);
  ZQ_REQUIRE(down_stride_bytes >= d_model * (d_ff / 32) * bb && down_stride_bytes % 2 == 0,
             ZQ_EINVAL);
  ZQ_REQUIRE((flags & ~uint32_t(ZQ_ACCUMULATE)) == 0, ZQ_EINVAL);
  const MoeWorkspace L = moe_layout(d_model, d_ff, n_sel);
  ZQ_REQUIRE(workspace_bytes >= L.total, ZQ_EINVAL);
  ZQ_REQUIRE(al(gu_bank, 4) && al(down_bank, 4) && al(ids, 4) && al(wts, 4) && al(x, 16) &&
                 al(workspace, kAlign) && al(y, 4) && al(dev_status, 4),
             ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  return moe_ffn_run(wtype, gu_bank, gu_stride_bytes, down_bank, down_stride_bytes, n_experts,
                     d_model, d_ff, const_cast<int32_t *>(ids), const_cast<float *>(wts), n_sel, x,
                     workspace, y, flags, dev_status, nullptr, S(stream));
}

int zq_moe_ffn_route(int wtype, const void *gu_bank, int64_t gu_stride_bytes,
                     const void *down_bank, int64_t down_stride_bytes, int64_t n_experts,
                     int64_t d_model, int64_t d_ff, const float *logits, int32_t n_routed,
                     int32_t top_k, const float *shared_gate, const float *x, int32_t *ids,
                     float *wts, void *workspace, size_t workspace_bytes, float *y,
                     uint32_t flags, void *stream) {
  const int64_t bb = block_bytes(wtype);
  ZQ_REQUIRE(bb > 0, ZQ_EINVAL);
  ZQ_REQUIRE(gu_bank && down_bank && logits && ids && wts && x && workspace && y, ZQ_ENULL);
  ZQ_REQUIRE(top_k >= 1 && top_k <= 64 && n_routed >= top_k && n_routed <= 1024, ZQ_EINVAL);
  const int32_t n_sel = top_k + (shared_gate ? 1 : 0);
  ZQ_REQUIRE(n_experts >= n_sel - top_k + n_routed && n_experts <= INT32_MAX && k_ok(d_model) &&
                 k_ok(d_ff),
             ZQ_EINVAL);
  ZQ_REQUIRE(gu_stride_bytes >= 2 * d_ff * (d_model / 32) * bb && gu_stride_bytes % 2 == 0,
             ZQ_EINVAL);
  ZQ_REQUIRE(down_stride_bytes >= d_model * (d_ff / 32) * bb && down_stride_bytes % 2 == 0,
             ZQ_EINVAL);
  ZQ_REQUIRE((flags & ~uint32_t(ZQ_ACCUMULATE)) == 0, ZQ_EINVAL);
  ZQ_REQUIRE(workspace_bytes >= moe_layout(d_model, d_ff, n_sel).total, ZQ_EINVAL);
  ZQ_REQUIRE(al(gu_bank, 4) && al(down_bank, 4) && al(logits, 4) && al(shared_gate, 4) &&
                 al(ids, 4) && al(wts, 4) && al(x, 16) && al(workspace, kAlign) && al(y, 4),
             ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  const MoeRoute route{logits, n_routed, top_k, shared_gate};
  return moe_ffn_run(wtype, gu_bank, gu_stride_bytes, down_bank, down_stride_bytes, n_experts,
                     d_model, d_ff, ids, wts, n_sel, x, workspace, y, flags, nullptr, &route,
                     S(stream));
}

int zq_moe_ffn_norm_route(int wtype, const void *gu_bank, int64_t gu_stride_bytes,
                          const void *down_bank, int64_t down_stride_bytes, int64_t n_experts,
                          int64_t d_model, int64_t d_ff, const void *router_w,
                          const float *norm_w, float eps, const float *x, int32_t n_routed,
                          int32_t top_k, const float *shared_gate, float *xn_out,
                          float *logits_out, int32_t *ids, float *wts, void *workspace,
                          size_t workspace_bytes, float *y, uint32_t flags, void *stream) {
  const int64_t bb = block_bytes(wtype);
  ZQ_REQUIRE(bb > 0, ZQ_EINVAL);
  ZQ_REQUIRE(gu_bank && down_bank && router_w && norm_w && x && xn_out && logits_out && ids &&
                 wts && workspace && y,
             ZQ_ENULL);
  ZQ_REQUIRE(top_k >= 1 && top_k <= 64 && n_routed >= top_k && n_routed <= 1024, ZQ_EINVAL);
  const int32_t n_sel = top_k + (shared_gate ? 1 : 0);
  ZQ_REQUIRE(n_experts >= n_sel - top_k + n_routed && n_experts <= INT32_MAX && k_ok(d_model) &&
                 d_model <= 16384 && k_ok(d_ff) && eps_ok(eps),
             ZQ_EINVAL);
  ZQ_REQUIRE(gu_stride_bytes >= 2 * d_ff * (d_model / 32) * bb && gu_stride_bytes % 2 == 0,
             ZQ_EINVAL);
  ZQ_REQUIRE(down_stride_bytes >= d_model * (d_ff / 32) * bb && down_stride_bytes % 2 == 0,
             ZQ_EINVAL);
  ZQ_REQUIRE((flags & ~uint32_t(ZQ_ACCUMULATE)) == 0, ZQ_EINVAL);
  ZQ_REQUIRE(workspace_bytes >= moe_layout(d_model, d_ff, n_sel).total, ZQ_EINVAL);
  ZQ_REQUIRE(al(gu_bank, 4) && al(down_bank, 4) && al(router_w, 4) && al(norm_w, 16) &&
                 al(x, 16) && al(shared_gate, 4) && al(xn_out, 16) && al(logits_out, 4) &&
                 al(ids, 4) && al(wts, 4) && al(workspace, kAlign) && al(y, 4),
             ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  const hipStream_t s = S(stream);
  const MoeRoute route{logits_out, n_routed, top_k, shared_gate};
  // the fused norm + router DMMV launch, then the block on xn
  zq::DmmvF32Args r{};
  r.w = static_cast<const uint8_t *>(router_w);
  r.x = x;
  r.y = logits_out;
  r.norm_w = norm_w;
  r.eps = eps;
  r.xn_out = xn_out;
  r.rows = n_routed;
  r.k = static_cast<int32_t>(d_model);
  r.nb = static_cast<int32_t>(d_model / 32);
  const int rc = zq::launch_dmmv_f32x(ZQ_Q8_0, r, s);
  if (rc != ZQ_OK) return rc;
  return moe_ffn_run(wtype, gu_bank, gu_stride_bytes, down_bank, down_stride_bytes, n_experts,
                     d_model, d_ff, ids, wts, n_sel, xn_out, workspace, y, flags, nullptr, &route,
                     s);
}

int zq_gemm_prefill(int wtype, const void *w, int64_t n, int64_t k, const int8_t *qx,
                    const float *dx, const int32_t *sx, int64_t m, float *y, uint32_t flags,
                    void *stream) {
  (void)sx;  // the kernel unpacks Q4_0 nibbles to signed values; no block sums needed
  ZQ_REQUIRE(block_bytes(wtype) > 0, ZQ_EINVAL);
  ZQ_REQUIRE(w && qx && dx && y, ZQ_ENULL);
  ZQ_REQUIRE(n >= 0 && m >= 0 && k_ok(k), ZQ_EINVAL);
  ZQ_REQUIRE(((n + 63) / 64) * ((m + 63) / 64) <= INT32_MAX, ZQ_EINVAL);
  ZQ_REQUIRE((flags & ~uint32_t(ZQ_ACCUMULATE)) == 0, ZQ_EINVAL);
  ZQ_REQUIRE(al(w, 4) && al(qx, 16) && al(dx, 4) && al(y, 4) && al(sx, 4), ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  return zq::launch_gemm(wtype, w, n, k, qx, dx, m, y, flags, nullptr, 0, m, 0, n, S(stream));
}

int zq_gemm_isums(int wtype, const void *w, int64_t n, int64_t k, const int8_t *qx,
                  const int32_t *sx, int64_t m, int64_t m0, int64_t m1, int64_t n0, int64_t n1,
                  int32_t *isums, void *stream) {
  (void)sx;
  ZQ_REQUIRE(block_bytes(wtype) > 0, ZQ_EINVAL);
  ZQ_REQUIRE(w && qx && isums, ZQ_ENULL);
  ZQ_REQUIRE(n >= 0 && m >= 0 && k_ok(k), ZQ_EINVAL);
  ZQ_REQUIRE(0 <= m0 && m0 <= m1 && m1 <= m && 0 <= n0 && n0 <= n1 && n1 <= n, ZQ_EINVAL);
  ZQ_REQUIRE(al(w, 4) && al(qx, 16) && al(isums, 4) && al(sx, 4), ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  // dx is not read by the isums variant's result; the scale loads use qx's
  // bytes as a readable stand-in (k >= 32 bytes per token >= k/32 floats).
  return zq::launch_gemm(wtype, w, n, k, qx, reinterpret_cast<const float *>(qx), m, nullptr, 0,
                         isums, m0, m1, n0, n1, S(stream));
}

namespace {

// Launch one expert-indexed DMMV stage in whichever kernel serves wtype
// (arguments already checked by the caller).
int moe_stage(int wtype, int mode, const void *bank, int64_t stride, int64_t n_experts,
              int32_t id_base, int64_t rows, int64_t k, const int32_t *ids, const float *wts,
              int32_t n_sel, const int8_t *qx, const float *dx, const int32_t *sx,
              int64_t x_stride, float *y, uint32_t flags, hipStream_t s) {
  zq::DmmvArgs a{};
  a.w = static_cast<const uint8_t *>(bank);
  a.qx = qx;
  a.dx = dx;
  a.sx = (wtype == ZQ_Q4_0 || wtype == ZQ_Q4_K || wtype == ZQ_Q5_K) ? sx : nullptr;
  a.y = y;
  a.ids = ids;
  a.wts = wts;
  a.rows = rows;
  a.expert_stride = stride;
  a.x_stride = x_stride;
  a.nb = static_cast<int32_t>(k / 32);
  a.n_experts = static_cast<int32_t>(n_experts);
  a.n_sel = n_sel;
  a.flags = flags;
  a.id_base = id_base;
  if (wtype == ZQ_Q4_K || wtype == ZQ_Q5_K || wtype == ZQ_Q6_K) return zq::launch_dmmv_k(wtype, mode, a, s);
  // the same dispatch as zq_dmmv_moe: the weighted sum over Q4_0 / Q8_0
  // experts takes the dedicated down kernel when it fits
  if (mode == zq::MODE_WEIGHTED && x_stride % 32 == 0 && zq::moe_down_fits(n_sel, k)) {
    zq::MoeDownArgs b{};
    b.bank = static_cast<const uint8_t *>(bank);
    b.expert_stride = stride;
    b.n_experts = static_cast<int32_t>(n_experts);
    b.ids = ids;
    b.wts = wts;
    b.n_sel = n_sel;
    b.qx = qx;
    b.dx = dx;
    b.sx = wtype == ZQ_Q4_0 ? sx : nullptr;
    b.x_stride = x_stride;
    b.k = static_cast<int32_t>(k);
    b.rows = rows;
    b.y = y;
    b.flags = flags;
    b.id_base = id_base;
    return zq::launch_moe_down(wtype, b, s);
  }
  return zq::launch_dmmv(wtype, mode, a, s);
}

}  // namespace

namespace {

struct MoeTokWorkspace {
  size_t mem, qx, dx, sx, qh, dh, sh, total;
};

MoeTokWorkspace moe_tok_layout(int64_t d_model, int64_t d_ff, int32_t n_tok, int32_t n_sel) {
  const size_t J = static_cast<size_t>(n_tok) * static_cast<size_t>(n_sel);
  const size_t T = static_cast<size_t>(n_tok);
  MoeTokWorkspace w;
  size_t off = 0;
  w.mem = off; off += round_up(zq::kTokMax * J * 4);
  w.qx = off; off += round_up(T * static_cast<size_t>(d_model));
  w.dx = off; off += round_up(T * static_cast<size_t>(d_model / 32) * 4);
  w.sx = off; off += round_up(T * static_cast<size_t>(d_model / 32) * 4);
  w.qh = off; off += round_up(J * static_cast<size_t>(d_ff));
  w.dh = off; off += round_up(J * static_cast<size_t>(d_ff / 32) * 4);
  w.sh = off; off += round_up(J * static_cast<size_t>(d_ff / 32) * 4);
  w.total = off;
  return w;
}

}  // namespace

size_t zq_moe_ffn_tokens_workspace_bytes(int64_t d_model, int64_t d_ff, int32_t n_tok,
                                         int32_t n_sel) {
  if (d_model <= 0 || d_ff <= 0 || n_tok < 0 || n_sel < 0) return 0;
  return moe_tok_layout(d_model, d_ff, n_tok, n_sel).total;
}

int zq_moe_ffn_tokens(int wtype, const void *gu_bank, int64_t gu_stride_bytes,
                      const void *down_bank, int64_t down_stride_bytes, int64_t n_experts,
                      int64_t d_model, int64_t d_ff, const float *logits, int32_t n_routed,
                      int32_t top_k, const float *shared_gate, const float *x, int32_t n_tok,
                      int32_t *ids, float *wts, void *workspace, size_t workspace_bytes, float *y,
                      uint32_t flags, void *stream) {
  const bool shared = shared_gate != nullptr;
  ZQ_REQUIRE(block_bytes(wtype) > 0, ZQ_EINVAL);
  ZQ_REQUIRE(gu_bank && down_bank && logits && x && ids && wts && workspace && y, ZQ_ENULL);
  ZQ_REQUIRE(n_tok >= 1 && n_tok <= zq::kTokMax && top_k >= 1 && top_k <= 64 &&
                 n_routed >= top_k && n_routed <= 1024 && n_experts >= n_routed + (shared ? 1 : 0) &&
                 n_experts <= INT32_MAX,
             ZQ_EINVAL);
  ZQ_REQUIRE(k_ok(d_model) && zq::moe_tok_fits(d_model, d_ff), ZQ_EINVAL);
  ZQ_REQUIRE(gu_stride_bytes >= matrix_bytes(wtype, 2 * d_ff, d_model) &&
                 down_stride_bytes >= matrix_bytes(wtype, d_model, d_ff),
             ZQ_EINVAL);
  ZQ_REQUIRE((flags & ~uint32_t(ZQ_ACCUMULATE)) == 0, ZQ_EINVAL);
  const int32_t n_sel = top_k + (shared ? 1 : 0);
  const MoeTokWorkspace L = moe_tok_layout(d_model, d_ff, n_tok, n_sel);
  ZQ_REQUIRE(workspace_bytes >= L.total, ZQ_EINVAL);
  ZQ_REQUIRE(bank_al(wtype, gu_bank, gu_stride_bytes) &&
                 bank_al(wtype, down_bank, down_stride_bytes) && al(logits, 4) &&
                 al(shared_gate, 4) && al(x, 16) && al(ids, 4) && al(wts, 4) &&
                 al(workspace, 256) && al(y, 4),
             ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  const int32_t J = n_tok * n_sel;
  zq::MoeTokArgs p{};
  p.logits = logits;
  p.n_routed = n_routed;
  p.top_k = top_k;
  p.shared_gate = shared_gate;
  p.n_tok = n_tok;
  p.ids = ids;
  p.wts = wts;
  p.x = x;
  p.d_model = static_cast<int32_t>(d_model);
  p.qx = reinterpret_cast<int8_t *>(ws + L.qx);
  p.dx = reinterpret_cast<float *>(ws + L.dx);
  p.sx = reinterpret_cast<int32_t *>(ws + L.sx);
  zq::MoeGateUpArgs g{};
  g.bank = static_cast<const uint8_t *>(gu_bank);
  g.expert_stride = gu_stride_bytes;
  g.n_experts = static_cast<int32_t>(n_experts);
  g.n_sel = J;
  g.k = static_cast<int32_t>(d_model);
  g.d_ff = static_cast<int32_t>(d_ff);
  g.qh = reinterpret_cast<int8_t *>(ws + L.qh);
  g.dh = reinterpret_cast<float *>(ws + L.dh);
  g.sh = reinterpret_cast<int32_t *>(ws + L.sh);
  zq::MoeDownTokArgs d{};
  d.bank = static_cast<const uint8_t *>(down_bank);
  d.expert_stride = down_stride_bytes;
  d.n_experts = static_cast<int32_t>(n_experts);
  d.mem = reinterpret_cast<int32_t *>(ws + L.mem);
  d.n_sel = J;
  d.n_tok = n_tok;
  d.qh = g.qh;
  d.dh = g.dh;
  d.sh = g.sh;
  d.wts = wts;
  d.n_sel_tok = n_sel;
  d.y = y;
  d.rows = d_model;
  d.k = static_cast<int32_t>(d_ff);
  d.flags = flags;
  return zq::launch_moe_ffn_tok(wtype, p, g, d, S(stream));
}

int zq_moe_ffn_mixed(int gu_wtype, const void *gu_bank, int64_t gu_stride_bytes, int down_wtype,
                     const void *down_bank, int64_t down_stride_bytes, int sh_wtype,
                     const void *sh_gu, const void *sh_down, int64_t d_model, int64_t d_ff,
                     const float *logits, int32_t n_routed, int32_t top_k,
                     const float *shared_gate, const float *x, int32_t *ids, float *wts,
                     void *workspace, size_t workspace_bytes, float *y, uint32_t flags,
                     void *stream) {
  const bool shared = shared_gate != nullptr;
  ZQ_REQUIRE(matrix_bytes(gu_wtype, 1, 256) > 0 && matrix_bytes(down_wtype, 1, 256) > 0 &&
                 (!shared || matrix_bytes(sh_wtype, 1, 256) > 0),
             ZQ_EINVAL);
  ZQ_REQUIRE(gu_bank && down_bank && logits && x && ids && wts && workspace && y, ZQ_ENULL);
  ZQ_REQUIRE(!shared || (sh_gu && sh_down), ZQ_ENULL);
  ZQ_REQUIRE(k_ok(d_model) && k_ok(d_ff) && d_model <= (int64_t(1) << 24) &&
                 d_ff <= (int64_t(1) << 24) && top_k >= 1 && top_k <= 64 && n_routed >= top_k &&
                 n_routed <= 1024,
             ZQ_EINVAL);
  // K-quant matrices take whole 256-element super-blocks along k
  ZQ_REQUIRE(!is_k(gu_wtype) || d_model % 256 == 0, ZQ_EINVAL);
  ZQ_REQUIRE(!is_k(down_wtype) || d_ff % 256 == 0, ZQ_EINVAL);
  ZQ_REQUIRE(!shared || !is_k(sh_wtype) || (d_model % 256 == 0 && d_ff % 256 == 0), ZQ_EINVAL);
  ZQ_REQUIRE(gu_stride_bytes >= matrix_bytes(gu_wtype, 2 * d_ff, d_model) &&
                 down_stride_bytes >= matrix_bytes(down_wtype, d_model, d_ff),
             ZQ_EINVAL);
  ZQ_REQUIRE((flags & ~uint32_t(ZQ_ACCUMULATE)) == 0, ZQ_EINVAL);
  const int32_t n_sel = top_k + (shared ? 1 : 0);
  ZQ_REQUIRE(workspace_bytes >= zq_moe_ffn_workspace_bytes(d_model, d_ff, n_sel), ZQ_EINVAL);
  ZQ_REQUIRE(bank_al(gu_wtype, gu_bank, gu_stride_bytes) &&
                 bank_al(down_wtype, down_bank, down_stride_bytes) &&
                 (!shared || (bank_al(sh_wtype, sh_gu, 0) && bank_al(sh_wtype, sh_down, 0))) &&
                 al(logits, 4) && al(shared_gate, 4) && al(x, 16) && al(ids, 4) && al(wts, 4) &&
                 al(workspace, 256) && al(y, 4),
             ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  hipStream_t s = S(stream);
  const MoeWorkspace L = moe_layout(d_model, d_ff, n_sel);
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  int8_t *qx = reinterpret_cast<int8_t *>(ws + L.qx);
  float *dx = reinterpret_cast<float *>(ws + L.dx);
  int32_t *sx = reinterpret_cast<int32_t *>(ws + L.sx);
  float *gu = reinterpret_cast<float *>(ws + L.gu);
  int8_t *qh = reinterpret_cast<int8_t *>(ws + L.qh);
  float *dh = reinterpret_cast<float *>(ws + L.dh);
  int32_t *sh = reinterpret_cast<int32_t *>(ws + L.sh);
  int rc;
  if (gate_up_fits(gu_wtype, d_model) && (!shared || gate_up_fits(sh_wtype, d_model))) {
    // fused: the routed experts' gate/up pass ranks the logits itself and
    // publishes ids / wts (the shared slot included); the shared expert
    // (id n_routed) runs in the same launch where the two row layouts fit
    // together, else in a launch of its own
    zq::MoeGateUpArgs a{};
    a.bank = static_cast<const uint8_t *>(gu_bank);
    a.expert_stride = gu_stride_bytes;
    a.n_experts = n_routed;
    a.ids = ids;
    a.n_sel = top_k;
    a.x = x;
    a.k = static_cast<int32_t>(d_model);
    a.d_ff = static_cast<int32_t>(d_ff);
    a.qh = qh;
    a.dh = dh;
    a.sh = sh;
    a.logits = logits;
    a.n_routed = n_routed;
    a.top_k = top_k;
    a.shared_gate = shared_gate;
    a.ids_out = ids;
    a.wts_out = wts;
    if (shared && zq::moe_gate_up_mix_fits(d_model)) {
      // both in one launch: slot top_k runs the shared matrix in its format
      a.bank2 = static_cast<const uint8_t *>(sh_gu);
      rc = zq::launch_moe_gate_up_mix(gu_wtype, sh_wtype, a, s);
    } else {
      rc = launch_gate_up(gu_wtype, a, s);
    }
    if (rc != ZQ_OK) return rc;
    if (shared && !zq::moe_gate_up_mix_fits(d_model)) {
      const int64_t h0 = static_cast<int64_t>(top_k) * d_ff;
      zq::MoeGateUpArgs b{};
      b.bank = static_cast<const uint8_t *>(sh_gu);
      b.n_experts = 1;
      b.ids = ids + top_k;
      b.id_base = n_routed;
      b.n_sel = 1;
      b.x = x;
      b.k = static_cast<int32_t>(d_model);
      b.d_ff = static_cast<int32_t>(d_ff);
      b.qh = qh + h0;
      b.dh = dh + h0 / 32;
      b.sh = sh + h0 / 32;
      rc = launch_gate_up(sh_wtype, b, s);
      if (rc != ZQ_OK) return rc;
    }
  } else {
    rc = zq::launch_moe_route(logits, n_routed, top_k, shared_gate, ids, wts, s);
    if (rc != ZQ_OK) return rc;
    rc = zq::launch_quantize_act(x, 1, d_model, d_model, qx, dx, sx, s);
    if (rc != ZQ_OK) return rc;
    // gate||up rows of every selected expert; the shared one (id n_routed)
    // from its own matrix
    rc = moe_stage(gu_wtype, zq::MODE_GATHER, gu_bank, gu_stride_bytes, n_routed, 0, 2 * d_ff,
                   d_model, ids, nullptr, top_k, qx, dx, sx, 0, gu, 0, s);
    if (rc != ZQ_OK) return rc;
    if (shared) {
      rc = moe_stage(sh_wtype, zq::MODE_GATHER, sh_gu, 0, 1, n_routed, 2 * d_ff, d_model,
                     ids + top_k, nullptr, 1, qx, dx, sx, 0,
                     gu + static_cast<int64_t>(top_k) * 2 * d_ff, 0, s);
      if (rc != ZQ_OK) return rc;
    }
    rc = zq::launch_swiglu_quantize(gu, n_sel, d_ff, qh, dh, sh, nullptr, s);
    if (rc != ZQ_OK) return rc;
  }
  if (shared && zq::dmmv_k_wsum_shared_fits(down_wtype, sh_wtype, d_ff)) {
    // K-quant routed down rows and a block-format shared expert: one launch,
    // one reduction over every term
    zq::DmmvArgs a{};
    a.w = static_cast<const uint8_t *>(down_bank);
    a.qx = qh;
    a.dx = dh;
    a.sx = sh;
    a.y = y;
    a.ids = ids;
    a.wts = wts;
    a.rows = d_model;
    a.expert_stride = down_stride_bytes;
    a.x_stride = d_ff;
    a.nb = static_cast<int32_t>(d_ff / 32);
    a.n_experts = n_routed;
    a.n_sel = top_k;
    a.flags = flags;
    a.w2 = static_cast<const uint8_t *>(sh_down);
    return zq::launch_dmmv_k_wsum_shared(down_wtype, sh_wtype, a, s);
  }
  // down rows: the weighted sum over the routed experts, then the shared one
  // added onto it
  rc = moe_stage(down_wtype, zq::MODE_WEIGHTED, down_bank, down_stride_bytes, n_routed, 0,
                 d_model, d_ff, ids, wts, top_k, qh, dh, sh, d_ff, y, flags, s);
  if (rc != ZQ_OK || !shared) return rc;
  const int64_t h0 = static_cast<int64_t>(top_k) * d_ff;
  return moe_stage(sh_wtype, zq::MODE_WEIGHTED, sh_down, 0, 1, n_routed, d_model, d_ff,
                   ids + top_k, wts + top_k, 1, qh + h0, dh + h0 / 32, sh + h0 / 32, d_ff, y,
                   ZQ_ACCUMULATE, s);
}

}  // extern "C"

namespace zq {
// probe.hip: a streaming read of `bytes` (a multiple of 16) with 16-byte loads.
int launch_read_probe(const void *buf, int64_t bytes, uint32_t *sink, hipStream_t stream);
}  // namespace zq

int zq_read_probe(const void *buf, int64_t bytes, uint32_t *sink, void *stream) {
  ZQ_REQUIRE(buf && sink, ZQ_ENULL);
  ZQ_REQUIRE(bytes >= 0 && bytes % 16 == 0, ZQ_EINVAL);
  ZQ_REQUIRE(al(buf, 16) && al(sink, 4), ZQ_EALIGN);
  const int dc = check_current_device();
  if (dc != ZQ_OK) return dc;
  return zq::launch_read_probe(buf, bytes, sink, S(stream));
}
