// qg_api.hip -- the C ABI of libqgguf.so (declared in include/qgguf.h).
//
// Every entry point validates its arguments before touching the HIP runtime:
// on any error nothing is launched and nothing is written.  Then it checks
// once per device that the current device is gfx950 and enqueues its kernels
// on the caller's stream.  The status codes mirror the pages' habit of one
// distinct, named error per failure class (blazr 0.4.0 release notes,
// "Changed": model lookup / load / out-of-memory errors).
#include <atomic>
#include <string.h>

#include "../../include/qgguf.h"
#include "qg_launch.h"

#define QG_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other arch
std::atomic<int> g_arch[kMaxDevices];

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

qg_status check_device() {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) return QG_ERR_NO_DEVICE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return QG_ERR_NO_DEVICE;
  if (dev >= kMaxDevices) return QG_ERR_ARCH;
  int state = g_arch[dev].load(std::memory_order_acquire);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return QG_ERR_NO_DEVICE;
    state = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch[dev].store(state, std::memory_order_release);
  }
  return state == 1 ? QG_OK : QG_ERR_ARCH;
}

qg_status launched(hipError_t e) { return e == hipSuccess ? QG_OK : QG_ERR_LAUNCH; }

constexpr int64_t kMaxK = int64_t(1) << 24;
constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;

// fmt 0 = Q8_0 (k % 32), 1 = Q4_K, 2 = Q6_K, 3 = Q5_K (k % 256), 4 = Q4_0,
// 5 = Q5_0 (k % 64: the kernel takes block pairs)
qg_status check_gemv(int fmt, const void *w, const void *xq, const void *out, int64_t n, int64_t k) {
  if (!w || !xq || !out) return QG_ERR_NULL;
  if (n < 0 || k < 0 || n > kMaxRows || k > kMaxK) return QG_ERR_SHAPE;
  if (k % (fmt == 0 ? 32 : (fmt >= 4 ? 64 : 256)) != 0) return QG_ERR_SHAPE;
  if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(out, 4)) return QG_ERR_ALIGN;
  return QG_OK;
}

qg_status run_gemv(int fmt, const void *w, const void *xq, float *y, int32_t *D, int32_t *S, int64_t n, int64_t k,
                   hipStream_t stream) {
  if (n == 0) return QG_OK;
  qg_status st = check_device();
  if (st != QG_OK) return st;
  return launched(qg::launch_qgemv(fmt, w, xq, y, D, S, n, k, stream));
}

constexpr int64_t kMaxBatch = 8;

qg_status check_gemv_batch(int fmt, const void *w, const void *xq, const void *out, int64_t nb, int64_t n,
                           int64_t k) {
  if (!w || !xq || !out) return QG_ERR_NULL;
  if (nb < 0 || nb > kMaxBatch || n < 0 || k < 0 || n > kMaxRows || k > kMaxK) return QG_ERR_SHAPE;
  if (nb * n > kMaxRows) return QG_ERR_SHAPE;
  if (k % (fmt == 0 ? 32 : 256) != 0) return QG_ERR_SHAPE;
  if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(out, 4)) return QG_ERR_ALIGN;
  return QG_OK;
}

// D non-null: the per-block dot dump of the kernel the product call would run.
qg_status run_gemv_batch(int fmt, const void *w, const void *xq, float *y, int32_t *D, int64_t nb, int64_t n,
                         int64_t k, hipStream_t stream) {
  qg_status st = check_gemv_batch(fmt, w, xq, y ? static_cast<const void *>(y) : D, nb, n, k);
  if (st != QG_OK) return st;
  if (D && k > 0 && nb * n > (int64_t(1) << 29) / (k / (fmt == 2 ? 16 : 32))) return QG_ERR_SHAPE;
  if (nb == 0 || n == 0 || (D && k == 0)) return QG_OK;  // k == 0 runs for y: the kernel writes y = 0
  st = check_device();
  if (st != QG_OK) return st;
  return launched(qg::launch_qgemv_batch(fmt, w, xq, y, D, nb, n, k, stream));
}

qg_status check_mmq(int fmt, const void *w, const void *aq, const void *out, int64_t m, int64_t n, int64_t k) {
  if (!w || !aq || !out) return QG_ERR_NULL;
  if (m < 0 || n < 0 || k < 0 || m > kMaxRows || n > kMaxRows || k > kMaxK) return QG_ERR_SHAPE;
  if (k % ((fmt == 0 || fmt >= 4) ? 32 : 256) != 0) return QG_ERR_SHAPE;  // 32-value block types: k % 32
  if (((m + 63) / 64) * ((n + 63) / 64) > kMaxRows) return QG_ERR_SHAPE;
  if (!aligned(w, 16) || !aligned(aq, 16) || !aligned(out, 4)) return QG_ERR_ALIGN;
  return QG_OK;
}

}  // namespace

QG_EXPORT const char *qg_status_str(qg_status s) {
  // read as an int: a C caller may pass any int, which as a C++ enum of this
  // range would be undefined
  int v = 0;
  memcpy(&v, &s, sizeof v);
  switch (v) {
    case QG_OK: return "ok";
    case QG_ERR_NULL: return "a required pointer is NULL";
    case QG_ERR_SHAPE: return "invalid shape (negative, not a multiple of the block size, or too large)";
    case QG_ERR_ALIGN: return "pointer not aligned (block buffers and f32 inputs 16 B, outputs 4 B)";
    case QG_ERR_WORKSPACE: return "workspace too small";
    case QG_ERR_NO_DEVICE: return "no HIP device available";
    case QG_ERR_ARCH: return "current device is not gfx950";
    case QG_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

QG_EXPORT qg_status quantize_q8_1(const float *x, void *xq, int64_t rows, int64_t k, hipStream_t stream) {
  if (!x || !xq) return QG_ERR_NULL;
  if (rows < 0 || k < 0 || k % 32 != 0 || k > (int64_t(1) << 30)) return QG_ERR_SHAPE;
  if (rows > 0 && k > 0 && rows > (int64_t(1) << 40) / k) return QG_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(xq, 16)) return QG_ERR_ALIGN;
  if (rows == 0 || k == 0) return QG_OK;
  qg_status st = check_device();
  if (st != QG_OK) return st;
  return launched(qg::launch_quantize_q8_1(x, xq, rows, k, stream));
}

QG_EXPORT qg_status rmsnorm_quantize_q8_1(const float *x, const float *gamma, float eps, void *xq, float *r_out,
                                          int64_t rows, int64_t k, hipStream_t stream) {
  if (!x || !gamma || !xq) return QG_ERR_NULL;
  if (rows < 0 || k < 0 || k % 32 != 0 || k > kMaxK || rows > kMaxRows) return QG_ERR_SHAPE;
  if (!(eps >= 0.f) || !__builtin_isfinite(eps)) return QG_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(gamma, 16) || !aligned(xq, 16) || (r_out && !aligned(r_out, 4)))
    return QG_ERR_ALIGN;
  if (rows == 0 || k == 0) return QG_OK;
  qg_status st = check_device();
  if (st != QG_OK) return st;
  return launched(qg::launch_rmsnorm_quantize_q8_1(x, gamma, eps, xq, r_out, rows, k, stream));
}

QG_EXPORT qg_status qgemv_q8_0(const void *w, const void *xq, float *y, int64_t n, int64_t k, hipStream_t stream) {
  qg_status st = check_gemv(0, w, xq, y, n, k);
  return st != QG_OK ? st : run_gemv(0, w, xq, y, nullptr, nullptr, n, k, stream);
}

QG_EXPORT qg_status qgemv_q4_k(const void *w, const void *xq, float *y, int64_t n, int64_t k, hipStream_t stream) {
  qg_status st = check_gemv(1, w, xq, y, n, k);
  return st != QG_OK ? st : run_gemv(1, w, xq, y, nullptr, nullptr, n, k, stream);
}

QG_EXPORT qg_status qgemv_q6_k(const void *w, const void *xq, float *y, int64_t n, int64_t k, hipStream_t stream) {
  qg_status st = check_gemv(2, w, xq, y, n, k);
  return st != QG_OK ? st : run_gemv(2, w, xq, y, nullptr, nullptr, n, k, stream);
}

QG_EXPORT qg_status qgemv_q5_k(const void *w, const void *xq, float *y, int64_t n, int64_t k, hipStream_t stream) {
  qg_status st = check_gemv(3, w, xq, y, n, k);
  return st != QG_OK ? st : run_gemv(3, w, xq, y, nullptr, nullptr, n, k, stream);
}

QG_EXPORT qg_status qgemv_q4_0(const void *w, const void *xq, float *y, int64_t n, int64_t k, hipStream_t stream) {
  qg_status st = check_gemv(4, w, xq, y, n, k);
  return st != QG_OK ? st : run_gemv(4, w, xq, y, nullptr, nullptr, n, k, stream);
}

QG_EXPORT qg_status qgemv_q5_0(const void *w, const void *xq, float *y, int64_t n, int64_t k, hipStream_t stream) {
  qg_status st = check_gemv(5, w, xq, y, n, k);
  return st != QG_OK ? st : run_gemv(5, w, xq, y, nullptr, nullptr, n, k, stream);
}

QG_EXPORT qg_status qgemv_q8_0_batch(const void *w, const void *xq, float *y, int64_t b, int64_t n, int64_t k,
                                     hipStream_t stream) {
  return run_gemv_batch(0, w, xq, y, nullptr, b, n, k, stream);
}

QG_EXPORT qg_status qg_blockdots_q8_0_batch(const void *w, const void *xq, int32_t *D, int64_t b, int64_t n, int64_t k,
                                          hipStream_t stream) {
  return run_gemv_batch(0, w, xq, nullptr, D, b, n, k, stream);
}

QG_EXPORT qg_status qgemv_q4_k_batch(const void *w, const void *xq, float *y, int64_t b, int64_t n, int64_t k,
                                     hipStream_t stream) {
  return run_gemv_batch(1, w, xq, y, nullptr, b, n, k, stream);
}

QG_EXPORT qg_status qg_blockdots_q4_k_batch(const void *w, const void *xq, int32_t *D, int64_t b, int64_t n, int64_t k,
                                          hipStream_t stream) {
  return run_gemv_batch(1, w, xq, nullptr, D, b, n, k, stream);
}

QG_EXPORT qg_status qgemv_q6_k_batch(const void *w, const void *xq, float *y, int64_t b, int64_t n, int64_t k,
                                     hipStream_t stream) {
  return run_gemv_batch(2, w, xq, y, nullptr, b, n, k, stream);
}

QG_EXPORT qg_status qg_blockdots_q6_k_batch(const void *w, const void *xq, int32_t *D, int64_t b, int64_t n, int64_t k,
                                          hipStream_t stream) {
  return run_gemv_batch(2, w, xq, nullptr, D, b, n, k, stream);
}

static qg_status run_mmq(int fmt, const void *w, const void *aq, float *c, int32_t *D, int64_t m, int64_t n, int64_t k,
                  hipStream_t stream) {
  qg_status st = check_mmq(fmt, w, aq, c ? static_cast<const void *>(c) : D, m, n, k);
  if (st != QG_OK) return st;
  // the dump holds m * n dots per block (Q6_K: per 16 values)
  if (D && m > 0 && n > 0 && k > 0 && m * n > (int64_t(1) << 28) / (k / (fmt == 2 ? 16 : 32))) return QG_ERR_SHAPE;
  if (m == 0 || n == 0) return QG_OK;
  st = check_device();
  if (st != QG_OK) return st;
  return launched(qg::launch_qgemm_mmq(fmt, w, aq, c, D, m, n, k, stream));
}

QG_EXPORT qg_status qgemm_q8_0_mmq(const void *w, const void *aq, float *c, int64_t m, int64_t n, int64_t k,
                                   hipStream_t stream) {
  return run_mmq(0, w, aq, c, nullptr, m, n, k, stream);
}

QG_EXPORT qg_status qgemm_q4_k_mmq(const void *w, const void *aq, float *c, int64_t m, int64_t n, int64_t k,
                                   hipStream_t stream) {
  return run_mmq(1, w, aq, c, nullptr, m, n, k, stream);
}

QG_EXPORT qg_status qgemm_q5_k_mmq(const void *w, const void *aq, float *c, int64_t m, int64_t n, int64_t k,
                                   hipStream_t stream) {
  return run_mmq(3, w, aq, c, nullptr, m, n, k, stream);
}

QG_EXPORT qg_status qgemm_q6_k_mmq(const void *w, const void *aq, float *c, int64_t m, int64_t n, int64_t k,
                                   hipStream_t stream) {
  return run_mmq(2, w, aq, c, nullptr, m, n, k, stream);
}

QG_EXPORT qg_status qgemm_q4_0_mmq(const void *w, const void *aq, float *c, int64_t m, int64_t n, int64_t k,
                                   hipStream_t stream) {
  return run_mmq(4, w, aq, c, nullptr, m, n, k, stream);
}

QG_EXPORT qg_status qgemm_q5_0_mmq(const void *w, const void *aq, float *c, int64_t m, int64_t n, int64_t k,
                                   hipStream_t stream) {
  return run_mmq(5, w, aq, c, nullptr, m, n, k, stream);
}

QG_EXPORT qg_status moe_router_topk(const float *w_router, const float *x, int32_t *ids, float *weights,
                                    float *logits, int64_t n_tok, int64_t n_expert, int64_t n_embd, int64_t top_k,
                                    hipStream_t stream) {
  if (!w_router || (n_tok > 0 && (!x || !ids || !weights || !logits))) return QG_ERR_NULL;  // may be null when empty
  if (n_tok < 0 || n_tok > kMaxRows || n_expert < 1 || n_expert > 256 || top_k < 1 || top_k > 64 ||
      top_k > n_expert || n_embd < 4 || n_embd % 4 != 0 || n_embd > 65536)
    return QG_ERR_SHAPE;
  if (!aligned(w_router, 16) || !aligned(x, 16) || !aligned(ids, 4) || !aligned(weights, 4) ||
      !aligned(logits, 4))
    return QG_ERR_ALIGN;
  if (n_tok == 0) return QG_OK;
  qg_status st = check_device();
  if (st != QG_OK) return st;
  return launched(qg::launch_router_topk(w_router, x, ids, weights, logits, n_tok, n_expert, n_embd, top_k, stream));
}

QG_EXPORT size_t moe_qgemv_q4_k_workspace_size(int64_t n_tok, int64_t top_k, int64_t n_expert, int64_t n_ff,
                                               int64_t n_embd) {
  (void)n_expert;
  if (n_tok < 0 || top_k < 0 || n_ff < 0 || n_embd < 0) return 0;
  return qg::moe_layout(n_tok, top_k, n_ff, n_embd).total;
}

namespace qg {

qg_status check_gfx950() { return check_device(); }

MoeLayout moe_layout(int64_t n_tok, int64_t top_k, int64_t n_ff, int64_t n_embd) {
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  const size_t P = (size_t)(n_tok * top_k);
  MoeLayout l;
  l.hq_off = 0;
  l.gu_off = up(P * (size_t)(n_ff / 32) * 36);  // Q8_1: 36 bytes per 32 values
  l.z_off = l.gu_off + up(P * (size_t)(2 * n_ff) * sizeof(float));
  l.total = l.z_off + up(P * (size_t)n_embd * sizeof(float));
  return l;
}

// Arguments of the MoE call other than the workspace: nulls, shapes, alignment.
qg_status moe_check(const void *w_gate_up, const void *w_down, const void *xq, const int32_t *ids,
                    const float *weights, const float *out, int64_t n_tok, int64_t top_k, int64_t n_expert,
                    int64_t n_ff, int64_t n_embd) {
  if (!w_gate_up || !w_down || !xq || !ids || !weights || !out) return QG_ERR_NULL;
  if (n_tok < 0 || top_k < 1 || top_k > 64 || n_expert < 1 || n_expert > (1 << 16) || n_ff < 0 || n_embd < 0)
    return QG_ERR_SHAPE;
  if (n_ff % 256 != 0 || n_embd % 256 != 0 || n_ff > (1 << 20) || n_embd > (1 << 20)) return QG_ERR_SHAPE;
  if (n_tok * top_k > (1 << 20)) return QG_ERR_SHAPE;
  if (n_ff == 0 || n_embd == 0) return QG_ERR_SHAPE;
  if (!aligned(w_gate_up, 16) || !aligned(w_down, 16) || !aligned(xq, 16) || !aligned(ids, 4) ||
      !aligned(weights, 4) || !aligned(out, 4))
    return QG_ERR_ALIGN;
  return QG_OK;
}

// Enqueues the MoE kernels with the workspace at ws (checked arguments, a
// workspace of at least moe_layout().total bytes, 256-byte aligned).
qg_status moe_enqueue(const void *w_gate_up, const void *w_down, const void *xq, const int32_t *ids,
                      const float *weights, float *out, int64_t n_tok, int64_t top_k, int64_t n_expert, int64_t n_ff,
                      int64_t n_embd, uint8_t *ws, hipStream_t stream, int32_t *D_gu, int32_t *D_dn) {
  const MoeLayout lay = moe_layout(n_tok, top_k, n_ff, n_embd);
  MoeArgs a;
  a.w_gu = w_gate_up;
  a.w_down = w_down;
  a.xq = xq;
  a.ids = ids;
  a.weights = weights;
  a.out = out;
  a.n_tok = n_tok;
  a.top_k = top_k;
  a.n_expert = n_expert;
  a.n_ff = n_ff;
  a.n_embd = n_embd;
  a.ws_hq = ws + lay.hq_off;
  a.ws_gu = reinterpret_cast<float *>(ws + lay.gu_off);
  a.ws_z = reinterpret_cast<float *>(ws + lay.z_off);
  if (D_gu) return launched(launch_moe_q4_k_dump(a, D_gu, D_dn, stream));
  return launched(launch_moe_q4_k(a, stream));
}

}  // namespace qg

QG_EXPORT qg_status moe_qgemv_q4_k(const void *w_gate_up, const void *w_down, const void *xq, const int32_t *ids,
                                   const float *weights, float *out, int64_t n_tok, int64_t top_k, int64_t n_expert,
                                   int64_t n_ff, int64_t n_embd, void *workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  qg_status st = qg::moe_check(w_gate_up, w_down, xq, ids, weights, out, n_tok, top_k, n_expert, n_ff, n_embd);
  if (st != QG_OK) return st;
  if (!workspace) return QG_ERR_NULL;
  if (!aligned(workspace, 256)) return QG_ERR_ALIGN;
  if (workspace_bytes < qg::moe_layout(n_tok, top_k, n_ff, n_embd).total) return QG_ERR_WORKSPACE;
  if (n_tok == 0) return QG_OK;
  st = check_device();
  if (st != QG_OK) return st;
  return qg::moe_enqueue(w_gate_up, w_down, xq, ids, weights, out, n_tok, top_k, n_expert, n_ff, n_embd,
                         static_cast<uint8_t *>(workspace), stream);
}

QG_EXPORT qg_status qg_blockdots_q8_0(const void *w, const void *xq, int32_t *D, int64_t n, int64_t k,
                                      hipStream_t stream) {
  qg_status st = check_gemv(0, w, xq, D, n, k);
  return st != QG_OK ? st : run_gemv(0, w, xq, nullptr, D, nullptr, n, k, stream);
}

QG_EXPORT qg_status qg_blockdots_q4_k(const void *w, const void *xq, int32_t *D, int32_t *S, int64_t n, int64_t k,
                                      hipStream_t stream) {
  if (!S) return QG_ERR_NULL;
  if (!aligned(S, 4)) return QG_ERR_ALIGN;
  qg_status st = check_gemv(1, w, xq, D, n, k);
  return st != QG_OK ? st : run_gemv(1, w, xq, nullptr, D, S, n, k, stream);
}

QG_EXPORT qg_status qg_blockdots_q5_k(const void *w, const void *xq, int32_t *D, int32_t *S, int64_t n, int64_t k,
                                      hipStream_t stream) {
  if (!S) return QG_ERR_NULL;
  if (!aligned(S, 4)) return QG_ERR_ALIGN;
  qg_status st = check_gemv(3, w, xq, D, n, k);
  return st != QG_OK ? st : run_gemv(3, w, xq, nullptr, D, S, n, k, stream);
}

QG_EXPORT qg_status qg_blockdots_q6_k(const void *w, const void *xq, int32_t *D, int64_t n, int64_t k,
                                      hipStream_t stream) {
  qg_status st = check_gemv(2, w, xq, D, n, k);
  return st != QG_OK ? st : run_gemv(2, w, xq, nullptr, D, nullptr, n, k, stream);
}

QG_EXPORT qg_status qg_blockdots_q4_0(const void *w, const void *xq, int32_t *D, int64_t n, int64_t k,
                                      hipStream_t stream) {
  qg_status st = check_gemv(4, w, xq, D, n, k);
  return st != QG_OK ? st : run_gemv(4, w, xq, nullptr, D, nullptr, n, k, stream);
}

QG_EXPORT qg_status qg_blockdots_q5_0(const void *w, const void *xq, int32_t *D, int64_t n, int64_t k,
                                      hipStream_t stream) {
  qg_status st = check_gemv(5, w, xq, D, n, k);
  return st != QG_OK ? st : run_gemv(5, w, xq, nullptr, D, nullptr, n, k, stream);
}

QG_EXPORT qg_status qg_blockdots_q4_0_mmq(const void *w, const void *aq, int32_t *D, int64_t m, int64_t n, int64_t k,
                                          hipStream_t stream) {
  return run_mmq(4, w, aq, nullptr, D, m, n, k, stream);
}

QG_EXPORT qg_status qg_blockdots_q5_0_mmq(const void *w, const void *aq, int32_t *D, int64_t m, int64_t n, int64_t k,
                                          hipStream_t stream) {
  return run_mmq(5, w, aq, nullptr, D, m, n, k, stream);
}

QG_EXPORT qg_status qg_blockdots_q8_0_mmq(const void *w, const void *aq, int32_t *D, int64_t m, int64_t n, int64_t k,
                                          hipStream_t stream) {
  return run_mmq(0, w, aq, nullptr, D, m, n, k, stream);
}

QG_EXPORT qg_status qg_blockdots_q4_k_mmq(const void *w, const void *aq, int32_t *D, int64_t m, int64_t n, int64_t k,
                                          hipStream_t stream) {
  return run_mmq(1, w, aq, nullptr, D, m, n, k, stream);
}

QG_EXPORT qg_status qg_blockdots_q5_k_mmq(const void *w, const void *aq, int32_t *D, int64_t m, int64_t n, int64_t k,
                                          hipStream_t stream) {
  return run_mmq(3, w, aq, nullptr, D, m, n, k, stream);
}

QG_EXPORT qg_status qg_blockdots_q6_k_mmq(const void *w, const void *aq, int32_t *D, int64_t m, int64_t n, int64_t k,
                                          hipStream_t stream) {
  return run_mmq(2, w, aq, nullptr, D, m, n, k, stream);
}

QG_EXPORT qg_status qg_peak_read(const void *src, int64_t bytes, uint32_t *sink, int64_t sink_entries, int32_t grid,
                                 int32_t threads, int32_t loads, int32_t nontemporal, hipStream_t stream) {
  if (!src || !sink) return QG_ERR_NULL;
  if (bytes <= 0 || bytes % 16 != 0 || grid < 1 || grid > (1 << 20) || threads < 64 || threads > 1024 ||
      threads % 64 != 0 || (loads != 4 && loads != 8) || sink_entries < grid)
    return QG_ERR_SHAPE;
  if (!aligned(src, 16) || !aligned(sink, 4)) return QG_ERR_ALIGN;
  qg_status st = check_device();
  if (st != QG_OK) return st;
  return launched(qg::launch_peak_read(src, bytes, sink, grid, threads, loads, nontemporal != 0, stream));
}

QG_EXPORT qg_status qg_peak_mfma_i8(int32_t *sink, int64_t sink_entries, int64_t iters, int64_t *ops,
                                    hipStream_t stream) {
  if (!sink || !ops) return QG_ERR_NULL;
  if (iters < 1 || iters > (int64_t(1) << 24)) return QG_ERR_SHAPE;
  if (!aligned(sink, 4)) return QG_ERR_ALIGN;
  qg_status st = check_device();
  if (st != QG_OK) return st;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess)
    return QG_ERR_NO_DEVICE;
  if (sink_entries < (int64_t)cus * 8) return QG_ERR_SHAPE;
  return launched(qg::launch_peak_mfma_i8(sink, iters, ops, stream));
}

QG_EXPORT qg_status qg_blockdots_moe_q4_k(const void *w_gate_up, const void *w_down, const void *xq,
                                          const int32_t *ids, const float *weights, int64_t n_tok, int64_t top_k,
                                          int64_t n_expert, int64_t n_ff, int64_t n_embd, void *workspace,
                                          size_t workspace_bytes, int32_t *D_gu, int32_t *D_dn, hipStream_t stream) {
  // D_gu stands in for out (checked for null and alignment; out is not written)
  qg_status st = qg::moe_check(w_gate_up, w_down, xq, ids, weights, reinterpret_cast<const float *>(D_gu), n_tok,
                               top_k, n_expert, n_ff, n_embd);
  if (st != QG_OK) return st;
  if (!workspace || !D_dn) return QG_ERR_NULL;
  if (!aligned(workspace, 256) || !aligned(D_dn, 4)) return QG_ERR_ALIGN;
  if (workspace_bytes < qg::moe_layout(n_tok, top_k, n_ff, n_embd).total) return QG_ERR_WORKSPACE;
  const int64_t P = n_tok * top_k;
  if (P * 2 * n_ff > (int64_t(1) << 29) / (n_embd / 32) || P * n_embd > (int64_t(1) << 29) / (n_ff / 32))
    return QG_ERR_SHAPE;
  if (n_tok == 0) return QG_OK;
  st = check_device();
  if (st != QG_OK) return st;
  return qg::moe_enqueue(w_gate_up, w_down, xq, ids, weights, nullptr, n_tok, top_k, n_expert, n_ff, n_embd,
                         static_cast<uint8_t *>(workspace), stream, D_gu, D_dn);
}

QG_EXPORT int qg_moe_q4_k_launches(int64_t n_tok, int64_t top_k, int64_t n_expert, int64_t n_ff, int64_t n_embd) {
  if (n_tok <= 0 || top_k < 1 || n_expert < 1 || n_ff <= 0 || n_embd <= 0 || n_ff % 256 || n_embd % 256) return 0;
  qg::MoeArgs a{};
  a.n_tok = n_tok;
  a.top_k = top_k;
  a.n_expert = n_expert;
  a.n_ff = n_ff;
  a.n_embd = n_embd;
  return qg::moe_two_kernel_path(a) ? 2 : 4;
}
