// qg_noalloc.hip -- moe_qgemv_q4_k_noalloc: the MoE expert FFN for callers
// that cannot allocate device memory (code under HIP graph capture, serving
// loops, harnesses that forbid hipMalloc).  Its workspace is a file-scope
// device array of kScratchBytes, one copy per GPU, held until the process
// ends; the entry point itself allocates nothing.
//
// Each GPU's copy is at its own device address.  The host-side name of the
// array is only a stand-in for it, so the address is asked for once per
// device (hipGetSymbolAddress, with that device current, on the first call
// there) and that address is what the kernels receive.  All calls on one GPU
// share its copy: calls that overlap on one GPU (different streams, no
// ordering between them) race.  The kernels write every workspace byte they
// read before reading it within the call, so nothing of an earlier call's
// contents needs clearing.
#include <atomic>
#include <mutex>

#include "qg_launch.h"

#define QG_EXPORT extern "C" __attribute__((visibility("default")))

// 32 MiB: 1000 (token, slot) pairs of a 768 x 2048 expert FFN fit.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<uint8_t *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's copy of scratch.
qg_status scratch_address(uint8_t **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return QG_ERR_NO_DEVICE;
  if (dev >= kMaxDevices) return QG_ERR_ARCH;
  uint8_t *p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      void *q = nullptr;
      if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return QG_ERR_LAUNCH;
      p = static_cast<uint8_t *>(q);
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return QG_OK;
}

}  // namespace

QG_EXPORT size_t moe_qgemv_q4_k_noalloc_max_workspace(void) { return kScratchBytes; }

QG_EXPORT qg_status moe_qgemv_q4_k_noalloc(const void *w_gate_up, const void *w_down, const void *xq,
                                           const int32_t *ids, const float *weights, float *out, int64_t n_tok,
                                           int64_t top_k, int64_t n_expert, int64_t n_ff, int64_t n_embd,
                                           hipStream_t stream) {
  qg_status st = qg::moe_check(w_gate_up, w_down, xq, ids, weights, out, n_tok, top_k, n_expert, n_ff, n_embd);
  if (st != QG_OK) return st;
  if (qg::moe_layout(n_tok, top_k, n_ff, n_embd).total > kScratchBytes) return QG_ERR_WORKSPACE;
  if (n_tok == 0) return QG_OK;
  st = qg::check_gfx950();
  if (st != QG_OK) return st;
  uint8_t *ws = nullptr;
  st = scratch_address(&ws);
  if (st != QG_OK) return st;
  return qg::moe_enqueue(w_gate_up, w_down, xq, ids, weights, out, n_tok, top_k, n_expert, n_ff, n_embd, ws, stream);
}
