// qg_launch.h -- internal launchers (validated arguments only; called by the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace qg {

// Workgroups of `Kernel` (`threads` per workgroup, `lds` bytes of dynamic LDS)
// resident on the current device at once, for sizing persistent grids.  The
// kernel is a template argument so that every kernel has a cache of its own
// (kernels of one signature would otherwise share it); per device it holds the
// last LDS size asked, as (lds << 32 | count) in one word so that readers never
// see a torn pair.
template <auto Kernel>
int64_t resident_blocks(int threads, size_t lds) {
  constexpr int kMaxDev = 64;
  static std::atomic<uint64_t> cached[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) dev = -1;
  const uint64_t c = dev >= 0 ? cached[dev].load(std::memory_order_relaxed) : 0;
  if (c != 0 && (c >> 32) == (uint64_t)lds) return (int64_t)(c & 0xffffffffu);
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, Kernel, threads, lds) != hipSuccess || per_cu < 1)
    per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev < 0 ? 0 : dev) != hipSuccess || cus < 1)
    cus = 1;
  const int64_t v = (int64_t)per_cu * cus;
  if (dev >= 0) cached[dev].store(((uint64_t)lds << 32) | (uint64_t)v, std::memory_order_relaxed);
  return v;
}

hipError_t launch_quantize_q8_1(const float *x, void *xq, int64_t rows, int64_t k, hipStream_t stream);

// fmt: 0 = Q8_0, 1 = Q4_K, 2 = Q6_K, 3 = Q5_K, 4 = Q4_0, 5 = Q5_0.  D/S
// non-null selects the per-block dot dump instead of y.
hipError_t launch_qgemv(int fmt, const void *w, const void *xq, float *y, int32_t *D, int32_t *S, int64_t n,
                        int64_t k, hipStream_t stream);

// f32 rows -> Q8_1 of x * r * gamma, r = 1 / sqrt(mean(x^2) + eps) per row
// (r_out nullable).
hipError_t launch_rmsnorm_quantize_q8_1(const float *x, const float *gamma, float eps, void *xq, float *r_out,
                                        int64_t rows, int64_t k, hipStream_t stream);

// Small-batch GEMV: nb (1..8) Q8_1 rows [nb][k/32] against the weights; y is
// [nb][n].  D non-null selects the per-block dot dump of the kernel the
// product call dispatches to for this nb: D[nb][n][k/32] (Q6_K: [k/16]).
hipError_t launch_qgemv_batch(int fmt, const void *w, const void *xq, float *y, int32_t *D, int64_t nb, int64_t n,
                              int64_t k, hipStream_t stream);

// Small-batch Q4_K / Q6_K GEMV on the int8 matrix cores (nb <= 8); D as above.
hipError_t launch_qgemv_batch_mfma_q8_0(const void *w, const void *xq, float *y, int32_t *D, int64_t nb, int64_t n,
                                        int64_t k, hipStream_t stream);
hipError_t launch_qgemv_batch_mfma_q4k(const void *w, const void *xq, float *y, int32_t *D, int64_t nb, int64_t n,
                                       int64_t k, hipStream_t stream);
hipError_t launch_qgemv_batch_mfma_q6k(const void *w, const void *xq, float *y, int32_t *D, int64_t nb, int64_t n,
                                       int64_t k, hipStream_t stream);

// Prefill product on the int8 matrix cores; fmt as for launch_qgemv.  D
// non-null selects the per-block (Q6_K: per 16-value sub-block) dot dump.
hipError_t launch_qgemm_mmq(int fmt, const void *w, const void *aq, float *c, int32_t *D, int64_t m, int64_t n,
                            int64_t k, hipStream_t stream);

// MoE router: logits, top-k, softmax per token (validated arguments).
hipError_t launch_router_topk(const float *w_router, const float *x, int32_t *ids, float *weights, float *logits,
                              int64_t n_tok, int64_t n_expert, int64_t n_embd, int64_t top_k, hipStream_t stream);

// Measurement references (not part of the product): a streaming read of
// `bytes` (a multiple of 16) with `grid` x `threads` threads and `loads` (4 or
// 8) loads in flight per thread, plain or non-temporal; and a loop of int8
// MFMAs on eight 4-wave workgroups per CU, whose int8 operation count is
// returned in *ops.  sink: grid entries (read) or 8 * CUs entries (MFMA).
hipError_t launch_peak_read(const void *src, int64_t bytes, uint32_t *sink, int grid, int threads, int loads, bool nt,
                            hipStream_t stream);
hipError_t launch_peak_mfma_i8(int32_t *sink, int64_t iters, int64_t *ops, hipStream_t stream);

struct MoeArgs {
  const void *w_gu, *w_down, *xq;
  const int32_t *ids;
  const float *weights;
  float *out;
  int64_t n_tok, top_k, n_expert, n_ff, n_embd;
  uint8_t *ws_hq;    // Q8_1 h^ per pair
  float *ws_gu;      // g|u per pair
  float *ws_z;       // weighted down projection per pair (four-kernel path)
};
hipError_t launch_moe_q4_k(const MoeArgs &a, hipStream_t stream);
// The same kernels' dump instances: exact dots of gate/up D_gu [P][2F][H/32]
// and of down D_dn [P][H][F/32] (after the gate/up product, which the down
// dump needs); out and z are not written.
hipError_t launch_moe_q4_k_dump(const MoeArgs &a, int32_t *D_gu, int32_t *D_dn, hipStream_t stream);
// True when the call runs the two-kernel path, false for the four-kernel one.
bool moe_two_kernel_path(const MoeArgs &a);

// Workspace region offsets for the MoE call (each 256-byte aligned).
struct MoeLayout {
  size_t hq_off, gu_off, z_off, total;
};
MoeLayout moe_layout(int64_t n_tok, int64_t top_k, int64_t n_ff, int64_t n_embd);

}  // namespace qg

#include "../../include/qgguf.h"

namespace qg {

// The C ABI's shared checks (qg_api.hip): the current device is gfx950; the
// MoE call's arguments other than its workspace.  moe_enqueue launches the
// MoE kernels with the workspace at ws (checked arguments; ws 256-byte aligned
// and at least moe_layout().total bytes).
qg_status check_gfx950();
qg_status moe_check(const void *w_gate_up, const void *w_down, const void *xq, const int32_t *ids,
                    const float *weights, const float *out, int64_t n_tok, int64_t top_k, int64_t n_expert,
                    int64_t n_ff, int64_t n_embd);
qg_status moe_enqueue(const void *w_gate_up, const void *w_down, const void *xq, const int32_t *ids,
                      const float *weights, float *out, int64_t n_tok, int64_t top_k, int64_t n_expert, int64_t n_ff,
                      int64_t n_embd, uint8_t *ws, hipStream_t stream, int32_t *D_gu = nullptr,
                      int32_t *D_dn = nullptr);

}  // namespace qg
