// Host-only stand-ins for the kernel launchers of libqgguf, so that the C
// ABI's argument checks (qg_api.hip, qg_noalloc.hip) can be built for the
// host alone under AddressSanitizer / UndefinedBehaviorSanitizer.  Nothing
// here runs a kernel: every launcher reports a launch failure.
#include "../../gemm_gguf_block_amd/csrc/qg_launch.h"

namespace qg {
hipError_t launch_quantize_q8_1(const float *, void *, int64_t, int64_t, hipStream_t) { return hipErrorLaunchFailure; }
hipError_t launch_qgemv(int, const void *, const void *, float *, int32_t *, int32_t *, int64_t, int64_t,
                        hipStream_t) { return hipErrorLaunchFailure; }
hipError_t launch_rmsnorm_quantize_q8_1(const float *, const float *, float, void *, float *, int64_t, int64_t,
                                        hipStream_t) { return hipErrorLaunchFailure; }
hipError_t launch_qgemv_batch(int, const void *, const void *, float *, int32_t *, int64_t, int64_t, int64_t,
                              hipStream_t) { return hipErrorLaunchFailure; }
hipError_t launch_qgemm_mmq(int, const void *, const void *, float *, int32_t *, int64_t, int64_t, int64_t,
                            hipStream_t) { return hipErrorLaunchFailure; }
hipError_t launch_router_topk(const float *, const float *, int32_t *, float *, float *, int64_t, int64_t, int64_t,
                              int64_t, hipStream_t) { return hipErrorLaunchFailure; }
hipError_t launch_moe_q4_k(const MoeArgs &, hipStream_t) { return hipErrorLaunchFailure; }
hipError_t launch_moe_q4_k_dump(const MoeArgs &, int32_t *, int32_t *, hipStream_t) { return hipErrorLaunchFailure; }
bool moe_two_kernel_path(const MoeArgs &) { return false; }
hipError_t launch_peak_read(const void *, int64_t, uint32_t *, int, int, int, bool, hipStream_t) {
  return hipErrorLaunchFailure;
}
hipError_t launch_peak_mfma_i8(int32_t *, int64_t, int64_t *, hipStream_t) { return hipErrorLaunchFailure; }
}  // namespace qg
