// qg_peak.hip -- measured ceilings for the roofline fractions: a streaming
// read of HBM and a loop of int8 MFMAs.  They compute nothing of the product;
// the bench times them beside the product kernels so that each kernel's rate
// can be set against what this GPU reaches, as well as against the published
// peaks (the per-kernel accounting of infr page, "Per-op device profiling").
#include "qg_device.h"
#include "qg_launch.h"

namespace qg {

namespace {

typedef uint32_t u32x4n __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// Every 16-byte word of src once: thread t of the grid reads words t,
// t + S, t + 2S, ... (S = threads in the grid), LOADS of them issued before
// any is used.  The words are folded into one value that is stored only if it
// equals a constant no input here produces, so no load can be dropped and the
// kernel writes (almost) nothing.
template <int LOADS, bool NT>
__global__ __launch_bounds__(1024) void peak_read_kernel(const u32x4n *__restrict__ src, int64_t nvec,
                                                         uint32_t *__restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  for (int64_t base = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; base < nvec; base += stride * LOADS) {
    u32x4n v[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int64_t idx = base + i * stride;
      if (idx < nvec)
        v[i] = NT ? __builtin_nontemporal_load(src + idx) : src[idx];
      else
        v[i] = u32x4n{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < LOADS; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

// Four independent chains of v_mfma_i32_32x32x32_i8 per wave, `iters` long:
// 4 * 2 * 32 * 32 * 32 int8 operations per wave and iteration.
__global__ __launch_bounds__(256) void peak_mfma_i8_kernel(int32_t *__restrict__ sink, int64_t iters) {
  const int l = (int)threadIdx.x;
  const v4i a = {l, l + 1, l + 2, l + 3}, b = {3 * l, l ^ 5, l + 7, l * l};
  v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int64_t i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
  }
  int s = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] ^ c1[r] ^ c2[r] ^ c3[r];
  if (s == 0x1b873593) sink[blockIdx.x] = s;
}

template <int LOADS, bool NT>
hipError_t read_launch(const void *src, int64_t bytes, uint32_t *sink, int grid, int threads, hipStream_t stream) {
  hipLaunchKernelGGL((peak_read_kernel<LOADS, NT>), dim3((unsigned)grid), dim3((unsigned)threads), 0, stream,
                     static_cast<const u32x4n *>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_peak_read(const void *src, int64_t bytes, uint32_t *sink, int grid, int threads, int loads, bool nt,
                            hipStream_t stream) {
  if (loads == 4) return nt ? read_launch<4, true>(src, bytes, sink, grid, threads, stream)
                            : read_launch<4, false>(src, bytes, sink, grid, threads, stream);
  return nt ? read_launch<8, true>(src, bytes, sink, grid, threads, stream)
            : read_launch<8, false>(src, bytes, sink, grid, threads, stream);
}

hipError_t launch_peak_mfma_i8(int32_t *sink, int64_t iters, int64_t *ops, hipStream_t stream) {
  int dev = 0, cus = 1;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 1;
  // eight 4-wave workgroups per CU: eight waves per SIMD
  const int64_t grid = (int64_t)cus * 8;
  *ops = grid * 4 * iters * 4 * (2LL * 32 * 32 * 32);
  hipLaunchKernelGGL(peak_mfma_i8_kernel, dim3((unsigned)grid), dim3(256), 0, stream, sink, iters);
  return hipGetLastError();
}

}  // namespace qg
