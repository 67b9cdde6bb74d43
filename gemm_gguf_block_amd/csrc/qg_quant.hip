// qg_quant.hip -- f32 activations -> Q8_1 blocks (one wave = 8 blocks).
#include "qg_launch.h"
#include "qg_quant.h"

namespace qg {

__global__ __launch_bounds__(256) void quantize_q8_1_kernel(const float *__restrict__ x, uint8_t *__restrict__ xq,
                                                            int64_t nblocks) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t b = t >> 3;  // block index over rows*k/32
  const int j = (int)(t & 7);
  const bool live = b < nblocks;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (live) v = *reinterpret_cast<const float4 *>(x + b * 32 + 4 * j);
  quantize_block_q8_1(v, xq + b * kQ8_1Bytes, j, live);
}

hipError_t launch_quantize_q8_1(const float *x, void *xq, int64_t rows, int64_t k, hipStream_t stream) {
  const int64_t nblocks = rows * (k / 32);
  const int64_t threads = nblocks * 8;
  const int64_t grid = (threads + 255) / 256;
  hipLaunchKernelGGL(quantize_q8_1_kernel, dim3((unsigned)grid), dim3(256), 0, stream, x,
                     static_cast<uint8_t *>(xq), nblocks);
  return hipGetLastError();
}

}  // namespace qg
