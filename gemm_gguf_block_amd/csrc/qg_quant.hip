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

// One workgroup (256 threads) per row: thread t sums the squares of float4s t,
// t + 256, ... in that order (so the fp32 sum, hence r, depends on k alone);
// then the row is read again (from cache) and quantized, 32 blocks per pass,
// 8 lanes per block.  Holding the row in registers between the passes, or
// loading gamma with the first pass, measured slower on MI355X (7.9 and
// 8.6 us against 7.5 us for 512 x 4096).
__global__ __launch_bounds__(256) void rmsnorm_quantize_q8_1_kernel(const float *__restrict__ x,
                                                                    const float *__restrict__ gamma, float eps,
                                                                    uint8_t *__restrict__ xq,
                                                                    float *__restrict__ r_out, int k) {
  __shared__ float red[4];
  const float *xr = x + (int64_t)blockIdx.x * k;
  float ss = 0.f;
  for (int i = threadIdx.x; i < k / 4; i += 256) ss = sumsq4(reinterpret_cast<const float4 *>(xr)[i], ss);
  const float r = rms_from_partial(ss, k, eps, red);
  if (r_out && threadIdx.x == 0) r_out[blockIdx.x] = r;
  const int nb = k / 32, j = threadIdx.x & 7;
  uint8_t *dst = xq + (int64_t)blockIdx.x * nb * kQ8_1Bytes;
  for (int base = 0; base < nb; base += 256 / 8) {
    const int b = base + (int)(threadIdx.x >> 3);
    const bool live = b < nb;  // uniform per group of 8
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (live) {
      const float4 a = reinterpret_cast<const float4 *>(xr)[b * 8 + j];
      const float4 g = reinterpret_cast<const float4 *>(gamma)[b * 8 + j];
      v = make_float4((a.x * r) * g.x, (a.y * r) * g.y, (a.z * r) * g.z, (a.w * r) * g.w);
    }
    quantize_block_q8_1(v, dst + (int64_t)b * kQ8_1Bytes, j, live);
  }
}

hipError_t launch_rmsnorm_quantize_q8_1(const float *x, const float *gamma, float eps, void *xq, float *r_out,
                                        int64_t rows, int64_t k, hipStream_t stream) {
  hipLaunchKernelGGL(rmsnorm_quantize_q8_1_kernel, dim3((unsigned)rows), dim3(256), 0, stream, x, gamma, eps,
                     static_cast<uint8_t *>(xq), r_out, (int)k);
  return hipGetLastError();
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
