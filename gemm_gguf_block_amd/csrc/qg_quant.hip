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
// then the row is scaled and quantized, 32 blocks per pass, 8 lanes per block.
// Float4 t + 256q is also the value quad the thread quantizes in pass q, so
// rows of up to 4096 values stay in registers between the two steps, loaded
// together with gamma (all eight loads in flight at once); longer rows are read
// again from cache, four passes' loads at a time.  (512 x 4096 on MI355X:
// 7.07 us with one load in flight per thread, 6.11 us as here.)
__global__ __launch_bounds__(256) void rmsnorm_quantize_q8_1_kernel(const float *__restrict__ x,
                                                                    const float *__restrict__ gamma, float eps,
                                                                    uint8_t *__restrict__ xq,
                                                                    float *__restrict__ r_out, int k) {
  __shared__ float red[4];
  const float *xr = x + (int64_t)blockIdx.x * k;
  float ss = 0.f;
  const int n4 = k / 4;
  if (n4 <= 4 * 256) {  // uniform: the whole row fits four float4 per thread
    // float4 t + 256q of the row is also the value quad (block 32q + t/8,
    // lane t%8) this thread quantizes: the row stays in registers, and the
    // gamma loads go out with it
    float4 a[4], g[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i4 = min((int)threadIdx.x + 256 * q, n4 - 1);
      a[q] = reinterpret_cast<const float4 *>(xr)[i4];
      g[q] = reinterpret_cast<const float4 *>(gamma)[i4];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if ((int)threadIdx.x + 256 * q < n4) ss = sumsq4(a[q], ss);
    const float r = rms_from_partial(ss, k, eps, red);
    if (r_out && threadIdx.x == 0) r_out[blockIdx.x] = r;
    const int nb = k / 32, j = threadIdx.x & 7;
    uint8_t *dst = xq + (int64_t)blockIdx.x * nb * kQ8_1Bytes;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int b = q * 32 + (int)(threadIdx.x >> 3);
      const bool live = b < nb;  // uniform per group of 8
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (live) v = make_float4((a[q].x * r) * g[q].x, (a[q].y * r) * g[q].y, (a[q].z * r) * g[q].z, (a[q].w * r) * g[q].w);
      quantize_block_q8_1(v, dst + (int64_t)b * kQ8_1Bytes, j, live);
    }
    return;
  }
  int i = threadIdx.x;
  // four loads in flight per thread, summed in index order
  for (; i + 3 * 256 < n4; i += 4 * 256) {
    const float4 v0 = reinterpret_cast<const float4 *>(xr)[i], v1 = reinterpret_cast<const float4 *>(xr)[i + 256],
                 v2 = reinterpret_cast<const float4 *>(xr)[i + 512], v3 = reinterpret_cast<const float4 *>(xr)[i + 768];
    ss = sumsq4(v0, ss);
    ss = sumsq4(v1, ss);
    ss = sumsq4(v2, ss);
    ss = sumsq4(v3, ss);
  }
  for (; i < n4; i += 256) ss = sumsq4(reinterpret_cast<const float4 *>(xr)[i], ss);
  const float r = rms_from_partial(ss, k, eps, red);
  if (r_out && threadIdx.x == 0) r_out[blockIdx.x] = r;
  const int nb = k / 32, j = threadIdx.x & 7;
  uint8_t *dst = xq + (int64_t)blockIdx.x * nb * kQ8_1Bytes;
  // four passes of 32 blocks per round, all their loads first (groups past
  // the last block read block 0 and store nothing)
  for (int base = 0; base < nb; base += 4 * (256 / 8)) {
    float4 a[4], g[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int b = base + q * 32 + (int)(threadIdx.x >> 3);
      const int bc = b < nb ? b : 0;
      a[q] = reinterpret_cast<const float4 *>(xr)[bc * 8 + j];
      g[q] = reinterpret_cast<const float4 *>(gamma)[bc * 8 + j];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int b = base + q * 32 + (int)(threadIdx.x >> 3);
      const bool live = b < nb;  // uniform per group of 8
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (live) v = make_float4((a[q].x * r) * g[q].x, (a[q].y * r) * g[q].y, (a[q].z * r) * g[q].z, (a[q].w * r) * g[q].w);
      quantize_block_q8_1(v, dst + (int64_t)b * kQ8_1Bytes, j, live);
    }
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
