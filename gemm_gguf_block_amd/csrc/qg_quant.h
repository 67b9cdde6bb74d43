// qg_quant.h -- Q8_1 quantization of one 32-value block by 8 lanes, and the
// RMS scale of an activation row.
//
// Rule (the activation side of every integer dot): amax = max|x|;
// d = amax/127 in fp32 (correctly rounded division); q = round half away from
// zero of x/d, from the fp32 d, clamped to [-127, 127]; s = d*sum(q) as an
// fp32 product; d and s stored as fp16, each rounded once (nearest even).
#pragma once
#include "qg_device.h"

namespace qg {

// One lane's share of a quantized block: its four codes packed in a dword,
// the fp32 d, and the sum of the codes of the lane's group of 8.
struct Q81Part {
  uint32_t packed;
  float d;
  int sum;
};

// Lanes work in aligned groups of 8; lane j of a group holds values 4j..4j+3
// of the block in v.  All 8 lanes of the group must call this together.
__device__ __forceinline__ Q81Part quantize_part_q8_1(float4 v) {
  float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  amax = group_max<8>(amax);
  const float d = amax / 127.0f;
  int q0 = 0, q1 = 0, q2 = 0, q3 = 0;
  if (amax != 0.0f) {
    q0 = (int)__builtin_roundf(v.x / d);
    q1 = (int)__builtin_roundf(v.y / d);
    q2 = (int)__builtin_roundf(v.z / d);
    q3 = (int)__builtin_roundf(v.w / d);
    q0 = min(127, max(-127, q0));
    q1 = min(127, max(-127, q1));
    q2 = min(127, max(-127, q2));
    q3 = min(127, max(-127, q3));
  }
  Q81Part r;
  r.packed = (uint32_t)(q0 & 0xff) | ((uint32_t)(q1 & 0xff) << 8) | ((uint32_t)(q2 & 0xff) << 16) |
             ((uint32_t)(q3 & 0xff) << 24);
  r.d = d;
  r.sum = group_isum<8>(q0 + q1 + q2 + q3);
  return r;
}

// The d|s dword of a block (lane 0 of the group writes it).
__device__ __forceinline__ uint32_t q81_header(const Q81Part &p) {
  // s is the fp32 product, rounded to fp16 afterwards.  The empty asm pins
  // the product in a VGPR so it cannot be fused with the conversion into one
  // v_fma_mix that would round only once.
  float s = p.d * (float)p.sum;
  asm volatile("" : "+v"(s));
  return f2h(p.d) | (f2h(s) << 16);
}

// If `store`, lane j writes qs dword j and lane 0 writes the d|s dword of the
// 36-byte block at blk (4-byte aligned).
__device__ __forceinline__ void quantize_block_q8_1(float4 v, uint8_t *blk, int j, bool store) {
  const Q81Part p = quantize_part_q8_1(v);
  if (store) {
    *reinterpret_cast<uint32_t *>(blk + 4 + 4 * j) = p.packed;
    if (j == 0) *reinterpret_cast<uint32_t *>(blk) = q81_header(p);
  }
}

// Sum of squares of one thread's float4s, in index order: the first term of
// the RMS scale below.
__device__ __forceinline__ float sumsq4(const float4 &v, float ss) {
  ss = fmaf(v.x, v.x, ss);
  ss = fmaf(v.y, v.y, ss);
  ss = fmaf(v.z, v.z, ss);
  return fmaf(v.w, v.w, ss);
}

// r = 1 / sqrt(total / k + eps) from each thread's partial sum of squares.
// Whole workgroup of 256 threads; `red` is 4 floats of LDS.  Butterfly within
// each wave, then the four wave sums in order.
__device__ __forceinline__ float rms_from_partial(float ss, int k, float eps, float *red) {
  ss = group_sum<64>(ss);
  __syncthreads();  // `red` may still be read by an earlier call
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float total = ((red[0] + red[1]) + red[2]) + red[3];
  return 1.0f / __builtin_sqrtf(total / (float)k + eps);
}

}  // namespace qg
