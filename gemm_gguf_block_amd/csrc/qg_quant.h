// qg_quant.h -- Q8_1 quantization of one 32-value block by 8 lanes.
//
// Rule (the activation side of every integer dot): amax = max|x|;
// d = amax/127 in fp32 (correctly rounded division); q = round half away from
// zero of x/d, from the fp32 d, clamped to [-127, 127]; s = d*sum(q) as an
// fp32 product; d and s stored as fp16, each rounded once (nearest even).
#pragma once
#include "qg_device.h"

namespace qg {

// Lanes work in aligned groups of 8; lane j of a group holds values 4j..4j+3
// of the block in v.  All 8 lanes of the group must call this together.
// If `store`, lane j writes qs dword j and lane 0 writes the d|s dword of the
// 36-byte block at blk (4-byte aligned).
__device__ __forceinline__ void quantize_block_q8_1(float4 v, uint8_t *blk, int j, bool store) {
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
  const int sum = group_isum<8>(q0 + q1 + q2 + q3);
  if (store) {
    const uint32_t packed = (uint32_t)(q0 & 0xff) | ((uint32_t)(q1 & 0xff) << 8) |
                            ((uint32_t)(q2 & 0xff) << 16) | ((uint32_t)(q3 & 0xff) << 24);
    *reinterpret_cast<uint32_t *>(blk + 4 + 4 * j) = packed;
    if (j == 0) {
      // s is the fp32 product, rounded to fp16 afterwards.  The empty asm pins
      // the product in a VGPR so it cannot be fused with the conversion into
      // one v_fma_mix that would round only once.
      float s = d * (float)sum;
      asm volatile("" : "+v"(s));
      *reinterpret_cast<uint32_t *>(blk) = f2h(d) | (f2h(s) << 16);
    }
  }
}

}  // namespace qg
