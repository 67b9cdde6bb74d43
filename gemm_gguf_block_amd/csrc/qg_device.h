// qg_device.h -- device helpers shared by the gfx950 kernels of libqgguf.
//
// Block layouts are GGUF's (the pages name the types only -- blazr README,
// "Model Formats > GGUF"):
//   Q8_0 34 B = fp16 d | int8 qs[32]
//   Q8_1 36 B = fp16 d | fp16 s | int8 qs[32]     (qs is dword-aligned in a block)
//   Q4_K 144 B = fp16 d | fp16 dmin | scales[12] | qs[128]   (9 x 16 B, aligned)
//   Q6_K 210 B = ql[128] | qh[64] | int8 scales[16] | fp16 d
//   Q5_K 176 B = fp16 d | fp16 dmin | scales[12] | qh[32] | qs[128]  (11 x 16 B, aligned)
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

constexpr int kQ8_0Bytes = 34;
constexpr int kQ8_1Bytes = 36;
constexpr int kQ4KBytes = 144;
constexpr int kQ6KBytes = 210;
constexpr int kQ5KBytes = 176;

// 16 bytes at a 4-byte aligned address: global_load_dwordx4 needs only dword
// alignment, and this type tells the compiler exactly that.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2), aligned(4)));

__device__ __forceinline__ u32x4 ld16(const uint8_t *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ u32x2 ld8(const uint8_t *p) { return *reinterpret_cast<const u32x2 *>(p); }
__device__ __forceinline__ uint32_t ld4(const uint8_t *p) { return *reinterpret_cast<const uint32_t *>(p); }
__device__ __forceinline__ uint32_t ld2(const uint8_t *p) { return *reinterpret_cast<const uint16_t *>(p); }

// binary16 bits (low 16 bits of `h`) -> f32, exact.
__device__ __forceinline__ float h2f(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xffffu));
}

// f32 with the bits of u.  A scalar parameter on purpose: with this compiler
// __builtin_bit_cast applied directly to an ext-vector element (v.y) reads
// element 0, so elements must be copied out before the cast.
__device__ __forceinline__ float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }

// f32 -> binary16 bits, round to nearest even (v_cvt_f16_f32 in the default
// rounding mode, with fp16 denormals preserved).
__device__ __forceinline__ uint32_t f2h(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// Signed int8x4 dot product with int32 accumulate (v_dot4c_i32_i8).
__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// Signed byte of w starting at bit `bit` (v_bfe_i32).  The builtin's result
// type is unsigned, so it is cast back to int here: converting it straight to
// float would read a negative byte as about 4.3e9.
__device__ __forceinline__ int sbyte(uint32_t w, uint32_t bit) {
  return (int)__builtin_amdgcn_sbfe((int)w, bit, 8u);
}

// Sum of the four signed bytes of `a`, added to c.
__device__ __forceinline__ int bsum4(uint32_t a, int c) { return dot4(a, 0x01010101u, c); }

// ({hi,lo} >> 8*shift)[31:0] for shift in 0..3 (v_alignbyte_b32).
__device__ __forceinline__ uint32_t align_bytes(uint32_t hi, uint32_t lo, uint32_t shift) {
  return __builtin_amdgcn_alignbyte(hi, lo, shift);
}

// 16 / 8 bytes at a 2-byte aligned address (Q6_K fields, 210-byte blocks).
// gfx950 under the HSA runtime runs with unaligned memory access enabled, and
// the compiler emits a single global_load_dwordx4 / dwordx2 for these; only the
// bytes named are read.
typedef uint32_t u32x4_a2 __attribute__((ext_vector_type(4), aligned(2)));
typedef uint32_t u32x2_a2 __attribute__((ext_vector_type(2), aligned(2)));
__device__ __forceinline__ u32x4 ld16_a2(const uint8_t *p) {
  const u32x4_a2 v = *reinterpret_cast<const u32x4_a2 *>(p);
  return u32x4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ u32x2 ld8_a2(const uint8_t *p) {
  const u32x2_a2 v = *reinterpret_cast<const u32x2_a2 *>(p);
  return u32x2{v.x, v.y};
}

// Butterfly sum over aligned groups of L lanes (L a power of two <= 64); every
// lane of a group gets the group's sum.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = L / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// DPP controls (gfx9 encoding): row_shr:n = 0x110 + n, row_bcast:15 = 0x142,
// row_bcast:31 = 0x143.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_or_zero(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, true));
}

// Sum over aligned groups of L lanes (L a power of two, 1 <= L <= 64) with DPP
// adds only (no LDS traffic): the result is exact in the LAST lane of each
// group (lane % L == L - 1); other lanes hold partial sums.  Rows of 16 lanes
// are summed by shift-right-and-add (lane i accumulates lanes i-15..i of its
// row); row totals are then carried across rows with row_bcast.
template <int L>
__device__ __forceinline__ float group_sum_last(float v) {
  static_assert(L >= 1 && L <= 64 && (L & (L - 1)) == 0, "group of 1..64 lanes, a power of two");
  if (L >= 2) v += dpp_or_zero<0x111, 0xf>(v);
  if (L >= 4) v += dpp_or_zero<0x112, 0xf>(v);
  if (L >= 8) v += dpp_or_zero<0x114, 0xf>(v);
  if (L >= 16) v += dpp_or_zero<0x118, 0xf>(v);
  if (L >= 32) v += dpp_or_zero<0x142, 0xa>(v);  // rows 1, 3 += lane 15 of rows 0, 2
  if (L >= 64) v += dpp_or_zero<0x143, 0x8>(v);  // row 3 += lane 31
  return v;
}

// Lane exchange within a row of 16 lanes for the butterflies below (every
// lane reads a lane of its own row): quad_perm [1,0,3,2] (xor 1), quad_perm
// [2,3,0,1] (xor 2), row_half_mirror (lane i of 8 <-> 7 - i), row_mirror
// (lane i of 16 <-> 15 - i).
template <int STEP>
__device__ __forceinline__ int dpp_swap(int v) {
  constexpr int kCtrl = STEP == 1 ? 0xB1 : STEP == 2 ? 0x4E : STEP == 4 ? 0x141 : 0x140;
  return __builtin_amdgcn_update_dpp(v, v, kCtrl, 0xf, 0xf, false);
}

// Max / integer sum over aligned groups of L lanes (L a power of two <= 64);
// every lane of a group gets the result.  Up to 16 lanes the partner values
// come by DPP (after the quad steps a lane's partner in the other half of its
// group, by mirror, already holds that half's result); wider groups use
// cross-lane shuffles for the steps past 16.
template <int L>
__device__ __forceinline__ float group_max(float v) {
  static_assert(L >= 1 && L <= 64 && (L & (L - 1)) == 0, "group of 1..64 lanes, a power of two");
#pragma unroll
  for (int step = 1; step < L && step <= 8; step <<= 1)
    v = fmaxf(v, __builtin_bit_cast(float, step == 1   ? dpp_swap<1>(__builtin_bit_cast(int, v))
                                           : step == 2 ? dpp_swap<2>(__builtin_bit_cast(int, v))
                                           : step == 4 ? dpp_swap<4>(__builtin_bit_cast(int, v))
                                                       : dpp_swap<8>(__builtin_bit_cast(int, v))));
#pragma unroll
  for (int off = 16; off < L; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

template <int L>
__device__ __forceinline__ int group_isum(int v) {
  static_assert(L >= 1 && L <= 64 && (L & (L - 1)) == 0, "group of 1..64 lanes, a power of two");
#pragma unroll
  for (int step = 1; step < L && step <= 8; step <<= 1)
    v += step == 1 ? dpp_swap<1>(v) : step == 2 ? dpp_swap<2>(v) : step == 4 ? dpp_swap<4>(v) : dpp_swap<8>(v);
#pragma unroll
  for (int off = 16; off < L; off <<= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace qg
