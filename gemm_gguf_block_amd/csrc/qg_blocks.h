// qg_blocks.h -- block-level helpers shared by the GEMV, MoE and mmq kernels.
#pragma once
#include "qg_device.h"

namespace qg {

// 72 bytes = two consecutive Q8_1 blocks: A[0] = d|s of the first, A[1..8] its
// qs, A[9] = d|s of the second, A[10..17] its qs.
__device__ __forceinline__ void load_q8_1_pair(const uint8_t *p, uint32_t A[18]) {
  const u32x4 a0 = ld16(p), a1 = ld16(p + 16), a2 = ld16(p + 32), a3 = ld16(p + 48);
  const u32x2 a4 = ld8(p + 64);
  A[0] = a0.x; A[1] = a0.y; A[2] = a0.z; A[3] = a0.w;
  A[4] = a1.x; A[5] = a1.y; A[6] = a1.z; A[7] = a1.w;
  A[8] = a2.x; A[9] = a2.y; A[10] = a2.z; A[11] = a2.w;
  A[12] = a3.x; A[13] = a3.y; A[14] = a3.z; A[15] = a3.w;
  A[16] = a4.x; A[17] = a4.y;
}

// Scale/min of sub-blocks 2g and 2g+1 from header dwords y, z, w (the 12
// packed bytes).  Bytes 0..3 of y/z carry sc/m of sub-blocks 0..3 in their low
// six bits; sub-blocks 4..7 take a nibble of w plus the spare top two bits.
__device__ __forceinline__ void q4k_scales(uint32_t hy, uint32_t hz, uint32_t hw, int g, int &sc0, int &sc1,
                                           int &m0, int &m1) {
  const uint32_t sc_lo = hy & 0x3F3F3F3Fu;
  const uint32_t m_lo = hz & 0x3F3F3F3Fu;
  const uint32_t sc_hi = (hw & 0x0F0F0F0Fu) | ((hy >> 2) & 0x30303030u);
  const uint32_t m_hi = ((hw >> 4) & 0x0F0F0F0Fu) | ((hz >> 2) & 0x30303030u);
  const uint32_t scw = g < 2 ? sc_lo : sc_hi;
  const uint32_t mw = g < 2 ? m_lo : m_hi;
  const uint32_t sh = (uint32_t)(g & 1) * 16u;
  sc0 = (int)((scw >> sh) & 0xFFu);
  sc1 = (int)((scw >> (sh + 8)) & 0xFFu);
  m0 = (int)((mw >> sh) & 0xFFu);
  m1 = (int)((mw >> (sh + 8)) & 0xFFu);
}

// Q6_K codes as int8 q - 32, four at a time: low nibbles of `lo` (ql) and the
// low bit pairs of `hi` (qh).  The high nibble comes from a 4-entry byte table
// indexed by the qh bits (v_perm_b32), since (q - 32) mod 256 = ql + 16 * ((qh -
// 2) mod 16); the table is given as both sources so that the selector 0..3
// names a table byte either way round.
__device__ __forceinline__ int q6k_codes4(uint32_t lo, uint32_t hi) {
  const uint32_t top = __builtin_amdgcn_perm(0x1000F0E0u, 0x1000F0E0u, hi & 0x03030303u);
  return (int)((lo & 0x0F0F0F0Fu) | top);
}

// Lanes sharing one row: the largest power of two <= 64 dividing the row's
// unit count, so every lane of a row does the same number of units.
inline int lanes_per_row(int64_t units) {
  int L = 64;
  while (L > 1 && (units % L) != 0) L >>= 1;
  return L;
}

}  // namespace qg
