// qg_mmq.hip -- prefill product C[m][n] = sum_k a^[m,k] w^[n,k] with Q4_K,
// Q5_K, Q6_K, Q8_0, Q4_0 or Q5_0 weights and Q8_1 activations on gfx950 int8
// matrix cores.
//
// The pages run this step as "in-shader dequant and dp4a mmq" (infr page,
// "models") and as cooperative-matrix matmul (infr page, "Vulkan-first, Metal
// too"); the blazr README ("Model Formats > GGUF") names Q4_K, Q6_K and Q8_0 as
// the integer-dot types.  Here a workgroup owns a 64 (tokens) x 128 (weight
// rows) output tile; each 32x32 of it belongs to a pair of waves.  Per 256-wide
// step of k (one K-quant superblock, eight Q8_0 blocks) the workgroup stages in
// LDS:
//   A  Q8_1 qs as int8, plus per (row, block) d_a (and d_a*sum(qa) for Q4_K)
//   B  the weight codes as int8 (Q4_K nibbles, Q6_K q - 32, Q8_0 qs, Q4_0
//      q - 8, Q5_0 q - 16), plus per (weight row, scale group) the group's
//      factor (d*sc_j, d*sc_j, d) and for Q4_K -dmin*m_j
// double-buffered: the global loads of step s+1 are in flight while the MFMAs
// of step s run.  Each 32-wide block of k is one v_mfma_i32_32x32x32_i8 -> the
// exact int32 dots D of that block for the wave's 32x32 tile; Q6_K's 16-wide
// sub-blocks are two v_mfma_i32_32x32x16_i8.  A dot's fp32 rescale is
// acc += F * D with F[m][n] = d_a[m] * f[n], a rank-1 outer product that the
// matrix core forms as well: d_a (fp16) is exactly the sum of two bf16 parts
// and f is two bf16 parts to 2^-17 (exactly, for Q8_0's fp16 d), so one
// v_mfma_f32_32x32x8_bf16 over those parts gives F in the MFMA output layout,
// leaving one convert and one fma per output on the VALU.  Q4_K's min term
// -sum_j (d_a*sum qa)_j (dmin*m_j) is a rank-8-per-superblock product of two
// small matrices and runs on the matrix core too, into the same accumulator.
#include "qg_blocks.h"
#include "qg_launch.h"

namespace qg {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4n __attribute__((ext_vector_type(4)));  // naturally aligned: one 16-byte LDS read

constexpr int kBM = 64, kBN = 128;
constexpr int kRow = 272;  // LDS bytes per staged row: 256 + 16 (spreads rows over banks)

// Formats, numbered as the GEMV entry points number them.
constexpr int kMQ8_0 = 0, kMQ4K = 1, kMQ6K = 2, kMQ5K = 3, kMQ4_0 = 4, kMQ5_0 = 5;

template <int FMT>
struct MmqFmt {
  static constexpr int kGroups = FMT == kMQ6K ? 16 : 8;  // scale groups per 256-wide step
  static constexpr bool kMin = FMT == kMQ4K || FMT == kMQ5K;
  // 32-value blocks: k need only be a multiple of 32 (the last step is ragged)
  static constexpr bool kBlk32 = FMT == kMQ8_0 || FMT == kMQ4_0 || FMT == kMQ5_0;
  static constexpr int kRegs = (FMT == kMQ8_0 || FMT == kMQ5K) ? 5 : (FMT == kMQ6K ? 4 : 3);  // u32x4 staging
};

// Per-group factor arrays are [group][row] so that the MFMA operand reads of a
// wave are contiguous; one spare entry per group row spreads the transposed
// staging writes over the LDS banks.  For Q6_K each 32-byte block of A and B
// is stored as bytes [0..7, 16..23, 8..15, 24..31]: lane half h then reads its
// 8-byte slice of both 16-wide sub-blocks as one 16-byte group.
template <int FMT>
struct MmqStage {
  uint8_t a[kBM * kRow];
  uint8_t b[kBN * kRow];
  uint32_t fa[8][kBM + 1][2];  // bf16 (ah, ah, al, al) of d_a = ah + al, per (block j, activation row)
  uint32_t fb[MmqFmt<FMT>::kGroups][kBN + 1][2];  // bf16 (fh, fl, fh, fl) of the group factor f = fh + fl
  uint32_t fs[MmqFmt<FMT>::kMin ? 8 : 1][kBM + 1][2];  // bf16 (sh, sh, sl, sl) of d_a * sum(qa)
  uint32_t fm[MmqFmt<FMT>::kMin ? 8 : 1][kBN + 1][2];  // bf16 (mh, ml, mh, ml) of -2 dmin m_j
};

__device__ __forceinline__ uint32_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// x = hi + lo with hi, lo bf16 (exact when x has <= 16 significant bits).
__device__ __forceinline__ void bf16_split(float x, uint32_t &hi, uint32_t &lo) {
  const __bf16 h = (__bf16)x;
  hi = __builtin_bit_cast(uint16_t, h);
  lo = bf16_bits(x - (float)h);
}

__device__ __forceinline__ void put_factor(uint32_t (&f)[2], float x) {
  uint32_t hi, lo;
  bf16_split(x, hi, lo);
  f[0] = f[1] = hi | (lo << 16);
}

// Global -> registers for one 256-wide step.  A staging thread and a weight
// staging thread use the same registers (a wave stages one or the other).
// Activation thread t (0..511) holds block t%8 of tile row t/8: x[0] = bytes
// 0-15, x[1] = 16-31, x[2].x = 32-35.  Rows past the end of A or B load the last
// row instead; they only feed outputs that are never stored.  Blocks past k
// (32-value block formats only) load as zeros.
template <int FMT>
struct MmqRegs {
  u32x4 x[MmqFmt<FMT>::kRegs];
};

template <int FMT>
__device__ __forceinline__ void load_act(MmqRegs<FMT> &g, const uint8_t *__restrict__ AQ, int M, int nblk, int m0,
                                         int s, int t) {
  const int gm = min(m0 + (t >> 3), M - 1);
  const int blk = 8 * s + (t & 7);
  if (MmqFmt<FMT>::kBlk32 && blk >= nblk) {
    g.x[0] = g.x[1] = u32x4{0u, 0u, 0u, 0u};
    g.x[2].x = 0u;
    return;
  }
  const uint8_t *ap = AQ + ((int64_t)gm * nblk + blk) * kQ8_1Bytes;
  g.x[0] = ld16(ap);
  g.x[1] = ld16(ap + 16);
  g.x[2].x = ld4(ap + 32);
}

// Weight thread t: tile row t/4 and part c = t%4 of its 256-wide step.
//   Q4_K: x[0] = header (d, dmin, scales), x[1], x[2] = qs bytes 32c..32c+31
//   Q5_K: as Q4_K (qs at byte 48), plus x[3], x[4] = qh[0..31]
//   Q8_0: blocks 2c, 2c+1: x[0..1] and x[2..3] their qs, x[4].x/.y their d
//   Q4_0: blocks 2c, 2c+1: x[0], x[1] their qs, x[2].x/.y their d
//   Q5_0: as Q4_0, plus x[2].z/.w their qh words
// With `al` (32-value block types, an even block count per row) the block
// pair starts on a dword boundary and is loaded as it is stored, in aligned
// dwords: x[0], x[1], ... hold bytes 0-15, 16-31, ... of the pair; the
// fields are realigned when the pair is staged.
//   Q6_K: 128-half h = c/2, positions l = 16(c%2)..+15 of all four 32-groups:
//         x[0] = ql[64h + l] (groups 0, 2), x[1] = ql[64h + 32 + l] (groups
//         1, 3), x[2] = qh[32h + l], x[3].x/.y = scales[8h..8h+7], x[3].z = d
template <int FMT>
__device__ __forceinline__ void load_wgt(MmqRegs<FMT> &g, const uint8_t *__restrict__ W, int N, int nblk, int n0,
                                         int s, int t, bool al) {
  const int gn = min(n0 + (t >> 2), N - 1);
  const int c = t & 3;
  if constexpr (MmqFmt<FMT>::kBlk32) {
    if (al) {
      constexpr int kPair = FMT == kMQ8_0 ? 2 * kQ8_0Bytes : (FMT == kMQ4_0 ? 36 : 44);
      const int b0 = 8 * s + 2 * c;
      const uint8_t *bp = W + ((int64_t)gn * nblk + b0) * (kPair / 2);
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < MmqFmt<FMT>::kRegs; ++i) g.x[i] = z;
      if (b0 < nblk) {  // then b0 + 1 < nblk as well: nblk is even
        g.x[0] = ld16(bp);
        g.x[1] = ld16(bp + 16);
        if constexpr (FMT == kMQ8_0) {
          g.x[2] = ld16(bp + 32);
          g.x[3] = ld16(bp + 48);
          g.x[4].x = ld4(bp + 64);
        } else if constexpr (FMT == kMQ4_0) {
          g.x[2].x = ld4(bp + 32);
        } else {
          g.x[2].x = ld4(bp + 32);
          g.x[2].y = ld4(bp + 36);
          g.x[2].z = ld4(bp + 40);
        }
      }
      return;
    }
  }
  if constexpr (FMT == kMQ4K || FMT == kMQ5K) {
    constexpr int kB = FMT == kMQ5K ? kQ5KBytes : kQ4KBytes, kQs = FMT == kMQ5K ? 48 : 16;
    const uint8_t *bp = W + ((int64_t)gn * (nblk / 8) + s) * kB;
    g.x[0] = ld16(bp);
    g.x[1] = ld16(bp + kQs + 32 * c);
    g.x[2] = ld16(bp + kQs + 16 + 32 * c);
    if constexpr (FMT == kMQ5K) {
      g.x[3] = ld16(bp + 16);
      g.x[4] = ld16(bp + 32);
    }
  } else if constexpr (FMT == kMQ6K) {
    const uint8_t *bp = W + ((int64_t)gn * (nblk / 8) + s) * kQ6KBytes;
    const int h = c >> 1, l = 16 * (c & 1);
    g.x[0] = ld16_a2(bp + 64 * h + l);
    g.x[1] = ld16_a2(bp + 64 * h + 32 + l);
    g.x[2] = ld16_a2(bp + 128 + 32 * h + l);
    const u32x2 sc = ld8_a2(bp + 192 + 8 * h);
    g.x[3].x = sc.x;
    g.x[3].y = sc.y;
    g.x[3].z = ld2(bp + 208);
  } else if constexpr (FMT == kMQ4_0 || FMT == kMQ5_0) {
    constexpr int kB = FMT == kMQ4_0 ? 18 : 22, kQs = FMT == kMQ4_0 ? 2 : 6;
    const int b0 = 8 * s + 2 * c;
    const uint8_t *bp = W + ((int64_t)gn * nblk + b0) * kB;
    const u32x4 z = {0u, 0u, 0u, 0u};
    g.x[0] = g.x[1] = g.x[2] = z;
    if (b0 < nblk) {
      g.x[2].x = ld2(bp);
      g.x[0] = ld16_a2(bp + kQs);
      if constexpr (FMT == kMQ5_0) g.x[2].z = ld2(bp + 2) | (ld2(bp + 4) << 16);
    }
    if (b0 + 1 < nblk) {
      g.x[2].y = ld2(bp + kB);
      g.x[1] = ld16_a2(bp + kB + kQs);
      if constexpr (FMT == kMQ5_0) g.x[2].w = ld2(bp + kB + 2) | (ld2(bp + kB + 4) << 16);
    }
  } else {
    const int b0 = 8 * s + 2 * c;
    const uint8_t *bp = W + ((int64_t)gn * nblk + b0) * kQ8_0Bytes;
    const u32x4 z = {0u, 0u, 0u, 0u};
    g.x[0] = g.x[1] = g.x[2] = g.x[3] = z;
    g.x[4].x = g.x[4].y = 0u;
    if (b0 < nblk) {
      g.x[4].x = ld2(bp);
      g.x[0] = ld16_a2(bp + 2);
      g.x[1] = ld16_a2(bp + 18);
    }
    if (b0 + 1 < nblk) {
      g.x[4].y = ld2(bp + kQ8_0Bytes);
      g.x[2] = ld16_a2(bp + kQ8_0Bytes + 2);
      g.x[3] = ld16_a2(bp + kQ8_0Bytes + 18);
    }
  }
}

// activation block: qs -> int8 row, factors
template <int FMT>
__device__ __forceinline__ void store_act(const MmqRegs<FMT> &g, MmqStage<FMT> &s, int t) {
  const int ar = t >> 3, ab = t & 7;
  const uint32_t q[8] = {g.x[0].y, g.x[0].z, g.x[0].w, g.x[1].x, g.x[1].y, g.x[1].z, g.x[1].w, g.x[2].x};
  u32x4 *dst = reinterpret_cast<u32x4 *>(s.a + ar * kRow + 32 * ab);
  if constexpr (FMT == kMQ6K) {
    dst[0] = u32x4{q[0], q[1], q[4], q[5]};
    dst[1] = u32x4{q[2], q[3], q[6], q[7]};
  } else {
    dst[0] = u32x4{q[0], q[1], q[2], q[3]};
    dst[1] = u32x4{q[4], q[5], q[6], q[7]};
  }
  const float da = h2f(g.x[0].x);
  uint32_t hi, lo;
  bf16_split(da, hi, lo);
  s.fa[ab][ar][0] = hi | (hi << 16);
  s.fa[ab][ar][1] = lo | (lo << 16);
  if constexpr (MmqFmt<FMT>::kMin) {
    int S = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) S = bsum4(q[i], S);
    bf16_split(da * (float)S, hi, lo);
    s.fs[ab][ar][0] = hi | (hi << 16);
    s.fs[ab][ar][1] = lo | (lo << 16);
  }
}

// weight part: codes -> int8 row, factors
template <int FMT>
__device__ __forceinline__ void store_wgt(const MmqRegs<FMT> &g, MmqStage<FMT> &s, int t, bool al) {
  const int br = t >> 2, c = t & 3;
  if constexpr (FMT == kMQ4K || FMT == kMQ5K) {
    // sub-block 2c in the low nibbles, 2c+1 in the high ones (Q5_K: plus bits
    // 2c and 2c+1 of qh[l] as the fifth code bit)
    const uint32_t Q[8] = {g.x[1].x, g.x[1].y, g.x[1].z, g.x[1].w, g.x[2].x, g.x[2].y, g.x[2].z, g.x[2].w};
    uint32_t lo[8], hi[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      lo[i] = Q[i] & 0x0F0F0F0Fu;
      hi[i] = (Q[i] >> 4) & 0x0F0F0F0Fu;
    }
    if constexpr (FMT == kMQ5K) {
      const uint32_t H[8] = {g.x[3].x, g.x[3].y, g.x[3].z, g.x[3].w, g.x[4].x, g.x[4].y, g.x[4].z, g.x[4].w};
      const uint32_t s0 = 2u * (uint32_t)c;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        lo[i] |= ((H[i] >> s0) & 0x01010101u) << 4;
        hi[i] |= ((H[i] >> (s0 + 1)) & 0x01010101u) << 4;
      }
    }
    u32x4 *dst = reinterpret_cast<u32x4 *>(s.b + br * kRow + 64 * c);
    dst[0] = u32x4{lo[0], lo[1], lo[2], lo[3]};
    dst[1] = u32x4{lo[4], lo[5], lo[6], lo[7]};
    dst[2] = u32x4{hi[0], hi[1], hi[2], hi[3]};
    dst[3] = u32x4{hi[4], hi[5], hi[6], hi[7]};
    int sc0, sc1, mn0, mn1;
    q4k_scales(g.x[0].y, g.x[0].z, g.x[0].w, c, sc0, sc1, mn0, mn1);
    const float d = h2f(g.x[0].x), dmin = h2f(g.x[0].x >> 16);
    put_factor(s.fb[2 * c][br], d * (float)sc0);
    put_factor(s.fb[2 * c + 1][br], d * (float)sc1);
    // doubled like the factor product 2F (exact); see the kernel's accumulator
    put_factor(s.fm[2 * c][br], -2.f * (dmin * (float)mn0));
    put_factor(s.fm[2 * c + 1][br], -2.f * (dmin * (float)mn1));
  } else if constexpr (FMT == kMQ6K) {
    // group gq (0..3) of half h is block j = 4h + gq; this thread's 16 values
    // are its sub-block 2j + (c & 1), stored at bytes 8(c&1) and 16 + 8(c&1)
    // of the block's permuted 32
    const int h = c >> 1, hl = c & 1;
    const float d = h2f(g.x[3].z);
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const u32x4 lo = g.x[gq & 1];
      const uint32_t ls = 4u * (uint32_t)(gq >> 1), hs = 2u * (uint32_t)gq;
      const int j = 4 * h + gq;
      uint8_t *dst = s.b + br * kRow + 32 * j + 8 * hl;
      *reinterpret_cast<u32x2 *>(dst) =
          u32x2{(uint32_t)q6k_codes4(lo.x >> ls, g.x[2].x >> hs), (uint32_t)q6k_codes4(lo.y >> ls, g.x[2].y >> hs)};
      *reinterpret_cast<u32x2 *>(dst + 16) =
          u32x2{(uint32_t)q6k_codes4(lo.z >> ls, g.x[2].z >> hs), (uint32_t)q6k_codes4(lo.w >> ls, g.x[2].w >> hs)};
      // scale of sub-block 8h + 2gq + hl: byte 2gq + hl of scales[8h..8h+7]
      const uint32_t scw = gq < 2 ? g.x[3].x : g.x[3].y;
      put_factor(s.fb[2 * j + hl][br], d * (float)sbyte(scw, 8u * (uint32_t)((2 * gq + hl) & 3)));
    }
  } else if constexpr (FMT == kMQ4_0 || FMT == kMQ5_0) {
    // the two blocks' qs dwords, qh words and d, from either load layout
    uint32_t Qb[2][4], qh[2] = {0u, 0u}, dd[2];
    if (al) {
      const uint32_t w[12] = {g.x[0].x, g.x[0].y, g.x[0].z, g.x[0].w, g.x[1].x, g.x[1].y,
                              g.x[1].z, g.x[1].w, g.x[2].x, g.x[2].y, g.x[2].z, g.x[2].w};
      if constexpr (FMT == kMQ4_0) {  // d0 | qs0[16] | d1 | qs1[16]
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          Qb[0][i] = align_bytes(w[i + 1], w[i], 2);
          Qb[1][i] = w[5 + i];
        }
        dd[0] = w[0];
        dd[1] = w[4] >> 16;
      } else {  // d0 | qh0 | qs0[16] | d1 | qh1 | qs1[16]
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          Qb[0][i] = align_bytes(w[i + 2], w[i + 1], 2);
          Qb[1][i] = w[7 + i];
        }
        qh[0] = align_bytes(w[1], w[0], 2);
        qh[1] = w[6];
        dd[0] = w[0];
        dd[1] = w[5] >> 16;
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        Qb[h][0] = g.x[h].x;
        Qb[h][1] = g.x[h].y;
        Qb[h][2] = g.x[h].z;
        Qb[h][3] = g.x[h].w;
      }
      dd[0] = g.x[2].x;
      dd[1] = g.x[2].y;
      if constexpr (FMT == kMQ5_0) {
        qh[0] = g.x[2].z;
        qh[1] = g.x[2].w;
      }
    }
    // codes j (low nibble of qs byte j) and 16 + j (high nibble), minus the
    // zero code, as int8: a byte b <= 31 plus 0x80 - off stays below 0x100,
    // and flipping bit 7 then leaves b - off in two's complement
    constexpr uint32_t kBias = FMT == kMQ4_0 ? 0x78787878u : 0x70707070u;
    u32x4 *dst = reinterpret_cast<u32x4 *>(s.b + br * kRow + 64 * c);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo[i] = Qb[h][i] & 0x0F0F0F0Fu;
        hi[i] = (Qb[h][i] >> 4) & 0x0F0F0F0Fu;
        if constexpr (FMT == kMQ5_0) {
          // bit i of the qh word is the fifth bit of code i: bits 4i..4i+3
          // land on bit 4 of the four bytes (the four shifted copies of the
          // group set disjoint bits)
          lo[i] |= ((qh[h] >> (4 * i)) & 0xFu) * 0x02040810u & 0x10101010u;
          hi[i] |= ((qh[h] >> (16 + 4 * i)) & 0xFu) * 0x02040810u & 0x10101010u;
        }
        lo[i] = (lo[i] + kBias) ^ 0x80808080u;
        hi[i] = (hi[i] + kBias) ^ 0x80808080u;
      }
      dst[2 * h] = u32x4{lo[0], lo[1], lo[2], lo[3]};
      dst[2 * h + 1] = u32x4{hi[0], hi[1], hi[2], hi[3]};
    }
    put_factor(s.fb[2 * c][br], h2f(dd[0]));
    put_factor(s.fb[2 * c + 1][br], h2f(dd[1]));
  } else {
    u32x4 *dst = reinterpret_cast<u32x4 *>(s.b + br * kRow + 64 * c);
    if (al) {  // d0 | qs0[32] | d1 | qs1[32]: 17 dwords in x[0..3], x[4].x
      const uint32_t w[17] = {g.x[0].x, g.x[0].y, g.x[0].z, g.x[0].w, g.x[1].x, g.x[1].y, g.x[1].z,
                              g.x[1].w, g.x[2].x, g.x[2].y, g.x[2].z, g.x[2].w, g.x[3].x, g.x[3].y,
                              g.x[3].z, g.x[3].w, g.x[4].x};
      uint32_t q0[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) q0[i] = align_bytes(w[i + 1], w[i], 2);
      dst[0] = u32x4{q0[0], q0[1], q0[2], q0[3]};
      dst[1] = u32x4{q0[4], q0[5], q0[6], q0[7]};
      dst[2] = u32x4{w[9], w[10], w[11], w[12]};
      dst[3] = u32x4{w[13], w[14], w[15], w[16]};
      put_factor(s.fb[2 * c][br], h2f(w[0]));
      put_factor(s.fb[2 * c + 1][br], h2f(w[8] >> 16));
    } else {
      dst[0] = g.x[0];
      dst[1] = g.x[1];
      dst[2] = g.x[2];
      dst[3] = g.x[3];
      put_factor(s.fb[2 * c][br], h2f(g.x[4].x));
      put_factor(s.fb[2 * c + 1][br], h2f(g.x[4].y));
    }
  }
}

// Two waves share each 32x32 output tile and split every step's eight blocks
// between them; the workgroup has 16 waves.  Waves 0-7 stage activations and
// waves 8-15 weights, and the two partial tiles are summed through LDS at the
// end.  With DUMP the exact dots are written instead of C: [m][n][k/32] per
// block, or [m][n][k/16] per Q6_K sub-block.
template <int FMT, bool DUMP>
__global__ __launch_bounds__(1024) void mmq_kernel(const uint8_t *__restrict__ W, const uint8_t *__restrict__ AQ,
                                                   float *__restrict__ C, int32_t *__restrict__ Dd, int M, int N,
                                                   int nblk) {
  constexpr int kJ = 4;  // blocks per step per wave
  __shared__ MmqStage<FMT> stage[2];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int kh = wv >> 3;                         // which half of each step
  const int wm = (wv >> 2) & 1, wn = wv & 3;      // 2 x 4 tiles of 32x32
  const int tiles_n = (N + kBN - 1) / kBN;
  const int m0 = (int)(blockIdx.x / tiles_n) * kBM, n0 = (int)(blockIdx.x % tiles_n) * kBN;
  const int lr = lane & 31, lh = lane >> 5;
  const int nsteps = (nblk + 7) / 8;
  const int st = tid & 511;
  const bool act = tid < 512;  // this wave stages activations, else weights
  // 32-value block types with an even block count per row: block pairs are
  // dword aligned and load as aligned dwords
  const bool al = MmqFmt<FMT>::kBlk32 && (nblk & 1) == 0;

  // acc = 2 * (sum of F*D over blocks + min term); halved at the end
  v16f acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  v16i zero;
  v16f fzero;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    zero[r] = 0;
    fzero[r] = 0.f;
  }

  // Step s + 1's global loads are issued at the start of step s and staged at
  // its end: one compute phase (about 2 us at 512 x 4096 x 4096) covers their
  // latency, and a single register set leaves room for the compute phase's
  // operand lookahead.  (Loading two steps ahead from two register sets
  // measured slower with the lookahead dropped: 34.3 against 32.7 us.)
  MmqRegs<FMT> R0;
  auto load = [&](MmqRegs<FMT> &g, int s) {
    if (act)
      load_act<FMT>(g, AQ, M, nblk, m0, s, st);
    else
      load_wgt<FMT>(g, W, N, nblk, n0, s, st, al);
  };
  auto store = [&](const MmqRegs<FMT> &g, MmqStage<FMT> &dst) {
    if (act)
      store_act<FMT>(g, dst, st);
    else
      store_wgt<FMT>(g, dst, st, al);
  };
  // output register r holds tile row 8(r/4) + 4*lh + r%4, column lr
  auto dump = [&](const v16i &D, int idx, int per_row) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int gm = m0 + wm * 32 + 8 * (r / 4) + 4 * lh + (r % 4), gn = n0 + wn * 32 + lr;
      if (gm < M && gn < N) Dd[((int64_t)gm * N + gn) * per_row + idx] = D[r];
    }
  };
  auto factor = [&](const uint32_t *pa, const uint32_t *pb) {
    const v4s fav = __builtin_bit_cast(v4s, u32x2{pa[0], pa[1]});
    const v4s fbv = __builtin_bit_cast(v4s, u32x2{pb[0], pb[1]});
    return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(fav, fbv, fzero, 0, 0, 0);
  };
  auto compute = [&](MmqStage<FMT> &cur, int s) {
    const int j0 = kh * kJ;
    const uint8_t *arow = cur.a + (wm * 32 + lr) * kRow + 16 * lh + 32 * j0;
    const uint8_t *brow = cur.b + (wn * 32 + lr) * kRow + 16 * lh + 32 * j0;
    if constexpr (MmqFmt<FMT>::kMin) {
      if (!DUMP) {
        // min term of this wave's four blocks, -sum_j (d_a S)_j (dmin m_j): a
        // rank-4 product, split hi + lo on both sides into K = 16 bf16 terms
        // (lanes 0-31 carry blocks j0, j0+1, lanes 32-63 blocks j0+2, j0+3),
        // accumulated straight into acc on the matrix core
        const uint32_t *ps = cur.fs[j0 + 2 * lh][wm * 32 + lr];
        const uint32_t *pm = cur.fm[j0 + 2 * lh][wn * 32 + lr];
        constexpr int sA = (kBM + 1) * 2, sB = (kBN + 1) * 2;
        const v8bf sv = __builtin_bit_cast(v8bf, u32x4{ps[0], ps[1], ps[sA], ps[sA + 1]});
        const v8bf mv = __builtin_bit_cast(v8bf, u32x4{pm[0], pm[1], pm[sB], pm[sB + 1]});
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sv, mv, acc, 0, 0, 0);
      }
    }
    if constexpr (FMT == kMQ6K) {
#pragma unroll
      for (int jj = 0; jj < kJ; ++jj) {
        const int j = j0 + jj;
        const uint32_t *pa = cur.fa[j][wm * 32 + lr];
        const u32x4n av = *reinterpret_cast<const u32x4n *>(arow + 32 * jj);
        const u32x4n bv = *reinterpret_cast<const u32x4n *>(brow + 32 * jj);
        // sub-blocks 2j and 2j+1: the lane's 8-byte slices are (x, y) and (z, w)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const uint32_t alo = hh ? av.z : av.x, ahi = hh ? av.w : av.y;
          const uint32_t blo = hh ? bv.z : bv.x, bhi = hh ? bv.w : bv.y;
          const v16i D = __builtin_amdgcn_mfma_i32_32x32x16_i8((long)(((uint64_t)ahi << 32) | alo),
                                                                (long)(((uint64_t)bhi << 32) | blo), zero, 0, 0, 0);
          if (DUMP) {
            dump(D, 16 * s + 2 * j + hh, 2 * nblk);
          } else {
            const v16f F2 = factor(pa, cur.fb[2 * j + hh][wn * 32 + lr]);
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] += F2[r] * (float)D[r];
          }
          asm volatile("" : "+v"(acc)::"memory");  // one sub-block's D and F live at a time
        }
        asm volatile("" : "+v"(acc)::"memory");
      }
    } else {
      // Block j + 1's LDS operands are read before block j's rescale, so their
      // latency runs under that vector work; its products are issued after it.
      struct Opnd {
        u32x4n a, b;
        u32x2 fa, fb;
      };
      auto rd = [&](int jj, Opnd &o) {
        const int j = j0 + jj;
        o.a = *reinterpret_cast<const u32x4n *>(arow + 32 * jj);
        o.b = *reinterpret_cast<const u32x4n *>(brow + 32 * jj);
        const uint32_t *pa = cur.fa[j][wm * 32 + lr];
        const uint32_t *pb = cur.fb[j][wn * 32 + lr];
        o.fa = u32x2{pa[0], pa[1]};
        o.fb = u32x2{pb[0], pb[1]};
      };
      const int nj = MmqFmt<FMT>::kBlk32 ? max(0, min(kJ, nblk - 8 * s - j0)) : kJ;  // ragged last step
      // Q5_K's fifth staging register leaves no room for the lookahead
      constexpr bool kLook = FMT != kMQ5K;
      Opnd o0, o1;
      if (nj > 0) rd(0, o0);
#pragma unroll
      for (int jj = 0; jj < kJ; ++jj) {
        if (jj >= nj) break;
        Opnd &oc = (!kLook || (jj & 1) == 0) ? o0 : o1;
        Opnd &on = (!kLook || (jj & 1) == 0) ? o1 : o0;
        if (!kLook && jj > 0) rd(jj, oc);
        const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(v4i, oc.a),
                                                              __builtin_bit_cast(v4i, oc.b), zero, 0, 0, 0);
        v16f F2;
        if (!DUMP) {
          const v4s fav = __builtin_bit_cast(v4s, oc.fa), fbv = __builtin_bit_cast(v4s, oc.fb);
          F2 = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(fav, fbv, fzero, 0, 0, 0);
        }
        if (kLook && jj + 1 < nj) rd(jj + 1, on);
        if (DUMP) {
          dump(D, 8 * s + j0 + jj, nblk);
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[r] += F2[r] * (float)D[r];
        }
        // Fence: block j + 1's products stay after block j's rescale
        asm volatile("" : "+v"(acc), "+v"(on.a), "+v"(on.b), "+v"(on.fa), "+v"(on.fb)::"memory");
      }
    }
  };
  // One step: s + 1 loads into R0 (free: it held s, staged one step earlier),
  // s computes from `cur`, and s + 1 is then staged into `other`, which
  // nobody reads during this step.
  auto step = [&](int s, MmqStage<FMT> &cur, MmqStage<FMT> &other) {
    if (s + 1 < nsteps) load(R0, s + 1);
    compute(cur, s);
    if (s + 1 < nsteps) store(R0, other);
    __syncthreads();
  };
  if (nsteps > 0) {
    load(R0, 0);
    store(R0, stage[0]);
  }
  __syncthreads();
  for (int s = 0; s < nsteps; s += 2) {
    step(s, stage[0], stage[1]);
    if (s + 1 < nsteps) step(s + 1, stage[1], stage[0]);
  }

  if (!DUMP) {
    v16f v;
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = 0.5f * acc[r];
    {
      // the second half's partial tile goes through LDS (the staging buffers
      // are free after the loop's last barrier) and is added by the first
      float *part = reinterpret_cast<float *>(&stage[0]) + (wv & 7) * 16 * 64;
      if (kh == 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) part[r * 64 + lane] = v[r];
      }
      __syncthreads();
      if (kh == 1) return;
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] += part[r * 64 + lane];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int gm = m0 + wm * 32 + 8 * (r / 4) + 4 * lh + (r % 4);
      const int gn = n0 + wn * 32 + lr;
      if (gm < M && gn < N) C[(int64_t)gm * N + gn] = v[r];
    }
  }
}

// One kernel for every format.  An 8-wave form (two waves per SIMD, each
// wave a 32x32 tile over all eight blocks of a step, one block of MFMA
// lookahead, loads two steps ahead) ran the 32-value types faster than this
// kernel did before its operand lookahead (us at 512 x 4096 x 4096: Q8_0 46.4
// against 54.4), and slower since (Q8_0 46.1 against 33.9, Q4_0 38.6 against
// 32.8, Q5_0 42.0 against 35.1), so it was retired.
template <int FMT>
static hipError_t launch_fmt(const void *w, const void *aq, float *c, int32_t *D, int64_t m, int64_t n, int64_t k,
                             hipStream_t stream) {
  const dim3 grid((unsigned)(((n + kBN - 1) / kBN) * ((m + kBM - 1) / kBM)));
  const uint8_t *W = static_cast<const uint8_t *>(w);
  const uint8_t *A = static_cast<const uint8_t *>(aq);
  if (D)
    hipLaunchKernelGGL((mmq_kernel<FMT, true>), grid, dim3(1024), 0, stream, W, A, c, D, (int)m, (int)n,
                       (int)(k / 32));
  else
    hipLaunchKernelGGL((mmq_kernel<FMT, false>), grid, dim3(1024), 0, stream, W, A, c, D, (int)m, (int)n,
                       (int)(k / 32));
  return hipGetLastError();
}

hipError_t launch_qgemm_mmq(int fmt, const void *w, const void *aq, float *c, int32_t *D, int64_t m, int64_t n,
                            int64_t k, hipStream_t stream) {
  if (fmt == kMQ4K) return launch_fmt<kMQ4K>(w, aq, c, D, m, n, k, stream);
  if (fmt == kMQ6K) return launch_fmt<kMQ6K>(w, aq, c, D, m, n, k, stream);
  if (fmt == kMQ5K) return launch_fmt<kMQ5K>(w, aq, c, D, m, n, k, stream);
  if (fmt == kMQ4_0) return launch_fmt<kMQ4_0>(w, aq, c, D, m, n, k, stream);
  if (fmt == kMQ5_0) return launch_fmt<kMQ5_0>(w, aq, c, D, m, n, k, stream);
  return launch_fmt<kMQ8_0>(w, aq, c, D, m, n, k, stream);
}

}  // namespace qg
