// qg_gemv.hip -- batch-1 decode GEMV over Q8_0 / Q4_K / Q6_K weight blocks
// against one Q8_1 activation row (the dp4a-style dot kernels the blazr README
// lists for these three types, "Model Formats > GGUF", re-designed for gfx950).
//
// Work decomposition (all three formats): a row is cut into units of 64
// weights; L lanes (a power of two, <= 64) share a row and walk its units with
// stride L; a wave holds 64/L rows.  Each lane streams its unit's bytes with
// dword/dwordx4 loads straight into VGPRs, unpacks them there, runs exact
// int8 dot products with v_dot4, applies the fp32 block scales, and the L
// lanes of a row finish with a butterfly reduction.
//
//   Q4_K unit (superblock sb, group g): the 16-byte header + qs[32g..32g+31],
//        i.e. sub-blocks 2g (low nibbles) and 2g+1 (high nibbles).
//   Q6_K unit (sb, half h, l-half): ql[64h+16l..], ql[64h+32+16l..],
//        qh[32h+16l..]: 16-value sub-blocks 8h+2g+l for g = 0..3.
//   Q8_0 unit: a pair of blocks (68 bytes, dword aligned when the row has an
//        even block count), else one block read with byte realignment.
//
// With DUMP the same code writes the exact per-block int32 dots instead of y.
#include "qg_device.h"
#include "qg_launch.h"

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

// ---------------------------------------------------------------- Q4_K
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

template <int L, bool DUMP>
__global__ __launch_bounds__(256) void gemv_q4k_kernel(const uint8_t *__restrict__ W, const uint8_t *__restrict__ XQ,
                                                       float *__restrict__ Y, int32_t *__restrict__ Dd,
                                                       int32_t *__restrict__ Sd, int n, int nsb) {
  constexpr int G = 64 / L;
  const int lane = threadIdx.x & 63;
  const int li = lane & (L - 1);
  const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * G + lane / L;
  const bool live = row < n;
  const int U = nsb * 4;
  const uint8_t *wrow = W + row * (int64_t)nsb * kQ4KBytes;
  float acc = 0.f;
  if (live) {
    for (int u = li; u < U; u += L) {
      const int sb = u >> 2, g = u & 3;
      const uint8_t *bp = wrow + (int64_t)sb * kQ4KBytes;
      const u32x4 hdr = ld16(bp);
      const u32x4 qa = ld16(bp + 16 + 32 * g), qb = ld16(bp + 32 + 32 * g);
      uint32_t A[18];
      load_q8_1_pair(XQ + (int64_t)(8 * sb + 2 * g) * kQ8_1Bytes, A);
      const uint32_t Q[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
      int D0 = 0, D1 = 0, S0 = 0, S1 = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        D0 = dot4(Q[i] & 0x0F0F0F0Fu, A[1 + i], D0);
        D1 = dot4((Q[i] >> 4) & 0x0F0F0F0Fu, A[10 + i], D1);
        S0 = bsum4(A[1 + i], S0);
        S1 = bsum4(A[10 + i], S1);
      }
      if (DUMP) {
        Dd[row * (int64_t)(nsb * 8) + 8 * sb + 2 * g] = D0;
        Dd[row * (int64_t)(nsb * 8) + 8 * sb + 2 * g + 1] = D1;
        if (row == 0) {
          Sd[8 * sb + 2 * g] = S0;
          Sd[8 * sb + 2 * g + 1] = S1;
        }
      } else {
        int sc0, sc1, m0, m1;
        q4k_scales(hdr.y, hdr.z, hdr.w, g, sc0, sc1, m0, m1);
        const float d = h2f(hdr.x), dmin = h2f(hdr.x >> 16);
        const float da0 = h2f(A[0]), da1 = h2f(A[9]);
        const float t = da0 * (float)(sc0 * D0) + da1 * (float)(sc1 * D1);
        const float mm = da0 * (float)(m0 * S0) + da1 * (float)(m1 * S1);
        acc += d * t - dmin * mm;
      }
    }
  }
  if (!DUMP) {
    acc = group_sum<L>(acc);
    if (live && li == 0) Y[row] = acc;
  }
}

// ---------------------------------------------------------------- Q6_K
template <int L, bool DUMP>
__global__ __launch_bounds__(256) void gemv_q6k_kernel(const uint8_t *__restrict__ W, const uint8_t *__restrict__ XQ,
                                                       float *__restrict__ Y, int32_t *__restrict__ Dd, int n,
                                                       int nsb) {
  constexpr int G = 64 / L;
  const int lane = threadIdx.x & 63;
  const int li = lane & (L - 1);
  const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * G + lane / L;
  const bool live = row < n;
  const int U = nsb * 4;
  const uint8_t *wrow = W + row * (int64_t)nsb * kQ6KBytes;
  float acc = 0.f;
  if (live) {
    for (int u = li; u < U; u += L) {
      const int sb = u >> 2, h = (u >> 1) & 1, l = u & 1;
      const uint8_t *bp = wrow + (int64_t)sb * kQ6KBytes;  // 2-byte aligned
      uint32_t qlA[4], qlB[4], qh[4];
      ld16_a2(bp + 64 * h + 16 * l, qlA);
      ld16_a2(bp + 64 * h + 32 + 16 * l, qlB);
      ld16_a2(bp + 128 + 32 * h + 16 * l, qh);
      // scales[8h .. 8h+7]: dwords around them, never past the superblock end
      const uint8_t *sp = bp + 192 + 8 * h;
      const uint32_t ssh = (uint32_t)(reinterpret_cast<uintptr_t>(sp) & 3u);
      const uint8_t *sa = sp - ssh;
      const uint32_t s0 = ld4(sa), s1 = ld4(sa + 4);
      const uint32_t s2 = ssh ? ld4(sa + 8) : 0u;
      const uint32_t scl = align_bytes(s1, s0, ssh), sch = align_bytes(s2, s1, ssh);
      const float d = h2f(ld2(bp + 208));
      // sub-block 8h + 2g + l has scale byte 2g + l of scales[8h..]
      const uint32_t lo8 = 8u * (uint32_t)l;
      const int sc[4] = {(int)__builtin_amdgcn_sbfe((int)scl, lo8, 8u), (int)__builtin_amdgcn_sbfe((int)scl, 16u + lo8, 8u),
                         (int)__builtin_amdgcn_sbfe((int)sch, lo8, 8u), (int)__builtin_amdgcn_sbfe((int)sch, 16u + lo8, 8u)};
      float t = 0.f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint8_t *ap = XQ + (int64_t)(8 * sb + 4 * h + g) * kQ8_1Bytes;
        const float da = h2f(ld4(ap));
        const u32x4 av = ld16(ap + 4 + 16 * l);
        const uint32_t a[4] = {av.x, av.y, av.z, av.w};
        int Dg = 0, Sg = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t q;
          if (g == 0) q = (qlA[i] & 0x0F0F0F0Fu) | ((qh[i] << 4) & 0x30303030u);
          else if (g == 1) q = (qlB[i] & 0x0F0F0F0Fu) | ((qh[i] << 2) & 0x30303030u);
          else if (g == 2) q = ((qlA[i] >> 4) & 0x0F0F0F0Fu) | (qh[i] & 0x30303030u);
          else q = ((qlB[i] >> 4) & 0x0F0F0F0Fu) | ((qh[i] >> 2) & 0x30303030u);
          Dg = dot4(q, a[i], Dg);  // codes 0..63 are non-negative int8
          Sg = bsum4(a[i], Sg);
        }
        Dg -= 32 * Sg;  // sum (q-32)*qa
        if (DUMP) {
          Dd[row * (int64_t)(nsb * 16) + 16 * sb + 8 * h + 2 * g + l] = Dg;
        } else {
          t += da * (float)(sc[g] * Dg);
        }
      }
      acc += d * t;
    }
  }
  if (!DUMP) {
    acc = group_sum<L>(acc);
    if (live && li == 0) Y[row] = acc;
  }
}

// ---------------------------------------------------------------- Q8_0
// Rows with an even block count: unit = block pair at a dword-aligned offset.
template <int L, bool DUMP>
__global__ __launch_bounds__(256) void gemv_q8_0_pair_kernel(const uint8_t *__restrict__ W,
                                                             const uint8_t *__restrict__ XQ, float *__restrict__ Y,
                                                             int32_t *__restrict__ Dd, int n, int npair) {
  constexpr int G = 64 / L;
  const int lane = threadIdx.x & 63;
  const int li = lane & (L - 1);
  const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * G + lane / L;
  const bool live = row < n;
  const uint8_t *wrow = W + row * (int64_t)npair * (2 * kQ8_0Bytes);
  float acc = 0.f;
  if (live) {
    for (int u = li; u < npair; u += L) {
      const uint8_t *bp = wrow + (int64_t)u * (2 * kQ8_0Bytes);
      const u32x4 w0 = ld16(bp), w1 = ld16(bp + 16), w2 = ld16(bp + 32), w3 = ld16(bp + 48);
      const uint32_t w4 = ld4(bp + 64);
      const uint32_t Wd[17] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w, w2.x,
                               w2.y, w2.z, w2.w, w3.x, w3.y, w3.z, w3.w, w4};
      uint32_t A[18];
      load_q8_1_pair(XQ + (int64_t)(2 * u) * kQ8_1Bytes, A);
      int D0 = 0, D1 = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        D0 = dot4(align_bytes(Wd[i + 1], Wd[i], 2), A[1 + i], D0);  // qs of block 0 at bytes 2..33
        D1 = dot4(Wd[9 + i], A[10 + i], D1);                         // qs of block 1 at bytes 36..67
      }
      if (DUMP) {
        Dd[row * (int64_t)(2 * npair) + 2 * u] = D0;
        Dd[row * (int64_t)(2 * npair) + 2 * u + 1] = D1;
      } else {
        acc += h2f(Wd[0]) * h2f(A[0]) * (float)D0 + h2f(Wd[8] >> 16) * h2f(A[9]) * (float)D1;
      }
    }
  }
  if (!DUMP) {
    acc = group_sum<L>(acc);
    if (live && li == 0) Y[row] = acc;
  }
}

// Rows with an odd block count: unit = one block at a 2-byte aligned offset.
template <int L, bool DUMP>
__global__ __launch_bounds__(256) void gemv_q8_0_single_kernel(const uint8_t *__restrict__ W,
                                                               const uint8_t *__restrict__ XQ,
                                                               float *__restrict__ Y, int32_t *__restrict__ Dd, int n,
                                                               int nb) {
  constexpr int G = 64 / L;
  const int lane = threadIdx.x & 63;
  const int li = lane & (L - 1);
  const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * G + lane / L;
  const bool live = row < n;
  const uint8_t *wrow = W + row * (int64_t)nb * kQ8_0Bytes;
  float acc = 0.f;
  if (live) {
    for (int u = li; u < nb; u += L) {
      const uint8_t *p = wrow + (int64_t)u * kQ8_0Bytes;
      const uint32_t sh = (uint32_t)(reinterpret_cast<uintptr_t>(p) & 3u);  // 0 or 2
      const uint32_t x0 = ld4(p - sh);
      const float dw = h2f(sh ? (x0 >> 16) : x0);
      // qs = bytes p+2 .. p+33; read dwords from (p+2) & ~3, the last two bytes
      // separately so nothing past the block is touched
      const uint32_t qsh = 2u - sh;
      const uint8_t *qa = p + 2 - qsh;
      const u32x4 v0 = ld16(qa), v1 = ld16(qa + 16);
      const uint32_t e = ld2(p + 32);
      const uint32_t V[9] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w, e};
      const uint8_t *ap = XQ + (int64_t)u * kQ8_1Bytes;
      const u32x4 a0 = ld16(ap), a1 = ld16(ap + 16);
      const uint32_t a2 = ld4(ap + 32);
      const uint32_t A[9] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w, a2};
      int D = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) D = dot4(align_bytes(V[i + 1], V[i], qsh), A[1 + i], D);
      if (DUMP) {
        Dd[row * (int64_t)nb + u] = D;
      } else {
        acc += dw * h2f(A[0]) * (float)D;
      }
    }
  }
  if (!DUMP) {
    acc = group_sum<L>(acc);
    if (live && li == 0) Y[row] = acc;
  }
}

// ---------------------------------------------------------------- dispatch
static int lanes_per_row(int64_t units) {
  int L = 64;
  while (L > 1 && (units % L) != 0) L >>= 1;
  return L;
}

#define QG_GEMV_CASE(KERNEL, LV, ...)                                                             \
  case LV:                                                                                        \
    if (dump)                                                                                     \
      hipLaunchKernelGGL((KERNEL<LV, true>), grid, dim3(256), 0, stream, __VA_ARGS__);            \
    else                                                                                          \
      hipLaunchKernelGGL((KERNEL<LV, false>), grid, dim3(256), 0, stream, __VA_ARGS__);           \
    break;

#define QG_GEMV_SWITCH(KERNEL, ...)          \
  switch (L) {                               \
    QG_GEMV_CASE(KERNEL, 64, __VA_ARGS__)    \
    QG_GEMV_CASE(KERNEL, 32, __VA_ARGS__)    \
    QG_GEMV_CASE(KERNEL, 16, __VA_ARGS__)    \
    QG_GEMV_CASE(KERNEL, 8, __VA_ARGS__)     \
    QG_GEMV_CASE(KERNEL, 4, __VA_ARGS__)     \
    QG_GEMV_CASE(KERNEL, 2, __VA_ARGS__)     \
    default:                                 \
      QG_GEMV_CASE_ONE(KERNEL, __VA_ARGS__)  \
  }

#define QG_GEMV_CASE_ONE(KERNEL, ...)                                                  \
  if (dump)                                                                            \
    hipLaunchKernelGGL((KERNEL<1, true>), grid, dim3(256), 0, stream, __VA_ARGS__);    \
  else                                                                                 \
    hipLaunchKernelGGL((KERNEL<1, false>), grid, dim3(256), 0, stream, __VA_ARGS__);

hipError_t launch_qgemv(int fmt, const void *w, const void *xq, float *y, int32_t *D, int32_t *S, int64_t n,
                        int64_t k, hipStream_t stream) {
  const bool dump = D != nullptr;
  const uint8_t *W = static_cast<const uint8_t *>(w);
  const uint8_t *X = static_cast<const uint8_t *>(xq);
  int64_t units;
  bool q8_pair = false;
  if (fmt == 0) {
    q8_pair = ((k / 32) % 2) == 0;
    units = q8_pair ? k / 64 : k / 32;
  } else {
    units = (k / 256) * 4;
  }
  const int L = lanes_per_row(units);
  const int64_t rows_per_block = 4 * (64 / L);
  const dim3 grid((unsigned)((n + rows_per_block - 1) / rows_per_block));
  const int ni = (int)n;
  if (fmt == 0 && q8_pair) {
    const int npair = (int)(k / 64);
    QG_GEMV_SWITCH(gemv_q8_0_pair_kernel, W, X, y, D, ni, npair)
  } else if (fmt == 0) {
    const int nb = (int)(k / 32);
    QG_GEMV_SWITCH(gemv_q8_0_single_kernel, W, X, y, D, ni, nb)
  } else if (fmt == 1) {
    const int nsb = (int)(k / 256);
    QG_GEMV_SWITCH(gemv_q4k_kernel, W, X, y, D, S, ni, nsb)
  } else {
    const int nsb = (int)(k / 256);
    QG_GEMV_SWITCH(gemv_q6k_kernel, W, X, y, D, ni, nsb)
  }
  return hipGetLastError();
}

}  // namespace qg
