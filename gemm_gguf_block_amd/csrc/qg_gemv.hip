// qg_gemv.hip -- batch-1 decode GEMV over Q8_0 / Q4_K / Q6_K weight blocks
// against one Q8_1 activation row (the dp4a-style dot kernels the blazr README
// lists for these three types, "Model Formats > GGUF", re-designed for gfx950),
// and over Q5_K, Q4_0 and Q5_0, GGUF types that README runs on its generic path.
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
//   Q4_0 / Q5_0 unit: a pair of blocks (36 / 44 bytes, dword aligned; rows
//        with an even block count only).
//
// With DUMP the same code writes the exact per-block int32 dots instead of y.
#include <algorithm>

#include "qg_blocks.h"
#include "qg_launch.h"

namespace qg {

// ------------------------------------------------------ activations in LDS
// Every row group reads the whole Q8_1 activation, so a workgroup stages it in
// (dynamic) LDS once per chunk of up to kXBlocks blocks.  The kernels read it
// in units of 64 values (four 16-value pieces) per lane, so it is stored
// unit-major for Q4_K: with U units in the chunk, piece c of unit u sits at
// qs[c*U + u] (16 bytes each), and a wave's 64 lanes read 64 consecutive
// pieces -- no LDS bank conflicts; unit u = blocks 2u, 2u+1 (pieces: halves
// of 2u, then of 2u+1), with the 16-byte record
//        rec[u] = {d_a(2u), d_a(2u+1), sum qs(2u), sum qs(2u+1)}.
// Q6_K keeps the blocks in order (block b at qs bytes 32b) with, per 16-value
// half h, the 8-byte record {d_a, sum of its 16 qs} at rec word pair 2b + h:
// its lanes read with bank conflicts, yet this measured faster for that
// kernel than the unit-major order.
// d_a is stored as f32 bits, sums as int32.
constexpr int kXBlocks = 512;
typedef uint32_t u32x4n __attribute__((ext_vector_type(4)));  // 16-byte aligned: ds_read/write_b128

// Blocks per staged chunk for a row of nb activation blocks, and its LDS
// bytes: 32 of qs and 16 of records per block.
__host__ __device__ inline int x_chunk_blocks(int64_t nb) { return nb < kXBlocks ? (int)nb : kXBlocks; }
inline size_t x_chunk_bytes(int64_t nb) { return (size_t)x_chunk_blocks(nb) * 48; }

struct XView {
  u32x4n *qs;   // 4U pieces of 16 bytes
  u32x4n *rec;  // 2U x 16 bytes (Q4_K uses the first U)
};

// View of a staged chunk of U units (2U blocks) at the start of the dynamic LDS.
__device__ __forceinline__ XView x_view(uint8_t *lds, int U) {
  u32x4n *p = reinterpret_cast<u32x4n *>(lds);
  return XView{p, p + 4 * U};
}

enum { kXQ4K = 1, kXQ6K = 2 };

// Stages activation blocks [b0, b0 + nb) (nb = 2U <= kXBlocks) in the layout
// of format FMT; all threads of the workgroup call it, between barriers.
template <int FMT>
__device__ __forceinline__ void stage_x(XView x, const uint8_t *__restrict__ XQ, int64_t b0, int nb) {
  const int U = nb / 2;
  for (int b = threadIdx.x; b < nb; b += blockDim.x) {
    const uint8_t *ap = XQ + (b0 + b) * kQ8_1Bytes;
    const u32x4 v0 = ld16(ap), v1 = ld16(ap + 16);
    const uint32_t v2 = ld4(ap + 32);
    const u32x4n lo = {v0.y, v0.z, v0.w, v1.x}, hi = {v1.y, v1.z, v1.w, v2};
    const uint32_t d = __builtin_bit_cast(uint32_t, h2f(v0.x));
    const int slo = bsum4(lo.w, bsum4(lo.z, bsum4(lo.y, bsum4(lo.x, 0))));
    const int shi = bsum4(hi.w, bsum4(hi.z, bsum4(hi.y, bsum4(hi.x, 0))));
    uint32_t *ra = reinterpret_cast<uint32_t *>(x.rec);
    if (FMT == kXQ4K) {
      const int u = b >> 1, bb = b & 1;
      x.qs[(2 * bb) * U + u] = lo;
      x.qs[(2 * bb + 1) * U + u] = hi;
      ra[4 * u + bb] = d;
      ra[4 * u + 2 + bb] = (uint32_t)(slo + shi);
    } else {
      x.qs[2 * b] = lo;
      x.qs[2 * b + 1] = hi;
      ra[4 * b] = d;
      ra[4 * b + 1] = (uint32_t)slo;
      ra[4 * b + 2] = d;
      ra[4 * b + 3] = (uint32_t)shi;
    }
  }
}

// ------------------------------------------------------------- Q4_K, Q5_K
// The K-quants with a min term share this kernel.  Q5_K (FMT 3) is Q4_K's
// block with qh[32] between the header and qs: element 32j + l of a
// superblock takes bit j of qh[l] as its fifth code bit.
template <int L, int R, bool DUMP, int FMT, int NWV>
__device__ __forceinline__ void gemv_kmin(const uint8_t *__restrict__ W, const uint8_t *__restrict__ XQ,
                                          float *__restrict__ Y, int32_t *__restrict__ Dd,
                                          int32_t *__restrict__ Sd, int n, int nsb) {
  constexpr bool Q5 = FMT == 3;
  constexpr int kBlockBytes = Q5 ? kQ5KBytes : kQ4KBytes;
  constexpr int kQsOff = Q5 ? 48 : 16;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int G = 64 / L;
  constexpr int kChunkSb = kXBlocks / 8;
  constexpr int kGroupRows = NWV * G * R;  // rows per workgroup per group
  const int lane = threadIdx.x & 63;
  const int li = lane & (L - 1);
  const int64_t rb = (int64_t)nsb * kBlockBytes;
  const int64_t ngroups = ((int64_t)n + kGroupRows - 1) / kGroupRows;
  int staged = -1;  // first superblock of the chunk in xs
  // persistent over row groups, like the Q6_K kernel
  for (int64_t grp = blockIdx.x; grp < ngroups; grp += gridDim.x) {
    const int64_t row0 = ((grp * NWV + (threadIdx.x >> 6)) * G + lane / L) * R;
    const uint8_t *wrow = W + row0 * rb;
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
    for (int c0 = 0; c0 < nsb; c0 += kChunkSb) {
      const int csb = min(kChunkSb, nsb - c0);
      const int U = 4 * csb;
      const XView xs = x_view(lds, U);
      // L divides 4*nsb and 4*kChunkSb, so every lane of the workgroup runs
      // the same number of units per chunk (rows past n included, masked):
      // the chunk's staging barrier can sit in the first one, after that
      // unit's weight loads are in flight
      for (int u = li; u < U; u += L) {
        const int sbl = u >> 2, g = u & 3;
        const int sb = c0 + sbl;
        // weights of this unit for the R rows, all loads issued before any use
        u32x4 hdr[R], qa[R], qb[R], ha[Q5 ? R : 1], hb[Q5 ? R : 1];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (row0 + r < n) {
            const uint8_t *bp = wrow + r * rb + sb * kBlockBytes;
            hdr[r] = ld16(bp);
            qa[r] = ld16(bp + kQsOff + 32 * g);
            qb[r] = ld16(bp + kQsOff + 16 + 32 * g);
            if constexpr (Q5) {
              ha[r] = ld16(bp + 16);  // qh[0..15]
              hb[r] = ld16(bp + 32);  // qh[16..31]
            }
          } else {
            hdr[r] = qa[r] = qb[r] = u32x4{0u, 0u, 0u, 0u};
            if constexpr (Q5) ha[r] = hb[r] = hdr[r];
          }
        }
        if (staged != c0) {
          if (staged >= 0) __syncthreads();  // the previous chunk is no longer read
          stage_x<kXQ4K>(xs, XQ, (int64_t)8 * c0, 8 * csb);
          __syncthreads();
          staged = c0;
        }
        if (row0 >= n) continue;
        // the activation slice: Q8_1 blocks 8sb + 2g (low nibbles) and +1
        // (high nibbles), shared by the R rows
        const u32x4n x0 = xs.qs[u], x1 = xs.qs[U + u], x2 = xs.qs[2 * U + u], x3 = xs.qs[3 * U + u];
        const u32x4n rec = xs.rec[u];
        const uint32_t A0[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        const uint32_t A1[8] = {x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
        const int S0 = (int)rec.z, S1 = (int)rec.w;
        const float da0 = as_f32(rec.x), da1 = as_f32(rec.y);
        const float dS0 = da0 * (float)S0, dS1 = da1 * (float)S1;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint32_t Q[8] = {qa[r].x, qa[r].y, qa[r].z, qa[r].w, qb[r].x, qb[r].y, qb[r].z, qb[r].w};
          int D0 = 0, D1 = 0;
          if constexpr (Q5) {
            // fifth bits of sub-blocks 2g and 2g+1: bits 2g, 2g+1 of qh[l]
            const uint32_t H[8] = {ha[r].x, ha[r].y, ha[r].z, ha[r].w, hb[r].x, hb[r].y, hb[r].z, hb[r].w};
            const uint32_t s0 = 2u * (uint32_t)g;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const uint32_t h0 = ((H[i] >> s0) & 0x01010101u) << 4, h1 = ((H[i] >> (s0 + 1)) & 0x01010101u) << 4;
              D0 = dot4((Q[i] & 0x0F0F0F0Fu) | h0, A0[i], D0);
              D1 = dot4(((Q[i] >> 4) & 0x0F0F0F0Fu) | h1, A1[i], D1);
            }
          } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              D0 = dot4(Q[i] & 0x0F0F0F0Fu, A0[i], D0);
              D1 = dot4((Q[i] >> 4) & 0x0F0F0F0Fu, A1[i], D1);
            }
          }
          if (DUMP) {
            if (row0 + r < n) {
              Dd[(row0 + r) * (int64_t)(nsb * 8) + 8 * sb + 2 * g] = D0;
              Dd[(row0 + r) * (int64_t)(nsb * 8) + 8 * sb + 2 * g + 1] = D1;
            }
          } else {
            int sc0, sc1, m0, m1;
            q4k_scales(hdr[r].y, hdr[r].z, hdr[r].w, g, sc0, sc1, m0, m1);
            const float d = h2f(hdr[r].x), dmin = h2f(hdr[r].x >> 16);
            const float t = da0 * (float)(sc0 * D0) + da1 * (float)(sc1 * D1);
            const float mm = dS0 * (float)m0 + dS1 * (float)m1;
            acc[r] += d * t - dmin * mm;
          }
        }
        if (DUMP && row0 == 0) {
          Sd[8 * sb + 2 * g] = S0;
          Sd[8 * sb + 2 * g + 1] = S1;
        }
      }
    }
    if (!DUMP && row0 < n) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float v = group_sum_last<L>(acc[r]);
        if (li == L - 1 && row0 + r < n) Y[row0 + r] = v;
      }
    }
  }
}

// Waves per workgroup of the Q4_K / Q5_K GEMV.
constexpr int kWavesQ4K = 4;

template <int L, int R, bool DUMP>
__global__ __launch_bounds__(64 * kWavesQ4K) void gemv_q4k_kernel(const uint8_t *__restrict__ W,
                                                                  const uint8_t *__restrict__ XQ,
                                                                  float *__restrict__ Y, int32_t *__restrict__ Dd,
                                                                  int32_t *__restrict__ Sd, int n, int nsb) {
  gemv_kmin<L, R, DUMP, 1, kWavesQ4K>(W, XQ, Y, Dd, Sd, n, nsb);
}

template <int L, int R, bool DUMP>
__global__ __launch_bounds__(64 * kWavesQ4K) void gemv_q5k_kernel(const uint8_t *__restrict__ W,
                                                                  const uint8_t *__restrict__ XQ,
                                                                  float *__restrict__ Y, int32_t *__restrict__ Dd,
                                                                  int32_t *__restrict__ Sd, int n, int nsb) {
  gemv_kmin<L, R, DUMP, 3, kWavesQ4K>(W, XQ, Y, Dd, Sd, n, nsb);
}

// ---------------------------------------------------------------- Q6_K
template <int L, int R, bool DUMP>
__global__ __launch_bounds__(256) void gemv_q6k_kernel(const uint8_t *__restrict__ W, const uint8_t *__restrict__ XQ,
                                                       float *__restrict__ Y, int32_t *__restrict__ Dd, int n,
                                                       int nsb) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int G = 64 / L;
  constexpr int kChunkSb = kXBlocks / 8;
  constexpr int kGroupRows = 4 * G * R;  // rows per workgroup per group
  const int lane = threadIdx.x & 63;
  const int li = lane & (L - 1);
  const int64_t rb = (int64_t)nsb * kQ6KBytes;
  const int64_t ngroups = ((int64_t)n + kGroupRows - 1) / kGroupRows;
  int staged = -1;  // first superblock of the chunk in xs
  // persistent: the grid holds what fits on the device and strides over row
  // groups, so the activation is staged once per workgroup when it fits in
  // one chunk
  for (int64_t grp = blockIdx.x; grp < ngroups; grp += gridDim.x) {
  const int64_t row0 = ((grp * 4 + (threadIdx.x >> 6)) * G + lane / L) * R;
  const uint8_t *wrow = W + row0 * rb;
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
  for (int c0 = 0; c0 < nsb; c0 += kChunkSb) {
    const int csb = min(kChunkSb, nsb - c0);
    const int U = 4 * csb;
    const XView xs = x_view(lds, U);
    if (staged != c0) {
      if (staged >= 0) __syncthreads();  // the previous chunk is no longer read
      stage_x<kXQ6K>(xs, XQ, (int64_t)8 * c0, 8 * csb);
      __syncthreads();
      staged = c0;
    }
    if (row0 >= n) continue;
    // L divides 4*nsb and 4*kChunkSb, hence the unit count of every chunk
    for (int u = li; u < U; u += L) {
      const int sbl = u >> 2, h = (u >> 1) & 1, l = u & 1;
      const int sb = c0 + sbl;
      u32x4 qlA[R], qlB[R], qh[R];
      u32x2 sc8[R];
      uint32_t dh[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (row0 + r < n) {
          const uint8_t *bp = wrow + r * rb + sb * kQ6KBytes;  // 2-byte aligned
          qlA[r] = ld16_a2(bp + 64 * h + 16 * l);
          qlB[r] = ld16_a2(bp + 64 * h + 32 + 16 * l);
          qh[r] = ld16_a2(bp + 128 + 32 * h + 16 * l);
          sc8[r] = ld8_a2(bp + 192 + 8 * h);  // scales[8h .. 8h+7]
          dh[r] = ld2(bp + 208);
        } else {
          qlA[r] = qlB[r] = qh[r] = u32x4{0u, 0u, 0u, 0u};
          sc8[r] = u32x2{0u, 0u};
          dh[r] = 0u;
        }
      }
      // activation: Q8_1 blocks 8sb + 4h + g, values 16l..16l+15 of each
      uint32_t a[4][4];
      float da[4];
      int S16[4];
      const uint8_t *xq = reinterpret_cast<const uint8_t *>(xs.qs);
      const u32x2 *xr = reinterpret_cast<const u32x2 *>(xs.rec);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int blk = 8 * sbl + 4 * h + g;
        const u32x4 av = *reinterpret_cast<const u32x4 *>(xq + 32 * blk + 16 * l);
        const u32x2 rec = xr[2 * blk + l];
        a[g][0] = av.x; a[g][1] = av.y; a[g][2] = av.z; a[g][3] = av.w;
        da[g] = as_f32(rec.x);
        S16[g] = 32 * (int)rec.y;
      }
      const uint32_t lo8 = 8u * (uint32_t)l;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        // sub-block 8h + 2g + l has scale byte 2g + l of scales[8h..]
        const int sc[4] = {sbyte(sc8[r].x, lo8), sbyte(sc8[r].x, 16u + lo8), sbyte(sc8[r].y, lo8),
                           sbyte(sc8[r].y, 16u + lo8)};
        const uint32_t A4[4] = {qlA[r].x, qlA[r].y, qlA[r].z, qlA[r].w};
        const uint32_t B4[4] = {qlB[r].x, qlB[r].y, qlB[r].z, qlB[r].w};
        const uint32_t H4[4] = {qh[r].x, qh[r].y, qh[r].z, qh[r].w};
        float t = 0.f;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          int Dg = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            uint32_t q;
            if (g == 0) q = (A4[i] & 0x0F0F0F0Fu) | ((H4[i] << 4) & 0x30303030u);
            else if (g == 1) q = (B4[i] & 0x0F0F0F0Fu) | ((H4[i] << 2) & 0x30303030u);
            else if (g == 2) q = ((A4[i] >> 4) & 0x0F0F0F0Fu) | (H4[i] & 0x30303030u);
            else q = ((B4[i] >> 4) & 0x0F0F0F0Fu) | ((H4[i] >> 2) & 0x30303030u);
            Dg = dot4(q, a[g][i], Dg);  // codes 0..63 are non-negative int8
          }
          Dg -= S16[g];  // sum (q-32)*qa
          if (DUMP) {
            if (row0 + r < n) Dd[(row0 + r) * (int64_t)(nsb * 16) + 16 * sb + 8 * h + 2 * g + l] = Dg;
          } else {
            t += da[g] * (float)(sc[g] * Dg);
          }
        }
        acc[r] += h2f(dh[r]) * t;
      }
    }
  }
  if (!DUMP && row0 < n) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float v = group_sum_last<L>(acc[r]);
      if (li == L - 1 && row0 + r < n) Y[row0 + r] = v;
    }
  }
  }
}

// ---------------------------------------------------------------- Q8_0
// Rows with an even block count: unit = block pair at a dword-aligned offset.
// Persistent like the K-quant kernels: the workgroup stages the Q8_1
// activation in LDS once per chunk, unit-major exactly as for Q4_K (a unit is
// two 32-value blocks there too), so a lane group reads its activation slice
// from LDS instead of every lane group fetching it from L2.
template <int L, int R, bool DUMP>
__global__ __launch_bounds__(256) void gemv_q8_0_pair_kernel(const uint8_t *__restrict__ W,
                                                             const uint8_t *__restrict__ XQ, float *__restrict__ Y,
                                                             int32_t *__restrict__ Dd, int n, int npair) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int G = 64 / L;
  constexpr int kChunkU = kXBlocks / 2;  // units (block pairs) per staged chunk
  constexpr int kGroupRows = 4 * G * R;  // rows per workgroup per group
  const int lane = threadIdx.x & 63;
  const int li = lane & (L - 1);
  const int64_t rb = (int64_t)npair * (2 * kQ8_0Bytes);
  const int64_t ngroups = ((int64_t)n + kGroupRows - 1) / kGroupRows;
  int staged = -1;  // first unit of the chunk in xs
  for (int64_t grp = blockIdx.x; grp < ngroups; grp += gridDim.x) {
    const int64_t row0 = ((grp * 4 + (threadIdx.x >> 6)) * G + lane / L) * R;
    const uint8_t *wrow = W + row0 * rb;
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
    for (int c0 = 0; c0 < npair; c0 += kChunkU) {
      const int U = min(kChunkU, npair - c0);
      const XView xs = x_view(lds, U);
      // L divides npair and kChunkU, so every lane of the workgroup runs the
      // same number of units per chunk (rows past n included, masked): the
      // staging barrier sits in the first one, after its weight loads
      for (int u = li; u < U; u += L) {
        uint32_t Wd[R][17];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (row0 + r < n) {
            const uint8_t *bp = wrow + r * rb + (int64_t)(c0 + u) * (2 * kQ8_0Bytes);
            const u32x4 w0 = ld16(bp), w1 = ld16(bp + 16), w2 = ld16(bp + 32), w3 = ld16(bp + 48);
            Wd[r][0] = w0.x; Wd[r][1] = w0.y; Wd[r][2] = w0.z; Wd[r][3] = w0.w;
            Wd[r][4] = w1.x; Wd[r][5] = w1.y; Wd[r][6] = w1.z; Wd[r][7] = w1.w;
            Wd[r][8] = w2.x; Wd[r][9] = w2.y; Wd[r][10] = w2.z; Wd[r][11] = w2.w;
            Wd[r][12] = w3.x; Wd[r][13] = w3.y; Wd[r][14] = w3.z; Wd[r][15] = w3.w;
            Wd[r][16] = ld4(bp + 64);
          } else {
#pragma unroll
            for (int i = 0; i < 17; ++i) Wd[r][i] = 0u;
          }
        }
        if (staged != c0) {
          if (staged >= 0) __syncthreads();  // the previous chunk is no longer read
          stage_x<kXQ4K>(xs, XQ, 2 * (int64_t)c0, 2 * U);
          __syncthreads();
          staged = c0;
        }
        if (row0 >= n) continue;
        // blocks 2u (pieces 0, 1) and 2u + 1 (pieces 2, 3) of the chunk
        const u32x4n x0 = xs.qs[u], x1 = xs.qs[U + u], x2 = xs.qs[2 * U + u], x3 = xs.qs[3 * U + u];
        const u32x4n rec = xs.rec[u];
        const uint32_t A0[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        const uint32_t A1[8] = {x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
        const float da0 = as_f32(rec.x), da1 = as_f32(rec.y);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          int D0 = 0, D1 = 0;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            D0 = dot4(align_bytes(Wd[r][i + 1], Wd[r][i], 2), A0[i], D0);  // qs of block 0: bytes 2..33
            D1 = dot4(Wd[r][9 + i], A1[i], D1);                            // qs of block 1: bytes 36..67
          }
          if (DUMP) {
            if (row0 + r < n) {
              Dd[(row0 + r) * (int64_t)(2 * npair) + 2 * (c0 + u)] = D0;
              Dd[(row0 + r) * (int64_t)(2 * npair) + 2 * (c0 + u) + 1] = D1;
            }
          } else {
            acc[r] += h2f(Wd[r][0]) * da0 * (float)D0 + h2f(Wd[r][8] >> 16) * da1 * (float)D1;
          }
        }
      }
    }
    if (!DUMP && row0 < n) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float v = group_sum_last<L>(acc[r]);
        if (li == L - 1 && row0 + r < n) Y[row0 + r] = v;
      }
    }
  }
}

// Rows with an odd block count: unit = one block at a 2-byte aligned offset.
// (Not tuned: the common row lengths have an even block count.)
template <int L, int R, bool DUMP>
__global__ __launch_bounds__(256) void gemv_q8_0_single_kernel(const uint8_t *__restrict__ W,
                                                               const uint8_t *__restrict__ XQ,
                                                               float *__restrict__ Y, int32_t *__restrict__ Dd, int n,
                                                               int nb) {
  static_assert(R == 1, "one row per lane group");
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
    acc = group_sum_last<L>(acc);
    if (live && li == L - 1) Y[row] = acc;
  }
}

// ---------------------------------------------------------------- Q4_0, Q5_0
// Bits b0..b3 of h moved to bit 0 of bytes 0..3 (the four shifted copies of h
// set disjoint bits, so the product carries nothing).
__device__ __forceinline__ uint32_t spread4(uint32_t h) { return (h * 0x00204081u) & 0x01010101u; }

// Rows with an even block count; unit = a block pair at a dword-aligned offset:
//   Q4_0 (36 bytes): d0 | qs0[16] | d1 | qs1[16]
//   Q5_0 (44 bytes): d0 | qh0[4] | qs0[16] | d1 | qh1[4] | qs1[16]
// Byte j of qs holds codes j (low nibble) and 16 + j (high nibble); Q5_0's
// fifth bits are bit i of the little-endian qh word.  The lane dots the stored
// codes (0..15 / 0..31, non-negative bytes) with v_dot4 and subtracts
// off * sum(qa): sum (q - off) qa exactly, off = 8 / 16.  sum(qa) is taken
// once per unit and reused for the R rows.
template <int FMT, int L, int R, bool DUMP>
__device__ __forceinline__ void gemv_legacy_pair(const uint8_t *__restrict__ W, const uint8_t *__restrict__ XQ,
                                                 float *__restrict__ Y, int32_t *__restrict__ Dd, int n, int npair) {
  constexpr bool kQ5 = FMT == 5;
  constexpr int kPair = kQ5 ? 44 : 36;   // bytes per block pair
  constexpr int kDw = kPair / 4;         // dwords per pair
  constexpr int kOff = kQ5 ? 16 : 8;
  constexpr int G = 64 / L;
  const int lane = threadIdx.x & 63;
  const int li = lane & (L - 1);
  const int64_t row0 = (((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * G + lane / L) * R;
  const int64_t rb = (int64_t)npair * kPair;
  const uint8_t *wrow = W + row0 * rb;
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
  if (row0 < n) {
    for (int u = li; u < npair; u += L) {
      uint32_t Wd[R][kDw];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (row0 + r < n) {
          const uint8_t *bp = wrow + r * rb + (int64_t)u * kPair;
          const u32x4 w0 = ld16(bp), w1 = ld16(bp + 16);
          Wd[r][0] = w0.x; Wd[r][1] = w0.y; Wd[r][2] = w0.z; Wd[r][3] = w0.w;
          Wd[r][4] = w1.x; Wd[r][5] = w1.y; Wd[r][6] = w1.z; Wd[r][7] = w1.w;
#pragma unroll
          for (int i = 8; i < kDw; ++i) Wd[r][i] = ld4(bp + 4 * i);
        } else {
#pragma unroll
          for (int i = 0; i < kDw; ++i) Wd[r][i] = 0u;
        }
      }
      uint32_t A[18];
      load_q8_1_pair(XQ + (int64_t)(2 * u) * kQ8_1Bytes, A);
      const float da0 = h2f(A[0]), da1 = h2f(A[9]);
      int sa0 = 0, sa1 = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        sa0 = bsum4(A[1 + i], sa0);
        sa1 = bsum4(A[10 + i], sa1);
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        // the two blocks' qs dwords, qh words and d halves
        uint32_t Q0[4], Q1[4], h0 = 0u, h1 = 0u, d0, d1;
        if constexpr (kQ5) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            Q0[i] = align_bytes(Wd[r][i + 2], Wd[r][i + 1], 2);  // bytes 6..21
            Q1[i] = Wd[r][7 + i];                                // bytes 28..43
          }
          h0 = align_bytes(Wd[r][1], Wd[r][0], 2);  // bytes 2..5
          h1 = Wd[r][6];                             // bytes 24..27
          d0 = Wd[r][0];
          d1 = Wd[r][5] >> 16;                       // bytes 22..23
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            Q0[i] = align_bytes(Wd[r][i + 1], Wd[r][i], 2);  // bytes 2..17
            Q1[i] = Wd[r][5 + i];                            // bytes 20..35
          }
          d0 = Wd[r][0];
          d1 = Wd[r][4] >> 16;                               // bytes 18..19
        }
        int D0 = 0, D1 = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t l0 = Q0[i] & 0x0F0F0F0Fu, u0 = (Q0[i] >> 4) & 0x0F0F0F0Fu;
          uint32_t l1 = Q1[i] & 0x0F0F0F0Fu, u1 = (Q1[i] >> 4) & 0x0F0F0F0Fu;
          if constexpr (kQ5) {
            l0 |= spread4((h0 >> (4 * i)) & 0xFu) << 4;
            u0 |= spread4((h0 >> (16 + 4 * i)) & 0xFu) << 4;
            l1 |= spread4((h1 >> (4 * i)) & 0xFu) << 4;
            u1 |= spread4((h1 >> (16 + 4 * i)) & 0xFu) << 4;
          }
          D0 = dot4(l0, A[1 + i], D0);   // codes 4i..4i+3
          D0 = dot4(u0, A[5 + i], D0);   // codes 16+4i..
          D1 = dot4(l1, A[10 + i], D1);
          D1 = dot4(u1, A[14 + i], D1);
        }
        D0 -= kOff * sa0;
        D1 -= kOff * sa1;
        if (DUMP) {
          if (row0 + r < n) {
            Dd[(row0 + r) * (int64_t)(2 * npair) + 2 * u] = D0;
            Dd[(row0 + r) * (int64_t)(2 * npair) + 2 * u + 1] = D1;
          }
        } else {
          acc[r] += h2f(d0) * da0 * (float)D0 + h2f(d1) * da1 * (float)D1;
        }
      }
    }
  }
  if (!DUMP) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float v = group_sum_last<L>(acc[r]);
      if (li == L - 1 && row0 + r < n) Y[row0 + r] = v;
    }
  }
}

template <int L, int R, bool DUMP>
__global__ __launch_bounds__(256) void gemv_q4_0_kernel(const uint8_t *__restrict__ W, const uint8_t *__restrict__ XQ,
                                                        float *__restrict__ Y, int32_t *__restrict__ Dd, int n,
                                                        int npair) {
  gemv_legacy_pair<4, L, R, DUMP>(W, XQ, Y, Dd, n, npair);
}

template <int L, int R, bool DUMP>
__global__ __launch_bounds__(256) void gemv_q5_0_kernel(const uint8_t *__restrict__ W, const uint8_t *__restrict__ XQ,
                                                        float *__restrict__ Y, int32_t *__restrict__ Dd, int n,
                                                        int npair) {
  gemv_legacy_pair<5, L, R, DUMP>(W, XQ, Y, Dd, n, npair);
}

// ---------------------------------------------------------------- dispatch
// Rows per lane group (R): each lane reuses its activation slice across R
// rows and keeps R rows' worth of weight loads in flight.
constexpr int kRowsQ8_0 = 1;    // the staged block-pair kernel (R = 2: 5.35 us, R = 1: 5.22 us at 4096 x 4096)
constexpr int kRowsLegacy = 2;  // Q4_0 / Q5_0 (R = 1: 8.00 us, R = 2: 7.22 us at 14336 x 4096)
constexpr int kRowsQ4K = 1;
constexpr int kRowsQ6K = 4;
// Q6_K grids hold this many workgroups per resident one: the queued ones start
// as others finish, which evens out the last round of row groups.
constexpr int64_t kOversubQ6K = 2;
constexpr int64_t kOversubQ8_0 = 1;

#define QG_LAUNCH(KERNEL, LV, RV, ...)                                                          \
  do {                                                                                          \
    if (dump)                                                                                   \
      hipLaunchKernelGGL((KERNEL<LV, RV, true>), grid, dim3(256), 0, stream, __VA_ARGS__);      \
    else                                                                                        \
      hipLaunchKernelGGL((KERNEL<LV, RV, false>), grid, dim3(256), 0, stream, __VA_ARGS__);     \
  } while (0)

#define QG_GEMV_SWITCH(KERNEL, RV, ...)                         \
  switch (L) {                                                  \
    case 64: QG_LAUNCH(KERNEL, 64, RV, __VA_ARGS__); break;     \
    case 32: QG_LAUNCH(KERNEL, 32, RV, __VA_ARGS__); break;     \
    case 16: QG_LAUNCH(KERNEL, 16, RV, __VA_ARGS__); break;     \
    case 8: QG_LAUNCH(KERNEL, 8, RV, __VA_ARGS__); break;       \
    case 4: QG_LAUNCH(KERNEL, 4, RV, __VA_ARGS__); break;       \
    case 2: QG_LAUNCH(KERNEL, 2, RV, __VA_ARGS__); break;       \
    default: QG_LAUNCH(KERNEL, 1, RV, __VA_ARGS__); break;      \
  }

// Persistent launch: at most `oversub` times the resident workgroups of
// `waves` waves, each striding over the row groups of waves * (64 / L) * R
// rows; `xlds` bytes of dynamic LDS.  The dump instance runs on the grid of
// the product instance (sized from the product kernel's occupancy), so a dump
// walks the row groups exactly as the product launch of that shape does.
#define QG_LAUNCH_PERSISTENT(KERNEL, LV, RV, ...)                                               \
  do {                                                                                          \
    const int64_t groups = (n + waves * (64 / LV) * RV - 1) / (waves * (64 / LV) * RV);                 \
    const int64_t g = std::min(groups, oversub * resident_blocks<KERNEL<LV, RV, false>>(64 * waves, xlds)); \
    if (dump)                                                                                   \
      hipLaunchKernelGGL((KERNEL<LV, RV, true>), dim3((unsigned)g), dim3(64 * waves), xlds, stream, __VA_ARGS__); \
    else                                                                                        \
      hipLaunchKernelGGL((KERNEL<LV, RV, false>), dim3((unsigned)g), dim3(64 * waves), xlds, stream, __VA_ARGS__); \
  } while (0)

#define QG_GEMV_SWITCH_PERSISTENT(KERNEL, RV, ...)                         \
  switch (L) {                                                             \
    case 64: QG_LAUNCH_PERSISTENT(KERNEL, 64, RV, __VA_ARGS__); break;     \
    case 32: QG_LAUNCH_PERSISTENT(KERNEL, 32, RV, __VA_ARGS__); break;     \
    case 16: QG_LAUNCH_PERSISTENT(KERNEL, 16, RV, __VA_ARGS__); break;     \
    case 8: QG_LAUNCH_PERSISTENT(KERNEL, 8, RV, __VA_ARGS__); break;       \
    case 4: QG_LAUNCH_PERSISTENT(KERNEL, 4, RV, __VA_ARGS__); break;       \
    case 2: QG_LAUNCH_PERSISTENT(KERNEL, 2, RV, __VA_ARGS__); break;       \
    default: QG_LAUNCH_PERSISTENT(KERNEL, 1, RV, __VA_ARGS__); break;      \
  }

static dim3 gemv_grid(int64_t n, int L, int R) {
  const int64_t rows_per_block = 4 * (64 / L) * (int64_t)R;
  return dim3((unsigned)((n + rows_per_block - 1) / rows_per_block));
}

hipError_t launch_qgemv(int fmt, const void *w, const void *xq, float *y, int32_t *D, int32_t *S, int64_t n,
                        int64_t k, hipStream_t stream) {
  const bool dump = D != nullptr;
  const uint8_t *W = static_cast<const uint8_t *>(w);
  const uint8_t *X = static_cast<const uint8_t *>(xq);
  const int ni = (int)n;
  if (fmt == 0 && ((k / 32) % 2) == 0) {
    const int npair = (int)(k / 64);
    const int L = lanes_per_row(npair);
    const size_t xlds = x_chunk_bytes(k / 32);
    const int64_t oversub = kOversubQ8_0;
    const int waves = 4;
    QG_GEMV_SWITCH_PERSISTENT(gemv_q8_0_pair_kernel, kRowsQ8_0, W, X, y, D, ni, npair)
  } else if (fmt == 0) {
    const int nb = (int)(k / 32);
    const int L = lanes_per_row(nb);
    const dim3 grid = gemv_grid(n, L, 1);
    QG_GEMV_SWITCH(gemv_q8_0_single_kernel, 1, W, X, y, D, ni, nb)
  } else if (fmt == 1) {
    const int nsb = (int)(k / 256);
    const int L = lanes_per_row((int64_t)nsb * 4);
    const size_t xlds = x_chunk_bytes(k / 32);
    const int64_t oversub = 1;
    const int waves = kWavesQ4K;
    QG_GEMV_SWITCH_PERSISTENT(gemv_q4k_kernel, kRowsQ4K, W, X, y, D, S, ni, nsb)
  } else if (fmt == 4 || fmt == 5) {
    const int npair = (int)(k / 64);
    const int L = lanes_per_row(npair);
    const dim3 grid = gemv_grid(n, L, kRowsLegacy);
    if (fmt == 4) {
      QG_GEMV_SWITCH(gemv_q4_0_kernel, kRowsLegacy, W, X, y, D, ni, npair)
    } else {
      QG_GEMV_SWITCH(gemv_q5_0_kernel, kRowsLegacy, W, X, y, D, ni, npair)
    }
  } else if (fmt == 3) {
    const int nsb = (int)(k / 256);
    const int L = lanes_per_row((int64_t)nsb * 4);
    const size_t xlds = x_chunk_bytes(k / 32);
    const int64_t oversub = 1;
    const int waves = kWavesQ4K;
    QG_GEMV_SWITCH_PERSISTENT(gemv_q5k_kernel, kRowsQ4K, W, X, y, D, S, ni, nsb)
  } else {
    const int nsb = (int)(k / 256);
    const int L = lanes_per_row((int64_t)nsb * 4);
    const size_t xlds = x_chunk_bytes(k / 32);
    const int64_t oversub = kOversubQ6K;
    const int waves = 4;
    QG_GEMV_SWITCH_PERSISTENT(gemv_q6k_kernel, kRowsQ6K, W, X, y, D, ni, nsb)
  }
  return hipGetLastError();
}

}  // namespace qg
