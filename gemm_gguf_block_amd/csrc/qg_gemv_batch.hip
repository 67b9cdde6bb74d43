// qg_gemv_batch.hip -- small-batch GEMV: b <= 8 Q8_1 activation rows against
// one read of Q8_0 / Q4_K / Q6_K weight rows, Y[i][r] = w^[r] . x^_i.
//
// This is the decode step of several concurrent sequences (the N generation
// slots of infr page, "Concurrent slots, many models"): every weight byte is
// fetched once and dotted against all b rows, so the call costs about one
// batch-1 GEMV of HBM traffic while the integer-dot work grows with b.
//
// Decomposition as in the batch-1 kernels: a row is cut into units (Q8_0: a
// pair of blocks read as stored in aligned dwords when the row has an even
// block count, else one 32-value block; Q4_K: a 64-value group = sub-blocks
// 2g, 2g+1; Q6_K: the 64-value (half h, l-half) set of four 16-value
// sub-blocks), L lanes share a
// row and walk its units.  A lane unpacks its unit's codes once into VGPRs and
// runs v_dot4 against each of the B activation rows, which the persistent
// workgroup stages in LDS once per chunk of k.  Rows i >= b of the batch
// template are staged as zeros and never written.
//
// LDS per activation row and chunk of U units: the unit's 16-value pieces
// unit-major, qs[(i * NP + p) * U + u] (NP = 2 pieces for Q8_0, 4 for the
// K-quants), so a wave's 64 lanes read consecutive 16-byte pieces, and
// per-unit records:
//   Q8_0  recf[i * U + u]  = d_a
//   Q4_K, Q8_0 pairs  rec4[i * U + u]  = {d_a(2u), d_a(2u+1), d_a*sum q (2u), d_a*sum q (2u+1)}
//   Q6_K  rec4[2(i * U + u)] = d_a of pieces 0..3, [+1] = sum of each piece's 16 qs
//
// With DUMP the same code writes the exact per-block int32 dots instead of Y:
// D[i][r][block] per 32-value block (Q8_0, Q4_K) or per 16-value sub-block
// (Q6_K).
#include <algorithm>

#include "qg_blocks.h"
#include "qg_launch.h"

namespace qg {

namespace {

typedef uint32_t u32x4n __attribute__((ext_vector_type(4)));  // 16-byte aligned: ds_read/write_b128

// kFmtQ8P: Q8_0 rows with an even block count, read as aligned block pairs.
enum { kFmtQ8_0 = 0, kFmtQ4K = 1, kFmtQ6K = 2, kFmtQ8P = 3 };

// Waves per workgroup.  Every workgroup stages all activation rows, so larger
// workgroups stage them fewer times; for Q8_0 with 5-8 rows that staging
// outweighs the workgroup's share of weight bytes, and 16 waves measured
// faster (8 rows at 4096 x 4096: 8.49 -> 7.78 us; 6 rows 8.18 -> 7.56), while
// 2 and 4 rows and the K-quants measured slower with 16 (Q8_0 b = 2: 6.63 ->
// 6.73 us; Q4_K b = 4: 11.1 -> 12.3; Q6_K b = 4: 99.1 -> 102.0).
template <int FMT, int B>
__host__ __device__ constexpr int batch_waves() {
  return (FMT == kFmtQ8_0 || FMT == kFmtQ8P) && B == 8 ? 16 : 8;
}

// Values per unit and 16-value pieces per unit.
template <int FMT> struct Unit {
  static constexpr int kValues = FMT == kFmtQ8_0 ? 32 : 64;  // Q8P: a block pair
  static constexpr int kPieces = kValues / 16;
};

// Activation blocks per staged chunk for a batch template of B rows: 1024/B
// blocks keeps LDS at <= 48 KB (32 B of qs + <= 16 B of records per block).
template <int B> constexpr int chunk_blocks() { return 1024 / B; }

template <int FMT> __host__ __device__ constexpr int rec_bytes_per_block() {
  return FMT == kFmtQ8_0 ? 4 : (FMT == kFmtQ4K || FMT == kFmtQ8P) ? 8 : 16;
}

// LDS bytes for nbk blocks of B rows.
template <int FMT, int B> size_t batch_lds_bytes(int64_t nbk) {
  const int64_t cb = std::min<int64_t>(nbk, chunk_blocks<B>());
  return (size_t)(B * cb * (32 + rec_bytes_per_block<FMT>()));
}

// Stages blocks [c0, c0 + cb) of every activation row i < nb (rows nb..B-1 as
// zeros); XQ row i starts at XQ + i * row_bytes.  All threads call it,
// between barriers.
template <int FMT, int B>
__device__ __forceinline__ void stage_batch(uint8_t *lds, const uint8_t *__restrict__ XQ, int64_t row_bytes, int nb,
                                            int64_t c0, int cb) {
  constexpr int NP = Unit<FMT>::kPieces;
  const int U = cb * 32 / Unit<FMT>::kValues;
  u32x4n *qs = reinterpret_cast<u32x4n *>(lds);
  uint8_t *rec = lds + (size_t)B * NP * U * 16;
  for (int t = threadIdx.x; t < B * cb; t += 64 * batch_waves<FMT, B>()) {
    const int i = t / cb, blk = t - i * cb;
    u32x4n lo = {0u, 0u, 0u, 0u}, hi = lo;
    float d = 0.f;
    if (i < nb) {
      const uint8_t *ap = XQ + i * row_bytes + (c0 + blk) * kQ8_1Bytes;
      const u32x4 v0 = ld16(ap), v1 = ld16(ap + 16);
      const uint32_t v2 = ld4(ap + 32);
      lo = u32x4n{v0.y, v0.z, v0.w, v1.x};
      hi = u32x4n{v1.y, v1.z, v1.w, v2};
      d = h2f(v0.x);
    }
    // code sums (the min and offset terms of the K-quants; Q8_0 has none)
    const bool sums = FMT == kFmtQ4K || FMT == kFmtQ6K;
    const int slo = sums ? bsum4(lo.w, bsum4(lo.z, bsum4(lo.y, bsum4(lo.x, 0)))) : 0;
    const int shi = sums ? bsum4(hi.w, bsum4(hi.z, bsum4(hi.y, bsum4(hi.x, 0)))) : 0;
    if (FMT == kFmtQ8_0) {
      qs[(i * NP + 0) * U + blk] = lo;
      qs[(i * NP + 1) * U + blk] = hi;
      reinterpret_cast<float *>(rec)[i * U + blk] = d;
    } else if (FMT == kFmtQ4K || FMT == kFmtQ8P) {
      const int u = blk >> 1, bb = blk & 1;
      qs[(i * NP + 2 * bb) * U + u] = lo;
      qs[(i * NP + 2 * bb + 1) * U + u] = hi;
      float *r = reinterpret_cast<float *>(rec) + 4 * (i * U + u);
      r[bb] = d;
      if (FMT == kFmtQ4K) r[2 + bb] = d * (float)(slo + shi);
    } else {
      const int sbl = blk >> 3, h = (blk >> 2) & 1, g = blk & 3;
      const int u0 = 4 * sbl + 2 * h;  // unit of half 0; half 1 is u0 + 1
      qs[(i * NP + g) * U + u0] = lo;
      qs[(i * NP + g) * U + u0 + 1] = hi;
      uint32_t *r0 = reinterpret_cast<uint32_t *>(rec) + 8 * (i * U + u0);
      r0[g] = __builtin_bit_cast(uint32_t, d);
      r0[4 + g] = (uint32_t)slo;
      r0[8 + g] = __builtin_bit_cast(uint32_t, d);
      r0[12 + g] = (uint32_t)shi;
    }
  }
}

// One workgroup of W = batch_waves waves strides over groups of W * (64/L) * R
// rows; the activation is staged per chunk of chunk_blocks<B>() Q8_1 blocks
// (c0 counts blocks for every format).
template <int FMT, int L, int B, int R, bool DUMP>
__global__ __launch_bounds__((64 * batch_waves<FMT, B>())) void gemv_batch_kernel(const uint8_t *__restrict__ W,
                                                              const uint8_t *__restrict__ XQ, float *__restrict__ Y,
                                                              int32_t *__restrict__ Dd, int nb, int n, int nblk) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int G = 64 / L;
  constexpr int NP = Unit<FMT>::kPieces;
  constexpr int kWaves = batch_waves<FMT, B>();
  constexpr int kGroupRows = kWaves * G * R;
  constexpr int CB = chunk_blocks<B>();  // activation blocks per chunk
  const int lane = threadIdx.x & 63;
  const int li = lane & (L - 1);
  // row bytes and activation row bytes
  const int64_t rb = (FMT == kFmtQ8_0 || FMT == kFmtQ8P) ? (int64_t)nblk * kQ8_0Bytes
                                     : (int64_t)(nblk / 8) * (FMT == kFmtQ4K ? kQ4KBytes : kQ6KBytes);
  const int64_t xrb = (int64_t)nblk * kQ8_1Bytes;
  const int64_t ngroups = ((int64_t)n + kGroupRows - 1) / kGroupRows;
  int64_t staged = -1;
  for (int64_t grp = blockIdx.x; grp < ngroups; grp += gridDim.x) {
    const int64_t row0 = ((grp * kWaves + (threadIdx.x >> 6)) * G + lane / L) * R;
    const uint8_t *wrow = W + row0 * rb;
    float acc[R][B];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < B; ++i) acc[r][i] = 0.f;
    for (int64_t c0 = 0; c0 < nblk; c0 += CB) {
      const int cb = (int)std::min<int64_t>(CB, nblk - c0);
      const int U = cb * 32 / Unit<FMT>::kValues;
      if (staged != c0) {
        if (staged >= 0) __syncthreads();  // the previous chunk is no longer read
        stage_batch<FMT, B>(lds, XQ, xrb, nb, c0, cb);
        __syncthreads();
        staged = c0;
      }
      if (row0 >= n) continue;
      const u32x4n *qs = reinterpret_cast<const u32x4n *>(lds);
      const uint8_t *rec = lds + (size_t)B * NP * U * 16;
      // L divides the unit count of every chunk (a power of two dividing both
      // the row's unit count and the full chunk's)
      for (int u = li; u < U; u += L) {
        // ---- this unit's codes, once per row: 16 dwords of int8 (Q8_0: 8)
        uint32_t q[R][16];
        float f[R][4];  // per-format scale factors
        int mi[R][2];   // Q4_K mins
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const bool live = row0 + r < n;
          if (FMT == kFmtQ8_0) {
            const uint8_t *bp = wrow + r * rb + (c0 + u) * kQ8_0Bytes;  // 2-byte aligned
            u32x4 a = {0u, 0u, 0u, 0u}, b = a;
            uint32_t dh = 0u;
            if (live) {
              dh = ld2(bp);
              a = ld16_a2(bp + 2);
              b = ld16_a2(bp + 18);
            }
            q[r][0] = a.x; q[r][1] = a.y; q[r][2] = a.z; q[r][3] = a.w;
            q[r][4] = b.x; q[r][5] = b.y; q[r][6] = b.z; q[r][7] = b.w;
            f[r][0] = h2f(dh);
          } else if (FMT == kFmtQ8P) {
            // blocks 2p, 2p + 1 (p = c0/2 + u) as stored, in aligned dwords:
            // d0 | qs0[32] | d1 | qs1[32]; qs0 realigned by two bytes
            const uint8_t *bp = wrow + r * rb + (c0 / 2 + u) * (2 * kQ8_0Bytes);  // 4-byte aligned
            u32x4 w0 = {0u, 0u, 0u, 0u}, w1 = w0, w2 = w0, w3 = w0;
            uint32_t w4 = 0u;
            if (live) {
              w0 = ld16(bp);
              w1 = ld16(bp + 16);
              w2 = ld16(bp + 32);
              w3 = ld16(bp + 48);
              w4 = ld4(bp + 64);
            }
            const uint32_t D[17] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w, w2.x,
                                    w2.y, w2.z, w2.w, w3.x, w3.y, w3.z, w3.w, w4};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              q[r][j] = align_bytes(D[j + 1], D[j], 2);
              q[r][8 + j] = D[9 + j];
            }
            f[r][0] = h2f(D[0] & 0xFFFFu);
            f[r][1] = h2f(D[8] >> 16);
          } else if (FMT == kFmtQ4K) {
            const int sb = (int)(c0 / 8) + (u >> 2), g = u & 3;
            const uint8_t *bp = wrow + r * rb + (int64_t)sb * kQ4KBytes;
            u32x4 hdr = {0u, 0u, 0u, 0u}, qa = hdr, qb = hdr;
            if (live) {
              hdr = ld16(bp);
              qa = ld16(bp + 16 + 32 * g);
              qb = ld16(bp + 32 + 32 * g);
            }
            const uint32_t Q[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              q[r][j] = Q[j] & 0x0F0F0F0Fu;             // sub-block 2g
              q[r][8 + j] = (Q[j] >> 4) & 0x0F0F0F0Fu;  // sub-block 2g+1
            }
            int sc0, sc1, m0, m1;
            q4k_scales(hdr.y, hdr.z, hdr.w, g, sc0, sc1, m0, m1);
            f[r][0] = h2f(hdr.x);        // d
            f[r][1] = h2f(hdr.x >> 16);  // dmin
            f[r][2] = (float)sc0;
            f[r][3] = (float)sc1;
            mi[r][0] = m0;
            mi[r][1] = m1;
          } else {
            const int sb = (int)(c0 / 8) + (u >> 2), h = (u >> 1) & 1, l = u & 1;
            const uint8_t *bp = wrow + r * rb + (int64_t)sb * kQ6KBytes;  // 2-byte aligned
            u32x4 qlA = {0u, 0u, 0u, 0u}, qlB = qlA, qh = qlA;
            u32x2 sc8 = {0u, 0u};
            uint32_t dh = 0u;
            if (live) {
              qlA = ld16_a2(bp + 64 * h + 16 * l);
              qlB = ld16_a2(bp + 64 * h + 32 + 16 * l);
              qh = ld16_a2(bp + 128 + 32 * h + 16 * l);
              sc8 = ld8_a2(bp + 192 + 8 * h);
              dh = ld2(bp + 208);
            }
            const uint32_t A4[4] = {qlA.x, qlA.y, qlA.z, qlA.w};
            const uint32_t B4[4] = {qlB.x, qlB.y, qlB.z, qlB.w};
            const uint32_t H4[4] = {qh.x, qh.y, qh.z, qh.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {  // piece g = 0..3: sub-block 8h + 2g + l
              q[r][j] = (A4[j] & 0x0F0F0F0Fu) | ((H4[j] << 4) & 0x30303030u);
              q[r][4 + j] = (B4[j] & 0x0F0F0F0Fu) | ((H4[j] << 2) & 0x30303030u);
              q[r][8 + j] = ((A4[j] >> 4) & 0x0F0F0F0Fu) | (H4[j] & 0x30303030u);
              q[r][12 + j] = ((B4[j] >> 4) & 0x0F0F0F0Fu) | ((H4[j] >> 2) & 0x30303030u);
            }
            const uint32_t lo8 = 8u * (uint32_t)l;
            const float d = h2f(dh);
            f[r][0] = d * (float)sbyte(sc8.x, lo8);
            f[r][1] = d * (float)sbyte(sc8.x, 16u + lo8);
            f[r][2] = d * (float)sbyte(sc8.y, lo8);
            f[r][3] = d * (float)sbyte(sc8.y, 16u + lo8);
          }
        }
        // ---- against each activation row
#pragma unroll
        for (int i = 0; i < B; ++i) {
          uint32_t a[16];
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            const u32x4n v = qs[(i * NP + p) * U + u];
            a[4 * p] = v.x; a[4 * p + 1] = v.y; a[4 * p + 2] = v.z; a[4 * p + 3] = v.w;
          }
          if (FMT == kFmtQ8_0) {
            const float da = reinterpret_cast<const float *>(rec)[i * U + u];
#pragma unroll
            for (int r = 0; r < R; ++r) {
              int D = 0;
#pragma unroll
              for (int j = 0; j < 8; ++j) D = dot4(q[r][j], a[j], D);
              if (DUMP) {
                if (row0 + r < n && i < nb) Dd[((int64_t)i * n + row0 + r) * nblk + c0 + u] = D;
              } else {
                acc[r][i] += f[r][0] * da * (float)D;
              }
            }
          } else if (FMT == kFmtQ8P) {
            const u32x4n rv = reinterpret_cast<const u32x4n *>(rec)[i * U + u];
            const float da0 = as_f32(rv.x), da1 = as_f32(rv.y);
#pragma unroll
            for (int r = 0; r < R; ++r) {
              int D0 = 0, D1 = 0;
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                D0 = dot4(q[r][j], a[j], D0);
                D1 = dot4(q[r][8 + j], a[8 + j], D1);
              }
              if (DUMP) {
                if (row0 + r < n && i < nb) {
                  int32_t *dp = Dd + ((int64_t)i * n + row0 + r) * nblk + c0 + 2 * u;
                  dp[0] = D0;
                  dp[1] = D1;
                }
              } else {
                acc[r][i] += f[r][0] * da0 * (float)D0;
                acc[r][i] += f[r][1] * da1 * (float)D1;
              }
            }
          } else if (FMT == kFmtQ4K) {
            const u32x4n rv = reinterpret_cast<const u32x4n *>(rec)[i * U + u];
            const float da0 = as_f32(rv.x), da1 = as_f32(rv.y), dS0 = as_f32(rv.z), dS1 = as_f32(rv.w);
#pragma unroll
            for (int r = 0; r < R; ++r) {
              int D0 = 0, D1 = 0;
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                D0 = dot4(q[r][j], a[j], D0);
                D1 = dot4(q[r][8 + j], a[8 + j], D1);
              }
              if (DUMP) {
                if (row0 + r < n && i < nb) {
                  int32_t *dp = Dd + ((int64_t)i * n + row0 + r) * nblk + c0 + 2 * u;  // blocks 8sb + 2g, + 1
                  dp[0] = D0;
                  dp[1] = D1;
                }
                continue;
              }
              const float t = da0 * (f[r][2] * (float)D0) + da1 * (f[r][3] * (float)D1);
              const float mm = dS0 * (float)mi[r][0] + dS1 * (float)mi[r][1];
              acc[r][i] += f[r][0] * t - f[r][1] * mm;
            }
          } else {
            const u32x4n rd = reinterpret_cast<const u32x4n *>(rec)[2 * (i * U + u)];
            const u32x4n rs = reinterpret_cast<const u32x4n *>(rec)[2 * (i * U + u) + 1];
            const uint32_t dd[4] = {rd.x, rd.y, rd.z, rd.w};
            const uint32_t ss[4] = {rs.x, rs.y, rs.z, rs.w};
#pragma unroll
            for (int r = 0; r < R; ++r) {
              float t = 0.f;
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                int Dg = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) Dg = dot4(q[r][4 * g + j], a[4 * g + j], Dg);
                Dg -= 32 * (int)ss[g];  // sum (q-32)*qa
                if (DUMP) {
                  // sub-block 8h + 2g + l of superblock c0/8 + u/4
                  if (row0 + r < n && i < nb)
                    Dd[((int64_t)i * n + row0 + r) * (2 * (int64_t)nblk) + 2 * c0 + 4 * (u & ~3) + 8 * ((u >> 1) & 1) +
                       2 * g + (u & 1)] = Dg;
                } else {
                  t += as_f32(dd[g]) * (f[r][g] * (float)Dg);
                }
              }
              acc[r][i] += t;
            }
          }
        }
      }
    }
    if (!DUMP && row0 < n) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < B; ++i) {
          const float v = group_sum_last<L>(acc[r][i]);
          if (li == L - 1 && row0 + r < n && i < nb) Y[(int64_t)i * n + row0 + r] = v;
        }
    }
  }
}

template <int FMT> constexpr int rows_per_lane() { return FMT == kFmtQ6K ? 2 : 1; }

// The dump instance runs on the grid of the product instance.
template <int FMT, int L, int B>
hipError_t launch_fmt_lb(const uint8_t *W, const uint8_t *X, float *y, int32_t *D, int nb, int64_t n, int nblk,
                         hipStream_t stream) {
  constexpr int R = rows_per_lane<FMT>();
  constexpr int kThreads = 64 * batch_waves<FMT, B>();
  constexpr int kGroupRows = batch_waves<FMT, B>() * (64 / L) * R;
  const size_t lds = batch_lds_bytes<FMT, B>(nblk);
  const int64_t groups = (n + kGroupRows - 1) / kGroupRows;
  const int64_t g = std::min(groups, resident_blocks<gemv_batch_kernel<FMT, L, B, R, false>>(kThreads, lds));
  if (D)
    hipLaunchKernelGGL((gemv_batch_kernel<FMT, L, B, R, true>), dim3((unsigned)g), dim3(kThreads), lds, stream, W, X,
                       y, D, nb, (int)n, nblk);
  else
    hipLaunchKernelGGL((gemv_batch_kernel<FMT, L, B, R, false>), dim3((unsigned)g), dim3(kThreads), lds, stream, W,
                       X, y, D, nb, (int)n, nblk);
  return hipGetLastError();
}

template <int FMT, int B>
hipError_t launch_fmt_b(const uint8_t *W, const uint8_t *X, float *y, int32_t *D, int nb, int64_t n, int nblk, int L,
                        hipStream_t stream) {
  switch (L) {
    case 64: return launch_fmt_lb<FMT, 64, B>(W, X, y, D, nb, n, nblk, stream);
    case 16: return launch_fmt_lb<FMT, 16, B>(W, X, y, D, nb, n, nblk, stream);
    case 4: return launch_fmt_lb<FMT, 4, B>(W, X, y, D, nb, n, nblk, stream);
    default: return launch_fmt_lb<FMT, 1, B>(W, X, y, D, nb, n, nblk, stream);
  }
}

template <int FMT>
hipError_t launch_fmt(const uint8_t *W, const uint8_t *X, float *y, int32_t *D, int nb, int64_t n, int nblk,
                      hipStream_t stream) {
  // lanes per row: the largest of 64, 16, 4, 1 dividing both the row's unit
  // count and a full chunk's (so every chunk's unit count too)
  const int units = nblk * 32 / Unit<FMT>::kValues;
  int L = 64;
  while (L > 1 && units % L != 0) L /= 4;
  if (nb <= 2) return launch_fmt_b<FMT, 2>(W, X, y, D, nb, n, nblk, L, stream);
  if (nb <= 4) return launch_fmt_b<FMT, 4>(W, X, y, D, nb, n, nblk, L, stream);
  return launch_fmt_b<FMT, 8>(W, X, y, D, nb, n, nblk, L, stream);
}

}  // namespace

hipError_t launch_qgemv_batch(int fmt, const void *w, const void *xq, float *y, int32_t *D, int64_t nb, int64_t n,
                              int64_t k, hipStream_t stream) {
  const uint8_t *W = static_cast<const uint8_t *>(w);
  const uint8_t *X = static_cast<const uint8_t *>(xq);
  const int nblk = (int)(k / 32);
  // Q8_0: int8 MFMA from 5 rows when k is a multiple of 256, so that 8 blocks
  // of a row are 16-byte aligned (the entry points require w to be) (same
  // process, us at 4096 x 4096: b = 8 7.67 -> 6.73; b = 4 6.58 against 7.12
  // and b = 2 5.69 against 7.07 stay on v_dot4); else aligned block pairs
  // against single 2-byte-aligned blocks (b = 2 6.65 -> 5.72, b = 4 6.98 ->
  // 6.81, b = 8 7.79 -> 7.69)
  if (fmt == 0 && nb > 4 && nblk % 8 == 0) return launch_qgemv_batch_mfma_q8_0(w, xq, y, D, nb, n, k, stream);
  if (fmt == 0 && nblk % 2 == 0) return launch_fmt<kFmtQ8P>(W, X, y, D, (int)nb, n, nblk, stream);
  if (fmt == 0) return launch_fmt<kFmtQ8_0>(W, X, y, D, (int)nb, n, nblk, stream);
  // Measured on MI355X (k = 4096, us per call): Q4_K 14336 rows takes v_dot4
  // for one row and the matrix cores from 2 (b = 2: 9.28 against 9.69, b = 3:
  // 9.57 against 10.59, b = 4: 10.18 against 10.75, b = 8: 10.3 against 16.0);
  // Q6_K 128256 rows takes v_dot4 up to 2 rows (b = 2: 86.1 against 87.2) and
  // the matrix cores from 3 (b = 3: 88.2 against 95.8, b = 4: 88.7 against
  // 98.3).
  if (fmt == 1) {
    if (nb > 1) return launch_qgemv_batch_mfma_q4k(w, xq, y, D, nb, n, k, stream);
    return launch_fmt<kFmtQ4K>(W, X, y, D, (int)nb, n, nblk, stream);
  }
  if (nb > 2) return launch_qgemv_batch_mfma_q6k(w, xq, y, D, nb, n, k, stream);
  return launch_fmt<kFmtQ6K>(W, X, y, D, (int)nb, n, nblk, stream);
}

}  // namespace qg
