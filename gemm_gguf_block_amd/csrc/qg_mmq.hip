// qg_mmq.hip -- prefill product C[m][n] = sum_k a^[m,k] w^[n,k] with Q4_K
// weights and Q8_1 activations on gfx950 int8 matrix cores.
//
// The pages run this step as "in-shader dequant and dp4a mmq" (infr page,
// "models") and as cooperative-matrix matmul (infr page, "Vulkan-first, Metal
// too").  Here: a 64x64 output tile per workgroup, four waves of 32x32.  Per
// 256-wide superblock of k, the workgroup stages A (Q8_1 qs as int8) and B
// (Q4_K nibbles widened to int8) in LDS together with the fp32 factors
// d_a, d_a*sum(qa) per activation block and d*sc_j, dmin*m_j per weight
// sub-block.  Each 32-wide sub-block j is exactly one
// v_mfma_i32_32x32x32_i8 -> the exact int32 dots D of that block for the
// 32x32 tile, which are then rescaled:
//   acc += d_a*(d*sc_j)*D - (d_a*S)*(dmin*m_j).
#include "qg_blocks.h"
#include "qg_launch.h"

namespace qg {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kBM = 64, kBN = 64;
constexpr int kRow = 272;  // LDS bytes per staged row: 256 + 16 padding (bank spread)

template <bool DUMP>
__global__ __launch_bounds__(256) void mmq_q4k_kernel(const uint8_t *__restrict__ W, const uint8_t *__restrict__ AQ,
                                                      float *__restrict__ C, int32_t *__restrict__ Dd, int M, int N,
                                                      int nsb) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[kBM * kRow];
  __shared__ __attribute__((aligned(16))) uint8_t sB[kBN * kRow];
  __shared__ __attribute__((aligned(16))) float sdA[8][kBM];   // d_a per (block j, row)
  __shared__ __attribute__((aligned(16))) float sSA[8][kBM];   // d_a * sum(qa)
  __shared__ __attribute__((aligned(16))) float sdsc[8][kBN];  // d * sc_j per (j, weight row)
  __shared__ __attribute__((aligned(16))) float sdmm[8][kBN];  // dmin * m_j

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int tiles_n = (N + kBN - 1) / kBN;
  const int m0 = (int)(blockIdx.x / tiles_n) * kBM, n0 = (int)(blockIdx.x % tiles_n) * kBN;
  const int lr = lane & 31, lh = lane >> 5;
  const int nbrow = nsb * 8;  // Q8_1 blocks per activation row

  float acc[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;

  for (int sb = 0; sb < nsb; ++sb) {
    // ---- stage A: thread -> activation row r, Q8_1 blocks 2p, 2p+1 of this superblock
    {
      const int r = tid >> 2, p = tid & 3;
      const int gm = m0 + r;
      uint32_t A[18];
      if (gm < M) {
        const uint8_t *ap = AQ + ((int64_t)gm * nbrow + sb * 8 + 2 * p) * kQ8_1Bytes;
        const u32x4 a0 = ld16(ap), a1 = ld16(ap + 16), a2 = ld16(ap + 32), a3 = ld16(ap + 48);
        const u32x2 a4 = ld8(ap + 64);
        A[0] = a0.x; A[1] = a0.y; A[2] = a0.z; A[3] = a0.w; A[4] = a1.x; A[5] = a1.y;
        A[6] = a1.z; A[7] = a1.w; A[8] = a2.x; A[9] = a2.y; A[10] = a2.z; A[11] = a2.w;
        A[12] = a3.x; A[13] = a3.y; A[14] = a3.z; A[15] = a3.w; A[16] = a4.x; A[17] = a4.y;
      } else {
#pragma unroll
        for (int i = 0; i < 18; ++i) A[i] = 0u;
      }
      int S0 = 0, S1 = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        S0 = bsum4(A[1 + i], S0);
        S1 = bsum4(A[10 + i], S1);
      }
      uint32_t *dst = reinterpret_cast<uint32_t *>(sA + r * kRow + 64 * p);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        dst[i] = A[1 + i];
        dst[8 + i] = A[10 + i];
      }
      const float da0 = h2f(A[0]), da1 = h2f(A[9]);
      sdA[2 * p][r] = da0;
      sdA[2 * p + 1][r] = da1;
      sSA[2 * p][r] = da0 * (float)S0;
      sSA[2 * p + 1][r] = da1 * (float)S1;
    }
    // ---- stage B: thread -> weight row r, byte group g (sub-blocks 2g, 2g+1)
    {
      const int r = tid >> 2, g = tid & 3;
      const int gn = n0 + r;
      u32x4 hdr = {0u, 0u, 0u, 0u}, qa = {0u, 0u, 0u, 0u}, qb = {0u, 0u, 0u, 0u};
      if (gn < N) {
        const uint8_t *bp = W + ((int64_t)gn * nsb + sb) * kQ4KBytes;
        hdr = ld16(bp);
        qa = ld16(bp + 16 + 32 * g);
        qb = ld16(bp + 32 + 32 * g);
      }
      const uint32_t Q[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
      uint32_t *dst = reinterpret_cast<uint32_t *>(sB + r * kRow + 64 * g);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        dst[i] = Q[i] & 0x0F0F0F0Fu;             // sub-block 2g, values 0..31
        dst[8 + i] = (Q[i] >> 4) & 0x0F0F0F0Fu;  // sub-block 2g+1
      }
      int sc0, sc1, mn0, mn1;
      q4k_scales(hdr.y, hdr.z, hdr.w, g, sc0, sc1, mn0, mn1);
      const float d = h2f(hdr.x), dmin = h2f(hdr.x >> 16);
      sdsc[2 * g][r] = d * (float)sc0;
      sdsc[2 * g + 1][r] = d * (float)sc1;
      sdmm[2 * g][r] = dmin * (float)mn0;
      sdmm[2 * g + 1][r] = dmin * (float)mn1;
    }
    __syncthreads();

    // ---- eight 32x32x32 int8 MFMAs, one per sub-block, each rescaled in fp32
    const uint8_t *arow = sA + (wm * 32 + lr) * kRow + 16 * lh;
    const uint8_t *brow = sB + (wn * 32 + lr) * kRow + 16 * lh;
#pragma unroll 2
    for (int j = 0; j < 8; ++j) {
      const v4i a = *reinterpret_cast<const v4i *>(arow + 32 * j);
      const v4i b = *reinterpret_cast<const v4i *>(brow + 32 * j);
      v16i zero;
#pragma unroll
      for (int r = 0; r < 16; ++r) zero[r] = 0;
      const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, zero, 0, 0, 0);
      // output register r holds row 8(r/4) + 4*lh + r%4 of the wave tile, column lr
      const float dsc = sdsc[j][wn * 32 + lr], dmm = sdmm[j][wn * 32 + lr];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 da4 = *reinterpret_cast<const float4 *>(&sdA[j][wm * 32 + 8 * q + 4 * lh]);
        const float4 sa4 = *reinterpret_cast<const float4 *>(&sSA[j][wm * 32 + 8 * q + 4 * lh]);
        const float da[4] = {da4.x, da4.y, da4.z, da4.w};
        const float sa[4] = {sa4.x, sa4.y, sa4.z, sa4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * q + i;
          if (DUMP) {
            const int gm = m0 + wm * 32 + 8 * q + 4 * lh + i, gn = n0 + wn * 32 + lr;
            if (gm < M && gn < N) Dd[((int64_t)gm * N + gn) * nbrow + sb * 8 + j] = D[r];
          } else {
            acc[r] += (da[i] * dsc) * (float)D[r] - sa[i] * dmm;
          }
        }
      }
    }
    __syncthreads();
  }

  if (!DUMP) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int gm = m0 + wm * 32 + 8 * (r / 4) + 4 * lh + (r % 4);
      const int gn = n0 + wn * 32 + lr;
      if (gm < M && gn < N) C[(int64_t)gm * N + gn] = acc[r];
    }
  }
}

hipError_t launch_qgemm_q4_k_mmq(const void *w, const void *aq, float *c, int32_t *D, int64_t m, int64_t n, int64_t k,
                                 hipStream_t stream) {
  const dim3 grid((unsigned)(((n + kBN - 1) / kBN) * ((m + kBM - 1) / kBM)));
  const uint8_t *W = static_cast<const uint8_t *>(w);
  const uint8_t *A = static_cast<const uint8_t *>(aq);
  if (D)
    hipLaunchKernelGGL(mmq_q4k_kernel<true>, grid, dim3(256), 0, stream, W, A, c, D, (int)m, (int)n, (int)(k / 256));
  else
    hipLaunchKernelGGL(mmq_q4k_kernel<false>, grid, dim3(256), 0, stream, W, A, c, D, (int)m, (int)n,
                       (int)(k / 256));
  return hipGetLastError();
}

}  // namespace qg
