// qg_mmq.hip -- prefill product C[m][n] = sum_k a^[m,k] w^[n,k] with Q4_K
// weights and Q8_1 activations on gfx950 int8 matrix cores.
//
// The pages run this step as "in-shader dequant and dp4a mmq" (infr page,
// "models") and as cooperative-matrix matmul (infr page, "Vulkan-first, Metal
// too").  Here a workgroup of 8 waves owns a 64 (tokens) x 128 (weight rows)
// output tile; each wave owns 32x32.  Per 256-wide superblock of k the
// workgroup stages in LDS:
//   A  Q8_1 qs as int8, plus per (row, block) d_a and d_a*sum(qa)
//   B  Q4_K nibbles widened to int8, plus per (weight row, sub-block) d*sc_j
//      and -dmin*m_j
// double-buffered: the global loads of superblock s+1 are in flight while the
// MFMAs of superblock s run.  Each 32-wide sub-block j is exactly one
// v_mfma_i32_32x32x32_i8 -> the exact int32 dots D of that block for the wave's
// 32x32 tile.  Its fp32 rescale is acc += F * D with F[m][n] = d_a[m] * (d*sc_j)[n],
// a rank-1 outer product that the matrix core forms as well: d_a (fp16) is
// exactly the sum of two bf16 parts and d*sc_j is two bf16 parts to 2^-17, so
// one v_mfma_f32_32x32x8_bf16 over those parts gives F in the MFMA output
// layout, leaving one convert and one fma per output on the VALU.  The min term
// -sum_j (d_a*sum qa)_j (dmin*m_j) is a rank-8-per-superblock product of two
// small fp32 matrices and runs on the matrix core too (v_mfma_f32_32x32x2_f32
// over pairs of sub-blocks) into a second accumulator.
#include "qg_blocks.h"
#include "qg_launch.h"

namespace qg {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));

constexpr int kBM = 64, kBN = 128;
constexpr int kRow = 272;  // LDS bytes per staged row: 256 + 16 (spreads rows over banks)

// Per-block factor arrays are [block][row] so that the MFMA operand reads of a
// wave are contiguous; one spare entry per block row spreads the transposed
// staging writes over the LDS banks.
struct MmqStage {
  uint8_t a[kBM * kRow];
  uint8_t b[kBN * kRow];
  uint32_t fa[8][kBM + 1][2];   // bf16 (ah, ah, al, al) of d_a = ah + al, per (block j, activation row)
  uint32_t fb[8][kBN + 1][2];   // bf16 (dh, dl, dh, dl) of d*sc_j = dh + dl, per (sub-block j, weight row)
  float SA[8][kBM + 1];         // d_a * sum(qa)
  float ndm[8][kBN + 1];        // -dmin * m_j
};

__device__ __forceinline__ uint32_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// x = hi + lo with hi, lo bf16 (exact when x has <= 16 significant bits).
__device__ __forceinline__ void bf16_split(float x, uint32_t &hi, uint32_t &lo) {
  const __bf16 h = (__bf16)x;
  hi = __builtin_bit_cast(uint16_t, h);
  lo = bf16_bits(x - (float)h);
}

// Global -> registers for one superblock: thread t stages activation block
// (row t/8, block t%8) and weight (row t/4, byte group t%4).
struct MmqRegs {
  u32x4 a0, a1;
  uint32_t a2;
  u32x4 hdr, qa, qb;
};

__device__ __forceinline__ void mmq_load(MmqRegs &g, const uint8_t *__restrict__ W, const uint8_t *__restrict__ AQ,
                                         int M, int N, int nsb, int m0, int n0, int sb, int tid) {
  const int ar = tid >> 3, ab = tid & 7;
  const int gm = m0 + ar;
  if (gm < M) {
    const uint8_t *ap = AQ + ((int64_t)gm * nsb * 8 + sb * 8 + ab) * kQ8_1Bytes;
    g.a0 = ld16(ap);
    g.a1 = ld16(ap + 16);
    g.a2 = ld4(ap + 32);
  } else {
    g.a0 = g.a1 = u32x4{0u, 0u, 0u, 0u};
    g.a2 = 0u;
  }
  const int br = tid >> 2, bg = tid & 3;
  const int gn = n0 + br;
  if (gn < N) {
    const uint8_t *bp = W + ((int64_t)gn * nsb + sb) * kQ4KBytes;
    g.hdr = ld16(bp);
    g.qa = ld16(bp + 16 + 32 * bg);
    g.qb = ld16(bp + 32 + 32 * bg);
  } else {
    g.hdr = g.qa = g.qb = u32x4{0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ void mmq_store(const MmqRegs &g, MmqStage &s, int tid) {
  {  // activation block: qs -> int8 row, factors
    const int ar = tid >> 3, ab = tid & 7;
    const uint32_t q[8] = {g.a0.y, g.a0.z, g.a0.w, g.a1.x, g.a1.y, g.a1.z, g.a1.w, g.a2};
    int S = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) S = bsum4(q[i], S);
    uint32_t *dst = reinterpret_cast<uint32_t *>(s.a + ar * kRow + 32 * ab);
    *reinterpret_cast<u32x4 *>(dst) = u32x4{q[0], q[1], q[2], q[3]};
    *reinterpret_cast<u32x4 *>(dst + 4) = u32x4{q[4], q[5], q[6], q[7]};
    const float da = h2f(g.a0.x);
    uint32_t hi, lo;
    bf16_split(da, hi, lo);
    s.fa[ab][ar][0] = hi | (hi << 16);
    s.fa[ab][ar][1] = lo | (lo << 16);
    s.SA[ab][ar] = da * (float)S;
  }
  {  // weight group: nibbles -> int8 (sub-block 2g low, 2g+1 high), factors
    const int br = tid >> 2, bg = tid & 3;
    const uint32_t Q[8] = {g.qa.x, g.qa.y, g.qa.z, g.qa.w, g.qb.x, g.qb.y, g.qb.z, g.qb.w};
    uint32_t *dst = reinterpret_cast<uint32_t *>(s.b + br * kRow + 64 * bg);
    *reinterpret_cast<u32x4 *>(dst) =
        u32x4{Q[0] & 0x0F0F0F0Fu, Q[1] & 0x0F0F0F0Fu, Q[2] & 0x0F0F0F0Fu, Q[3] & 0x0F0F0F0Fu};
    *reinterpret_cast<u32x4 *>(dst + 4) =
        u32x4{Q[4] & 0x0F0F0F0Fu, Q[5] & 0x0F0F0F0Fu, Q[6] & 0x0F0F0F0Fu, Q[7] & 0x0F0F0F0Fu};
    *reinterpret_cast<u32x4 *>(dst + 8) = u32x4{(Q[0] >> 4) & 0x0F0F0F0Fu, (Q[1] >> 4) & 0x0F0F0F0Fu,
                                                (Q[2] >> 4) & 0x0F0F0F0Fu, (Q[3] >> 4) & 0x0F0F0F0Fu};
    *reinterpret_cast<u32x4 *>(dst + 12) = u32x4{(Q[4] >> 4) & 0x0F0F0F0Fu, (Q[5] >> 4) & 0x0F0F0F0Fu,
                                                 (Q[6] >> 4) & 0x0F0F0F0Fu, (Q[7] >> 4) & 0x0F0F0F0Fu};
    int sc0, sc1, mn0, mn1;
    q4k_scales(g.hdr.y, g.hdr.z, g.hdr.w, bg, sc0, sc1, mn0, mn1);
    const float d = h2f(g.hdr.x), dmin = h2f(g.hdr.x >> 16);
    uint32_t hi, lo;
    bf16_split(d * (float)sc0, hi, lo);
    s.fb[2 * bg][br][0] = s.fb[2 * bg][br][1] = hi | (lo << 16);
    bf16_split(d * (float)sc1, hi, lo);
    s.fb[2 * bg + 1][br][0] = s.fb[2 * bg + 1][br][1] = hi | (lo << 16);
    s.ndm[2 * bg][br] = -(dmin * (float)mn0);
    s.ndm[2 * bg + 1][br] = -(dmin * (float)mn1);
  }
}

template <bool DUMP>
__global__ __launch_bounds__(512) void mmq_q4k_kernel(const uint8_t *__restrict__ W, const uint8_t *__restrict__ AQ,
                                                      float *__restrict__ C, int32_t *__restrict__ Dd, int M, int N,
                                                      int nsb) {
  __shared__ MmqStage stage[2];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 2, wn = wv & 3;  // 2 x 4 waves of 32x32
  const int tiles_n = (N + kBN - 1) / kBN;
  const int m0 = (int)(blockIdx.x / tiles_n) * kBM, n0 = (int)(blockIdx.x % tiles_n) * kBN;
  const int lr = lane & 31, lh = lane >> 5;
  const int nbrow = nsb * 8;

  v16f acc, accm;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = accm[r] = 0.f;
  v16i zero;
  v16f fzero;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    zero[r] = 0;
    fzero[r] = 0.f;
  }

  MmqRegs g;
  if (nsb > 0) {
    mmq_load(g, W, AQ, M, N, nsb, m0, n0, 0, tid);
    mmq_store(g, stage[0], tid);
  }
  __syncthreads();
  for (int sb = 0; sb < nsb; ++sb) {
    MmqStage &cur = stage[sb & 1];
    const bool more = sb + 1 < nsb;
    if (more) mmq_load(g, W, AQ, M, N, nsb, m0, n0, sb + 1, tid);

    const uint8_t *arow = cur.a + (wm * 32 + lr) * kRow + 16 * lh;
    const uint8_t *brow = cur.b + (wn * 32 + lr) * kRow + 16 * lh;
#pragma unroll 2  // full unrolling keeps all eight MFMA results live and spills
    for (int j = 0; j < 8; ++j) {
      const v4i a = *reinterpret_cast<const v4i *>(arow + 32 * j);
      const v4i b = *reinterpret_cast<const v4i *>(brow + 32 * j);
      const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, zero, 0, 0, 0);
      if (!DUMP && (j & 1) == 0) {
        // min term for sub-blocks j, j+1: (32 x 2) x (2 x 32) fp32 MFMA;
        // lane l supplies row/column l%32 at k = l/32
        const float sa = cur.SA[j + lh][wm * 32 + lr];
        const float nd = cur.ndm[j + lh][wn * 32 + lr];
        accm = __builtin_amdgcn_mfma_f32_32x32x2f32(sa, nd, accm, 0, 0, 0);
      }
      // 2F for this block: lanes 32-63 (k = 4..7) repeat the four parts of
      // lanes 0-31, so the MFMA returns exactly twice the outer product
      const uint32_t *fa = cur.fa[j][wm * 32 + lr];
      const uint32_t *fb = cur.fb[j][wn * 32 + lr];
      const v4s fav = __builtin_bit_cast(v4s, u32x2{fa[0], fa[1]});
      const v4s fbv = __builtin_bit_cast(v4s, u32x2{fb[0], fb[1]});
      const v16f F2 = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(fav, fbv, fzero, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // output register r holds tile row 8(r/4) + 4*lh + r%4, column lr
        if (DUMP) {
          const int gm = m0 + wm * 32 + 8 * (r / 4) + 4 * lh + (r % 4), gn = n0 + wn * 32 + lr;
          if (gm < M && gn < N) Dd[((int64_t)gm * N + gn) * nbrow + sb * 8 + j] = D[r];
        } else {
          acc[r] += F2[r] * (float)D[r];
        }
      }
    }
    if (more) mmq_store(g, stage[(sb + 1) & 1], tid);
    __syncthreads();
  }

  if (!DUMP) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int gm = m0 + wm * 32 + 8 * (r / 4) + 4 * lh + (r % 4);
      const int gn = n0 + wn * 32 + lr;
      if (gm < M && gn < N) C[(int64_t)gm * N + gn] = 0.5f * acc[r] + accm[r];
    }
  }
}

hipError_t launch_qgemm_q4_k_mmq(const void *w, const void *aq, float *c, int32_t *D, int64_t m, int64_t n, int64_t k,
                                 hipStream_t stream) {
  const dim3 grid((unsigned)(((n + kBN - 1) / kBN) * ((m + kBM - 1) / kBM)));
  const uint8_t *W = static_cast<const uint8_t *>(w);
  const uint8_t *A = static_cast<const uint8_t *>(aq);
  if (D)
    hipLaunchKernelGGL(mmq_q4k_kernel<true>, grid, dim3(512), 0, stream, W, A, c, D, (int)m, (int)n, (int)(k / 256));
  else
    hipLaunchKernelGGL(mmq_q4k_kernel<false>, grid, dim3(512), 0, stream, W, A, c, D, (int)m, (int)n,
                       (int)(k / 256));
  return hipGetLastError();
}

}  // namespace qg
