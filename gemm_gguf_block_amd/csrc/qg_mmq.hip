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
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

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
  uint32_t fs[8][kBM + 1][2];   // bf16 (sh, sh, sl, sl) of d_a * sum(qa) = sh + sl
  uint32_t fm[8][kBN + 1][2];   // bf16 (mh, ml, mh, ml) of -2 dmin m_j = mh + ml
};

__device__ __forceinline__ uint32_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// x = hi + lo with hi, lo bf16 (exact when x has <= 16 significant bits).
__device__ __forceinline__ void bf16_split(float x, uint32_t &hi, uint32_t &lo) {
  const __bf16 h = (__bf16)x;
  hi = __builtin_bit_cast(uint16_t, h);
  lo = bf16_bits(x - (float)h);
}

// Global -> registers for one superblock.  Activation staging thread t
// (0..511) holds block t%8 of tile row t/8: x0 = bytes 0-15, x1 = 16-31,
// x2.x = 32-35.  Weight staging thread t holds tile row t/4, qs byte group t%4:
// x0 = header (d, dmin, scales), x1, x2 = its 32 qs bytes.  Rows past the end
// of A or B load the last row instead; they only feed outputs that are never
// stored.
struct MmqRegs {
  u32x4 x0, x1, x2;
};

__device__ __forceinline__ void load_act(MmqRegs &g, const uint8_t *__restrict__ AQ, int M, int nsb, int m0, int sb,
                                         int t) {
  const int gm = min(m0 + (t >> 3), M - 1);
  const uint8_t *ap = AQ + ((int64_t)gm * nsb * 8 + sb * 8 + (t & 7)) * kQ8_1Bytes;
  g.x0 = ld16(ap);
  g.x1 = ld16(ap + 16);
  g.x2.x = ld4(ap + 32);
}

__device__ __forceinline__ void load_wgt(MmqRegs &g, const uint8_t *__restrict__ W, int N, int nsb, int n0, int sb,
                                         int t) {
  const int gn = min(n0 + (t >> 2), N - 1);
  const uint8_t *bp = W + ((int64_t)gn * nsb + sb) * kQ4KBytes;
  g.x0 = ld16(bp);
  g.x1 = ld16(bp + 16 + 32 * (t & 3));
  g.x2 = ld16(bp + 32 + 32 * (t & 3));
}

// activation block: qs -> int8 row, factors
__device__ __forceinline__ void store_act(const MmqRegs &g, MmqStage &s, int t) {
  const int ar = t >> 3, ab = t & 7;
  const uint32_t q[8] = {g.x0.y, g.x0.z, g.x0.w, g.x1.x, g.x1.y, g.x1.z, g.x1.w, g.x2.x};
  int S = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) S = bsum4(q[i], S);
  uint32_t *dst = reinterpret_cast<uint32_t *>(s.a + ar * kRow + 32 * ab);
  *reinterpret_cast<u32x4 *>(dst) = u32x4{q[0], q[1], q[2], q[3]};
  *reinterpret_cast<u32x4 *>(dst + 4) = u32x4{q[4], q[5], q[6], q[7]};
  const float da = h2f(g.x0.x);
  uint32_t hi, lo;
  bf16_split(da, hi, lo);
  s.fa[ab][ar][0] = hi | (hi << 16);
  s.fa[ab][ar][1] = lo | (lo << 16);
  bf16_split(da * (float)S, hi, lo);
  s.fs[ab][ar][0] = hi | (hi << 16);
  s.fs[ab][ar][1] = lo | (lo << 16);
}

// weight group: nibbles -> int8 (sub-block 2g low, 2g+1 high), factors
__device__ __forceinline__ void store_wgt(const MmqRegs &g, MmqStage &s, int t) {
  const int br = t >> 2, bg = t & 3;
  const uint32_t Q[8] = {g.x1.x, g.x1.y, g.x1.z, g.x1.w, g.x2.x, g.x2.y, g.x2.z, g.x2.w};
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
  q4k_scales(g.x0.y, g.x0.z, g.x0.w, bg, sc0, sc1, mn0, mn1);
  const float d = h2f(g.x0.x), dmin = h2f(g.x0.x >> 16);
  uint32_t hi, lo;
  bf16_split(d * (float)sc0, hi, lo);
  s.fb[2 * bg][br][0] = s.fb[2 * bg][br][1] = hi | (lo << 16);
  bf16_split(d * (float)sc1, hi, lo);
  s.fb[2 * bg + 1][br][0] = s.fb[2 * bg + 1][br][1] = hi | (lo << 16);
  // doubled like the factor product 2F (exact); see the kernel's accumulator
  bf16_split(-2.f * (dmin * (float)mn0), hi, lo);
  s.fm[2 * bg][br][0] = s.fm[2 * bg][br][1] = hi | (lo << 16);
  bf16_split(-2.f * (dmin * (float)mn1), hi, lo);
  s.fm[2 * bg + 1][br][0] = s.fm[2 * bg + 1][br][1] = hi | (lo << 16);
}

// Two waves share each 32x32 output tile and split every superblock's eight
// blocks between them; the workgroup has 16 waves.  Waves 0-7 stage
// activations and waves 8-15 weights, and the two partial tiles are summed
// through LDS at the end.
constexpr bool kPipe = false;  // issue block j+1's MFMAs before block j's rescale

template <bool DUMP>
__global__ __launch_bounds__(1024) void mmq_q4k_kernel(const uint8_t *__restrict__ W,
                                                           const uint8_t *__restrict__ AQ, float *__restrict__ C,
                                                           int32_t *__restrict__ Dd, int M, int N, int nsb) {
  constexpr int kJ = 4;  // blocks per superblock per wave
  __shared__ MmqStage stage[2];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int kh = wv >> 3;                         // which part of each superblock
  const int wm = (wv >> 2) & 1, wn = wv & 3;      // 2 x 4 tiles of 32x32
  const int tiles_n = (N + kBN - 1) / kBN;
  const int m0 = (int)(blockIdx.x / tiles_n) * kBM, n0 = (int)(blockIdx.x % tiles_n) * kBN;
  const int lr = lane & 31, lh = lane >> 5;
  const int nbrow = nsb * 8;
  const int st = tid & 511;
  const bool act = tid < 512;  // this wave stages activations, else weights

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

  // Superblock s is staged from registers R[s & 1]: its global loads are
  // issued two superblocks ahead, so two compute phases cover their latency.
  MmqRegs R0, R1;
  auto load = [&](MmqRegs &g, int s) {
    if (act)
      load_act(g, AQ, M, nsb, m0, s, st);
    else
      load_wgt(g, W, N, nsb, n0, s, st);
  };
  auto store = [&](const MmqRegs &g, MmqStage &dst) {
    if (act)
      store_act(g, dst, st);
    else
      store_wgt(g, dst, st);
  };
  auto compute = [&](MmqStage &cur, int sb) {
    const int j0 = kh * kJ;
    const uint8_t *arow = cur.a + (wm * 32 + lr) * kRow + 16 * lh + 32 * j0;
    const uint8_t *brow = cur.b + (wn * 32 + lr) * kRow + 16 * lh + 32 * j0;
    const uint32_t *fa = cur.fa[j0][wm * 32 + lr];
    const uint32_t *fb = cur.fb[j0][wn * 32 + lr];
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
#pragma unroll
    for (int jj = 0; jj < kJ; ++jj) {
      // D = exact int32 dots of block j0+jj; F2 = 2F for its rescale: lanes
      // 32-63 (k = 4..7) of the bf16 MFMA repeat the four parts of lanes 0-31,
      // so it returns exactly twice the outer product
      const v4i av = *reinterpret_cast<const v4i *>(arow + 32 * jj);
      const v4i bv = *reinterpret_cast<const v4i *>(brow + 32 * jj);
      const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv, zero, 0, 0, 0);
      v16f F2 = fzero;
      if (!DUMP) {
        const uint32_t *pa = fa + jj * (kBM + 1) * 2, *pb = fb + jj * (kBN + 1) * 2;
        const v4s fav = __builtin_bit_cast(v4s, u32x2{pa[0], pa[1]});
        const v4s fbv = __builtin_bit_cast(v4s, u32x2{pb[0], pb[1]});
        F2 = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(fav, fbv, fzero, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // output register r holds tile row 8(r/4) + 4*lh + r%4, column lr
        if (DUMP) {
          const int gm = m0 + wm * 32 + 8 * (r / 4) + 4 * lh + (r % 4), gn = n0 + wn * 32 + lr;
          if (gm < M && gn < N) Dd[((int64_t)gm * N + gn) * nbrow + sb * 8 + j0 + jj] = D[r];
        } else {
          acc[r] += F2[r] * (float)D[r];
        }
      }
      // Fence: the MFMA builtins carry no memory dependence, so without it
      // every block's products would be hoisted to the top of the
      // superblock, with all their results live at once.
      asm volatile("" : "+v"(acc)::"memory");
    }
  };
  // One step: superblock s+2 loads into `mine` (free: it held s, staged one
  // step earlier), s computes from `cur`, and s+1 (loaded one step earlier,
  // in `next`) is staged into `other`, which nobody reads during this step.
  auto step = [&](int s, MmqRegs &mine, const MmqRegs &next, MmqStage &cur, MmqStage &other) {
    if (s + 2 < nsb) load(mine, s + 2);
    compute(cur, s);
    if (s + 1 < nsb) store(next, other);
    __syncthreads();
  };
  if (nsb > 0) load(R0, 0);
  if (nsb > 1) load(R1, 1);
  if (nsb > 0) store(R0, stage[0]);
  __syncthreads();
  for (int sb = 0; sb < nsb; sb += 2) {
    step(sb, R0, R1, stage[0], stage[1]);
    if (sb + 1 < nsb) step(sb + 1, R1, R0, stage[1], stage[0]);
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

hipError_t launch_qgemm_q4_k_mmq(const void *w, const void *aq, float *c, int32_t *D, int64_t m, int64_t n, int64_t k,
                                 hipStream_t stream) {
  const dim3 grid((unsigned)(((n + kBN - 1) / kBN) * ((m + kBM - 1) / kBM)));
  const uint8_t *W = static_cast<const uint8_t *>(w);
  const uint8_t *A = static_cast<const uint8_t *>(aq);
  if (D)
    hipLaunchKernelGGL((mmq_q4k_kernel<true>), grid, dim3(1024), 0, stream, W, A, c, D, (int)m,
                       (int)n, (int)(k / 256));
  else
    hipLaunchKernelGGL((mmq_q4k_kernel<false>), grid, dim3(1024), 0, stream, W, A, c, D, (int)m,
                       (int)n, (int)(k / 256));
  return hipGetLastError();
}

}  // namespace qg
