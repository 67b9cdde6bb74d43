// qg_gemv_mfma.hip -- small-batch Q4_K GEMV on the int8 matrix cores.
//
// With b <= 8 activation rows the dot4 kernels spend VALU per (row, block,
// activation row).  Here the b rows form the M side of
// v_mfma_i32_32x32x32_i8 (rows b..31 are zero) and 32 weight rows the N side,
// so one MFMA gives the exact int32 block dots of 32 weight rows against all b
// activation rows, and the fp32 rescale costs the same few VALU per block
// whatever b is.
//
// A workgroup of 8 waves owns a tile of 32 weight rows.  k is walked in
// chunks of 16 superblocks: the workgroup stages the chunk's activation blocks
// in LDS, wave w takes superblocks w and w + 8 of the chunk (32 rows x 144
// bytes each, loaded before the staging barrier), and runs their blocks on the
// matrix core.  The 8 waves' partial tiles are summed through LDS at the end.
// Two such workgroups fit on a CU, so 14336 rows (448 tiles) run in one pass.
//
// Output register r of a lane holds activation row 8(r/4) + 4(lane/32) + r%4,
// so for b <= 8 only r = 0..3 carry rows (4(lane/32) + r) and are rescaled.
#include "qg_blocks.h"
#include "qg_launch.h"

namespace qg {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4n __attribute__((ext_vector_type(4)));
typedef float f32x4n __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kSbPerWave = 2;
constexpr int kChunkSb = kWaves * kSbPerWave;  // superblocks per chunk
constexpr int kChunkBlk = 8 * kChunkSb;
constexpr int kMaxB = 8;

// Dynamic LDS for b activation rows: qs [blk][m][half] (16 B), d_a [blk][m],
// d_a*sum(qa) [blk][m] (rows padded to 4 so lanes read 16-byte groups), then
// the waves' partial tiles [wave][lane] (16 B).
__host__ __device__ constexpr int rows_padded(int nb) { return nb <= 4 ? 4 : 8; }
inline size_t lds_bytes(int nb) {
  const int bp = rows_padded(nb);
  return (size_t)kChunkBlk * bp * 32 + 2 * (size_t)kChunkBlk * bp * 4 + (size_t)kWaves * 64 * 16;
}

__global__ __launch_bounds__(kThreads) void gemv_batch_mfma_q4k(const uint8_t *__restrict__ W,
                                                                const uint8_t *__restrict__ XQ,
                                                                float *__restrict__ Y, int nb, int n, int nsb) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int bp = rows_padded(nb);
  u32x4n *act = reinterpret_cast<u32x4n *>(lds);
  float *da = reinterpret_cast<float *>(lds + (size_t)kChunkBlk * bp * 32);
  float *das = da + kChunkBlk * bp;
  f32x4n *part = reinterpret_cast<f32x4n *>(das + kChunkBlk * bp);

  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int nl = lane & 31, lh = lane >> 5;  // weight row in the tile / k half; also activation row (A side)
  const int64_t row = (int64_t)blockIdx.x * 32 + nl;
  const bool live_row = row < n;
  const int64_t rb = (int64_t)nsb * kQ4KBytes;
  const int64_t xrb = (int64_t)nsb * 8 * kQ8_1Bytes;
  const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < nsb; c0 += kChunkSb) {
    const int csb = min(kChunkSb, nsb - c0);
    // this wave's superblocks wv and wv + kWaves of the chunk; weights first,
    // so their latency overlaps the staging
    u32x4 hdr[kSbPerWave], q[kSbPerWave][4];
#pragma unroll
    for (int s = 0; s < kSbPerWave; ++s) {
      const int sbl = wv + kWaves * s;
      hdr[s] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int g = 0; g < 4; ++g) q[s][g] = hdr[s];
      if (sbl < csb && live_row) {
        const uint8_t *bp8 = W + row * rb + (int64_t)(c0 + sbl) * kQ4KBytes;
        hdr[s] = ld16(bp8);
#pragma unroll
        for (int g = 0; g < 4; ++g) q[s][g] = ld16(bp8 + 16 + 32 * g + 16 * lh);
      }
    }
    if (c0 > 0) __syncthreads();  // the previous chunk is no longer read
    for (int t = tid; t < nb * 8 * csb; t += kThreads) {
      const int m = t / (8 * csb), blk = t - m * (8 * csb);
      const uint8_t *ap = XQ + m * xrb + (int64_t)(8 * c0 + blk) * kQ8_1Bytes;
      const u32x4 v0 = ld16(ap), v1 = ld16(ap + 16);
      const uint32_t v2 = ld4(ap + 32);
      const u32x4n lo = {v0.y, v0.z, v0.w, v1.x}, hi = {v1.y, v1.z, v1.w, v2};
      act[(blk * bp + m) * 2] = lo;
      act[(blk * bp + m) * 2 + 1] = hi;
      const int S = bsum4(hi.w, bsum4(hi.z, bsum4(hi.y, bsum4(hi.x,
                    bsum4(lo.w, bsum4(lo.z, bsum4(lo.y, bsum4(lo.x, 0))))))));
      const float d = h2f(v0.x);
      da[blk * bp + m] = d;
      das[blk * bp + m] = d * (float)S;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kSbPerWave; ++s) {
      const int sbl = wv + kWaves * s;
      if (sbl >= csb) break;
      int sc[8], mn[8];
#pragma unroll
      for (int g = 0; g < 4; ++g)
        q4k_scales(hdr[s].y, hdr[s].z, hdr[s].w, g, sc[2 * g], sc[2 * g + 1], mn[2 * g], mn[2 * g + 1]);
      const float d = h2f(hdr[s].x), dmin = h2f(hdr[s].x >> 16);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int blk = 8 * sbl + j;
        const u32x4 qg = q[s][j >> 1];
        const uint32_t sh = 4u * (uint32_t)(j & 1);  // sub-block 2g: low nibbles, 2g+1: high
        const v4i b = {(int)((qg.x >> sh) & 0x0F0F0F0Fu), (int)((qg.y >> sh) & 0x0F0F0F0Fu),
                       (int)((qg.z >> sh) & 0x0F0F0F0Fu), (int)((qg.w >> sh) & 0x0F0F0F0Fu)};
        v4i a = {0, 0, 0, 0};
        if (nl < nb) a = __builtin_bit_cast(v4i, act[(blk * bp + nl) * 2 + lh]);
        const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, zero, 0, 0, 0);
        // activation rows 4*lh + r, r = 0..3 (broadcast reads; rows >= nb
        // only reach registers that are never stored)
        f32x4n a4 = {0.f, 0.f, 0.f, 0.f}, s4 = a4;
        if (4 * lh < bp) {
          a4 = *reinterpret_cast<const f32x4n *>(da + blk * bp + 4 * lh);
          s4 = *reinterpret_cast<const f32x4n *>(das + blk * bp + 4 * lh);
        }
        const float dsc = d * (float)sc[j], dm = dmin * (float)mn[j];
        acc[0] += (a4.x * dsc) * (float)D[0] - s4.x * dm;
        acc[1] += (a4.y * dsc) * (float)D[1] - s4.y * dm;
        acc[2] += (a4.z * dsc) * (float)D[2] - s4.z * dm;
        acc[3] += (a4.w * dsc) * (float)D[3] - s4.w * dm;
        // Fence: MFMA builtins carry no memory dependence; without it every
        // block's MFMA is hoisted with all results live at once.
        asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3])::"memory");
      }
    }
  }
  // sum the waves' partial tiles; thread t < 32 * nb owns output (m, nl) with
  // m = t / 32: lane nl + 32 * (m / 4), register m % 4 of every wave
  part[wv * 64 + lane] = f32x4n{acc[0], acc[1], acc[2], acc[3]};
  __syncthreads();
  if (tid < 32 * nb) {
    const int m = tid >> 5, nn = tid & 31;
    const int64_t r = (int64_t)blockIdx.x * 32 + nn;
    if (r < n) {
      float s = 0.f;
      for (int w = 0; w < kWaves; ++w) s += part[w * 64 + nn + 32 * (m >> 2)][m & 3];
      Y[(int64_t)m * n + r] = s;
    }
  }
}

}  // namespace

hipError_t launch_qgemv_batch_mfma_q4k(const void *w, const void *xq, float *y, int64_t nb, int64_t n, int64_t k,
                                       hipStream_t stream) {
  const dim3 grid((unsigned)((n + 31) / 32));
  hipLaunchKernelGGL(gemv_batch_mfma_q4k, grid, dim3(kThreads), lds_bytes((int)nb), stream,
                     static_cast<const uint8_t *>(w),
                     static_cast<const uint8_t *>(xq), y, (int)nb, (int)n, (int)(k / 256));
  return hipGetLastError();
}

}  // namespace qg
