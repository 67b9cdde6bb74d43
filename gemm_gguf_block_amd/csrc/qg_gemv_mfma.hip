// qg_gemv_mfma.hip -- small-batch Q4_K and Q6_K GEMV on the int8 matrix cores.
//
// With b <= 8 activation rows the dot4 kernels spend VALU per (row, block,
// activation row).  Here the activation rows form the M side of
// v_mfma_i32_32x32x32_i8 (unused rows are zero) and 32 weight rows the N side,
// so one MFMA gives the exact int32 block dots of 32 weight rows against all
// activation rows, and the fp32 rescale costs the same few VALU per block
// whatever b is.
//
// MFMA 32x32 output layout: register r of lane l holds row 8(r/4) + 4(l/32) +
// r%4, column l%32.  The A operand of lane l is row l%32, k half l/32; the B
// operand of lane l is column l%32, the same k half.
//
// Q4_K: a workgroup of 8 waves owns a tile of 32 weight rows.  k is walked in
// chunks of 16 superblocks: the workgroup stages the chunk's activation blocks
// in LDS, wave w takes superblocks w and w + 8 of the chunk (32 rows x 144
// bytes each, loaded before the staging barrier), and runs their blocks on the
// matrix core.  The 8 waves' partial tiles are summed through LDS at the end.
// Two such workgroups fit on a CU, so 14336 rows (448 tiles) run in one pass.
// For b <= 8 only registers r = 0..3 carry rows (4(lane/32) + r).
//
// With DUMP the same code writes the exact int32 dots of every MFMA instead of
// Y: D[i][r][block] per 32-value block (Q4_K) or per 16-value sub-block (Q6_K).
#include "qg_blocks.h"
#include "qg_launch.h"

#include <algorithm>

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

template <bool DUMP>
__global__ __launch_bounds__(kThreads) void gemv_batch_mfma_q4k(const uint8_t *__restrict__ W,
                                                                const uint8_t *__restrict__ XQ,
                                                                float *__restrict__ Y, int32_t *__restrict__ Dd,
                                                                int nb, int n, int nsb) {
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
        if (DUMP) {
          // register r: activation row 4*lh + r, weight row `row`
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (4 * lh + r < nb && live_row)
              Dd[((int64_t)(4 * lh + r) * n + row) * (8 * (int64_t)nsb) + 8 * (c0 + sbl) + j] = D[r];
          asm volatile("" ::: "memory");
          continue;
        }
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
  if (DUMP) return;
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

// ---------------------------------------------------------------------------
// Q6_K.  A scale covers 16 values, half a Q8_1 block, so a block's MFMA
// carries each activation row twice: A row 2m + h holds activation row m in k
// half h and zeros in the other half (those lanes read a zero unit in LDS).
// Output registers 2j and 2j + 1 then hold the two sub-block dots of one
// activation row.  They are combined with the sub-blocks' int8 scales in fp32:
// each product is exact (a sub-block dot is at most 16 * 32 * 128 in
// magnitude), so the pair's sum is rounded once, and not at all below 2^24.
// (The MFMA results are read by compiler-generated code only: an inline-asm
// reader gets none of the wait states an MFMA result needs.)
//
// B takes the codes as q - 32 in int8 (q6k_codes4).
//
// A persistent workgroup of 8 waves takes one 32-row tile at a time; wave w
// runs superblocks w, w + 8, ... of it (all of a 4096-wide row's superblocks
// are in flight at once), the 8 partial tiles are summed through LDS, and the
// next tile's first superblock is loaded before that reduction.  The
// activation rows are staged in LDS once when k fits a chunk (7168 values),
// else once per chunk and tile.
namespace q6 {

constexpr int kChunkBlk = 224;           // Q8_1 blocks per LDS chunk
constexpr int kChunkSb = kChunkBlk / 8;  // superblocks per chunk

// Per chunk block: 2 * BP units of 16 bytes (activation row m, k half h at
// unit 2m + h) and a zero unit; after all units, 8 d_a per block, row m at
// position pos(m) so that lane half lh reads rows {2lh, 2lh+1, 2lh+4, 2lh+5}
// as one group at 4 * lh; then the waves' partial tiles, BP / 2 floats per
// lane.
__host__ __device__ constexpr int unit_stride(int bp) { return 2 * bp + 1; }
__device__ __forceinline__ int pos(int m) { return (m & 1) | ((m & 2) << 1) | ((m & 4) >> 1); }
__host__ __device__ constexpr size_t part_offset(int bp) { return (size_t)kChunkBlk * ((size_t)unit_stride(bp) * 16 + 32); }
inline size_t lds_bytes(int bp) { return part_offset(bp) + (size_t)kWaves * 64 * (bp / 2) * 4; }

// One superblock as lane half lh needs it: block j (k 32j..32j+31) takes its
// half-lh codes from ql[2(j/4) + j%2] (nibble (j/2)%2) and qh[j/4] (bit pair
// j%4); all 16 scales and d are read by both halves.
struct Sb {
  u32x4 ql[4];
  u32x4 qh[2];
  u32x4 sc;
  uint32_t d;
};

__device__ __forceinline__ void load_sb(const uint8_t *p, int lh, Sb &s) {
#pragma unroll
  for (int i = 0; i < 4; ++i) s.ql[i] = ld16_a2(p + 64 * (i >> 1) + 32 * (i & 1) + 16 * lh);
#pragma unroll
  for (int h = 0; h < 2; ++h) s.qh[h] = ld16_a2(p + 128 + 32 * h + 16 * lh);
  s.sc = ld16_a2(p + 192);
  s.d = ld2(p + 208);
}

template <int BP, bool DUMP>
__global__ __launch_bounds__(kThreads) void gemv_batch_mfma_q6k(const uint8_t *__restrict__ W,
                                                                const uint8_t *__restrict__ XQ,
                                                                float *__restrict__ Y, int32_t *__restrict__ Dd,
                                                                int nb, int n, int nsb) {
  constexpr int S = unit_stride(BP);
  constexpr int NJ = BP / 2;  // activation rows per lane
  typedef float fNJ __attribute__((ext_vector_type(NJ)));
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  u32x4n *act = reinterpret_cast<u32x4n *>(lds);
  float *da = reinterpret_cast<float *>(lds + (size_t)kChunkBlk * S * 16);
  fNJ *part = reinterpret_cast<fNJ *>(lds + part_offset(BP));

  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int nl = lane & 31, lh = lane >> 5;
  // A row nl is activation row nl / 2 in k half nl % 2
  const int aunit = ((nl & 1) == lh && (nl >> 1) < nb) ? nl : 2 * BP;
  const int64_t rb = (int64_t)nsb * kQ6KBytes;
  const int64_t xrb = (int64_t)nsb * 8 * kQ8_1Bytes;
  const int ntiles = (n + 31) / 32;
  const int nchunk = (nsb + kChunkSb - 1) / kChunkSb;
  const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
  auto wrow = [&](int tile) { return W + min((int64_t)tile * 32 + nl, (int64_t)n - 1) * rb; };

  // zero units and the d_a of rows >= nb; never written by the staging
  for (int t = tid; t < kChunkBlk; t += kThreads) {
    act[t * S + 2 * BP] = u32x4n{0u, 0u, 0u, 0u};
    for (int m = nb; m < 8; ++m) da[t * 8 + pos(m)] = 0.f;
  }

  // c0 and tile of the superblock being run, for the dump
  int dump_c0 = 0, dump_tile = 0;
  auto step = [&](const Sb &w, int sbl, fNJ &acc) {
    fNJ p = {};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int blk = 8 * sbl + j;
      const u32x4 lo = w.ql[2 * (j >> 2) + (j & 1)], hi = w.qh[j >> 2];
      const uint32_t ls = 4u * (uint32_t)((j >> 1) & 1), hs = 2u * (uint32_t)(j & 3);
      const v4i b = {q6k_codes4(lo.x >> ls, hi.x >> hs), q6k_codes4(lo.y >> ls, hi.y >> hs),
                     q6k_codes4(lo.z >> ls, hi.z >> hs), q6k_codes4(lo.w >> ls, hi.w >> hs)};
      const v4i a = __builtin_bit_cast(v4i, act[blk * S + aunit]);
      const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, zero, 0, 0, 0);
      if (DUMP) {
        // registers 2q + h: activation row 4(q/2) + 2lh + q%2, k half h =
        // sub-block 2j + h of the superblock
        const int64_t r = (int64_t)dump_tile * 32 + nl;
#pragma unroll
        for (int q = 0; q < NJ; ++q) {
          const int m = 4 * (q >> 1) + 2 * lh + (q & 1);
          if (m < nb && r < n) {
            int32_t *dp = Dd + ((int64_t)m * n + r) * (16 * (int64_t)nsb) + 16 * (dump_c0 + sbl) + 2 * j;
            dp[0] = D[2 * q];
            dp[1] = D[2 * q + 1];
          }
        }
        asm volatile("" ::: "memory");
        continue;
      }
      const uint32_t scw = w.sc[j >> 1];
      const float sc0 = (float)sbyte(scw, 16u * (uint32_t)(j & 1));
      const float sc1 = (float)sbyte(scw, 16u * (uint32_t)(j & 1) + 8u);
      const fNJ dv = *reinterpret_cast<const fNJ *>(da + blk * 8 + 4 * lh);
#pragma unroll
      for (int q = 0; q < NJ; ++q) p[q] = fmaf(dv[q], fmaf((float)D[2 * q + 1], sc1, (float)D[2 * q] * sc0), p[q]);
      asm volatile("" : "+v"(p)::"memory");
    }
    acc += h2f(w.d) * p;
  };

  Sb cur, nxt;
  int tile = (int)blockIdx.x;
  if (tile < ntiles && wv < min(kChunkSb, nsb)) load_sb(wrow(tile) + (int64_t)wv * kQ6KBytes, lh, cur);
  for (int rnd = 0; tile < ntiles; ++rnd, tile += (int)gridDim.x) {  // tile is uniform in the workgroup
    const uint8_t *wr = wrow(tile);
    fNJ acc = {};
    dump_tile = tile;
    for (int c0 = 0; c0 < nsb; c0 += kChunkSb) {
      const int csb = min(kChunkSb, nsb - c0);
      dump_c0 = c0;
      if (c0 > 0 && wv < csb) load_sb(wr + (int64_t)(c0 + wv) * kQ6KBytes, lh, cur);
      if (nchunk > 1 || rnd == 0) {
        if (rnd > 0 || c0 > 0) __syncthreads();  // the previous chunk is no longer read
        for (int t = tid; t < nb * 8 * csb; t += kThreads) {
          const int m = t / (8 * csb), blk = t - m * (8 * csb);
          const uint8_t *ap = XQ + m * xrb + (int64_t)(8 * c0 + blk) * kQ8_1Bytes;
          const u32x4 v0 = ld16(ap), v1 = ld16(ap + 16);
          const uint32_t v2 = ld4(ap + 32);
          act[blk * S + 2 * m] = u32x4n{v0.y, v0.z, v0.w, v1.x};
          act[blk * S + 2 * m + 1] = u32x4n{v1.y, v1.z, v1.w, v2};
          da[blk * 8 + pos(m)] = h2f(v0.x);
        }
        __syncthreads();
      }
      // superblocks wv, wv + 8, ... of the chunk, the next one loaded ahead
      for (int s = wv; s < csb; s += 2 * kWaves) {
        if (s + kWaves < csb) load_sb(wr + (int64_t)(c0 + s + kWaves) * kQ6KBytes, lh, nxt);
        step(cur, s, acc);
        if (s + kWaves >= csb) break;
        if (s + 2 * kWaves < csb) load_sb(wr + (int64_t)(c0 + s + 2 * kWaves) * kQ6KBytes, lh, cur);
        step(nxt, s + kWaves, acc);
      }
    }
    const int next = tile + (int)gridDim.x;
    if (next < ntiles && wv < min(kChunkSb, nsb)) load_sb(wrow(next) + (int64_t)wv * kQ6KBytes, lh, cur);
    if (DUMP) continue;  // tile is uniform in the workgroup: no barrier is skipped by part of it
    // sum the waves' partial tiles: thread t < 32 * nb owns activation row
    // m = t / 32, weight row nn = t % 32, held by lane nn + 32 * ((m / 2) % 2),
    // element (m % 2) + 2 * (m / 4) of every wave
    part[wv * 64 + lane] = acc;
    __syncthreads();
    if (tid < 32 * nb) {
      const int m = tid >> 5, nn = tid & 31;
      const int src = nn + 32 * ((m >> 1) & 1), q = (m & 1) + 2 * (m >> 2);
      const int64_t r = (int64_t)tile * 32 + nn;
      if (r < n) {
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) sum += part[w * 64 + src][q];
        Y[(int64_t)m * n + r] = sum;
      }
    }
    __syncthreads();  // part is rewritten next round
  }
}

// The dump instance runs on the grid of the product instance.
template <int BP>
hipError_t launch_bp(const void *w, const void *xq, float *y, int32_t *D, int64_t nb, int64_t n, int64_t k,
                     hipStream_t stream) {
  const size_t lds = lds_bytes(BP);
  const int64_t groups = (n + 31) / 32;
  const int64_t g = std::min(groups, resident_blocks<gemv_batch_mfma_q6k<BP, false>>(kThreads, lds));
  const uint8_t *W = static_cast<const uint8_t *>(w), *X = static_cast<const uint8_t *>(xq);
  if (D)
    hipLaunchKernelGGL((gemv_batch_mfma_q6k<BP, true>), dim3((unsigned)g), dim3(kThreads), lds, stream, W, X, y, D,
                       (int)nb, (int)n, (int)(k / 256));
  else
    hipLaunchKernelGGL((gemv_batch_mfma_q6k<BP, false>), dim3((unsigned)g), dim3(kThreads), lds, stream, W, X, y, D,
                       (int)nb, (int)n, (int)(k / 256));
  return hipGetLastError();
}

}  // namespace q6

}  // namespace

hipError_t launch_qgemv_batch_mfma_q4k(const void *w, const void *xq, float *y, int32_t *D, int64_t nb, int64_t n,
                                       int64_t k, hipStream_t stream) {
  const dim3 grid((unsigned)((n + 31) / 32));
  const uint8_t *W = static_cast<const uint8_t *>(w), *X = static_cast<const uint8_t *>(xq);
  if (D)
    hipLaunchKernelGGL(gemv_batch_mfma_q4k<true>, grid, dim3(kThreads), lds_bytes((int)nb), stream, W, X, y, D,
                       (int)nb, (int)n, (int)(k / 256));
  else
    hipLaunchKernelGGL(gemv_batch_mfma_q4k<false>, grid, dim3(kThreads), lds_bytes((int)nb), stream, W, X, y, D,
                       (int)nb, (int)n, (int)(k / 256));
  return hipGetLastError();
}

hipError_t launch_qgemv_batch_mfma_q6k(const void *w, const void *xq, float *y, int32_t *D, int64_t nb, int64_t n,
                                       int64_t k, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  return nb <= 4 ? q6::launch_bp<4>(w, xq, y, D, nb, n, k, stream) : q6::launch_bp<8>(w, xq, y, D, nb, n, k, stream);
}

}  // namespace qg
