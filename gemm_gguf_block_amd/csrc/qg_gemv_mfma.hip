// qg_gemv_mfma.hip -- small-batch Q4_K, Q6_K and Q8_0 GEMV on the int8 matrix
// cores.
//
// With b <= 8 activation rows the dot4 kernels spend VALU per (row, block,
// activation row).  Here the activation rows form the M side of
// v_mfma_i32_32x32x32_i8 and 32 weight rows the N side, so one MFMA gives the
// exact int32 block dots of 32 weight rows against all activation rows, and
// the fp32 rescale costs the same few VALU per block whatever b is.
//
// MFMA 32x32 output layout: register r of lane l holds row 8(r/4) + 4(l/32) +
// r%4, column l%32.  The A operand of lane l is row l%32, k half l/32; the B
// operand of lane l is column l%32, the same k half.  For b <= 8 only
// registers r = 0..3 carry rows (4(lane/32) + r).
//
// With DUMP the same code writes the exact int32 dots of every MFMA instead of
// Y: D[i][r][block] per 32-value block (Q4_K, Q8_0) or per 16-value sub-block
// (Q6_K).  (Q8_0 runs 16-row tiles on v_mfma_i32_16x16x64_i8; see below.)
#include "qg_blocks.h"
#include "qg_launch.h"

#include <algorithm>

namespace qg {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4n __attribute__((ext_vector_type(4)));
typedef float f32x4n __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

// ---------------------------------------------------------------------------
// Q4_K.  A workgroup of 8 waves owns a tile of 32 weight rows; two fit on a
// CU, so 14336 rows (448 tiles) run in one pass.  k is walked in chunks of 16
// superblocks, and wave w takes superblocks w and w + 8 of a chunk.
//
// Weights: the tile's 32 rows of one superblock are 288 16-byte pieces.  A
// wave reads them in address order (lane l: pieces l + 64q, q = 0..4), which
// touches a third as many cache lines per load instruction as reading them
// straight in the MFMA B layout, writes them to its own LDS buffer as
// [piece][row], and reads back the B layout (header of row l%32, code piece
// 1 + 2g + l/32).  One superblock is in flight per wave: the next one is
// loaded as soon as the current one has gone through LDS.
//
// Activations: the chunk's Q8_1 blocks are staged once per workgroup:
//   act  [blk][m][half]  16 B  int8 codes, the A operand;
//   da   [blk][m]        f32   d_a;
//   mina [sb][m][half]   16 B  bf16 (hi, lo) of d_a * sum(qa) for blocks
//                              4 half .. 4 half + 3 of superblock sb.
// Their loads are issued before the weights', and the staging writes wait
// for them alone.
//
// Per superblock the int8 MFMAs give the block dots D_j; the lane's four
// activation rows take d * sum_j d_a (sc_j D_j) on the VALU, with block j+1's
// MFMA issued before block j's rescale, and the min term dmin * sum_j
// (d_a sum qa)_j m_j on the matrix core: one bf16 MFMA over the (hi, lo)
// split of d_a sum(qa) (2^-16 relative) against the integer m_j, lanes 0-31
// carrying blocks 0-3 and lanes 32-63 blocks 4-7 (k slots 2i, 2i + 1 of
// block 4 l/32 + i).  The 8 waves' partial tiles are summed through LDS.
namespace q4 {

constexpr int kSbPerWave = 2;
constexpr int kChunkSb = kWaves * kSbPerWave;  // superblocks per chunk
constexpr int kChunkBlk = 8 * kChunkSb;
constexpr int kWbUnits = 9 * 33;  // per wave: [piece][row], rows padded to 33 units of 16 bytes
constexpr size_t kDaOff = (size_t)kChunkBlk * 8 * 32;
constexpr size_t kMinOff = kDaOff + (size_t)kChunkBlk * 8 * 4;
constexpr size_t kWbOff = kMinOff + (size_t)kChunkSb * 8 * 2 * 16;
constexpr size_t kPartOff = kWbOff;  // the partial tiles reuse the weight buffers
constexpr size_t kLds = kWbOff + (size_t)kWaves * kWbUnits * 16;
static_assert(kWaves * 64 <= kWaves * kWbUnits, "the partial tiles fit in the weight buffers");
static_assert(2 * kLds <= 160 * 1024, "two workgroups per CU");
constexpr int kStageIters = (8 * kChunkBlk + kThreads - 1) / kThreads;

// Five 16-byte pieces of one superblock.  As loaded (load_sb): the lane's
// address-ordered pieces l + 64q of the tile's 32 rows.  After to_mfma: what
// lane l needs in the B layout, the header of row l%32 and, per 32-byte code
// group, the 16 bytes that fall in k half l/32.
struct Sb {
  u32x4 hdr, q[4];
};

// bf16 bits of x with the low mantissa bits cut off (hi) and of the rest
// rounded to nearest (lo), packed lo << 16 | hi: x = hi + lo to 2^-16.
__device__ __forceinline__ uint32_t bf16_hilo(float x) {
  const uint32_t hb = __builtin_bit_cast(uint32_t, x) & 0xFFFF0000u;
  const uint32_t lb = __builtin_bit_cast(uint32_t, x - __builtin_bit_cast(float, hb));
  const uint32_t lr = (lb + 0x7FFFu + ((lb >> 16) & 1u)) >> 16;
  return (hb >> 16) | (lr << 16);
}

// W and XQ are not declared __restrict__: that keeps the activation loads
// ahead of the weight loads and both ahead of the staging barrier (loads the
// compiler may treat as invariant are otherwise scheduled next to their uses).
template <bool DUMP>
__global__ __launch_bounds__(kThreads, 4) void gemv_batch_mfma_q4k(const uint8_t *W, const uint8_t *XQ, float *Y,
                                                                   int32_t *Dd, int nb, int n, int nsb) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  u32x4n *act = reinterpret_cast<u32x4n *>(lds);
  float *da = reinterpret_cast<float *>(lds + kDaOff);
  const u32x4n *mina = reinterpret_cast<const u32x4n *>(lds + kMinOff);
  uint32_t *minw = reinterpret_cast<uint32_t *>(lds + kMinOff);
  f32x4n *part = reinterpret_cast<f32x4n *>(lds + kPartOff);
  u32x4n *wb = reinterpret_cast<u32x4n *>(lds + kWbOff) + (threadIdx.x >> 6) * kWbUnits;

  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int nl = lane & 31, lh = lane >> 5;  // weight row in the tile / k half; also activation row (A side)
  const int tile = (int)blockIdx.x;
  const int64_t rb = (int64_t)nsb * kQ4KBytes;
  const int64_t xrb = (int64_t)nsb * 8 * kQ8_1Bytes;
  const int nchunk = (nsb + kChunkSb - 1) / kChunkSb;
  const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
  const v16f fzero = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

  // Byte offsets of this lane's pieces from the tile's first row (rows past n
  // read row n - 1; the last 32 lanes of q = 4 repeat piece 287), and their
  // LDS units.  k <= 2^24 keeps 32 rows of offsets within 31 bits.
  uint32_t off[5], wbi[5];
  {
    const int rowlim = n - 1 - tile * 32;
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      const int pc = min(lane + 64 * q, 287), pr = pc / 9, pp = pc - 9 * pr;
      off[q] = (uint32_t)(min(pr, rowlim) * (int)rb + 16 * pp);
      wbi[q] = (uint32_t)(pp * 33 + pr);
    }
  }
  const uint8_t *tw = W + (int64_t)tile * 32 * rb;
  // superblock i of this wave in chunk c (past the chunk's end: its last one,
  // never used)
  auto load_sb = [&](Sb &R, int c, int i) __attribute__((always_inline)) {
    const int c0 = c * kChunkSb, last = min(kChunkSb, nsb - c0) - 1;
    const uint8_t *p = tw + (int64_t)(c0 + min(wv + kWaves * i, last)) * kQ4KBytes;
    R.hdr = ld16(p + off[0]);
#pragma unroll
    for (int g = 0; g < 4; ++g) R.q[g] = ld16(p + off[g + 1]);
  };
  // R through this wave's LDS buffer into the B layout (a wave's LDS
  // accesses complete in order, so no barrier is needed)
  auto to_mfma = [&](const Sb &R) __attribute__((always_inline)) {
    const u32x4 v[5] = {R.hdr, R.q[0], R.q[1], R.q[2], R.q[3]};
#pragma unroll
    for (int q = 0; q < 5; ++q) wb[wbi[q]] = u32x4n{v[q].x, v[q].y, v[q].z, v[q].w};
    Sb O;
    const u32x4n h = wb[nl];
    O.hdr = u32x4{h.x, h.y, h.z, h.w};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x4n t = wb[(1 + 2 * g + lh) * 33 + nl];
      O.q[g] = u32x4{t.x, t.y, t.z, t.w};
    }
    return O;
  };

  // Activation staging of chunk c: all loads first (threads past the last
  // block repeat it, so the loads are a fixed sequence), then the writes.
  u32x4 sv0[kStageIters], sv1[kStageIters];
  uint32_t sv2[kStageIters];
  auto stage_load = [&](int c) __attribute__((always_inline)) {
    const int c0 = c * kChunkSb, csb = min(kChunkSb, nsb - c0), items = nb * 8 * csb;
#pragma unroll
    for (int it = 0; it < kStageIters; ++it) {
      const int t = min(tid + it * kThreads, items - 1);
      const int m = t / (8 * csb), blk = t - m * (8 * csb);
      const uint8_t *ap = XQ + m * xrb + (int64_t)(8 * c0 + blk) * kQ8_1Bytes;
      sv0[it] = ld16(ap);
      sv1[it] = ld16(ap + 16);
      sv2[it] = ld4(ap + 32);
    }
  };
  auto stage_write = [&](int c) __attribute__((always_inline)) {
    const int c0 = c * kChunkSb, csb = min(kChunkSb, nsb - c0), items = nb * 8 * csb;
#pragma unroll
    for (int it = 0; it < kStageIters; ++it) {
      const int t = min(tid + it * kThreads, items - 1);
      const int m = t / (8 * csb), blk = t - m * (8 * csb);
      const u32x4 v0 = sv0[it], v1 = sv1[it];
      const u32x4n lo = {v0.y, v0.z, v0.w, v1.x}, hi = {v1.y, v1.z, v1.w, sv2[it]};
      act[(blk * 8 + m) * 2] = lo;
      act[(blk * 8 + m) * 2 + 1] = hi;
      const int S = bsum4(hi.w, bsum4(hi.z, bsum4(hi.y, bsum4(hi.x,
                    bsum4(lo.w, bsum4(lo.z, bsum4(lo.y, bsum4(lo.x, 0))))))));
      const float d = h2f(v0.x);
      da[blk * 8 + m] = d;
      const int sbl = blk >> 3, j = blk & 7;
      minw[((sbl * 8 + m) * 2 + (j >> 2)) * 4 + (j & 3)] = bf16_hilo(d * (float)S);
    }
  };

  f32x4n acc = {0.f, 0.f, 0.f, 0.f};
  // superblock sbl of chunk c0, accumulated into acc
  auto run_sb = [&](const Sb &w, int sbl, int c0) __attribute__((always_inline)) {
    int sc[8], mn[8];
#pragma unroll
    for (int g = 0; g < 4; ++g)
      q4k_scales(w.hdr.y, w.hdr.z, w.hdr.w, g, sc[2 * g], sc[2 * g + 1], mn[2 * g], mn[2 * g + 1]);
    // A rows 8..31 reach only output registers 4..15, which are never read,
    // so those lanes take rows nl % 8; rows nb..7 are never stored
    const u32x4n *ap = act + (64 * sbl + (nl & 7)) * 2 + lh;
    const f32x4n *dp = reinterpret_cast<const f32x4n *>(da + 64 * sbl + 4 * lh);
    auto bops = [&](int j) __attribute__((always_inline)) {
      const u32x4 qg = w.q[j >> 1];
      const uint32_t sh = 4u * (uint32_t)(j & 1);  // sub-block 2g: low nibbles, 2g+1: high
      return v4i{(int)((qg.x >> sh) & 0x0F0F0F0Fu), (int)((qg.y >> sh) & 0x0F0F0F0Fu),
                 (int)((qg.z >> sh) & 0x0F0F0F0Fu), (int)((qg.w >> sh) & 0x0F0F0F0Fu)};
    };
    f32x4n t = {0.f, 0.f, 0.f, 0.f};
    v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(v4i, ap[0]), bops(0), zero, 0, 0, 0);
    f32x4n a4c = dp[0], a4n = dp[2];
    v4i an = __builtin_bit_cast(v4i, ap[16]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v16i Dn = zero;
      if (j + 1 < 8) Dn = __builtin_amdgcn_mfma_i32_32x32x32_i8(an, bops(j + 1), zero, 0, 0, 0);
      const f32x4n a4 = a4c;  // d_a of activation rows 4 lh + r (broadcast read)
      a4c = a4n;
      if (j + 2 < 8) {
        an = __builtin_bit_cast(v4i, ap[(j + 2) * 16]);
        a4n = dp[2 * (j + 2)];
      }
      if (DUMP) {
        const int64_t row = (int64_t)tile * 32 + nl;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * lh + r < nb && row < n)
            Dd[((int64_t)(4 * lh + r) * n + row) * (8 * (int64_t)nsb) + 8 * (c0 + sbl) + j] = D[r];
      } else {
        t.x = fmaf(a4.x, (float)__mul24(sc[j], D[0]), t.x);
        t.y = fmaf(a4.y, (float)__mul24(sc[j], D[1]), t.y);
        t.z = fmaf(a4.z, (float)__mul24(sc[j], D[2]), t.z);
        t.w = fmaf(a4.w, (float)__mul24(sc[j], D[3]), t.w);
      }
      // Fence: MFMA builtins carry no memory dependence; without it every
      // block's MFMA is hoisted with all results live at once.
      asm volatile("" : "+v"(t)::"memory");
      D = Dn;
    }
    if (DUMP) return;
    // min term: B k slots 2i, 2i + 1 hold m of block 4lh + i as bf16 (exact)
    uint32_t bm[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t h = __builtin_bit_cast(uint32_t, (float)(lh ? mn[4 + i] : mn[i])) >> 16;
      bm[i] = h | (h << 16);
    }
    const v16f M = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        __builtin_bit_cast(v8bf, mina[(sbl * 8 + (nl & 7)) * 2 + lh]),
        __builtin_bit_cast(v8bf, u32x4n{bm[0], bm[1], bm[2], bm[3]}), fzero, 0, 0, 0);
    const float d = h2f(w.hdr.x), dmin = h2f(w.hdr.x >> 16);
    acc.x = fmaf(d, t.x, fmaf(-dmin, M[0], acc.x));
    acc.y = fmaf(d, t.y, fmaf(-dmin, M[1], acc.y));
    acc.z = fmaf(d, t.z, fmaf(-dmin, M[2], acc.z));
    acc.w = fmaf(d, t.w, fmaf(-dmin, M[3], acc.w));
  };

  // (k = 0 runs no chunk and stores zeros)
  // prologue: the first chunk's activation loads, then the first superblock
  // of weights, then the staging writes
  Sb cur;
  if (nchunk > 0) {  // uniform in the workgroup
    stage_load(0);
    asm volatile("" ::: "memory");
    load_sb(cur, 0, 0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);  // nothing that waits for the activation moves above the weight loads
    stage_write(0);
    __syncthreads();
  }
  for (int c = 0; c < nchunk; ++c) {
    const int c0 = c * kChunkSb, csb = min(kChunkSb, nsb - c0);
    if (c > 0) {         // uniform in the workgroup
      __syncthreads();   // the previous chunk is no longer read
      stage_load(c);
      stage_write(c);
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < kSbPerWave; ++i) {
      // cur goes through LDS, then the next superblock is loaded into it
      // while this one runs
      const Sb O = to_mfma(cur);
      if (i + 1 < kSbPerWave) load_sb(cur, c, i + 1);
      else if (c + 1 < nchunk) load_sb(cur, c + 1, 0);
      if (wv + kWaves * i < csb) run_sb(O, wv + kWaves * i, c0);
    }
  }
  if (DUMP) return;
  // sum the waves' partial tiles; thread t < 32 * nb owns output (m, nn) with
  // m = t / 32: lane nn + 32 * (m / 4), register m % 4 of every wave.  part
  // overlays the weight buffers, so every wave first finishes with them.
  __syncthreads();
  part[wv * 64 + lane] = acc;
  __syncthreads();
  if (tid < 32 * nb) {
    const int m = tid >> 5, nn = tid & 31;
    const int64_t r = (int64_t)tile * 32 + nn;
    if (r < n) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) sum += part[w * 64 + nn + 32 * (m >> 2)][m & 3];
      Y[(int64_t)m * n + r] = sum;
    }
  }
}

}  // namespace q4

// ---------------------------------------------------------------------------
// Q6_K.  A scale covers 16 values, half a Q8_1 block, so a block's MFMA
// carries each activation row twice: A row 2m + h holds activation row m in k
// half h and zeros in the other half (those lanes read a zero unit in LDS).
// Output registers 2j and 2j + 1 then hold the two sub-block dots of one
// activation row.  They are combined with the sub-blocks' int8 scales in
// integers (exact, at most 2^24, so the fp32 convert is exact too).  (The
// MFMA results are read by compiler-generated code only: an inline-asm reader
// gets none of the wait states an MFMA result needs.)
//
// B takes the codes as q - 32 in int8 (q6k_codes4).
//
// Workgroups of 16 waves, one per CU, persistent; every wave owns whole
// 32-row tiles and walks all superblocks of its tile itself, so there is no
// reduction across waves.  The tile's 32 rows of a superblock (210 bytes
// each, 2-byte aligned) are read as 448 16-byte pieces in address order, 14
// per row starting at the row's superblock (the last one at byte 194, so
// that it ends with d inside the superblock): a third as many cache lines per
// load instruction as reading the MFMA layout straight from memory.  They go
// to the wave's LDS buffer as [piece][row], where every field the B layout
// needs starts a piece.  The next superblock is loaded while the current one
// runs.  The activation rows are staged in LDS once when k fits a chunk
// (16 superblocks), else once per chunk and round of tiles.
namespace q6 {

constexpr int kWaves6 = 16;
constexpr int kThreads6 = 64 * kWaves6;
constexpr int kChunkSb = kWaves6;       // superblocks per chunk: one per wave
constexpr int kChunkBlk = 8 * kChunkSb;  // Q8_1 blocks per LDS chunk
constexpr int kPieces = 14;             // 16-byte pieces per superblock row (the last one at byte 194)
constexpr int kWbUnits = kPieces * 33;  // per wave: [piece][row], rows padded to 33 units

// Per chunk block: 2 * BP units of 16 bytes (activation row m, k half h at
// unit 2m + h) and a zero unit; after all units, 8 d_a per block, row m at
// position pos(m) so that lane half lh reads rows {2lh, 2lh+1, 2lh+4, 2lh+5}
// as one group at 4 * lh; then the waves' weight buffers.
__host__ __device__ constexpr int unit_stride(int bp) { return 2 * bp + 1; }
__device__ __forceinline__ int pos(int m) { return (m & 1) | ((m & 2) << 1) | ((m & 4) >> 1); }
__host__ __device__ constexpr size_t wb_offset(int bp) { return (size_t)kChunkBlk * ((size_t)unit_stride(bp) * 16 + 32); }
inline size_t lds_bytes(int bp) { return wb_offset(bp) + (size_t)kWaves6 * kWbUnits * 16; }

// The same superblock of the tile's 32 rows as loaded: 448 pieces in address
// order, lane l holding pieces l + 64q (q = 0..6).
struct Raw {
  u32x4 v[7];
};

template <int BP, bool DUMP>
__global__ __launch_bounds__(kThreads6) void gemv_batch_mfma_q6k(const uint8_t *W, const uint8_t *XQ, float *Y,
                                                                 int32_t *Dd, int nb, int n, int nsb) {
  constexpr int S = unit_stride(BP);
  constexpr int NJ = BP / 2;  // activation rows per lane
  typedef float fNJ __attribute__((ext_vector_type(NJ)));
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  u32x4n *act = reinterpret_cast<u32x4n *>(lds);
  float *da = reinterpret_cast<float *>(lds + (size_t)kChunkBlk * S * 16);
  u32x4n *wb = reinterpret_cast<u32x4n *>(lds + wb_offset(BP)) + (threadIdx.x >> 6) * kWbUnits;

  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int nl = lane & 31, lh = lane >> 5;
  // A row nl is activation row nl / 2 in k half nl % 2
  const int aunit = ((nl & 1) == lh && (nl >> 1) < nb) ? nl : 2 * BP;
  const int64_t rb = (int64_t)nsb * kQ6KBytes;
  const int64_t xrb = (int64_t)nsb * 8 * kQ8_1Bytes;
  const int ntiles = (n + 31) / 32;
  const int nchunk = (nsb + kChunkSb - 1) / kChunkSb;
  const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

  // A tile's first row: the last tile is moved back to end at row n - 1
  // (its rows that the previous tile also has come out bit-identical, and
  // both store them), so every row read is a row of W; with n < 32 the rows
  // past n - 1 read row n - 1 instead.
  auto row0 = [&](int tile) __attribute__((always_inline)) { return n >= 32 ? min(tile * 32, n - 32) : 0; };
  // this lane's pieces pc = lane + 64q: row pc / 14 of the tile, byte 16 *
  // (pc % 14) of its superblock (the last piece at 194, so that it ends with
  // d and stays inside the superblock); poff[q] is its byte offset from the
  // tile's first row (k <= 2^24 keeps it within 31 bits)
  uint32_t poff[7];
#pragma unroll
  for (int q = 0; q < 7; ++q) {
    const int pc = lane + 64 * q, pr = pc / kPieces, pp = pc - kPieces * pr;
    poff[q] = (uint32_t)(min(pr, n - 1) * (int)rb + (pp == kPieces - 1 ? 194 : 16 * pp));
  }
  // superblock sb of `tile` (both wave-uniform: p is a scalar base)
  auto load_raw = [&](Raw &R, int tile, int sb) __attribute__((always_inline)) {
    const uint8_t *p = W + (int64_t)row0(tile) * rb + (int64_t)sb * kQ6KBytes;
#pragma unroll
    for (int q = 0; q < 7; ++q) {
      uint32_t o = poff[q];
      asm volatile("" : "+v"(o));  // one scalar base plus a 32-bit offset per load, not hoisted 64-bit addresses
      R.v[q] = ld16_a2(p + o);
    }
  };
  // R into this wave's LDS buffer as [piece][row]; the B layout is read back
  // from there as the blocks need it (piece pp of row nl)
  auto put_raw = [&](const Raw &R) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 7; ++q) {
      const int pc = lane + 64 * q, pr = pc / kPieces, pp = pc - kPieces * pr;
      wb[pp * 33 + pr] = u32x4n{R.v[q].x, R.v[q].y, R.v[q].z, R.v[q].w};
    }
  };
  auto rd = [&](int pp) __attribute__((always_inline)) {
    const u32x4n t = wb[pp * 33 + nl];
    return u32x4{t.x, t.y, t.z, t.w};
  };

  // zero units and the d_a of rows >= nb; never written by the staging
  for (int t = tid; t < kChunkBlk; t += kThreads6) {
    act[t * S + 2 * BP] = u32x4n{0u, 0u, 0u, 0u};
    for (int m = nb; m < 8; ++m) da[t * 8 + pos(m)] = 0.f;
  }

  // c0 and tile of the superblock being run, for the dump
  int dump_c0 = 0, dump_tile = 0;
  // One superblock of this wave's tile from its LDS buffer.  Block j + 1's
  // MFMA is issued before block j's rescale; the code pieces of blocks 4..7
  // replace those of blocks 0..3 once block 3's operand is built.
  auto step = [&](int sbl, fNJ &acc) {
    fNJ p = {};
    const u32x4 scv = rd(12);
    const uint32_t dw = rd(13).w >> 16;
    u32x4 ql0 = rd(lh), ql1 = rd(2 + lh), qh = rd(8 + lh);
    auto bops = [&](int j) __attribute__((always_inline)) {
      const u32x4 lo = (j & 1) ? ql1 : ql0, hi = qh;
      const uint32_t ls = 4u * (uint32_t)((j >> 1) & 1), hs = 2u * (uint32_t)(j & 3);
      return v4i{q6k_codes4(lo.x >> ls, hi.x >> hs), q6k_codes4(lo.y >> ls, hi.y >> hs),
                 q6k_codes4(lo.z >> ls, hi.z >> hs), q6k_codes4(lo.w >> ls, hi.w >> hs)};
    };
    auto aops = [&](int j) __attribute__((always_inline)) {
      return __builtin_bit_cast(v4i, act[(8 * sbl + j) * S + aunit]);
    };
    v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(aops(0), bops(0), zero, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int blk = 8 * sbl + j;
      if (j == 3) {
        ql0 = rd(4 + lh);
        ql1 = rd(6 + lh);
        qh = rd(10 + lh);
      }
      v16i Dn = zero;
      if (j + 1 < 8) Dn = __builtin_amdgcn_mfma_i32_32x32x32_i8(aops(j + 1), bops(j + 1), zero, 0, 0, 0);
      if (DUMP) {
        // registers 2q + h: activation row 4(q/2) + 2lh + q%2, k half h =
        // sub-block 2j + h of the superblock
        const int64_t r = (int64_t)row0(dump_tile) + nl;
#pragma unroll
        for (int q = 0; q < NJ; ++q) {
          const int m = 4 * (q >> 1) + 2 * lh + (q & 1);
          if (m < nb && r < n) {
            int32_t *dp = Dd + ((int64_t)m * n + r) * (16 * (int64_t)nsb) + 16 * (dump_c0 + sbl) + 2 * j;
            dp[0] = D[2 * q];
            dp[1] = D[2 * q + 1];
          }
        }
      } else {
        // sc0 D0 + sc1 D1 in integers: |D| <= 16 * 32 * 128, |sc| <= 128, so
        // the sum is at most 2^24 and exact in int32 and in its fp32 convert
        const uint32_t scw = scv[j >> 1];
        const int sc0 = sbyte(scw, 16u * (uint32_t)(j & 1));
        const int sc1 = sbyte(scw, 16u * (uint32_t)(j & 1) + 8u);
        const fNJ dv = *reinterpret_cast<const fNJ *>(da + blk * 8 + 4 * lh);
#pragma unroll
        for (int q = 0; q < NJ; ++q)
          p[q] = fmaf(dv[q], (float)(__mul24(D[2 * q + 1], sc1) + __mul24(D[2 * q], sc0)), p[q]);
      }
      asm volatile("" : "+v"(p)::"memory");
      D = Dn;
    }
    acc += h2f(dw) * p;
  };

  // Every wave owns whole tiles: wave gw = 16 blockIdx.x + wv of the grid
  // takes tiles gw, gw + TW, ... (TW waves in the grid), one round at a time,
  // and walks all superblocks of its tile itself, the next one loaded while
  // the current one runs.  Past the last tile a wave repeats it and stores
  // nothing (the rounds are uniform in the workgroup, for the staging
  // barriers).
  const int gw = (int)blockIdx.x * kWaves6 + __builtin_amdgcn_readfirstlane(wv);
  const int TW = (int)gridDim.x * kWaves6;
  const int rounds = (ntiles + TW - 1) / TW;
  auto round_tile = [&](int r) __attribute__((always_inline)) { return min(gw + r * TW, ntiles - 1); };
  Raw cur;
  if (rounds > 0) load_raw(cur, round_tile(0), 0);
  for (int r = 0; r < rounds; ++r) {
    const int tile = round_tile(r);
    const bool live = gw + r * TW < ntiles;
    fNJ acc = {};
    dump_tile = tile;
    for (int c0 = 0; c0 < nsb; c0 += kChunkSb) {
      const int csb = min(kChunkSb, nsb - c0);
      dump_c0 = c0;
      if (nchunk > 1 || r == 0) {
        if (r > 0 || c0 > 0) __syncthreads();  // the previous chunk is no longer read
        for (int t = tid; t < nb * 8 * csb; t += kThreads6) {
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
#pragma unroll 1
      for (int sl = 0; sl < csb; ++sl) {
        put_raw(cur);
        // the next superblock of this wave: this tile's next, else the next round's first
        if (c0 + sl + 1 < nsb) load_raw(cur, tile, c0 + sl + 1);
        else if (r + 1 < rounds) load_raw(cur, round_tile(r + 1), 0);
        step(sl, acc);
      }
    }
    if (DUMP || !live) continue;
    // element q of acc: activation row 4(q/2) + 2lh + q%2, weight row
    // row0(tile) + nl
    const int64_t row = (int64_t)row0(tile) + nl;
#pragma unroll
    for (int q = 0; q < NJ; ++q) {
      const int m = 4 * (q >> 1) + 2 * lh + (q & 1);
      if (m < nb && row < n) Y[(int64_t)m * n + row] = acc[q];
    }
  }
}

// The dump instance runs on the grid of the product instance.
template <int BP>
hipError_t launch_bp(const void *w, const void *xq, float *y, int32_t *D, int64_t nb, int64_t n, int64_t k,
                     hipStream_t stream) {
  const size_t lds = lds_bytes(BP);
  const int64_t waves = (n + 31) / 32;  // one per tile at most
  const int64_t g = std::min((waves + kWaves6 - 1) / kWaves6,
                             resident_blocks<gemv_batch_mfma_q6k<BP, false>>(kThreads6, lds));
  const uint8_t *W = static_cast<const uint8_t *>(w), *X = static_cast<const uint8_t *>(xq);
  if (D)
    hipLaunchKernelGGL((gemv_batch_mfma_q6k<BP, true>), dim3((unsigned)g), dim3(kThreads6), lds, stream, W, X, y, D,
                       (int)nb, (int)n, (int)(k / 256));
  else
    hipLaunchKernelGGL((gemv_batch_mfma_q6k<BP, false>), dim3((unsigned)g), dim3(kThreads6), lds, stream, W, X, y, D,
                       (int)nb, (int)n, (int)(k / 256));
  return hipGetLastError();
}

}  // namespace q6

// ---------------------------------------------------------------------------
// Q8_0 (k a multiple of 256).  A workgroup of 16 waves owns a tile of 16
// weight rows: 4096 rows give 256 workgroups.  v_mfma_i32_16x16x64_i8 takes
// two blocks per instruction: A rows 0-7 hold the activation rows in k 0..31
// (block j) and zeros in k 32..63, rows 8-15 the same rows in k 32..63 (block
// j + 1) and zeros below, so output rows 0-7 are block j's dots and 8-15 block
// j + 1's.  Register r of lane l is output row 4(l/16) + r, column l%16: the
// lane holds activation rows 4((l/16)%2) + r of block j + l/32 against weight
// row l%16, and its B operand is that same weight row and block (16 of the
// code bytes, k half (l/16)%2).
//
// Weights: 8 blocks of a row are 272 bytes, 16-byte aligned; the tile's 16
// rows of them are 272 pieces of 16 bytes.  Wave w takes blocks 8w..8w+7 of
// every 128-block activation chunk, loads the pieces in address order (lane l:
// pieces l + 64q), and writes them to its LDS buffer as [piece][row] (rows
// padded to 17).  A block's 32 code bytes start 2 bytes past its d, so a lane
// reads the two pieces its 16 bytes fall in and shifts them into place: by a
// whole number of dwords for an odd block, with v_alignbyte for an even one
// (the offsets are fixed per block pair, one choice per lane half).
namespace q8 {

constexpr int kWaves8 = 16;
constexpr int kThreads8 = 64 * kWaves8;
constexpr int kChunkBlk = 8 * kWaves8;       // activation blocks per staged chunk
constexpr int kRowPad = 17;                  // 16 rows + 1
constexpr int kWbDwords = 68 * kRowPad;      // per wave: 17 pieces (68 dwords) of each of 16 rows
constexpr size_t kZeroUnit = (size_t)kChunkBlk * 8 * 2;  // act unit index of a zero unit
constexpr size_t kDaOff = (kZeroUnit + 1) * 16;
constexpr size_t kWbOff = kDaOff + (size_t)kChunkBlk * 8 * 4;
constexpr size_t kPartOff = kWbOff;  // the partial tiles reuse the weight buffers
constexpr size_t kLds = kWbOff + (size_t)kWaves8 * kWbDwords * 4;
static_assert(kWaves8 * 64 * 16 <= kWaves8 * kWbDwords * 4, "the partial tiles fit in the weight buffers");
static_assert(kLds <= 160 * 1024, "one workgroup per CU");

// W and XQ are not declared __restrict__, as in the Q4_K kernel: the loads
// then stay in the order written around the staging barrier.
template <bool DUMP>
__global__ __launch_bounds__(kThreads8) void gemv_batch_mfma_q8_0(const uint8_t *W, const uint8_t *XQ, float *Y,
                                                                  int32_t *Dd, int nb, int n, int nblk) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  u32x4n *act = reinterpret_cast<u32x4n *>(lds);  // [blk][m][half], 16 bytes
  float *da = reinterpret_cast<float *>(lds + kDaOff);
  uint32_t *wb = reinterpret_cast<uint32_t *>(lds + kWbOff) + (threadIdx.x >> 6) * kWbDwords;
  f32x4n *part = reinterpret_cast<f32x4n *>(lds + kPartOff);

  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int nl = lane & 15, sl = lane >> 4;  // weight row in the tile (B column) / k slice; A row is nl too
  const int tile = (int)blockIdx.x;
  const int64_t rb = (int64_t)nblk * kQ8_0Bytes;
  const int64_t xrb = (int64_t)nblk * kQ8_1Bytes;
  const int nsub = nblk / 8;  // 8-block pieces of a row
  const int nchunk = (nblk + kChunkBlk - 1) / kChunkBlk;
  const v4i izero = {0, 0, 0, 0};

  // this lane's pieces: pc = lane + 64q (the last 48 lanes of q = 4 repeat
  // piece 271), row pc / 17, piece pc % 17; rows past n read row n - 1.
  // Offsets from the tile's first row, k <= 2^24 keeping them in 32 bits.
  uint32_t goff[5];
  {
    const int rowlim = n - 1 - tile * 16;
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      const int pc = min(lane + 64 * q, 271), pr = pc / 17, pp = pc - 17 * pr;
      goff[q] = (uint32_t)(min(pr, rowlim) * (int)rb + 16 * pp);
    }
  }
  const uint8_t *tw = W + (int64_t)tile * 16 * rb;
  u32x4 P[5];
  // the wave's 8 blocks of chunk c (past the row's end: its last 8, never used)
  auto load_w = [&](int c) __attribute__((always_inline)) {
    const uint8_t *p = tw + (int64_t)min(c * kWaves8 + wv, nsub - 1) * 272;
#pragma unroll
    for (int q = 0; q < 5; ++q) P[q] = ld16(p + goff[q]);
  };
  auto put_w = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      const int pc = lane + 64 * q;
      if (pc < 272) {
        const int pr = pc / 17, pp = pc - 17 * pr;
        reinterpret_cast<u32x4n *>(wb)[pp * kRowPad + pr] = u32x4n{P[q].x, P[q].y, P[q].z, P[q].w};
      }
    }
  };

  // Activation staging of chunk c: item t = (row m, block) with its loads first.
  constexpr int kStageIters = (8 * kChunkBlk + kThreads8 - 1) / kThreads8;
  u32x4 sv0[kStageIters], sv1[kStageIters];
  uint32_t sv2[kStageIters];
  auto stage_load = [&](int c) __attribute__((always_inline)) {
    const int b0 = c * kChunkBlk, cb = min(kChunkBlk, nblk - b0), items = nb * cb;
#pragma unroll
    for (int it = 0; it < kStageIters; ++it) {
      const int t = min(tid + it * kThreads8, items - 1);
      const int m = t / cb, blk = t - m * cb;
      const uint8_t *ap = XQ + m * xrb + (int64_t)(b0 + blk) * kQ8_1Bytes;
      sv0[it] = ld16(ap);
      sv1[it] = ld16(ap + 16);
      sv2[it] = ld4(ap + 32);
    }
  };
  auto stage_write = [&](int c) __attribute__((always_inline)) {
    const int b0 = c * kChunkBlk, cb = min(kChunkBlk, nblk - b0), items = nb * cb;
#pragma unroll
    for (int it = 0; it < kStageIters; ++it) {
      const int t = min(tid + it * kThreads8, items - 1);
      const int m = t / cb, blk = t - m * cb;
      const u32x4 v0 = sv0[it], v1 = sv1[it];
      act[(blk * 8 + m) * 2] = u32x4n{v0.y, v0.z, v0.w, v1.x};
      act[(blk * 8 + m) * 2 + 1] = u32x4n{v1.y, v1.z, v1.w, sv2[it]};
      da[blk * 8 + m] = h2f(v0.x);
    }
  };

  f32x4n acc = {0.f, 0.f, 0.f, 0.f};
  // the wave's 8 blocks (chunk-local blocks 8wv .. 8wv + 7) from its buffer
  auto run = [&](int c) __attribute__((always_inline)) {
#pragma unroll
    for (int jp = 0; jp < 4; ++jp) {
      // B: weight row nl, block jj = 2jp + sl/2, k half sl%2
      const int jj = 2 * jp + (sl >> 1);
      const int o = 34 * jj + 2 + 16 * (sl & 1), p0 = o >> 4;
      const u32x4n *wu = reinterpret_cast<const u32x4n *>(wb);
      const u32x4n u0 = wu[p0 * kRowPad + nl], u1 = wu[min(p0 + 1, 16) * kRowPad + nl];
      const uint32_t X[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
      // the byte shift within the two pieces: (4jp + 2) mod 16 for the even
      // block (lanes with sl < 2), (4jp + 4) mod 16 for the odd one
      const int se = (4 * jp + 2) & 15, so = (4 * jp + 4) & 15;
      v4i bv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t ev = align_bytes(X[(se >> 2) + i + 1], X[(se >> 2) + i], 2);
        const uint32_t od = X[(so >> 2) + i];
        bv[i] = (int)((sl >> 1) ? od : ev);
      }
      const uint32_t dword = wb[(((34 * jj) >> 4) * kRowPad + nl) * 4 + (((34 * jj) & 15) >> 2)];
      const float dw = h2f((jj & 1) ? (dword >> 16) : dword);
      // A: row nl = activation row nl % 8 of block 2jp + nl/8, nonzero in
      // the k slices of that block only
      const bool av = (sl >> 1) == (nl >> 3);
      const int ab = 8 * wv + 2 * jp + (nl >> 3);
      const u32x4n a = act[av ? (size_t)((ab * 8 + (nl & 7)) * 2 + (sl & 1)) : kZeroUnit];
      const v4i D = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, a), bv, izero, 0, 0, 0);
      const int bo = 8 * wv + 2 * jp + (lane >> 5);  // this lane's output block (chunk-local)
      const int m0 = 4 * (sl & 1);
      if (DUMP) {
        const int64_t row = (int64_t)tile * 16 + nl;
        const int64_t blk = (int64_t)c * kChunkBlk + bo;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (m0 + r < nb && row < n) Dd[((int64_t)(m0 + r) * n + row) * nblk + blk] = D[r];
      } else {
        const f32x4n a4 = *reinterpret_cast<const f32x4n *>(da + bo * 8 + m0);
        acc.x = fmaf(dw * a4.x, (float)D[0], acc.x);
        acc.y = fmaf(dw * a4.y, (float)D[1], acc.y);
        acc.z = fmaf(dw * a4.z, (float)D[2], acc.z);
        acc.w = fmaf(dw * a4.w, (float)D[3], acc.w);
      }
    }
  };

  if (tid == 0) act[kZeroUnit] = u32x4n{0u, 0u, 0u, 0u};
  for (int c = 0; c < nchunk; ++c) {
    if (c > 0) __syncthreads();  // the previous chunk is no longer read
    stage_load(c);
    asm volatile("" ::: "memory");
    load_w(c);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);  // nothing that waits for the activation moves above the weight loads
    stage_write(c);
    __syncthreads();
    put_w();  // the wave's own buffer: its LDS accesses complete in order
    if (c * kWaves8 + wv < nsub) run(c);
  }
  if (DUMP) return;
  // sum the waves' partial tiles and both block parities: output (m, row
  // nn) is register m%4 of lanes nn + 16(m/4) and nn + 16(m/4) + 32
  __syncthreads();
  part[wv * 64 + lane] = acc;
  __syncthreads();
  if (tid < 16 * nb) {
    const int m = tid >> 4, nn = tid & 15;
    const int64_t r = (int64_t)tile * 16 + nn;
    if (r < n) {
      const int l0 = nn + 16 * (m >> 2);
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves8; ++w) sum += part[w * 64 + l0][m & 3] + part[w * 64 + l0 + 32][m & 3];
      Y[(int64_t)m * n + r] = sum;
    }
  }
}

}  // namespace q8

}  // namespace

hipError_t launch_qgemv_batch_mfma_q4k(const void *w, const void *xq, float *y, int32_t *D, int64_t nb, int64_t n,
                                       int64_t k, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 31) / 32));
  const uint8_t *W = static_cast<const uint8_t *>(w), *X = static_cast<const uint8_t *>(xq);
  if (D)
    hipLaunchKernelGGL(q4::gemv_batch_mfma_q4k<true>, grid, dim3(kThreads), q4::kLds, stream, W, X, y, D, (int)nb,
                       (int)n, (int)(k / 256));
  else
    hipLaunchKernelGGL(q4::gemv_batch_mfma_q4k<false>, grid, dim3(kThreads), q4::kLds, stream, W, X, y, D, (int)nb,
                       (int)n, (int)(k / 256));
  return hipGetLastError();
}

hipError_t launch_qgemv_batch_mfma_q8_0(const void *w, const void *xq, float *y, int32_t *D, int64_t nb, int64_t n,
                                        int64_t k, hipStream_t stream) {
  if (n == 0 || nb == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 15) / 16));
  const uint8_t *W = static_cast<const uint8_t *>(w), *X = static_cast<const uint8_t *>(xq);
  if (D)
    hipLaunchKernelGGL(q8::gemv_batch_mfma_q8_0<true>, grid, dim3(q8::kThreads8), q8::kLds, stream, W, X, y, D,
                       (int)nb, (int)n, (int)(k / 32));
  else
    hipLaunchKernelGGL(q8::gemv_batch_mfma_q8_0<false>, grid, dim3(q8::kThreads8), q8::kLds, stream, W, X, y, D,
                       (int)nb, (int)n, (int)(k / 32));
  return hipGetLastError();
}

hipError_t launch_qgemv_batch_mfma_q6k(const void *w, const void *xq, float *y, int32_t *D, int64_t nb, int64_t n,
                                       int64_t k, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  return nb <= 4 ? q6::launch_bp<4>(w, xq, y, D, nb, n, k, stream) : q6::launch_bp<8>(w, xq, y, D, nb, n, k, stream);
}

}  // namespace qg
