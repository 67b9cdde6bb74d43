// qg_moe.hip -- MoE expert FFN with Q4_K experts (the expert_gateup and down
// calls an MoE decode step spends its time in; infr page, "Per-op device
// profiling" and "Paged experts").
//
// Four kernels on one stream, no host round trip:
//   1. gate/up: work items (touched expert, row tile).  A workgroup finds the
//      (token, slot) pairs routed to its item's expert and runs the Q4_K GEMV
//      rows of its tile against each such token's Q8_1 row (staged in LDS).
//      An expert nobody routed to reads no weights, and a touched expert's
//      weights are streamed once for all of its pairs.
//   2. act: per pair, h = silu(g)*u in fp32, requantized to Q8_1 exactly as
//      quantize_q8_1 does; written as Q8_1 rows and again unit-major with
//      ready {d, code sum} records for kernel 3.
//   3. down: like 1, over the down weights and each pair's h^ (the unit-major
//      copy), scaled by the pair's routing weight.
//   4. combine: out[t] = sum over t's slots in slot order (deterministic).
// Large routing tables take the (expert x tile) grid form of 1 and 3 instead
// of the persistent one, reading the Q8_1 rows.
#include "qg_blocks.h"
#include "qg_launch.h"
#include "qg_quant.h"

namespace qg {

// Kernels 1 and 3.  blockIdx.x = expert * tiles + row tile; each wave covers
// (64/L)*R rows of the expert's [rows][nsb] matrix, a lane the units
// li, li + L, ... (UPL of them; lanes with nothing to do stay idle).  The
// routing table is scanned 64 ids per vector load + ballot.  If any pair is
// routed to the expert, the lane loads its weight units for all R rows into
// VGPRs once; then, for every pair p with ids[p] == expert,
//   out[p][row] = scale(p) * dot(row, act + act_row(p))
// with act_row(p) = p / top_k (token rows, kernel 1) or p (h^ rows, kernel 3),
// scale(p) = 1 (kernel 1) or weights[p] (kernel 3).  An expert nobody routed
// to reads no weights; a touched expert's weights are read once.
template <int L, int R, int UPL>
__global__ __launch_bounds__(256) void moe_expert_gemv_kernel(const uint8_t *__restrict__ W,
                                                              const uint8_t *__restrict__ act,
                                                              const int32_t *__restrict__ ids,
                                                              const float *__restrict__ weights,
                                                              float *__restrict__ out, int rows, int nsb,
                                                              int npairs, int top_k, int act_per_token,
                                                              int64_t expert_bytes, int64_t act_row_bytes,
                                                              int tiles) {
  constexpr int G = 64 / L;
  const int e = (int)(blockIdx.x / (unsigned)tiles);
  const int tile = (int)(blockIdx.x % (unsigned)tiles);
  const int lane = threadIdx.x & 63;
  const int li = lane & (L - 1);
  const int row0 = ((tile * 4 + (threadIdx.x >> 6)) * G + lane / L) * R;
  const int64_t rb = (int64_t)nsb * kQ4KBytes;
  const uint8_t *wexp = W + (int64_t)e * expert_bytes;
  const int U = nsb * 4;

  constexpr int NV = UPL > 0 ? UPL : 1;
  bool loaded = false;
  u32x4 hdr[NV][R], qa[NV][R], qb[NV][R];
  for (int c0 = 0; c0 < npairs; c0 += 64) {
    const int id = c0 + lane < npairs ? ids[c0 + lane] : -1;
    uint64_t mask = __ballot(id == e);
    if (UPL > 0 && mask && !loaded) {
      loaded = true;
#pragma unroll
      for (int v = 0; v < UPL; ++v) {
        const int u = li + v * L;
        const int sb = u >> 2, g = u & 3;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (u < U && row0 + r < rows) {
            const uint8_t *bp = wexp + (int64_t)(row0 + r) * rb + (int64_t)sb * kQ4KBytes;
            hdr[v][r] = ld16(bp);
            qa[v][r] = ld16(bp + 16 + 32 * g);
            qb[v][r] = ld16(bp + 32 + 32 * g);
          } else {
            hdr[v][r] = qa[v][r] = qb[v][r] = u32x4{0u, 0u, 0u, 0u};
          }
        }
      }
    }
    while (mask) {
      const int p = c0 + __builtin_ctzll(mask);
      mask &= mask - 1;
      const uint8_t *xr = act + (int64_t)(act_per_token ? p / top_k : p) * act_row_bytes;
      float acc[R];
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = 0.f;
      // UPL > 0: the lane's UPL units were loaded above; UPL == 0: walk the
      // row's units with stride L, loading each unit's weights here
      const int nv = UPL > 0 ? UPL : (U - li + L - 1) / L;
      // fully unrolled when the count is the constant UPL; a plain loop for long rows
      constexpr int kUnroll = UPL > 0 ? UPL : 1;
#pragma unroll kUnroll
      for (int v = 0; v < nv; ++v) {
        const int u = li + v * L;
        if (u < U) {
          const int sb = u >> 2, g = u & 3;
          if (UPL == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
              if (row0 + r < rows) {
                const uint8_t *bp = wexp + (int64_t)(row0 + r) * rb + (int64_t)sb * kQ4KBytes;
                hdr[0][r] = ld16(bp);
                qa[0][r] = ld16(bp + 16 + 32 * g);
                qb[0][r] = ld16(bp + 32 + 32 * g);
              } else {
                hdr[0][r] = qa[0][r] = qb[0][r] = u32x4{0u, 0u, 0u, 0u};
              }
            }
          }
          const int vi = UPL > 0 ? v : 0;
          uint32_t A[18];
          load_q8_1_pair(xr + (int64_t)(8 * sb + 2 * g) * kQ8_1Bytes, A);
          int S0 = 0, S1 = 0;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            S0 = bsum4(A[1 + i], S0);
            S1 = bsum4(A[10 + i], S1);
          }
          const float da0 = h2f(A[0]), da1 = h2f(A[9]);
          const float dS0 = da0 * (float)S0, dS1 = da1 * (float)S1;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const uint32_t Q[8] = {qa[vi][r].x, qa[vi][r].y, qa[vi][r].z, qa[vi][r].w,
                                   qb[vi][r].x, qb[vi][r].y, qb[vi][r].z, qb[vi][r].w};
            int D0 = 0, D1 = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              D0 = dot4(Q[i] & 0x0F0F0F0Fu, A[1 + i], D0);
              D1 = dot4((Q[i] >> 4) & 0x0F0F0F0Fu, A[10 + i], D1);
            }
            int sc0, sc1, m0, m1;
            q4k_scales(hdr[vi][r].y, hdr[vi][r].z, hdr[vi][r].w, g, sc0, sc1, m0, m1);
            const float d = h2f(hdr[vi][r].x), dmin = h2f(hdr[vi][r].x >> 16);
            acc[r] += d * (da0 * (float)(sc0 * D0) + da1 * (float)(sc1 * D1)) -
                      dmin * (dS0 * (float)m0 + dS1 * (float)m1);
          }
        }
      }
      const float scale = weights ? weights[p] : 1.0f;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float v = group_sum_last<L>(acc[r]);
        if (li == L - 1 && row0 + r < rows) out[(int64_t)p * rows + row0 + r] = scale * v;
      }
    }
  }
}

// Persistent form of kernels 1 and 3 for small routing tables (npairs <=
// 64*kMaxIdWords, n_expert <= 64*kMaxExpertWords).  Every wave loads the whole
// routing table into VGPRs once and builds the bitmap of touched experts with
// ballots; the workgroups then stride over the work items (touched expert x
// row tile) only, so an untouched expert costs nothing and every resident
// workgroup is streaming some expert's weights.  Per item the pairs routed to
// the expert come from ballots over the ids already in registers.
constexpr int kMaxIdWords = 4;      // up to 256 (token, slot) pairs
constexpr int kMaxExpertWords = 4;  // up to 256 experts
static_assert(kMaxIdWords == kMaxExpertWords, "one word count serves both");

//
// Item bookkeeping stays off the scalar unit's critical path: the expert of an
// item comes from per-lane ranks of the touched experts (one compare and ballot
// per bitmap word), the item's (expert, tile) pair advances by the grid size
// without dividing, and the token row of a pair is read from a VGPR with
// v_readlane.  Bit scans and divisions per item and per pair had cost each wave
// about as many scalar as vector instructions.
//
// With UMX (the down call) `act` holds the activation rows in that same
// unit-major layout in global memory (written by the act kernel), so the pair
// loop loads aligned 16-byte pieces and ready code sums instead of Q8_1 blocks.
//
// With STAGE (the gate/up call when the token rows fit in LDS) the workgroup
// first stages every activation row, unit-major: piece c of unit u of row t at
// slot t*5U + c*U + u (16 bytes: half c%2 of block 2u + c/2), and the record
// {d_a(2u), d_a(2u+1), sum qa(2u), sum qa(2u+1)} at slot t*5U + 4U + u.  The
// pair loop then reads its activation from LDS instead of L2.
template <int L, int R, bool STAGE, int NT, int WPE, bool UMX, int NW>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(WPE))) void moe_expert_gemv_persistent(
    const uint8_t *__restrict__ W, const uint8_t *__restrict__ act, const int32_t *__restrict__ ids,
    const float *__restrict__ weights, float *__restrict__ out, int rows, int nsb, int npairs, int top_k,
    int act_per_token, int64_t expert_bytes, int64_t act_row_bytes, int tiles, int n_expert, int n_act) {
  typedef uint32_t u32x4n __attribute__((ext_vector_type(4)));
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  u32x4n *xs = reinterpret_cast<u32x4n *>(lds);
  constexpr int G = 64 / L;
  const int lane = threadIdx.x & 63;
  const int li = lane & (L - 1);
  const int64_t rb = (int64_t)nsb * kQ4KBytes;
  const int U = nsb * 4;
  // routing table in registers: id[w] = ids[64w + lane]
  int id[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int p = 64 * w + lane;
    id[w] = p < npairs ? ids[p] : -1;
  }
  // touched[x] bit b  <=>  expert 64x + b has a pair: each lane sets the bits
  // of its ids, then a butterfly ORs the words over the wave
  uint64_t touched[NW];
#pragma unroll
  for (int x = 0; x < NW; ++x) touched[x] = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int e = id[w];
    const bool ok = e >= 0 && e < n_expert;
#pragma unroll
    for (int x = 0; x < NW; ++x)
      if (ok && (e >> 6) == x) touched[x] |= 1ull << (e & 63);
  }
#pragma unroll
  for (int x = 0; x < NW; ++x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) touched[x] |= __shfl_xor(touched[x], off, 64);
    // the same in every lane now: keep it in scalar registers
    touched[x] = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(touched[x] >> 32)) << 32) |
                 (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)touched[x]);
  }
  // rank[x] = position of expert 64x + lane among the touched experts, or -1
  // if it is untouched; the expert at position k is then the one lane whose
  // rank equals k (one compare and ballot per word)
  int rank[NW];
  int active = 0;
#pragma unroll
  for (int x = 0; x < NW; ++x) {
    const uint64_t t = touched[x];
    const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(t >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)t, 0u));
    rank[x] = ((t >> lane) & 1) ? active + below : -1;
    active += __builtin_popcountll(t);
  }
  const int items = active * tiles;
  // token row of pair 64w + lane (the activation row of the staged form)
  int tok[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) tok[w] = STAGE ? (64 * w + lane) / top_k : 0;

  const int u = li;  // this lane's unit (L >= U here, so at most one)
  const int sb = u >> 2, g = u & 3;
  if constexpr (STAGE) {
    for (int t = threadIdx.x; t < n_act * U; t += NT) {
      const int row = t / U, uu = t - row * U;
      uint32_t A[18];
      load_q8_1_pair(act + (int64_t)row * act_row_bytes + (int64_t)(2 * uu) * kQ8_1Bytes, A);
      int S0 = 0, S1 = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        S0 = bsum4(A[1 + i], S0);
        S1 = bsum4(A[10 + i], S1);
      }
      u32x4n *base = xs + row * 5 * U;
      base[uu] = u32x4n{A[1], A[2], A[3], A[4]};
      base[U + uu] = u32x4n{A[5], A[6], A[7], A[8]};
      base[2 * U + uu] = u32x4n{A[10], A[11], A[12], A[13]};
      base[3 * U + uu] = u32x4n{A[14], A[15], A[16], A[17]};
      base[4 * U + uu] = u32x4n{__builtin_bit_cast(uint32_t, h2f(A[0])), __builtin_bit_cast(uint32_t, h2f(A[9])),
                                (uint32_t)S0, (uint32_t)S1};
    }
    __syncthreads();
  }
  // item = k * tiles + t, advanced by the grid size without dividing
  const int kstep = (int)gridDim.x / tiles, tstep = (int)gridDim.x - kstep * tiles;
  int ik = (int)blockIdx.x / tiles, it = (int)blockIdx.x - ik * tiles;
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    int e = -1;
#pragma unroll
    for (int x = 0; x < NW; ++x) {
      const uint64_t m = __ballot(rank[x] == ik);
      if (m) e = 64 * x + __builtin_ctzll(m);
    }
    const int row0 = ((it * (NT / 64) + (threadIdx.x >> 6)) * G + lane / L) * R;
    ik += kstep;
    it += tstep;
    if (it >= tiles) {
      it -= tiles;
      ++ik;
    }
    const uint8_t *wu = W + (int64_t)e * expert_bytes + (int64_t)row0 * rb + sb * kQ4KBytes;
    u32x4 hdr[R], qa[R], qb[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (u < U && row0 + r < rows) {
        const uint8_t *bp = wu + r * rb;
        hdr[r] = ld16(bp);
        qa[r] = ld16(bp + 16 + 32 * g);
        qb[r] = ld16(bp + 32 + 32 * g);
      } else {
        hdr[r] = qa[r] = qb[r] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      uint64_t mask = __ballot(id[w] == e);
      while (mask) {
        const int p = 64 * w + __builtin_ctzll(mask);
        mask &= mask - 1;
        const int arow = STAGE ? __builtin_amdgcn_readlane(tok[w], p - 64 * w) : act_per_token ? p / top_k : p;
        const uint8_t *xr = act + (int64_t)arow * act_row_bytes;
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0.f;
        if (u < U) {
          uint32_t A[18];
          int S0 = 0, S1 = 0;
          float da0, da1;
          if constexpr (STAGE || UMX) {
            // the unit-major row: staged in LDS, or (UMX) in global memory
            const u32x4n *base =
                (STAGE ? xs : reinterpret_cast<const u32x4n *>(act)) + (int64_t)arow * 5 * U;
            const u32x4n x0 = base[u], x1 = base[U + u], x2 = base[2 * U + u], x3 = base[3 * U + u];
            const u32x4n rec = base[4 * U + u];
            A[1] = x0.x; A[2] = x0.y; A[3] = x0.z; A[4] = x0.w;
            A[5] = x1.x; A[6] = x1.y; A[7] = x1.z; A[8] = x1.w;
            A[10] = x2.x; A[11] = x2.y; A[12] = x2.z; A[13] = x2.w;
            A[14] = x3.x; A[15] = x3.y; A[16] = x3.z; A[17] = x3.w;
            da0 = as_f32(rec.x);
            da1 = as_f32(rec.y);
            S0 = (int)rec.z;
            S1 = (int)rec.w;
          } else {
            load_q8_1_pair(xr + (int64_t)(8 * sb + 2 * g) * kQ8_1Bytes, A);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              S0 = bsum4(A[1 + i], S0);
              S1 = bsum4(A[10 + i], S1);
            }
            da0 = h2f(A[0]);
            da1 = h2f(A[9]);
          }
          const float dS0 = da0 * (float)S0, dS1 = da1 * (float)S1;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const uint32_t Q[8] = {qa[r].x, qa[r].y, qa[r].z, qa[r].w, qb[r].x, qb[r].y, qb[r].z, qb[r].w};
            int D0 = 0, D1 = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              D0 = dot4(Q[i] & 0x0F0F0F0Fu, A[1 + i], D0);
              D1 = dot4((Q[i] >> 4) & 0x0F0F0F0Fu, A[10 + i], D1);
            }
            int sc0, sc1, m0, m1;
            q4k_scales(hdr[r].y, hdr[r].z, hdr[r].w, g, sc0, sc1, m0, m1);
            const float d = h2f(hdr[r].x), dmin = h2f(hdr[r].x >> 16);
            acc[r] += d * (da0 * (float)(sc0 * D0) + da1 * (float)(sc1 * D1)) -
                      dmin * (dS0 * (float)m0 + dS1 * (float)m1);
          }
        }
        const float scale = weights ? weights[p] : 1.0f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float v = group_sum_last<L>(acc[r]);
          if (li == L - 1 && row0 + r < rows) out[(int64_t)p * rows + row0 + r] = scale * v;
        }
      }
    }
  }
}

// Kernel 2: h = silu(g) * u per pair, requantized to Q8_1.  One 8-lane group
// per 32-value block of h; pairs with an out-of-range id are skipped.  The
// block also goes to hx in the unit-major layout the staged gate/up kernel
// keeps in LDS (unit = blocks 2u, 2u+1: pieces c = 0..3 of 16 bytes, then the
// record {d(2u), d(2u+1), sum(2u), sum(2u+1)}), which the down GEMV reads.
__global__ __launch_bounds__(256) void moe_act_quant_kernel(const float *__restrict__ gu,
                                                            const int32_t *__restrict__ ids,
                                                            uint8_t *__restrict__ hq, uint8_t *__restrict__ hx,
                                                            int npairs, int n_ff, int n_expert) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int nbp = n_ff / 32, U = n_ff / 64;
  const int64_t b = t >> 3;
  const int j = (int)(t & 7);
  const int p = (int)(b / nbp), bi = (int)(b % nbp);
  bool live = false;
  if (p < npairs) {
    const int e = ids[p];
    live = e >= 0 && e < n_expert;
  }
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (live) {
    const float *g = gu + (int64_t)p * 2 * n_ff + bi * 32 + 4 * j;
    const float *u = g + n_ff;
    const float4 g4 = *reinterpret_cast<const float4 *>(g);
    const float4 u4 = *reinterpret_cast<const float4 *>(u);
    v.x = g4.x / (1.0f + expf(-g4.x)) * u4.x;
    v.y = g4.y / (1.0f + expf(-g4.y)) * u4.y;
    v.z = g4.z / (1.0f + expf(-g4.z)) * u4.z;
    v.w = g4.w / (1.0f + expf(-g4.w)) * u4.w;
  }
  const Q81Part q = quantize_part_q8_1(v);
  if (live) {
    uint8_t *blk = hq + ((int64_t)p * nbp + bi) * kQ8_1Bytes;
    const uint32_t hdr = q81_header(q);
    *reinterpret_cast<uint32_t *>(blk + 4 + 4 * j) = q.packed;
    if (j == 0) *reinterpret_cast<uint32_t *>(blk) = hdr;
    uint32_t *row = reinterpret_cast<uint32_t *>(hx + (int64_t)p * U * 80);
    const int uu = bi >> 1, bb = bi & 1;
    row[4 * ((2 * bb + (j >> 2)) * U + uu) + (j & 3)] = q.packed;
    if (j == 0) {
      row[4 * (4 * U + uu) + bb] = __builtin_bit_cast(uint32_t, h2f(hdr));
      row[4 * (4 * U + uu) + 2 + bb] = (uint32_t)q.sum;
    }
  }
}

// Kernel 4: out[t][i] = sum over slots s (in order) of z[t*top_k + s][i].
__global__ __launch_bounds__(256) void moe_combine_kernel(const float *__restrict__ z, const int32_t *__restrict__ ids,
                                                          float *__restrict__ out, int n_tok, int top_k, int n_embd,
                                                          int n_expert) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)n_tok * n_embd) return;
  const int t = (int)(i / n_embd), c = (int)(i % n_embd);
  float acc = 0.f;
  for (int s = 0; s < top_k; ++s) {
    const int p = t * top_k + s;
    const int e = ids[p];
    if (e >= 0 && e < n_expert) acc += z[(int64_t)p * n_embd + c];
  }
  out[i] = acc;
}

template <int L, int R, int UPL>
static void launch_expert_gemv(const uint8_t *W, const uint8_t *act, const int32_t *ids, const float *weights,
                               float *out, int rows, int nsb, int npairs, int top_k, int act_per_token,
                               int64_t expert_bytes, int64_t act_row_bytes, int n_expert, hipStream_t stream) {
  const int rows_per_block = 4 * (64 / L) * R;
  const int tiles = (rows + rows_per_block - 1) / rows_per_block;
  const dim3 grid((unsigned)((int64_t)tiles * n_expert));
  hipLaunchKernelGGL((moe_expert_gemv_kernel<L, R, UPL>), grid, dim3(256), 0, stream, W, act, ids, weights, out,
                     rows, nsb, npairs, top_k, act_per_token, expert_bytes, act_row_bytes, tiles);
}

// Rows per lane group of the grid-form expert GEMV.
constexpr int kMoeRows = 2;

// Lanes per row: the smallest power of two >= the row's unit count, capped at
// 64 (lanes past the last unit idle); each lane then keeps ceil(U/L) units'
// weights for R rows in VGPRs (up to two units; longer rows reload per pair).
// LDS for staging all activation rows of a gate/up call: 5 x 16 bytes per unit
// of each row.  Up to this much, four workgroups still fit on a CU.
constexpr size_t kMoeStageBytes = 40 * 1024;

// Launch shape of the persistent expert GEMV: workgroup size, rows per lane
// group, and the waves per SIMD its register allocation must leave room for.
// The staged gate/up call runs 8-wave workgroups, two per CU: 16 waves, as
// with four 4-wave ones, but each CU stages the token rows twice, not four
// times.  The down call runs four waves per SIMD (held to the 96 VGPRs of
// five it spills) and three rows per lane group.  The grid is the number of
// workgroups resident at once.
constexpr int kGuThreads = 512, kGuRows = 2, kGuWaves = 4;
constexpr int kDnThreads = 256, kDnRows = 3, kDnWaves = 4;

template <int L, int R, bool STAGE, int NT, int WPE, bool UMX, int NW>
static void launch_persistent_shape(const uint8_t *W, const uint8_t *act, const int32_t *ids, const float *weights,
                                    float *out, int rows, int nsb, int npairs, int top_k, int act_per_token,
                                    int64_t expert_bytes, int64_t act_row_bytes, int n_expert, int n_act,
                                    size_t stage, hipStream_t stream) {
  constexpr auto kern = moe_expert_gemv_persistent<L, R, STAGE, NT, WPE, UMX, NW>;
  const int rows_per_block = (NT / 64) * (64 / L) * R;
  const int tiles = (rows + rows_per_block - 1) / rows_per_block;
  const int64_t max_items = (int64_t)tiles * n_expert;
  const int64_t resident = resident_blocks<kern>(NT, stage);
  const dim3 grid((unsigned)(max_items < resident ? max_items : resident));
  hipLaunchKernelGGL(kern, grid, dim3(NT), stage, stream, W, act, ids, weights, out, rows, nsb, npairs, top_k,
                     act_per_token, expert_bytes, act_row_bytes, tiles, n_expert, n_act);
}

// act_um (nullable): the activation rows in the unit-major layout, used
// instead of the Q8_1 rows by the unstaged form.
template <int L, int NW>
static void launch_expert_gemv_persistent_nw(const uint8_t *W, const uint8_t *act, const uint8_t *act_um,
                                          const int32_t *ids, const float *weights, float *out, int rows, int nsb,
                                          int npairs, int top_k, int act_per_token, int64_t expert_bytes,
                                          int64_t act_row_bytes, int n_expert, hipStream_t stream) {
  const int n_act = act_per_token ? (npairs + top_k - 1) / top_k : npairs;
  const size_t stage = (size_t)n_act * nsb * 4 * 80;
  if (act_per_token && stage <= kMoeStageBytes)
    launch_persistent_shape<L, kGuRows, true, kGuThreads, kGuWaves, false, NW>(
        W, act, ids, weights, out, rows, nsb, npairs, top_k, act_per_token, expert_bytes, act_row_bytes, n_expert,
        n_act, stage, stream);
  else if (act_um)
    launch_persistent_shape<L, kDnRows, false, kDnThreads, kDnWaves, true, NW>(
        W, act_um, ids, weights, out, rows, nsb, npairs, top_k, act_per_token, expert_bytes, (int64_t)nsb * 4 * 80,
        n_expert, n_act, 0, stream);
  else
    launch_persistent_shape<L, kDnRows, false, kDnThreads, kDnWaves, false, NW>(
        W, act, ids, weights, out, rows, nsb, npairs, top_k, act_per_token, expert_bytes, act_row_bytes, n_expert,
        n_act, 0, stream);
}

// Routing tables of up to 128 pairs over up to 128 experts keep two words of
// ids and of the touched-expert bitmap per lane instead of four: four VGPRs
// fewer, which the down call needs to hold five waves per SIMD without spills.
template <int L>
static void launch_expert_gemv_persistent(const uint8_t *W, const uint8_t *act, const uint8_t *act_um,
                                          const int32_t *ids, const float *weights, float *out, int rows, int nsb,
                                          int npairs, int top_k, int act_per_token, int64_t expert_bytes,
                                          int64_t act_row_bytes, int n_expert, hipStream_t stream) {
  if (npairs <= 128 && n_expert <= 128)
    launch_expert_gemv_persistent_nw<L, 2>(W, act, act_um, ids, weights, out, rows, nsb, npairs, top_k,
                                           act_per_token, expert_bytes, act_row_bytes, n_expert, stream);
  else
    launch_expert_gemv_persistent_nw<L, kMaxIdWords>(W, act, act_um, ids, weights, out, rows, nsb, npairs, top_k,
                                                     act_per_token, expert_bytes, act_row_bytes, n_expert, stream);
}

static void expert_gemv(const uint8_t *W, const uint8_t *act, const uint8_t *act_um, const int32_t *ids,
                        const float *weights, float *out, int rows, int nsb, int npairs, int top_k,
                        int act_per_token, int64_t act_row_bytes, int n_expert, hipStream_t stream) {
  const int64_t expert_bytes = (int64_t)rows * nsb * kQ4KBytes;
  const int U = nsb * 4;
  int L = 4;
  while (L < U && L < 64) L <<= 1;
  const int upl = (U + L - 1) / L;
  if (upl == 1 && npairs <= 64 * kMaxIdWords && n_expert <= 64 * kMaxExpertWords) {
#define QG_MOE_PERSIST(LV)                                                                                        \
  launch_expert_gemv_persistent<LV>(W, act, act_um, ids, weights, out, rows, nsb, npairs, top_k, act_per_token, \
                                              expert_bytes, act_row_bytes, n_expert, stream)
    if (L == 4) QG_MOE_PERSIST(4);
    else if (L == 8) QG_MOE_PERSIST(8);
    else if (L == 16) QG_MOE_PERSIST(16);
    else if (L == 32) QG_MOE_PERSIST(32);
    else QG_MOE_PERSIST(64);
#undef QG_MOE_PERSIST
    return;
  }
#define QG_MOE_LAUNCH(LV, RV, UV)                                                                                 \
  launch_expert_gemv<LV, RV, UV>(W, act, ids, weights, out, rows, nsb, npairs, top_k, act_per_token,             \
                                 expert_bytes, act_row_bytes, n_expert, stream)
  if (L == 4) QG_MOE_LAUNCH(4, kMoeRows, 1);
  else if (L == 8) QG_MOE_LAUNCH(8, kMoeRows, 1);
  else if (L == 16) QG_MOE_LAUNCH(16, kMoeRows, 1);
  else if (L == 32) QG_MOE_LAUNCH(32, kMoeRows, 1);
  else if (upl == 1) QG_MOE_LAUNCH(64, kMoeRows, 1);
  else if (upl == 2) QG_MOE_LAUNCH(64, 2, 2);
  else QG_MOE_LAUNCH(64, 1, 0);  // long rows: weights reloaded per pair
#undef QG_MOE_LAUNCH
}

MoeLayout moe_layout(int64_t n_tok, int64_t top_k, int64_t n_ff, int64_t n_embd) {
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  const size_t P = (size_t)(n_tok * top_k);
  MoeLayout l;
  l.hq_off = 0;
  l.gu_off = up(P * (size_t)(n_ff / 32) * kQ8_1Bytes);
  l.z_off = l.gu_off + up(P * (size_t)(2 * n_ff) * sizeof(float));
  l.hx_off = l.z_off + up(P * (size_t)n_embd * sizeof(float));
  l.total = l.hx_off + up(P * (size_t)(n_ff / 64) * 80);
  return l;
}

hipError_t launch_moe_q4_k(const MoeArgs &a, hipStream_t stream) {
  const int P = (int)(a.n_tok * a.top_k);
  const int F = (int)a.n_ff, H = (int)a.n_embd, E = (int)a.n_expert, K = (int)a.top_k;
  // 1. gate|up rows [2F] of each touched expert against token rows of xq
  expert_gemv(static_cast<const uint8_t *>(a.w_gu), static_cast<const uint8_t *>(a.xq), nullptr, a.ids, nullptr, a.ws_gu,
              2 * F, H / 256, P, K, 1, (int64_t)(H / 32) * kQ8_1Bytes, E, stream);
  // 2. h^ = Q8_1(silu(g) * u)
  {
    const int64_t threads = (int64_t)P * (F / 32) * 8;
    hipLaunchKernelGGL(moe_act_quant_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a.ws_gu,
                       a.ids, a.ws_hq, a.ws_hx, P, F, E);
  }
  // 3. z[p] = weights[p] * (Wdown[e] . h^[p])
  expert_gemv(static_cast<const uint8_t *>(a.w_down), a.ws_hq, a.ws_hx, a.ids, a.weights, a.ws_z, H, F / 256, P, K, 0,
              (int64_t)(F / 32) * kQ8_1Bytes, E, stream);
  // 4. out[t] = sum of its slots
  {
    const int64_t total = (int64_t)a.n_tok * H;
    if (total > 0)
      hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, a.ws_z,
                         a.ids, a.out, (int)a.n_tok, K, H, E);
  }
  return hipGetLastError();
}

}  // namespace qg
