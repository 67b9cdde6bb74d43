// qg_moe.hip -- MoE expert FFN with Q4_K experts (the expert_gateup and down
// calls an MoE decode step spends its time in; infr page, "Per-op device
// profiling" and "Paged experts").
//
// Two kernels on one stream when the routing table is small (<= 256 pairs
// over <= 256 experts), the token rows are <= 4096 wide and the down rows
// split evenly over lane groups:
//   1. gate/up: work items (touched expert, row tile).  A workgroup finds the
//      (token, slot) pairs routed to its item's expert and runs the Q4_K GEMV
//      rows of its tile against each such token's Q8_1 row (staged in LDS).
//      An expert nobody routed to reads no weights, and a touched expert's
//      weights are streamed once for all of its pairs.  Writes g|u per pair.
//   2. down, token-major: a workgroup per (token, row tile) forms h = silu(g)
//      * u of the token's slots, quantizes it to Q8_1 in LDS (the rule of
//      quantize_q8_1), and sums weights[p] * (Wdown[e] . h^_p) over the slots
//      in slot order straight into out: no combine step, no cross-workgroup
//      traffic, deterministic.  An expert row tile is read once per token
//      routed to it, the repeats from cache.
// Larger tables, and down rows that do not split evenly, take four kernels:
// the (expert x tile) grid form or the persistent form of the expert GEMV for
// gate/up and for down, with the activation step and the combine as kernels
// of their own.
//
// Every expert GEMV has a DUMP instance that writes the exact per-block int32
// dots instead of its outputs, for the tests.
#include "qg_blocks.h"
#include "qg_launch.h"
#include "qg_quant.h"

namespace qg {

typedef uint32_t u32x4n __attribute__((ext_vector_type(4)));  // 16-byte aligned: ds_read/write_b128

// R rows of one lane unit (64 weights: superblock sb, group g) of a Q4_K row
// against one activation unit: A[1..8] / A[10..17] the qs of Q8_1 blocks 2u
// and 2u + 1, da0/da1 their d, dS0/dS1 their d times their code sum (formed
// once per activation unit, for the min term).  D0/D1 are the exact block dots
// of each row.
struct ActUnit {
  uint32_t A[18];
  float da0, da1;
  float dS0, dS1;
};

__device__ __forceinline__ void unit_dots(const u32x4 &qa, const u32x4 &qb, const ActUnit &x, int &D0, int &D1) {
  const uint32_t Q[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
  D0 = 0;
  D1 = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    D0 = dot4(Q[i] & 0x0F0F0F0Fu, x.A[1 + i], D0);
    D1 = dot4((Q[i] >> 4) & 0x0F0F0F0Fu, x.A[10 + i], D1);
  }
}

__device__ __forceinline__ float unit_value(const u32x4 &hdr, int g, const ActUnit &x, int D0, int D1) {
  int sc0, sc1, m0, m1;
  q4k_scales(hdr.y, hdr.z, hdr.w, g, sc0, sc1, m0, m1);
  const float d = h2f(hdr.x), dmin = h2f(hdr.x >> 16);
  return d * (x.da0 * (float)(sc0 * D0) + x.da1 * (float)(sc1 * D1)) - dmin * (x.dS0 * (float)m0 + x.dS1 * (float)m1);
}

// Activation unit from Q8_1 blocks 2u, 2u + 1 at p.
__device__ __forceinline__ void act_from_q8_1(const uint8_t *p, ActUnit &x) {
  load_q8_1_pair(p, x.A);
  int S0 = 0, S1 = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    S0 = bsum4(x.A[1 + i], S0);
    S1 = bsum4(x.A[10 + i], S1);
  }
  x.da0 = h2f(x.A[0]);
  x.da1 = h2f(x.A[9]);
  x.dS0 = x.da0 * (float)S0;
  x.dS1 = x.da1 * (float)S1;
}

// Activation unit u from a unit-major row of U units at base: piece c of unit
// u at base[c*U + u] (16 bytes: half c%2 of block 2u + c/2), the record
// {d(2u), d(2u+1), d*sum(2u), d*sum(2u+1)} at base[4U + u] (sum: the block's code sum).
__device__ __forceinline__ void act_from_unit_major(const u32x4n *base, int U, int u, ActUnit &x) {
  const u32x4n x0 = base[u], x1 = base[U + u], x2 = base[2 * U + u], x3 = base[3 * U + u];
  const u32x4n rec = base[4 * U + u];
  x.A[1] = x0.x; x.A[2] = x0.y; x.A[3] = x0.z; x.A[4] = x0.w;
  x.A[5] = x1.x; x.A[6] = x1.y; x.A[7] = x1.z; x.A[8] = x1.w;
  x.A[10] = x2.x; x.A[11] = x2.y; x.A[12] = x2.z; x.A[13] = x2.w;
  x.A[14] = x3.x; x.A[15] = x3.y; x.A[16] = x3.z; x.A[17] = x3.w;
  x.da0 = as_f32(rec.x);
  x.da1 = as_f32(rec.y);
  x.dS0 = as_f32(rec.z);
  x.dS1 = as_f32(rec.w);
}

// Writes the two block dots of unit u (blocks 2u, 2u + 1) of row `row` of
// pair p into a dump [P][rows][U*2].
__device__ __forceinline__ void dump_unit(int32_t *Dd, int p, int rows, int row, int U, int u, int D0, int D1) {
  int32_t *dp = Dd + ((int64_t)p * rows + row) * (2 * U) + 2 * u;
  dp[0] = D0;
  dp[1] = D1;
}

// ------------------------------------------------------------------------
// Grid form of the expert GEMV.  blockIdx.x = expert * tiles + row tile; each
// wave covers (64/L)*R rows of the expert's [rows][nsb] matrix, a lane the
// units li, li + L, ... (UPL of them; lanes with nothing to do stay idle).
// The routing table is scanned 64 ids per vector load + ballot.  If any pair
// is routed to the expert, the lane loads its weight units for all R rows into
// VGPRs once; then, for every pair p with ids[p] == expert,
//   out[p][row] = scale(p) * dot(row, act + act_row(p))
// with act_row(p) = p / top_k (token rows, gate/up) or p (h^ rows, down),
// scale(p) = 1 (gate/up) or weights[p] (down).
template <int L, int R, int UPL, bool DUMP>
__global__ __launch_bounds__(256) void moe_expert_gemv_kernel(const uint8_t *__restrict__ W,
                                                              const uint8_t *__restrict__ act,
                                                              const int32_t *__restrict__ ids,
                                                              const float *__restrict__ weights,
                                                              float *__restrict__ out, int32_t *__restrict__ Dd,
                                                              int rows, int nsb, int npairs, int top_k,
                                                              int act_per_token, int64_t expert_bytes,
                                                              int64_t act_row_bytes, int tiles) {
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
          const int g = u & 3;
          if (UPL == 0) {
            const int sb = u >> 2;
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
          ActUnit x;
          act_from_q8_1(xr + (int64_t)(2 * u) * kQ8_1Bytes, x);
#pragma unroll
          for (int r = 0; r < R; ++r) {
            int D0, D1;
            unit_dots(qa[vi][r], qb[vi][r], x, D0, D1);
            if (DUMP) {
              if (row0 + r < rows) dump_unit(Dd, p, rows, row0 + r, U, u, D0, D1);
            } else {
              acc[r] += unit_value(hdr[vi][r], g, x, D0, D1);
            }
          }
        }
      }
      if (!DUMP) {
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

// ------------------------------------------------------------------------
// Routing state of the persistent kernels for small tables (npairs <=
// 64*NW, n_expert <= 64*NW).  Every wave loads the whole routing table into
// VGPRs once and builds the bitmap of touched experts with ballots; the
// workgroups then stride over the work items (touched expert x row tile)
// only, so an untouched expert costs nothing.
//
// Item bookkeeping stays off the scalar unit's critical path: the expert of an
// item comes from per-lane ranks of the touched experts (one compare and
// ballot per bitmap word), the item's (expert, tile) pair advances by the grid
// size without dividing.  Bit scans and divisions per item had cost each wave
// about as many scalar as vector instructions.
constexpr int kMaxIdWords = 4;  // up to 256 (token, slot) pairs and 256 experts

template <int NW>
struct Routing {
  int id[NW];    // ids[64w + lane], -1 past the table
  int rank[NW];  // rank of expert 64x + lane among the touched experts, -1 if untouched
  int active;    // touched experts
};

template <int NW>
__device__ __forceinline__ void load_routing(Routing<NW> &rt, const int32_t *__restrict__ ids, int npairs,
                                             int n_expert) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int p = 64 * w + lane;
    rt.id[w] = p < npairs ? ids[p] : -1;
  }
  // touched[x] bit b  <=>  expert 64x + b has a pair: each lane sets the bits
  // of its ids, then a butterfly ORs the words over the wave
  uint64_t touched[NW];
#pragma unroll
  for (int x = 0; x < NW; ++x) touched[x] = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int e = rt.id[w];
    const bool ok = e >= 0 && e < n_expert;
#pragma unroll
    for (int x = 0; x < NW; ++x)
      if (ok && (e >> 6) == x) touched[x] |= 1ull << (e & 63);
  }
  rt.active = 0;
#pragma unroll
  for (int x = 0; x < NW; ++x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) touched[x] |= __shfl_xor(touched[x], off, 64);
    // the same in every lane now: keep it in scalar registers
    const uint64_t t = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(touched[x] >> 32)) << 32) |
                       (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)touched[x]);
    const int below =
        (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(t >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)t, 0u));
    rt.rank[x] = ((t >> lane) & 1) ? rt.active + below : -1;
    rt.active += __builtin_popcountll(t);
  }
}

// The expert of rank k among the touched ones (wave-uniform).
template <int NW>
__device__ __forceinline__ int expert_of_rank(const Routing<NW> &rt, int k) {
  int e = -1;
#pragma unroll
  for (int x = 0; x < NW; ++x) {
    const uint64_t m = __ballot(rt.rank[x] == k);
    if (m) e = 64 * x + __builtin_ctzll(m);
  }
  return e;
}

// Persistent form of the expert GEMV (gate/up always, when the table is
// small; down in the four-kernel path).  With STAGE (gate/up, token rows that
// fit in LDS) the workgroup first stages every activation row, unit-major:
// piece c of unit u of row t at slot t*5U + c*U + u, and the record at slot
// t*5U + 4U + u.  The pair loop then reads its activation from LDS instead of
// L2.
template <int L, int R, bool STAGE, int NT, int WPE, int NW, bool DUMP>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(WPE))) void moe_expert_gemv_persistent(
    const uint8_t *__restrict__ W, const uint8_t *__restrict__ act, const int32_t *__restrict__ ids,
    const float *__restrict__ weights, float *__restrict__ out, int32_t *__restrict__ Dd,
    int rows, int nsb, int npairs, int top_k, int act_per_token,
    int64_t expert_bytes, int64_t act_row_bytes, int tiles, int n_expert, int n_act) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  u32x4n *xs = reinterpret_cast<u32x4n *>(lds);
  constexpr int G = 64 / L;
  const int lane = threadIdx.x & 63;
  const int li = lane & (L - 1);
  const int64_t rb = (int64_t)nsb * kQ4KBytes;
  const int U = nsb * 4;
  Routing<NW> rt;
  load_routing<NW>(rt, ids, npairs, n_expert);
  const int items = rt.active * tiles;
  // token row of pair 64w + lane (the activation row of the staged form)
  int tok[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) tok[w] = STAGE ? (64 * w + lane) / top_k : 0;

  const int u = li;  // this lane's unit (L >= U here, so at most one)
  const int sb = u >> 2, g = u & 3;
  if constexpr (STAGE) {
    for (int t = threadIdx.x; t < n_act * U; t += NT) {
      const int row = t / U, uu = t - row * U;
      ActUnit x;
      act_from_q8_1(act + (int64_t)row * act_row_bytes + (int64_t)(2 * uu) * kQ8_1Bytes, x);
      u32x4n *base = xs + row * 5 * U;
      base[uu] = u32x4n{x.A[1], x.A[2], x.A[3], x.A[4]};
      base[U + uu] = u32x4n{x.A[5], x.A[6], x.A[7], x.A[8]};
      base[2 * U + uu] = u32x4n{x.A[10], x.A[11], x.A[12], x.A[13]};
      base[3 * U + uu] = u32x4n{x.A[14], x.A[15], x.A[16], x.A[17]};
      base[4 * U + uu] = u32x4n{__builtin_bit_cast(uint32_t, x.da0), __builtin_bit_cast(uint32_t, x.da1),
                                __builtin_bit_cast(uint32_t, x.dS0), __builtin_bit_cast(uint32_t, x.dS1)};
    }
    __syncthreads();
  }
  // item = k * tiles + t, advanced by the grid size without dividing
  const int kstep = (int)gridDim.x / tiles, tstep = (int)gridDim.x - kstep * tiles;
  int ik = (int)blockIdx.x / tiles, it = (int)blockIdx.x - ik * tiles;
  // the next item's expert and first row of this lane group
  auto next_item = [&](int &e, int &row0) __attribute__((always_inline)) {
    e = expert_of_rank<NW>(rt, ik);
    row0 = ((it * (NT / 64) + (threadIdx.x >> 6)) * G + lane / L) * R;
    ik += kstep;
    it += tstep;
    if (it >= tiles) {
      it -= tiles;
      ++ik;
    }
  };
  // the lane's unit of the item's R rows: w[3r] header, w[3r+1], w[3r+2] the
  // unit's two 16-byte qs pieces
  auto load_item = [&](u32x4 (&w)[3 * R], int e, int row0) __attribute__((always_inline)) {
    const uint8_t *wu = W + (int64_t)e * expert_bytes + (int64_t)row0 * rb + sb * kQ4KBytes;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (u < U && row0 + r < rows) {
        const uint8_t *bp = wu + r * rb;
        w[3 * r] = ld16(bp);
        w[3 * r + 1] = ld16(bp + 16 + 32 * g);
        w[3 * r + 2] = ld16(bp + 32 + 32 * g);
      } else {
        w[3 * r] = w[3 * r + 1] = w[3 * r + 2] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  // the item's rows against every pair routed to its expert
  auto run_item = [&](const u32x4 (&w)[3 * R], int e, int row0) __attribute__((always_inline)) {
#pragma unroll
    for (int wd = 0; wd < NW; ++wd) {
      uint64_t mask = __ballot(rt.id[wd] == e);
      while (mask) {
        const int p = 64 * wd + __builtin_ctzll(mask);
        mask &= mask - 1;
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0.f;
        if (u < U) {
          ActUnit x;
          if constexpr (STAGE) {
            const int arow = __builtin_amdgcn_readlane(tok[wd], p - 64 * wd);
            act_from_unit_major(xs + arow * 5 * U, U, u, x);
          } else {
            const int arow = act_per_token ? p / top_k : p;
            act_from_q8_1(act + (int64_t)arow * act_row_bytes + (int64_t)(2 * u) * kQ8_1Bytes, x);
          }
#pragma unroll
          for (int r = 0; r < R; ++r) {
            int D0, D1;
            unit_dots(w[3 * r + 1], w[3 * r + 2], x, D0, D1);
            if (DUMP) {
              if (row0 + r < rows) dump_unit(Dd, p, rows, row0 + r, U, u, D0, D1);
            } else {
              acc[r] += unit_value(w[3 * r], g, x, D0, D1);
            }
          }
        }
        if (!DUMP) {
          const float scale = weights ? weights[p] : 1.0f;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const float v = group_sum_last<L>(acc[r]);
            if (li == L - 1 && row0 + r < rows) out[(int64_t)p * rows + row0 + r] = scale * v;
          }
        }
      }
    }
  };
  // One item at a time.  Loading the next item's weights during this item's
  // pairs measured slower: the pairs' stores, a number known only at run
  // time, sit between the two sets of loads in the vector memory counter, so
  // waiting for this item's weights waits for the next item's as well.
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    int e, row0;
    next_item(e, row0);
    u32x4 w[3 * R];
    load_item(w, e, row0);
    run_item(w, e, row0);
  }
}

// ------------------------------------------------------------------------
// The down kernel of the two-kernel path: one 8-wave workgroup per (token t,
// row tile of 4 * (64/L) rows); lane li of a row's group of L lanes owns units
// li, li + L, ..., li + (UPL-1)L, with L * UPL = U = n_ff / 64 (all lanes
// busy).  Waves w and w + 4 share rows: the first runs the even valid slots,
// the second the odd ones.
//   1. the token's valid slots (ids in range) in slot order, with their
//      experts and routing weights, into LDS;
//   2. each wave's first slot's weight loads are issued;
//   3. for every valid slot, h = silu(g) * u from g|u of its pair, quantized
//      to Q8_1 (8 lanes per 32-value block, the rule of quantize_q8_1) into
//      LDS, unit-major with the record {d(2u), d(2u+1), d*sum(2u), d*sum(2u+1)};
//      row tile 0 also writes the Q8_1 rows to hq;
//   4. each wave runs its slots in order (its next slot's weights loading
//      during this one's dots), acc += weights[p] * (Wdown[e] . h^_p); then
//      out[t][row] = acc(even slots) + acc(odd slots).
// Out-of-range slots contribute nothing; a token without a valid slot gets
// zeros.  Nothing is shared between workgroups, so the sum is deterministic.
// A touched expert's row tile is read by every token routed to it; the grid
// puts all tokens of a row tile on one XCD (workgroups go to XCDs round robin
// and the tile count is a multiple of 8 there), where the repeats hit L2.
template <int L, int UPL, bool DUMP>
__global__ __launch_bounds__(512) void moe_down_token_kernel(
    const uint8_t *__restrict__ W, const float *__restrict__ gu, const int32_t *__restrict__ ids,
    const float *__restrict__ weights, float *__restrict__ out, uint8_t *__restrict__ hq, int32_t *__restrict__ Dd,
    int H, int F, int top_k, int n_expert, int tiles) {
  constexpr int NT = 512, G = 64 / L;
  constexpr int kRowsItem = 4 * G;  // waves w and w + 4 share rows
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int U = L * UPL;  // == F / 64
  const int nq = F / 4;   // value quads per pair
  u32x4n *xs = reinterpret_cast<u32x4n *>(lds);                          // [top_k][5U]
  int *vs = reinterpret_cast<int *>(lds + (size_t)top_k * 5 * U * 16);  // valid slots, in order
  int *ve = vs + top_k;                                                  // their experts
  float *vw = reinterpret_cast<float *>(ve + top_k);                     // their routing weights
  float *part = vw + top_k;                                              // [4][64] odd-slot sums
  int *nv_s = reinterpret_cast<int *>(part + 4 * 64);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int li = lane & (L - 1);
  const int t = (int)(blockIdx.x / (unsigned)tiles), tile = (int)(blockIdx.x % (unsigned)tiles);
  const int rg = wv & 3, sp = wv >> 2;  // row group; slot parity this wave runs
  const int row = (tile * 4 + rg) * G + lane / L;
  const int64_t rb = (int64_t)(F / 256) * kQ4KBytes;
  const int64_t expert_bytes = (int64_t)H * rb;

  // 1. valid slots, with their experts and routing weights (in LDS, so that
  // the slot loop below issues no global load besides the weights it streams)
  if (wv == 0) {
    int n = 0;
    for (int s0 = 0; s0 < top_k; s0 += 64) {
      const int s = s0 + lane;
      const int e = s < top_k ? ids[t * top_k + s] : -1;
      const bool ok = s < top_k && e >= 0 && e < n_expert;
      const uint64_t m = __ballot(ok);
      const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      if (ok) {
        vs[n + below] = s;
        ve[n + below] = e;
        vw[n + below] = weights[t * top_k + s];
      }
      n += __builtin_popcountll(m);
    }
    if (lane == 0) *nv_s = n;
  }
  __syncthreads();
  const int nv = *nv_s;

  // weights of valid slot j's expert for this lane's units: w[3v] header,
  // w[3v+1] and w[3v+2] the unit's two 16-byte qs pieces
  // A slot's 3 * UPL loads are issued by every lane (rows past H read row
  // H - 1 and are never stored): without a per-lane branch around them the
  // compiler's waits for one slot leave more of the next slot's loads in
  // flight (53.6 -> 52.2 us).
  const int64_t row_off = (int64_t)min(row, H - 1) * rb;
  auto load_w = [&](u32x4 (&w)[3 * UPL], int j) __attribute__((always_inline)) {
    const uint8_t *we = W + (int64_t)ve[j] * expert_bytes + row_off;
#pragma unroll
    for (int v = 0; v < UPL; ++v) {
      const int u = li + v * L, sb = u >> 2, g = u & 3;
      const uint8_t *bp = we + sb * kQ4KBytes;
      w[3 * v] = ld16(bp);
      w[3 * v + 1] = ld16(bp + 16 + 32 * g);
      w[3 * v + 2] = ld16(bp + 32 + 32 * g);
    }
  };
  // 2. this wave's first slot's weights in flight during the activation step
  u32x4 cur[3 * UPL];
  if (sp < nv) load_w(cur, sp);

  // 3. h^ of every valid slot into LDS; 8 consecutive threads per block.  A
  // thread takes up to kActUnroll quads per round, all their g|u loads issued
  // before any is used (a round is uniform over each 8-thread group: the
  // quad count and the thread stride are multiples of 8).
  constexpr int kActUnroll = 3;  // 8 slots of 768 values: every quad of a thread in one round
  for (int q0 = tid; q0 < nv * nq; q0 += kActUnroll * NT) {
    float4 g4[kActUnroll], u4[kActUnroll];
#pragma unroll
    for (int k = 0; k < kActUnroll; ++k) {
      const int qq = q0 + k * NT;
      if (qq < nv * nq) {
        const int j = qq / nq, q = qq - j * nq;
        const float *gp = gu + (int64_t)(t * top_k + vs[j]) * 2 * F + 4 * q;
        g4[k] = *reinterpret_cast<const float4 *>(gp);
        u4[k] = *reinterpret_cast<const float4 *>(gp + F);
      }
    }
#pragma unroll
    for (int k = 0; k < kActUnroll; ++k) {
      const int qq = q0 + k * NT;
      if (qq >= nv * nq) break;
      const int j = qq / nq, q = qq - j * nq;
      const int p = t * top_k + vs[j];
      float4 h;
      h.x = g4[k].x / (1.0f + expf(-g4[k].x)) * u4[k].x;
      h.y = g4[k].y / (1.0f + expf(-g4[k].y)) * u4[k].y;
      h.z = g4[k].z / (1.0f + expf(-g4[k].z)) * u4[k].z;
      h.w = g4[k].w / (1.0f + expf(-g4[k].w)) * u4[k].w;
      const Q81Part qp = quantize_part_q8_1(h);
      const int blk = q >> 3, j8 = q & 7, uu = blk >> 1, bb = blk & 1;
      uint32_t *xr = reinterpret_cast<uint32_t *>(xs + j * 5 * U);
      xr[4 * ((2 * bb + (j8 >> 2)) * U + uu) + (j8 & 3)] = qp.packed;
      const uint32_t head = q81_header(qp);
      if (j8 == 0) {
        xr[4 * (4 * U + uu) + bb] = __builtin_bit_cast(uint32_t, h2f(head));
        xr[4 * (4 * U + uu) + 2 + bb] = __builtin_bit_cast(uint32_t, h2f(head) * (float)qp.sum);
      }
      if (tile == 0) {
        uint8_t *qb8 = hq + ((int64_t)p * (F / 32) + blk) * kQ8_1Bytes;
        *reinterpret_cast<uint32_t *>(qb8 + 4 + 4 * j8) = qp.packed;
        if (j8 == 0) *reinterpret_cast<uint32_t *>(qb8) = head;
      }
    }
  }
  __syncthreads();

  // 4. this wave's slots (parity sp) in order, the next one's weights loading
  // during each; then the odd slots' sum joins the even slots' in LDS
  float acc = 0.f;
  auto run_slot = [&](const u32x4 (&w)[3 * UPL], int j) __attribute__((always_inline)) {
    const int p = t * top_k + vs[j];
    const u32x4n *base = xs + j * 5 * U;
    float pt = 0.f;
#pragma unroll
    for (int v = 0; v < UPL; ++v) {
      const int u = li + v * L, g = u & 3;
      ActUnit x;
      act_from_unit_major(base, U, u, x);
      int D0, D1;
      unit_dots(w[3 * v + 1], w[3 * v + 2], x, D0, D1);
      if (DUMP) {
        if (row < H) dump_unit(Dd, p, H, row, U, u, D0, D1);
      } else {
        pt += unit_value(w[3 * v], g, x, D0, D1);
      }
    }
    if (!DUMP) acc += vw[j] * group_sum_last<L>(pt);
  };
  // Two register sets in turn (no copies between them).  (Issuing the next
  // slot's loads even when there is none, repeating the last slot, so that
  // every wait is a fixed count, measured slower: 55.3 against 53.0 us.)
  u32x4 nxt[3 * UPL];
  for (int j = sp; j < nv; j += 4) {
    if (j + 2 < nv) load_w(nxt, j + 2);
    run_slot(cur, j);
    if (j + 2 >= nv) break;
    if (j + 4 < nv) load_w(cur, j + 4);
    run_slot(nxt, j + 2);
  }
  if (DUMP) return;
  if (sp == 1) part[rg * 64 + lane] = acc;
  __syncthreads();
  if (sp == 0 && li == L - 1 && row < H) out[(int64_t)t * H + row] = acc + part[rg * 64 + lane];
}

// ------------------------------------------------------------------------
// Activation step of the four-kernel path: h = silu(g) * u per pair,
// requantized to Q8_1.  One 8-lane group per 32-value block of h; pairs with
// an out-of-range id are skipped.
__global__ __launch_bounds__(256) void moe_act_quant_kernel(const float *__restrict__ gu,
                                                            const int32_t *__restrict__ ids,
                                                            uint8_t *__restrict__ hq, int npairs, int n_ff,
                                                            int n_expert) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int nbp = n_ff / 32;
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
  quantize_block_q8_1(v, hq + ((int64_t)p * nbp + bi) * kQ8_1Bytes, j, live);
}

// Combine of the four-kernel path: out[t][i] = sum over slots s (in order) of
// z[t*top_k + s][i].
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

// ------------------------------------------------------------------ launch
// Everything one expert-GEMV launch needs besides its kernel shape.
struct GemvCall {
  const uint8_t *W, *act;
  const int32_t *ids;
  const float *weights;  // nullptr: scale 1 (gate/up)
  float *out;
  int32_t *D;            // non-null: the dump instance
  int rows, nsb, npairs, top_k, act_per_token;
  int64_t act_row_bytes;
  int n_expert;
};

// Rows per lane group of the grid-form expert GEMV.
constexpr int kMoeRows = 2;

template <int L, int R, int UPL>
static void launch_grid_form(const GemvCall &c, hipStream_t stream) {
  const int rows_per_block = 4 * (64 / L) * R;
  const int tiles = (c.rows + rows_per_block - 1) / rows_per_block;
  const dim3 grid((unsigned)((int64_t)tiles * c.n_expert));
  const int64_t expert_bytes = (int64_t)c.rows * c.nsb * kQ4KBytes;
  if (c.D)
    hipLaunchKernelGGL((moe_expert_gemv_kernel<L, R, UPL, true>), grid, dim3(256), 0, stream, c.W, c.act, c.ids,
                       c.weights, c.out, c.D, c.rows, c.nsb, c.npairs, c.top_k, c.act_per_token, expert_bytes,
                       c.act_row_bytes, tiles);
  else
    hipLaunchKernelGGL((moe_expert_gemv_kernel<L, R, UPL, false>), grid, dim3(256), 0, stream, c.W, c.act, c.ids,
                       c.weights, c.out, c.D, c.rows, c.nsb, c.npairs, c.top_k, c.act_per_token, expert_bytes,
                       c.act_row_bytes, tiles);
}

// LDS for staging all activation rows of a gate/up call: 5 x 16 bytes per
// unit of each row.  Up to this much, four workgroups still fit on a CU.
constexpr size_t kMoeStageBytes = 40 * 1024;

// Launch shape of the persistent expert GEMV: workgroup size, rows per lane
// group, and the waves per SIMD its register allocation must leave room for.
// The staged gate/up call runs 8-wave workgroups, two per CU: 16 waves, as
// with four 4-wave ones, but each CU stages the token rows twice, not four
// times.  The unstaged form (down in the four-kernel path, or token rows past
// the staging limit) runs four waves per SIMD and three rows per lane group.
// The grid is the number of workgroups resident at once (the dump instance
// runs on the product instance's grid).
constexpr int kGuThreads = 512, kGuRows = 2, kGuWaves = 4;
constexpr int kDnThreads = 256, kDnRows = 3, kDnWaves = 4;

template <int L, int R, bool STAGE, int NT, int WPE, int NW>
static void launch_persistent_shape(const GemvCall &c, size_t stage, int n_act, hipStream_t stream) {
  constexpr auto kern = moe_expert_gemv_persistent<L, R, STAGE, NT, WPE, NW, false>;
  constexpr auto kdump = moe_expert_gemv_persistent<L, R, STAGE, NT, WPE, NW, true>;
  const int rows_per_block = (NT / 64) * (64 / L) * R;
  const int tiles = (c.rows + rows_per_block - 1) / rows_per_block;
  const int64_t max_items = (int64_t)tiles * c.n_expert;
  const int64_t resident = resident_blocks<kern>(NT, stage);
  const dim3 grid((unsigned)(max_items < resident ? max_items : resident));
  const int64_t expert_bytes = (int64_t)c.rows * c.nsb * kQ4KBytes;
  hipLaunchKernelGGL(c.D ? kdump : kern, grid, dim3(NT), stage, stream, c.W, c.act, c.ids, c.weights, c.out, c.D,
                     c.rows, c.nsb, c.npairs, c.top_k, c.act_per_token, expert_bytes,
                     c.act_row_bytes, tiles, c.n_expert, n_act);
}

template <int L, int NW>
static void launch_persistent_nw(const GemvCall &c, hipStream_t stream) {
  const int n_act = c.act_per_token ? (c.npairs + c.top_k - 1) / c.top_k : c.npairs;
  const size_t stage = (size_t)n_act * c.nsb * 4 * 80;
  if (c.act_per_token && stage <= kMoeStageBytes)
    launch_persistent_shape<L, kGuRows, true, kGuThreads, kGuWaves, NW>(c, stage, n_act, stream);
  else
    launch_persistent_shape<L, kDnRows, false, kDnThreads, kDnWaves, NW>(c, 0, n_act, stream);
}

// Routing tables of up to 128 pairs over up to 128 experts keep two words of
// ids and of the touched-expert bitmap per lane instead of four.
template <int L>
static void launch_persistent(const GemvCall &c, hipStream_t stream) {
  if (c.npairs <= 128 && c.n_expert <= 128)
    launch_persistent_nw<L, 2>(c, stream);
  else
    launch_persistent_nw<L, kMaxIdWords>(c, stream);
}

// Lanes per row of the gate/up and four-kernel down GEMVs: the smallest power
// of two >= the row's unit count, capped at 64 (lanes past the last unit
// idle); each lane then keeps ceil(U/L) units' weights for R rows in VGPRs
// (up to two units; longer rows reload per pair).
static bool persistent_fits(const GemvCall &c, int *L_out) {
  const int U = c.nsb * 4;
  int L = 4;
  while (L < U && L < 64) L <<= 1;
  *L_out = L;
  return (U + L - 1) / L == 1 && c.npairs <= 64 * kMaxIdWords && c.n_expert <= 64 * kMaxIdWords;
}

static void expert_gemv(const GemvCall &c, hipStream_t stream) {
  const int U = c.nsb * 4;
  int L = 4;
  if (persistent_fits(c, &L)) {
    if (L == 4) launch_persistent<4>(c, stream);
    else if (L == 8) launch_persistent<8>(c, stream);
    else if (L == 16) launch_persistent<16>(c, stream);
    else if (L == 32) launch_persistent<32>(c, stream);
    else launch_persistent<64>(c, stream);
    return;
  }
  const int upl = (U + L - 1) / L;
  if (L == 4) launch_grid_form<4, kMoeRows, 1>(c, stream);
  else if (L == 8) launch_grid_form<8, kMoeRows, 1>(c, stream);
  else if (L == 16) launch_grid_form<16, kMoeRows, 1>(c, stream);
  else if (L == 32) launch_grid_form<32, kMoeRows, 1>(c, stream);
  else if (upl == 1) launch_grid_form<64, kMoeRows, 1>(c, stream);
  else if (upl == 2) launch_grid_form<64, 2, 2>(c, stream);
  else launch_grid_form<64, 1, 0>(c, stream);  // long rows: weights reloaded per pair
}

// Shape of the token-major down kernel: L lanes per row with UPL units each,
// L * UPL = U = n_ff / 64, L a power of two in 4..64 and UPL in 1..3.  0 if
// no such split exists.
static int down_split(int U, int *upl) {
  for (int u = 1; u <= 3; ++u) {
    if (U % u) continue;
    const int L = U / u;
    if (L >= 4 && L <= 64 && (L & (L - 1)) == 0) {
      *upl = u;
      return L;
    }
  }
  return 0;
}

// LDS of the token-major down kernel: h^ of top_k slots (U * 80 bytes each)
// and the slot list.  It runs only when this fits in 32 KB.
constexpr size_t kDownLds = 32 * 1024;
static size_t down_lds(int U, int top_k) { return (size_t)top_k * U * 80 + (size_t)(3 * top_k + 4 * 64 + 1) * 4; }

template <int L, int UPL>
static void launch_down_token_lu(const MoeArgs &a, int32_t *D, hipStream_t stream) {
  const int U = (int)(a.n_ff / 64);
  const int rows = 4 * (64 / L);
  const int tiles = (int)((a.n_embd + rows - 1) / rows);
  const dim3 grid((unsigned)(a.n_tok * tiles));  // 512 threads each
  const size_t lds = down_lds(U, (int)a.top_k);
  if (D)
    hipLaunchKernelGGL((moe_down_token_kernel<L, UPL, true>), grid, dim3(512), lds, stream,
                       static_cast<const uint8_t *>(a.w_down), a.ws_gu, a.ids, a.weights, a.out, a.ws_hq, D,
                       (int)a.n_embd, (int)a.n_ff, (int)a.top_k, (int)a.n_expert, tiles);
  else
    hipLaunchKernelGGL((moe_down_token_kernel<L, UPL, false>), grid, dim3(512), lds, stream,
                       static_cast<const uint8_t *>(a.w_down), a.ws_gu, a.ids, a.weights, a.out, a.ws_hq, D,
                       (int)a.n_embd, (int)a.n_ff, (int)a.top_k, (int)a.n_expert, tiles);
}

static void launch_down_token(const MoeArgs &a, int32_t *D, int L, int upl, hipStream_t stream) {
#define QG_DT(LV, UV) \
  if (L == LV && upl == UV) return launch_down_token_lu<LV, UV>(a, D, stream)
  QG_DT(4, 1); QG_DT(4, 2); QG_DT(4, 3);
  QG_DT(8, 1); QG_DT(8, 2); QG_DT(8, 3);
  QG_DT(16, 1); QG_DT(16, 2); QG_DT(16, 3);
  QG_DT(32, 1); QG_DT(32, 2); QG_DT(32, 3);
  QG_DT(64, 1); QG_DT(64, 2); QG_DT(64, 3);
#undef QG_DT
}

// Which path a call takes: the two-kernel one needs the small-table
// persistent gate/up and a down row that splits evenly over lane groups.
static bool two_kernel_path(const MoeArgs &a, int *L, int *upl) {
  GemvCall gu{};
  gu.nsb = (int)(a.n_embd / 256);
  gu.npairs = (int)(a.n_tok * a.top_k);
  gu.n_expert = (int)a.n_expert;
  int lg = 0;
  if (!persistent_fits(gu, &lg)) return false;
  *L = down_split((int)(a.n_ff / 64), upl);
  return *L != 0 && down_lds((int)(a.n_ff / 64), (int)a.top_k) <= kDownLds;
}

// D_gu / D_dn non-null: the dump run (gate/up product first, so that the down
// dump has its g|u; then the dump instances).
static hipError_t run_moe(const MoeArgs &a, int32_t *D_gu, int32_t *D_dn, hipStream_t stream) {
  const int P = (int)(a.n_tok * a.top_k);
  const int F = (int)a.n_ff, H = (int)a.n_embd, E = (int)a.n_expert, K = (int)a.top_k;
  int L = 0, upl = 0;
  const bool two = two_kernel_path(a, &L, &upl);
  GemvCall gu{};
  gu.W = static_cast<const uint8_t *>(a.w_gu);
  gu.act = static_cast<const uint8_t *>(a.xq);
  gu.ids = a.ids;
  gu.weights = nullptr;
  gu.out = a.ws_gu;
  gu.rows = 2 * F;
  gu.nsb = H / 256;
  gu.npairs = P;
  gu.top_k = K;
  gu.act_per_token = 1;
  gu.act_row_bytes = (int64_t)(H / 32) * kQ8_1Bytes;
  gu.n_expert = E;
  // 1. gate|up rows [2F] of each touched expert against token rows of xq
  expert_gemv(gu, stream);
  if (D_gu) {
    GemvCall d = gu;
    d.D = D_gu;
    expert_gemv(d, stream);
  }
  if (two) {
    // 2. h^, down, routed sum
    launch_down_token(a, D_dn, L, upl, stream);
    return hipGetLastError();
  }
  // 2. h^ = Q8_1(silu(g) * u)
  {
    const int64_t threads = (int64_t)P * (F / 32) * 8;
    hipLaunchKernelGGL(moe_act_quant_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a.ws_gu,
                       a.ids, a.ws_hq, P, F, E);
  }
  // 3. z[p] = weights[p] * (Wdown[e] . h^[p])
  GemvCall dn{};
  dn.W = static_cast<const uint8_t *>(a.w_down);
  dn.act = a.ws_hq;
  dn.ids = a.ids;
  dn.weights = a.weights;
  dn.out = a.ws_z;
  dn.D = D_dn;
  dn.rows = H;
  dn.nsb = F / 256;
  dn.npairs = P;
  dn.top_k = K;
  dn.act_per_token = 0;
  dn.act_row_bytes = (int64_t)(F / 32) * kQ8_1Bytes;
  dn.n_expert = E;
  expert_gemv(dn, stream);
  // 4. out[t] = sum of its slots
  const int64_t total = (int64_t)a.n_tok * H;
  if (!D_dn && total > 0)
    hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, a.ws_z,
                       a.ids, a.out, (int)a.n_tok, K, H, E);
  return hipGetLastError();
}

hipError_t launch_moe_q4_k(const MoeArgs &a, hipStream_t stream) { return run_moe(a, nullptr, nullptr, stream); }

hipError_t launch_moe_q4_k_dump(const MoeArgs &a, int32_t *D_gu, int32_t *D_dn, hipStream_t stream) {
  return run_moe(a, D_gu, D_dn, stream);
}

bool moe_two_kernel_path(const MoeArgs &a) {
  int L = 0, upl = 0;
  return two_kernel_path(a, &L, &upl);
}

}  // namespace qg
