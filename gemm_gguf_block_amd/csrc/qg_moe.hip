// qg_moe.hip -- MoE expert FFN with Q4_K experts (the expert_gateup and down
// calls an MoE decode step spends its time in; infr page, "Per-op device
// profiling" and "Paged experts").
//
// Four kernels on one stream, no host round trip:
//   1. gate/up: grid over (expert, row tile).  A workgroup scans the routing
//      table for its expert and, for each (token, slot) pair routed to it,
//      runs the Q4_K GEMV rows of its tile against that token's Q8_1 row.  An
//      expert nobody routed to reads no weights, and a touched expert's
//      weights are streamed once for all of its pairs (later pairs hit cache).
//   2. act: per pair, h = silu(g)*u in fp32, requantized to Q8_1 exactly as
//      quantize_q8_1 does.
//   3. down: like 1, over the down weights and each pair's h^, scaled by the
//      pair's routing weight.
//   4. combine: out[t] = sum over t's slots in slot order (deterministic).
#include "qg_blocks.h"
#include "qg_launch.h"
#include "qg_quant.h"

namespace qg {

// Kernels 1 and 3.  blockIdx.x = expert * tiles + row tile; each wave covers
// (64/L)*R rows of the expert's [rows][nsb] matrix.  The routing table is
// scanned 64 ids at a time with one vector load and a ballot, so a workgroup
// whose expert nobody routed to finishes after npairs/64 loads.  For every pair
// p with ids[p] == expert:
//   out[p][row] = scale(p) * dot(row, act + act_row(p))
// with act_row(p) = p / top_k (token rows, kernel 1) or p (h^ rows, kernel 3),
// scale(p) = 1 (kernel 1) or weights[p] (kernel 3).
template <int L, int R>
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
  for (int c0 = 0; c0 < npairs; c0 += 64) {
    const int id = c0 + lane < npairs ? ids[c0 + lane] : -1;
    uint64_t mask = __ballot(id == e);
    while (mask) {
      const int p = c0 + __builtin_ctzll(mask);
      mask &= mask - 1;
      const uint8_t *xr = act + (int64_t)(act_per_token ? p / top_k : p) * act_row_bytes;
      float acc[R];
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = 0.f;
      if (row0 < rows) {
        for (int u = li; u < U; u += L) {
          const int sb = u >> 2, g = u & 3;
          u32x4 hdr[R], qa[R], qb[R];
#pragma unroll
          for (int r = 0; r < R; ++r) {
            if (row0 + r < rows) {
              const uint8_t *bp = wexp + (int64_t)(row0 + r) * rb + (int64_t)sb * kQ4KBytes;
              hdr[r] = ld16(bp);
              qa[r] = ld16(bp + 16 + 32 * g);
              qb[r] = ld16(bp + 32 + 32 * g);
            } else {
              hdr[r] = qa[r] = qb[r] = u32x4{0u, 0u, 0u, 0u};
            }
          }
          const uint8_t *ap = xr + (int64_t)(8 * sb + 2 * g) * kQ8_1Bytes;
          const u32x4 a0 = ld16(ap), a1 = ld16(ap + 16), a2 = ld16(ap + 32), a3 = ld16(ap + 48);
          const u32x2 a4 = ld8(ap + 64);
          const uint32_t A[18] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w, a2.x,
                                  a2.y, a2.z, a2.w, a3.x, a3.y, a3.z, a3.w, a4.x, a4.y};
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
      }
      const float scale = weights ? weights[p] : 1.0f;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float v = group_sum<L>(acc[r]);
        if (li == 0 && row0 + r < rows) out[(int64_t)p * rows + row0 + r] = scale * v;
      }
    }
  }
}

// Kernel 2: h = silu(g) * u per pair, requantized to Q8_1.  One 8-lane group
// per 32-value block of h; pairs with an out-of-range id are skipped.
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

template <int L, int R>
static void launch_expert_gemv(const uint8_t *W, const uint8_t *act, const int32_t *ids, const float *weights,
                               float *out, int rows, int nsb, int npairs, int top_k, int act_per_token,
                               int64_t expert_bytes, int64_t act_row_bytes, int n_expert, hipStream_t stream) {
  const int rows_per_block = 4 * (64 / L) * R;
  const int tiles = (rows + rows_per_block - 1) / rows_per_block;
  const dim3 grid((unsigned)((int64_t)tiles * n_expert));
  hipLaunchKernelGGL((moe_expert_gemv_kernel<L, R>), grid, dim3(256), 0, stream, W, act, ids, weights, out, rows,
                     nsb, npairs, top_k, act_per_token, expert_bytes, act_row_bytes, tiles);
}

// Rows per lane group for the expert GEMVs (activation reuse, loads in flight).
constexpr int kMoeRows = 2;

static void expert_gemv(const uint8_t *W, const uint8_t *act, const int32_t *ids, const float *weights, float *out,
                        int rows, int nsb, int npairs, int top_k, int act_per_token, int64_t act_row_bytes,
                        int n_expert, hipStream_t stream) {
  const int64_t expert_bytes = (int64_t)rows * nsb * kQ4KBytes;
  switch (lanes_per_row((int64_t)nsb * 4)) {
#define QG_MOE_CASE(LV)                                                                                          \
  case LV:                                                                                                       \
    launch_expert_gemv<LV, kMoeRows>(W, act, ids, weights, out, rows, nsb, npairs, top_k, act_per_token,         \
                                     expert_bytes, act_row_bytes, n_expert, stream);                             \
    break;
    QG_MOE_CASE(64)
    QG_MOE_CASE(32)
    QG_MOE_CASE(16)
    QG_MOE_CASE(8)
    default:
      QG_MOE_CASE(4)
#undef QG_MOE_CASE
  }
}

MoeLayout moe_layout(int64_t n_tok, int64_t top_k, int64_t n_ff, int64_t n_embd) {
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  const size_t P = (size_t)(n_tok * top_k);
  MoeLayout l;
  l.hq_off = 0;
  l.gu_off = up(P * (size_t)(n_ff / 32) * kQ8_1Bytes);
  l.z_off = l.gu_off + up(P * (size_t)(2 * n_ff) * sizeof(float));
  l.total = l.z_off + up(P * (size_t)n_embd * sizeof(float));
  return l;
}

hipError_t launch_moe_q4_k(const MoeArgs &a, hipStream_t stream) {
  const int P = (int)(a.n_tok * a.top_k);
  const int F = (int)a.n_ff, H = (int)a.n_embd, E = (int)a.n_expert, K = (int)a.top_k;
  // 1. gate|up rows [2F] of each touched expert against token rows of xq
  expert_gemv(static_cast<const uint8_t *>(a.w_gu), static_cast<const uint8_t *>(a.xq), a.ids, nullptr, a.ws_gu,
              2 * F, H / 256, P, K, 1, (int64_t)(H / 32) * kQ8_1Bytes, E, stream);
  // 2. h^ = Q8_1(silu(g) * u)
  {
    const int64_t threads = (int64_t)P * (F / 32) * 8;
    hipLaunchKernelGGL(moe_act_quant_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a.ws_gu,
                       a.ids, a.ws_hq, P, F, E);
  }
  // 3. z[p] = weights[p] * (Wdown[e] . h^[p])
  expert_gemv(static_cast<const uint8_t *>(a.w_down), a.ws_hq, a.ids, a.weights, a.ws_z, H, F / 256, P, K, 0,
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
