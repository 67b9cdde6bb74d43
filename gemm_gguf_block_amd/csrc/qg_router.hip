// qg_router.hip -- the MoE router: per token, the router logits Wr . x, the
// top-k experts and their softmax weights -- the routing table the expert FFN
// (moe_qgemv_q4_k) takes.  The router matrix stays f32, as it does in Q4_K_M
// files of the MoE models the infr page runs ("models").
//
// Two launches on the caller's stream.
//
// router_logits_kernel: a workgroup (256 threads) owns a tile of kRouterTT
// tokens x kRouterEW experts.  Thread i walks float4 columns i, i + 256, ...
// of its experts' rows and of the tile's token rows, keeping one partial sum
// per (expert, token) -- 16 values per thread, all of the tile's loads of one
// column in flight together.  A wave then reduces its 16 values across the 64
// lanes by a transposing butterfly (at each of the first four exchanges a lane
// keeps half of its values and adds the partner's half, so lane l ends with
// value l/4 summed over 16 lanes; two plain exchanges finish it), and the four
// wave sums are added in wave order.  Every logit therefore has a fixed
// summation order that depends on H alone.  Several hundred workgroups at
// decode shapes keep enough loads in flight for the weight stream; one
// workgroup per token would read the whole router matrix through one CU.
//
// router_select_kernel: one wave per token.  Each lane holds the keys of
// experts l, l + 64, ...; K times, the wave maximum of the keys is taken and
// its expert's key cleared.  A key orders by logit (larger first) and, for
// equal logits, by expert (lower first).  The softmax runs over the selected
// logits, shifted by the largest.
#include "qg_device.h"
#include "qg_launch.h"

namespace qg {

namespace {

constexpr int kRouterEW = 2;                       // experts per workgroup
constexpr int kRouterTT = 8;                       // tokens per workgroup
constexpr int kRouterV = kRouterEW * kRouterTT;    // partial sums per thread (16)
constexpr int kRouterMaxE = 256;                   // 4 keys per lane of one wave
constexpr int kRouterKeys = kRouterMaxE / 64;
static_assert(kRouterV == 16, "the reduction below halves 16 values four times");

__device__ __forceinline__ float dot4(float4 a, float4 b, float acc) {
  acc = fmaf(a.x, b.x, acc);
  acc = fmaf(a.y, b.y, acc);
  acc = fmaf(a.z, b.z, acc);
  return fmaf(a.w, b.w, acc);
}

// Lane exchange of the transposing butterfly.  Lanes whose bit `o` is clear
// keep `lo` and receive the partner's `lo`; the others keep `hi` and receive
// the partner's `hi`; the sum of kept and received is returned.  Offsets 32
// and 16 use the gfx950 permlane swaps (vdst's upper 32 lanes / odd rows trade
// places with src's lower 32 lanes / even rows), 8 and 4 row rotations.
template <int O>
__device__ __forceinline__ float xchg_sum(float lo, float hi, int lane) {
  const unsigned a = __builtin_bit_cast(unsigned, lo), b = __builtin_bit_cast(unsigned, hi);
  if constexpr (O == 32 || O == 16) {
    const auto r = O == 32 ? __builtin_amdgcn_permlane32_swap(a, b, false, false)
                           : __builtin_amdgcn_permlane16_swap(a, b, false, false);
    // the elements are copied out first: bit-casting r[1] in place reads r[0]
    // (hipcc of ROCm 7.2)
    const unsigned r0 = r[0], r1 = r[1];
    return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
  } else {
    const bool up = (lane & O) != 0;
    const int send = (int)(up ? a : b);
    // row_ror:n (0x120 + n): lane i reads lane (i - n) mod 16 of its row
    const int from_above = __builtin_amdgcn_update_dpp(0, send, 0x120 + (16 - O), 0xf, 0xf, false);
    const int from_below = __builtin_amdgcn_update_dpp(0, send, 0x120 + O, 0xf, 0xf, false);
    return (up ? hi : lo) + __builtin_bit_cast(float, up ? from_below : from_above);
  }
}

__global__ __launch_bounds__(256) void router_logits_kernel(const float *__restrict__ Wr, const float *__restrict__ X,
                                                            float *__restrict__ logits, int E, int H, int64_t T) {
  __shared__ float red[4][kRouterV];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int64_t t0 = (int64_t)blockIdx.x * kRouterTT;
  const int e0 = blockIdx.y * kRouterEW;
  const int nt = (int)min<int64_t>(kRouterTT, T - t0);
  const int ne = min(kRouterEW, E - e0);
  const int h4 = H / 4;
  // rows past the tile's end repeat its last row, so every load is in bounds
  // and unconditional; their sums are never stored
  const float4 *wrow[kRouterEW];
  const float4 *xrow[kRouterTT];
#pragma unroll
  for (int e = 0; e < kRouterEW; ++e)
    wrow[e] = reinterpret_cast<const float4 *>(Wr + (int64_t)(e0 + min(e, ne - 1)) * H);
#pragma unroll
  for (int j = 0; j < kRouterTT; ++j) xrow[j] = reinterpret_cast<const float4 *>(X + (t0 + min(j, nt - 1)) * H);

  float v[kRouterV];  // v[e * kRouterTT + j]: expert e0 + e, token t0 + j
#pragma unroll
  for (int q = 0; q < kRouterV; ++q) v[q] = 0.f;
#pragma unroll 2
  for (int i = tid; i < h4; i += 256) {
    float4 w[kRouterEW], x[kRouterTT];
#pragma unroll
    for (int e = 0; e < kRouterEW; ++e) w[e] = wrow[e][i];
#pragma unroll
    for (int j = 0; j < kRouterTT; ++j) x[j] = xrow[j][i];
#pragma unroll
    for (int e = 0; e < kRouterEW; ++e)
#pragma unroll
      for (int j = 0; j < kRouterTT; ++j) v[e * kRouterTT + j] = dot4(w[e], x[j], v[e * kRouterTT + j]);
  }
  // transposing butterfly: after the exchange at offset o (32, 16, 8, 4) a
  // lane holds half as many values, the half selected by its bit o
#pragma unroll
  for (int q = 0; q < 8; ++q) v[q] = xchg_sum<32>(v[q], v[q + 8], lane);
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = xchg_sum<16>(v[q], v[q + 4], lane);
#pragma unroll
  for (int q = 0; q < 2; ++q) v[q] = xchg_sum<8>(v[q], v[q + 2], lane);
  float s = xchg_sum<4>(v[0], v[1], lane);  // value lane >> 2, summed over the 16 lanes that share lane & 3
  // quad_perm [2,3,0,1] then [1,0,3,2]: the four lanes of a quad
  s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x4E, 0xf, 0xf, false));
  s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0xB1, 0xf, 0xf, false));
  if ((lane & 3) == 0) red[wv][lane >> 2] = s;
  __syncthreads();
  if (tid < kRouterV) {
    const int e = tid / kRouterTT, j = tid % kRouterTT;
    if (e < ne && j < nt) logits[(t0 + j) * E + e0 + e] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
  }
}

// (logit, expert) -> a key whose unsigned order is: larger logit, then lower
// expert.  Float bits are mapped to an order-preserving unsigned code; 0 is
// below every key (the cleared value).  The logit is recovered from the key.
__device__ __forceinline__ uint64_t route_key(float v, int e) {
  if (v == 0.f) v = 0.f;  // -0 ranks as +0
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

// Wave maximum of an unsigned value, returned to every lane: DPP shift-right
// maxima within rows of 16, row broadcasts across rows (0 is the identity of
// the unsigned maximum and fills lanes outside the source), then lane 63.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32_or_zero(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xf, true);
}

__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  v = max(v, dpp_u32_or_zero<0x111, 0xf>(v));
  v = max(v, dpp_u32_or_zero<0x112, 0xf>(v));
  v = max(v, dpp_u32_or_zero<0x114, 0xf>(v));
  v = max(v, dpp_u32_or_zero<0x118, 0xf>(v));
  v = max(v, dpp_u32_or_zero<0x142, 0xa>(v));
  v = max(v, dpp_u32_or_zero<0x143, 0x8>(v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__global__ __launch_bounds__(256) void router_select_kernel(const float *__restrict__ logits, int32_t *__restrict__ ids,
                                                            float *__restrict__ weights, int E, int K, int64_t T) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float *lg = logits + t * E;
  uint64_t key[kRouterKeys];
#pragma unroll
  for (int j = 0; j < kRouterKeys; ++j) {
    const int e = lane + 64 * j;
    key[j] = e < E ? route_key(lg[e], e) : 0ull;
  }
  // lane i keeps the i-th selected expert and its logit; `top` is the largest
  int mine = 0;
  float mine_l = 0.f, top = 0.f;
  for (int i = 0; i < K; ++i) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < kRouterKeys; ++j) best = key[j] > best ? key[j] : best;
    // the wave's largest key: its high word first, then the low word among
    // the lanes that hold that high word
    const uint32_t u = wave_umax((uint32_t)(best >> 32));
    const uint32_t lo = wave_umax((uint32_t)(best >> 32) == u ? (uint32_t)best : 0u);
    const int e = (int)(0xFFFFFFFFu - lo);
    const float l = __builtin_bit_cast(float, (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
    if (lane == (e & 63)) {
#pragma unroll
      for (int j = 0; j < kRouterKeys; ++j)
        if (j == (e >> 6)) key[j] = 0ull;
    }
    if (lane == i) {
      mine = e;
      mine_l = l;
    }
    if (i == 0) top = l;
  }
  const float p = lane < K ? expf(mine_l - top) : 0.f;
  const float s = group_sum<64>(p);
  if (lane < K) {
    ids[t * K + lane] = mine;
    weights[t * K + lane] = p / s;
  }
}

}  // namespace

hipError_t launch_router_topk(const float *w_router, const float *x, int32_t *ids, float *weights, float *logits,
                              int64_t n_tok, int64_t n_expert, int64_t n_embd, int64_t top_k, hipStream_t stream) {
  const dim3 grid_l((unsigned)((n_tok + kRouterTT - 1) / kRouterTT), (unsigned)((n_expert + kRouterEW - 1) / kRouterEW));
  hipLaunchKernelGGL(router_logits_kernel, grid_l, dim3(256), 0, stream, w_router, x, logits, (int)n_expert,
                     (int)n_embd, n_tok);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(router_select_kernel, dim3((unsigned)((n_tok + 3) / 4)), dim3(256), 0, stream, logits, ids,
                     weights, (int)n_expert, (int)top_k, n_tok);
  return hipGetLastError();
}

}  // namespace qg
