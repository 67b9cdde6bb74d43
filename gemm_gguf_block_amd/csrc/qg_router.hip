// qg_router.hip -- the MoE router in one launch: per token, the router logits
// Wr . x, the top-k experts and their softmax weights -- the routing table the
// expert FFN (moe_qgemv_q4_k) takes.  The router matrix stays f32, as it does
// in Q4_K_M files of the MoE models the infr page runs ("models").
//
// One workgroup (256 threads) per token.  x is staged in LDS; wave w takes
// experts w, w + 4, ... and lane l float4s l, l + 64, ... of each row, summed
// in that order and then by a butterfly, so a logit's bits depend on H alone.
// Wave 0 then selects: each lane holds the keys of experts l, l + 64, ...; K
// times, the wave maximum of the keys is taken and its expert's key cleared.
// A key orders by logit (larger first) and, for equal logits, by expert
// (lower first).  The softmax runs over the selected logits, shifted by the
// largest.
#include "qg_device.h"
#include "qg_launch.h"

namespace qg {

namespace {

constexpr int kRouterMaxE = 256;  // 4 keys per lane of one wave
constexpr int kRouterKeys = kRouterMaxE / 64;

// (logit, expert) -> a key whose unsigned order is: larger logit, then lower
// expert.  Float bits are mapped to an order-preserving unsigned code; 0 is
// below every key (the cleared value).
__device__ __forceinline__ uint64_t route_key(float v, int e) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint64_t o = __shfl_xor(v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}

__global__ __launch_bounds__(256) void router_topk_kernel(const float *__restrict__ Wr, const float *__restrict__ X,
                                                          int32_t *__restrict__ ids, float *__restrict__ weights,
                                                          float *__restrict__ logits_out, int E, int H, int K) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float4 *xs = reinterpret_cast<float4 *>(lds);
  float *lg = reinterpret_cast<float *>(lds) + H;  // E logits
  const int t = blockIdx.x, tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int h4 = H / 4;
  const float4 *x4 = reinterpret_cast<const float4 *>(X + (int64_t)t * H);
  for (int i = tid; i < h4; i += 256) xs[i] = x4[i];
  __syncthreads();
  for (int e = wv; e < E; e += 4) {
    const float4 *w4 = reinterpret_cast<const float4 *>(Wr + (int64_t)e * H);
    float acc = 0.f;
    for (int i = lane; i < h4; i += 64) {
      const float4 a = w4[i], b = xs[i];
      acc = fmaf(a.x, b.x, acc);
      acc = fmaf(a.y, b.y, acc);
      acc = fmaf(a.z, b.z, acc);
      acc = fmaf(a.w, b.w, acc);
    }
    acc = group_sum<64>(acc);
    if (lane == 0) {
      lg[e] = acc;
      if (logits_out) logits_out[(int64_t)t * E + e] = acc;
    }
  }
  __syncthreads();
  if (wv != 0) return;
  uint64_t key[kRouterKeys];
#pragma unroll
  for (int j = 0; j < kRouterKeys; ++j) {
    const int e = lane + 64 * j;
    key[j] = e < E ? route_key(lg[e], e) : 0ull;
  }
  // lane i keeps the i-th selected expert; `first` is the largest (uniform)
  int mine = 0, first = 0;
  for (int i = 0; i < K; ++i) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < kRouterKeys; ++j) best = key[j] > best ? key[j] : best;
    best = wave_max_u64(best);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
    if (lane == (e & 63)) {
#pragma unroll
      for (int j = 0; j < kRouterKeys; ++j)
        if (j == (e >> 6)) key[j] = 0ull;
    }
    if (lane == i) mine = e;
    if (i == 0) first = e;
  }
  const int e = mine;
  const float m = lg[first];
  const float v = lane < K ? expf(lg[e] - m) : 0.f;
  const float s = group_sum<64>(v);
  if (lane < K) {
    ids[(int64_t)t * K + lane] = e;
    weights[(int64_t)t * K + lane] = v / s;
  }
}

}  // namespace

static size_t router_lds_bytes(int64_t n_expert, int64_t n_embd) { return (size_t)(n_embd + n_expert) * 4; }

hipError_t launch_router_topk(const float *w_router, const float *x, int32_t *ids, float *weights, float *logits,
                              int64_t n_tok, int64_t n_expert, int64_t n_embd, int64_t top_k, hipStream_t stream) {
  hipLaunchKernelGGL(router_topk_kernel, dim3((unsigned)n_tok), dim3(256), router_lds_bytes(n_expert, n_embd), stream,
                     w_router, x, ids, weights, logits, (int)n_expert, (int)n_embd, (int)top_k);
  return hipGetLastError();
}

}  // namespace qg
