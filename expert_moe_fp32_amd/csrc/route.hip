// Router top-k: one wavefront per token.
//
// Each token's scores s = fl32(logit + bias) are spread over the 64 lanes
// (E/64 per lane).  A score becomes a 64-bit key whose high word is the
// score's bits mapped to an unsigned order (larger float -> larger word,
// -0.0 folded onto +0.0) and whose low word is the complemented expert id, so
// one unsigned max picks the largest score and, among equal scores, the
// lowest id.  k rounds of a wave-wide max select the experts in slot order;
// the gate weights are exp(s_j - s_0) / sum_i exp(s_i - s_0) (the softmax over
// E renormalised over the k chosen -- "6.4 Data parallelism and expert
// parallelism", section 3.1, step 1, with the renormalisation of the workload
// definition).  Lanes 0..k-1 write the outputs and bump the expert counts.
#include "common.h"

namespace moe {

__device__ __forceinline__ uint32_t order_bits(float s) {
  if (s == 0.0f) s = 0.0f;                  // -0.0 and +0.0 are one score
  uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_order_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
    uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
    uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

template <int EPL>
__global__ __launch_bounds__(256) void k_route_topk(
    const float* __restrict__ logits, const float* __restrict__ bias, int T,
    int E, int k, int32_t* __restrict__ ids, float* __restrict__ w,
    int32_t* __restrict__ counts) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  uint64_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    int e = lane + 64 * i;
    key[i] = 0;
    if (e < E) {
      float s = row[e];
      if (bias) s = s + bias[e];
      key[i] = ((uint64_t)order_bits(s) << 32) | (uint32_t)(~(uint32_t)e);
    }
  }
  int my_id = -1;
  float my_score = 0.0f, top = 0.0f, denom = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < EPL; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int e = (int)(~(uint32_t)best);
    const float s = from_order_bits((uint32_t)(best >> 32));
    if (j == 0) top = s;
    denom += expf(s - top);
#pragma unroll
    for (int i = 0; i < EPL; ++i)              // the owner drops the winner
      if (lane + 64 * i == e) key[i] = 0;
    if (lane == j) { my_id = e; my_score = s; }
  }
  if (lane < k) {
    const size_t o = (size_t)t * k + lane;
    ids[o] = my_id;
    w[o] = expf(my_score - top) / denom;
    if (counts) atomicAdd(&counts[my_id], 1);
  }
}

hipError_t launch_route_topk(const float* logits, const float* bias, int T,
                             int E, int k, int32_t* ids, float* w,
                             int32_t* counts, hipStream_t s) {
  dim3 grid((T + 3) / 4), block(256);
  if (E <= 64)
    k_route_topk<1><<<grid, block, 0, s>>>(logits, bias, T, E, k, ids, w, counts);
  else if (E <= 128)
    k_route_topk<2><<<grid, block, 0, s>>>(logits, bias, T, E, k, ids, w, counts);
  else if (E <= 256)
    k_route_topk<4><<<grid, block, 0, s>>>(logits, bias, T, E, k, ids, w, counts);
  else if (E <= 512)
    k_route_topk<8><<<grid, block, 0, s>>>(logits, bias, T, E, k, ids, w, counts);
  else
    k_route_topk<16><<<grid, block, 0, s>>>(logits, bias, T, E, k, ids, w, counts);
  return hipGetLastError();
}

}  // namespace moe
