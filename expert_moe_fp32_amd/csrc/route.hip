// Router top-k: the per-token selection and weights of route_row.h, on one
// 16-lane DPP row per token, or on a whole wavefront for E > 256.
//
// E <= 256: a token owns one 16-lane row of a wavefront (four tokens per
// wavefront) and the max runs as four DPP row rotations, with no LDS
// traffic.  Larger E: a token owns a whole wavefront (shuffle butterfly).
//
// The per-expert counts (the load an EPLB records) are a separate
// single-workgroup histogram of the chosen ids with one LDS copy per
// wavefront; it stores the counts, so no atomics reach global memory (on
// skewed routing the hot experts' counters would serialise them).
#include "route_row.h"

namespace moe {

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

// One token per 16-lane row (route_row.h), four tokens per wavefront.
template <int KPL, bool BIAS>
__global__ __launch_bounds__(256) void k_route_rows(
    const float* __restrict__ logits, const float* __restrict__ bias, int T,
    int E, int k, int32_t* __restrict__ ids, float* __restrict__ w) {
  route_rows_block<KPL, BIAS>(logits, bias, T, E, k, ids, w, blockIdx.x);
}

// counts[e] = number of entries equal to e among ids[0 .. n); one workgroup,
// one LDS histogram per wavefront, summed at the end and stored.
__global__ __launch_bounds__(1024) void k_count_ids(
    const int32_t* __restrict__ ids, int n, int E,
    int32_t* __restrict__ counts) {
  __shared__ int32_t h[16][MOE_EMAX];
  const int tid = threadIdx.x, wv = tid >> 6;
  for (int i = tid; i < 16 * E; i += 1024) h[i / E][i % E] = 0;
  __syncthreads();
  int32_t* mine = h[wv];
  const bool aligned = ((uintptr_t)ids & 15) == 0;   // 16-B loads need it
  const int n4 = aligned ? n >> 2 : 0;
  const int4* ids4 = (const int4*)ids;
  // ids outside [0, E) are not counted (they never come from the router,
  // but a stray one must not write past the histogram)
  auto count = [&](int e) {
    if ((unsigned)e < (unsigned)E) atomicAdd(&mine[e], 1);
  };
#pragma unroll 4
  for (int i = tid; i < n4; i += 1024) {
    const int4 v = ids4[i];
    count(v.x);
    count(v.y);
    count(v.z);
    count(v.w);
  }
  for (int i = 4 * n4 + tid; i < n; i += 1024) count(ids[i]);
  __syncthreads();
  for (int e = tid; e < E; e += 1024) {
    int c = 0;
#pragma unroll
    for (int v = 0; v < 16; ++v) c += h[v][e];
    counts[e] = c;
  }
}

template <int EPL, bool BIAS>
__global__ __launch_bounds__(256) void k_route_topk(
    const float* __restrict__ logits, const float* __restrict__ bias, int T,
    int E, int k, int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  uint64_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    const int ec = e < E ? e : 0;
    float s = row[ec];
    if (BIAS) s = s + bias[ec];
    const uint64_t kv = ((uint64_t)order_bits(s) << 32) | (uint32_t)(~(uint32_t)e);
    key[i] = e < E ? kv : 0;
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
  }
}

hipError_t launch_route_topk(const float* logits, const float* bias, int T,
                             int E, int k, int32_t* ids, float* w,
                             int32_t* counts, hipStream_t s) {
  if (E <= 256) {
    dim3 grid((T + 15) / 16), block(256);
#define ROUTE_ROWS(KPL)                                                        \
  (bias ? k_route_rows<KPL, true><<<grid, block, 0, s>>>(logits, bias, T, E, k, ids, w) \
        : k_route_rows<KPL, false><<<grid, block, 0, s>>>(logits, bias, T, E, k, ids, w))
    if (E <= 16) ROUTE_ROWS(1);
    else if (E <= 32) ROUTE_ROWS(2);
    else if (E <= 64) ROUTE_ROWS(4);
    else if (E <= 128) ROUTE_ROWS(8);
    else ROUTE_ROWS(16);
#undef ROUTE_ROWS
  } else {
    dim3 grid((T + 3) / 4), block(256);
#define ROUTE_WAVE(EPL)                                                        \
  (bias ? k_route_topk<EPL, true><<<grid, block, 0, s>>>(logits, bias, T, E, k, ids, w) \
        : k_route_topk<EPL, false><<<grid, block, 0, s>>>(logits, bias, T, E, k, ids, w))
    if (E <= 512) ROUTE_WAVE(8);
    else ROUTE_WAVE(16);
#undef ROUTE_WAVE
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !counts) return e;
  k_count_ids<<<1, 1024, 0, s>>>(ids, T * k, E, counts);
  return hipGetLastError();
}

}  // namespace moe
