// Router top-k.
//
// Each token's scores s = fl32(logit + bias) become 64-bit keys whose high
// word is the score's bits mapped to an unsigned order (larger float ->
// larger word, -0.0 folded onto +0.0) and whose low word is the complemented
// expert id, so one unsigned max picks the largest score and, among equal
// scores, the lowest id.  k rounds of a max over the token's lanes select
// the experts in slot order; the gate weights are exp(s_j - s_0) /
// sum_i exp(s_i - s_0) (the softmax over E renormalised over the k chosen --
// "6.4 Data parallelism and expert parallelism", section 3.1, step 1, with
// the renormalisation of the workload definition).
//
// E <= 256: a token owns one 16-lane row of a wavefront (four tokens per
// wavefront) and the max runs as four DPP row rotations, with no LDS
// traffic.  Larger E: a token owns a whole wavefront (shuffle butterfly).
//
// The per-expert counts (the load an EPLB records) are a separate
// single-workgroup histogram of the chosen ids with one LDS copy per
// wavefront; it stores the counts, so no atomics reach global memory (on
// skewed routing the hot experts' counters would serialise them).
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

// max over the 16 lanes of a DPP row: rotations by 8, 4, 2 and 1 lanes
__device__ __forceinline__ uint64_t row_max_u64(uint64_t v) {
#define ROW_STEP(ctrl)                                                        \
  {                                                                           \
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(                \
        0, (int)(uint32_t)(v >> 32), ctrl, 0xF, 0xF, false);                   \
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(                \
        0, (int)(uint32_t)v, ctrl, 0xF, 0xF, false);                           \
    const uint64_t o = ((uint64_t)hi << 32) | lo;                             \
    v = o > v ? o : v;                                                        \
  }
  ROW_STEP(0x128)  // row_ror:8
  ROW_STEP(0x124)  // row_ror:4
  ROW_STEP(0x122)  // row_ror:2
  ROW_STEP(0x121)  // row_ror:1
#undef ROW_STEP
  return v;
}

// One token per 16-lane row; lane r of the row holds experts r + 16 i.
// Loads are unconditional (clamped addresses) and the key is a select, so
// the key array stays in registers without per-key branches.
template <int KPL, bool BIAS>
__global__ __launch_bounds__(256) void k_route_rows(
    const float* __restrict__ logits, const float* __restrict__ bias, int T,
    int E, int k, int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63, r = lane & 15;
  const int t = (blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
  const bool valid = t < T;                // every lane joins the DPP steps
  const float* row = logits + (size_t)(valid ? t : 0) * E;
  uint64_t key[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int e = r + 16 * i;
    const int ec = e < E ? e : 0;
    float s = row[ec];
    if (BIAS) s = s + bias[ec];
    const uint64_t kv = ((uint64_t)order_bits(s) << 32) | (uint32_t)(~(uint32_t)e);
    key[i] = (valid && e < E) ? kv : 0;
  }
  int my_id = -1;
  float my_score = 0.0f, top = 0.0f, denom = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < KPL; ++i) best = key[i] > best ? key[i] : best;
    best = row_max_u64(best);
    const int e = (int)(~(uint32_t)best);
    const float s = from_order_bits((uint32_t)(best >> 32));
    if (j == 0) top = s;
    denom += expf(s - top);
#pragma unroll
    for (int i = 0; i < KPL; ++i)              // the owner drops the winner
      if (r + 16 * i == e) key[i] = 0;
    if (r == j) { my_id = e; my_score = s; }
  }
  if (valid && r < k) {
    const size_t o = (size_t)t * k + r;
    ids[o] = my_id;
    w[o] = expf(my_score - top) / denom;
  }
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
