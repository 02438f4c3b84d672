// Router top-k of one token on one 16-lane DPP row, shared by the router
// kernel (route.hip) and the FP8 layer's fused router + activation
// quantiser (dispatch.hip).
//
// Each token's scores s = fl32(logit + bias) become 64-bit keys whose high
// word is the score's bits mapped to an unsigned order (larger float ->
// larger word, -0.0 folded onto +0.0) and whose low word is the complemented
// expert id, so one unsigned max picks the largest score and, among equal
// scores, the lowest id.  k rounds of a max over the row select the experts
// in slot order; the gate weights are exp(s_j - s_0) / sum_i exp(s_i - s_0)
// (the softmax over E renormalised over the k chosen -- "6.4 Data
// parallelism and expert parallelism", section 3.1, step 1, with the
// renormalisation of the workload definition).
#pragma once

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

// Tokens of a 256-thread workgroup: token 16 blockIdx.x + threadIdx.x / 16
// on each 16-lane row (every lane of the row joins the DPP steps, valid or
// not); lane r of the row holds experts r + 16 i, i < KPL (E <= 16 KPL).
// Loads are unconditional (clamped addresses) and the key is a select, so
// the keys stay in registers without per-key branches.  Lane r < k of a
// valid token stores slot r's expert and weight.
template <int KPL, bool BIAS>
__device__ __forceinline__ void route_rows_block(
    const float* __restrict__ logits, const float* __restrict__ bias, int T,
    int E, int k, int32_t* __restrict__ ids, float* __restrict__ w,
    int block) {
  const int lane = threadIdx.x & 63, r = lane & 15;
  const int t = (block * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
  const bool valid = t < T;
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

}  // namespace moe
