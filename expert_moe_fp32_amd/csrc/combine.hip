// Combine: un-permute and sum each token's expert outputs weighted by its
// route weights ("6.4 Data parallelism and expert parallelism", section 3.1,
// step 4), plus the shared expert's output with weight 1 (section 2.1).
// Workgroup = (token, column slice); a slice is the whole row unless the
// batch is too small to fill the GPU.  The first wavefront compacts the
// token's local slots (slot order kept) into LDS while every thread already
// loads its columns of the shared expert's row; then each thread owns
// groups of 4 columns, CPT groups per pass, and issues all of a pass's row
// loads before it accumulates, in float32 and slot order, with one rounding
// to the output type.
#include "common.h"

namespace moe {

typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
static constexpr int kCombineCPT = 4;      // column groups per thread per pass

// Streaming (large batches): the expert outputs are read once and the output
// written once, so both go through non-temporal accesses, which keep them
// from displacing the L2's other lines (prefill combine 117 -> 88 us).
template <int STREAM, typename V>
__device__ __forceinline__ V ld(const V* p) {
  if (STREAM) return __builtin_nontemporal_load(p);
  return *p;
}
template <int STREAM, typename V>
__device__ __forceinline__ void st(V v, V* p) {
  if (STREAM) __builtin_nontemporal_store(v, p);
  else *p = v;
}

template <int OUT_BF16, int STREAM>
__global__ __launch_bounds__(256) void k_combine(
    const float* __restrict__ y, const int32_t* __restrict__ pair_row,
    const float* __restrict__ w, const float* __restrict__ y_shared, int T,
    int H, int k, int cw, void* __restrict__ out) {
  constexpr int CPT = kCombineCPT;
  const int t = blockIdx.x;
  const int H4 = H >> 2;
  const int cbeg = blockIdx.y * cw, cend = min(H4, cbeg + cw);
  __shared__ int32_t rows[MOE_KMAX];
  __shared__ float wts[MOE_KMAX];
  __shared__ int nloc;
  if (threadIdx.x < 64) {     // lanes j < k load slot j; local slots keep order
    const int j = threadIdx.x;
    const int r = j < k ? pair_row[(size_t)t * k + j] : -1;
    const float wj = j < k ? w[(size_t)t * k + j] : 0.0f;
    const uint64_t m = __ballot(r >= 0);
    if (r >= 0) {
      const int pos = __popcll(m & ((1ull << j) - 1ull));
      rows[pos] = r;
      wts[pos] = wj;
    }
    if (j == 0) nloc = __popcll(m);
  }
  // the first pass's shared-expert columns do not depend on the slots
  const float* ys = y_shared ? y_shared + (size_t)t * H : nullptr;
  f32x4_t sh0[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = cbeg + threadIdx.x + 256 * i;
    sh0[i] = (ys && c < cend) ? ld<STREAM>((const f32x4_t*)(ys + 4 * c)) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();
  const int n = nloc;
  for (int c0 = cbeg + threadIdx.x; c0 < cend; c0 += 256 * CPT) {
    f32x4_t acc[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    f32x4_t shv[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = c0 + 256 * i;
      shv[i] = c0 == cbeg + (int)threadIdx.x ? sh0[i]
               : (ys && c < cend) ? ld<STREAM>((const f32x4_t*)(ys + 4 * c))
                                : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    for (int j = 0; j < n; ++j) {
      const float* yr = y + (size_t)rows[j] * H;
      const float wj = wts[j];
      f32x4_t v[CPT];
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = c0 + 256 * i;
        v[i] = c < cend ? ld<STREAM>((const f32x4_t*)(yr + 4 * c)) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        acc[i].x = __builtin_fmaf(wj, v[i].x, acc[i].x);
        acc[i].y = __builtin_fmaf(wj, v[i].y, acc[i].y);
        acc[i].z = __builtin_fmaf(wj, v[i].z, acc[i].z);
        acc[i].w = __builtin_fmaf(wj, v[i].w, acc[i].w);
      }
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = c0 + 256 * i;
      if (c >= cend) continue;
      f32x4_t s = acc[i];
      if (ys) {
        s.x += shv[i].x; s.y += shv[i].y; s.z += shv[i].z; s.w += shv[i].w;
      }
      if (OUT_BF16) {
        u32x2_t pk;
        pk.x = (uint32_t)f32_to_bf16(s.x) | ((uint32_t)f32_to_bf16(s.y) << 16);
        pk.y = (uint32_t)f32_to_bf16(s.z) | ((uint32_t)f32_to_bf16(s.w) << 16);
        st<STREAM>(pk, (u32x2_t*)((bf16_t*)out + (size_t)t * H + 4 * c));
      } else {
        st<STREAM>(s, (f32x4_t*)((float*)out + (size_t)t * H + 4 * c));
      }
    }
  }
}

hipError_t launch_combine(const float* y_perm, const int32_t* pair_row,
                          const float* w, const float* y_shared, int T, int H,
                          int k, int out_dtype, void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  // column slices (multiples of 256 groups of 4) so that small batches
  // still launch about 2048 workgroups
  const int H4 = H / 4;
  const int groups = (H4 + 255) / 256;
  const int want = T >= 2048 ? 1 : min(groups, (2048 + T - 1) / T);
  const int cw = ((groups + want - 1) / want) * 256;
  const dim3 grid(T, (H4 + cw - 1) / cw);
  // (the decode-sized path reads outputs the expert kernels just left in L2)
  const bool stream = T >= 2048;
  if (out_dtype == MOE_BF16) {
    if (stream)
      k_combine<1, 1><<<grid, 256, 0, s>>>(y_perm, pair_row, w, y_shared, T, H, k, cw, out);
    else
      k_combine<1, 0><<<grid, 256, 0, s>>>(y_perm, pair_row, w, y_shared, T, H, k, cw, out);
  } else {
    if (stream)
      k_combine<0, 1><<<grid, 256, 0, s>>>(y_perm, pair_row, w, y_shared, T, H, k, cw, out);
    else
      k_combine<0, 0><<<grid, 256, 0, s>>>(y_perm, pair_row, w, y_shared, T, H, k, cw, out);
  }
  return hipGetLastError();
}

}  // namespace moe
