// Combine: un-permute and sum each token's expert outputs weighted by its
// route weights ("6.4 Data parallelism and expert parallelism", section 3.1,
// step 4), plus the shared expert's output with weight 1 (section 2.1).
// Workgroup (token t, 1024-column chunk); each thread owns 4 columns and
// issues the loads of all the token's local rows before it accumulates, in
// float32 and slot order, with one rounding to the output type.
#include "common.h"

namespace moe {

template <int OUT_BF16>
__global__ __launch_bounds__(256) void k_combine(
    const float* __restrict__ y, const int32_t* __restrict__ pair_row,
    const float* __restrict__ w, const float* __restrict__ y_shared, int T,
    int H, int k, void* __restrict__ out) {
  const int t = blockIdx.x;
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
  __syncthreads();
  const int n = nloc;
  const int H4 = H >> 2;
  const int c = blockIdx.y * blockDim.x + threadIdx.x;
  if (c < H4) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < n; j0 += 4) {      // four rows' loads in flight
      f32x4_t v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {          // past n: re-read the last row
        const int j = min(j0 + q, n - 1);
        v[q] = *(const f32x4_t*)(y + (size_t)rows[j] * H + 4 * c);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (j0 + q < n) {
          const float wj = wts[j0 + q];
          acc.x = __builtin_fmaf(wj, v[q].x, acc.x);
          acc.y = __builtin_fmaf(wj, v[q].y, acc.y);
          acc.z = __builtin_fmaf(wj, v[q].z, acc.z);
          acc.w = __builtin_fmaf(wj, v[q].w, acc.w);
        }
      }
    }
    if (y_shared) {
      const f32x4_t v = *(const f32x4_t*)(y_shared + (size_t)t * H + 4 * c);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    if (OUT_BF16) {
      uint2 pk;
      pk.x = (uint32_t)f32_to_bf16(acc.x) | ((uint32_t)f32_to_bf16(acc.y) << 16);
      pk.y = (uint32_t)f32_to_bf16(acc.z) | ((uint32_t)f32_to_bf16(acc.w) << 16);
      *(uint2*)((bf16_t*)out + (size_t)t * H + 4 * c) = pk;
    } else {
      *(f32x4_t*)((float*)out + (size_t)t * H + 4 * c) = acc;
    }
  }
}

hipError_t launch_combine(const float* y_perm, const int32_t* pair_row,
                          const float* w, const float* y_shared, int T, int H,
                          int k, int out_dtype, void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid(T, (H / 4 + 255) / 256);
  if (out_dtype == MOE_BF16)
    k_combine<1><<<grid, 256, 0, s>>>(y_perm, pair_row, w, y_shared, T, H, k, out);
  else
    k_combine<0><<<grid, 256, 0, s>>>(y_perm, pair_row, w, y_shared, T, H, k, out);
  return hipGetLastError();
}

}  // namespace moe
