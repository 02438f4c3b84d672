// Combine: un-permute and sum each token's expert outputs weighted by its
// route weights ("6.4 Data parallelism and expert parallelism", section 3.1,
// step 4), plus the shared expert's output with weight 1 (section 2.1).
// One workgroup per token; float32 accumulation in slot order, one rounding
// to the output type.
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
  if (threadIdx.x == 0) {
    int n = 0;
    for (int j = 0; j < k; ++j) {
      const int r = pair_row[(size_t)t * k + j];
      if (r >= 0) {
        rows[n] = r;
        wts[n] = w[(size_t)t * k + j];
        ++n;
      }
    }
    nloc = n;
  }
  __syncthreads();
  const int n = nloc;
  const int H4 = H >> 2;
  for (int c = threadIdx.x; c < H4; c += blockDim.x) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < n; ++j) {
      const f32x4_t v = *(const f32x4_t*)(y + (size_t)rows[j] * H + 4 * c);
      const float wj = wts[j];
      acc.x = __builtin_fmaf(wj, v.x, acc.x);
      acc.y = __builtin_fmaf(wj, v.y, acc.y);
      acc.z = __builtin_fmaf(wj, v.z, acc.z);
      acc.w = __builtin_fmaf(wj, v.w, acc.w);
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
  if (out_dtype == MOE_BF16)
    k_combine<1><<<T, 256, 0, s>>>(y_perm, pair_row, w, y_shared, T, H, k, out);
  else
    k_combine<0><<<T, 256, 0, s>>>(y_perm, pair_row, w, y_shared, T, H, k, out);
  return hipGetLastError();
}

}  // namespace moe
