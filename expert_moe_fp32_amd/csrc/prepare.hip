// One-time weight preparation: the storage orders a caller may hold an
// expert matrix in, turned into the form the expert kernels read.
//
// An expert is three matrices ("6.4 Data parallelism and expert
// parallelism", section 2.1: gate, up, down).  For one matrix with reduction
// size K and N output channels the caller stores either the logical layout
// [K][N] (layout KN: h = silu(x W_gate) * (x W_up), y = h W_down) or its
// transpose [N][K] (layout NK, a linear layer's output-major weight).
//
// Prepared forms (include/moe.h, moe_prepack_weights):
//  * float32: [K][N];
//  * bf16: 16 x 32 operand blocks, block (n/16, k/32) at block index
//    (n/16) * (K/32) + k/32, 16-byte lane L = n%16 + 16 * ((k%32)/8) holding
//    k%8 = 0..7;
//  * fp8 codes: 16 x 128 blocks of 2 KiB, block (n/16, k/128) at block index
//    (n/16) * (K/128) + k/128, lane L = n%16 + 16 * ((k%128)/32) owning 32
//    codes, the first 16 at byte L*16 and the rest at 1024 + L*16.
// These run once per weight upload, not on the layer's path: a packed chunk
// from a KN source is gathered value by value (strided reads), which is
// simple and fast enough for a one-time pass.
#include "common.h"

namespace moe {

// element (k, n) of a source matrix in either storage order
__device__ __forceinline__ size_t src_index(int layout, size_t k, size_t n,
                                            int K, int N) {
  return layout == MOE_LAYOUT_KN ? k * (size_t)N + n : n * (size_t)K + k;
}

// One thread per 16-byte chunk of the packed bf16 output.
__global__ __launch_bounds__(256) void k_pack_bf16(const bf16_t* __restrict__ src,
                                                   int K, int N, int layout,
                                                   u32x4_t* __restrict__ dst) {
  const size_t total = (size_t)K * N / 8;
  const int KB = K / 32;
  for (size_t gi = (size_t)blockIdx.x * 256 + threadIdx.x; gi < total;
       gi += (size_t)gridDim.x * 256) {
    const size_t blk = gi >> 6;
    const int lane = (int)(gi & 63);
    const size_t nb = blk / KB, kb = blk - nb * KB;
    const size_t n = nb * 16 + (lane & 15), k = kb * 32 + (lane >> 4) * 8;
    if (layout == MOE_LAYOUT_NK) {
      dst[gi] = *(const u32x4_t*)(src + n * K + k);
    } else {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = (uint32_t)src[(k + 2 * i) * N + n] |
               ((uint32_t)src[(k + 2 * i + 1) * N + n] << 16);
      dst[gi] = u32x4_t{w[0], w[1], w[2], w[3]};
    }
  }
}

// One thread per 16-byte chunk of the packed fp8 output.
__global__ __launch_bounds__(256) void k_pack_fp8(const uint8_t* __restrict__ src,
                                                  int K, int N, int layout,
                                                  u32x4_t* __restrict__ dst) {
  const size_t total = (size_t)K * N / 16;
  const int KB = K / 128;
  for (size_t gi = (size_t)blockIdx.x * 256 + threadIdx.x; gi < total;
       gi += (size_t)gridDim.x * 256) {
    const size_t blk = gi >> 7;
    const int idx = (int)(gi & 127);
    const int L = idx & 63, half = idx >> 6;
    const size_t nb = blk / KB, kb = blk - nb * KB;
    const size_t n = nb * 16 + (L & 15);
    const size_t k = kb * 128 + 32 * (L >> 4) + 16 * half;
    if (layout == MOE_LAYOUT_NK) {
      dst[gi] = *(const u32x4_t*)(src + n * K + k);
    } else {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b)
          v |= (uint32_t)src[(k + 4 * i + b) * N + n] << (8 * b);
        w[i] = v;
      }
      dst[gi] = u32x4_t{w[0], w[1], w[2], w[3]};
    }
  }
}

// float32: dst[k][n] from either order.
__global__ __launch_bounds__(256) void k_prep_f32(const float* __restrict__ src,
                                                  int K, int N, int layout,
                                                  float* __restrict__ dst) {
  const size_t total = (size_t)K * N;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (size_t)gridDim.x * 256) {
    const size_t k = i / N, n = i - k * N;
    dst[i] = src[src_index(layout, k, n, K, N)];
  }
}

hipError_t launch_prepack(const void* src, int K, int N, int dtype, int layout,
                          void* dst, hipStream_t s) {
  const size_t elems = (size_t)K * N;
  if (elems == 0) return hipSuccess;
  const size_t chunks = dtype == MOE_F32 ? elems
                        : dtype == MOE_BF16 ? elems / 8 : elems / 16;
  size_t grid = (chunks + 255) / 256;
  if (grid > 8192) grid = 8192;
  if (dtype == MOE_F32)
    k_prep_f32<<<(unsigned)grid, 256, 0, s>>>((const float*)src, K, N, layout,
                                              (float*)dst);
  else if (dtype == MOE_BF16)
    k_pack_bf16<<<(unsigned)grid, 256, 0, s>>>((const bf16_t*)src, K, N,
                                               layout, (u32x4_t*)dst);
  else
    k_pack_fp8<<<(unsigned)grid, 256, 0, s>>>((const uint8_t*)src, K, N,
                                              layout, (u32x4_t*)dst);
  return hipGetLastError();
}

// FP8 block quantisation: one workgroup per 128 x 128 block of the source
// (rows x cols as stored).  scale = amax/448 (1 for an all-zero block),
// code = RNE of fl32(w/scale) saturated; the scale is stored at
// [n-block][k-block] for either storage order.
__global__ __launch_bounds__(256) void k_quant_blocks_fp8(
    const float* __restrict__ w, int K, int N, int layout,
    uint8_t* __restrict__ codes, float* __restrict__ scales) {
  __shared__ float red[4];
  const int cols = layout == MOE_LAYOUT_KN ? N : K;
  const int bc = cols / 128;
  const int bi = blockIdx.x / bc, bj = blockIdx.x % bc;
  const float* base = w + (size_t)bi * 128 * cols + (size_t)bj * 128;
  float amax = 0.0f;
  for (int i = threadIdx.x; i < 128 * 128; i += 256)
    amax = fmaxf(amax, fabsf(base[(size_t)(i >> 7) * cols + (i & 127)]));
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = amax == 0.0f ? 1.0f : __fdiv_rn(amax, 448.0f);
  uint8_t* cb = codes + (size_t)bi * 128 * cols + (size_t)bj * 128;
  for (int i = threadIdx.x; i < 128 * 128; i += 256) {
    const size_t o = (size_t)(i >> 7) * cols + (i & 127);
    cb[o] = f32_to_e4m3(__fdiv_rn(base[o], sc));
  }
  // source block (bi, bj) is (k-block, n-block) for KN, (n-block, k-block)
  // for NK
  const int kb = layout == MOE_LAYOUT_KN ? bi : bj;
  const int nb = layout == MOE_LAYOUT_KN ? bj : bi;
  if (threadIdx.x == 0) scales[(size_t)nb * (K / 128) + kb] = sc;
}

hipError_t launch_quant_blocks_fp8(const float* w, int K, int N, int layout,
                                   uint8_t* codes, float* scales,
                                   hipStream_t s) {
  const int nb = (K / 128) * (N / 128);
  if (nb == 0) return hipSuccess;
  k_quant_blocks_fp8<<<nb, 256, 0, s>>>(w, K, N, layout, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
