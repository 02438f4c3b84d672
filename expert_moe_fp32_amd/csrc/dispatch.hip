// Dispatch: local filter, logical-to-physical replica remap and a
// deterministic expert-contiguous permutation, plus the row gather.
//
// Order ("6.4 Data parallelism and expert parallelism", section 3.1, step 2,
// on one rank; section 5.3 for replicas): walking the (token, slot) pairs in
// token order, the n-th pair of local expert e goes to replica n mod R_e at
// position floor(n / R_e) of that replica's segment.  Positions come from
// ranks, never from atomic slot grabbing, so the permutation is the same on
// every run:
//   1. k_local_hist: a workgroup covers 256 consecutive tokens; for every
//      local expert each wavefront ballots which of its 64 tokens picked it.
//      The per-block counts go to block_counts[block][e].
//   2. k_scan (one workgroup): per expert an exclusive scan over the blocks
//      (block_base), the expert's total n_e, the replica split
//      ceil((n_e - r) / R_e) and the exclusive scan over physical ids
//      (offsets).
//   3. k_permute: the ballots again give each pair its rank inside the
//      wavefront; block base + earlier wavefronts + that rank is n.
#include "common.h"

namespace moe {

static constexpr int kTokPerBlock = 256;

int dispatch_blocks(int T) { return (T + kTokPerBlock - 1) / kTokPerBlock; }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Each thread loads its token's local expert ids (-1 where not local).
__device__ __forceinline__ void load_local_ids(const int32_t* ids, int t,
                                               int T, int k, int e0, int L,
                                               int (&le)[MOE_KMAX]) {
#pragma unroll
  for (int j = 0; j < MOE_KMAX; ++j) {
    le[j] = -1;
    if (j < k && t < T) {
      int e = ids[(size_t)t * k + j] - e0;
      le[j] = (e >= 0 && e < L) ? e : -1;
    }
  }
}

__global__ __launch_bounds__(256) void k_local_hist(
    const int32_t* __restrict__ ids, int T, int k, int e0, int L,
    int32_t* __restrict__ block_counts) {
  extern __shared__ int32_t wave_cnt[];     // [4][L]
  const int t = blockIdx.x * kTokPerBlock + threadIdx.x;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int le[MOE_KMAX];
  load_local_ids(ids, t, T, k, e0, L, le);
  bool any_local = false;
#pragma unroll
  for (int j = 0; j < MOE_KMAX; ++j) any_local |= le[j] >= 0;
  const bool wave_has = __ballot(any_local) != 0ull;
  for (int e = 0; e < L; ++e) {
    int c = 0;
    if (wave_has) {
      bool has = false;
#pragma unroll
      for (int j = 0; j < MOE_KMAX; ++j) has |= le[j] == e;
      c = __popcll(__ballot(has));
    }
    if (lane == 0) wave_cnt[wv * L + e] = c;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < L; e += blockDim.x)
    block_counts[(size_t)blockIdx.x * L + e] =
        wave_cnt[e] + wave_cnt[L + e] + wave_cnt[2 * L + e] + wave_cnt[3 * L + e];
}

__global__ __launch_bounds__(1024) void k_scan(
    const int32_t* __restrict__ block_counts, int nblk, int L, int P,
    int max_rep, const int32_t* __restrict__ l2p,
    const int32_t* __restrict__ rep, int32_t* __restrict__ block_base,
    int32_t* __restrict__ offsets) {
  __shared__ int32_t pc[MOE_LMAX];
  for (int p = threadIdx.x; p < P; p += blockDim.x) pc[p] = 0;
  __syncthreads();
  for (int e = threadIdx.x; e < L; e += blockDim.x) {
    int run = 0;
    for (int b = 0; b < nblk; ++b) {
      const int c = block_counts[(size_t)b * L + e];
      block_base[(size_t)b * L + e] = run;
      run += c;
    }
    const int R = rep ? min(max(rep[e], 1), max_rep) : 1;
    for (int r = 0; r < R; ++r) {
      const int p = l2p ? l2p[e * max_rep + r] : e;
      if (p >= 0 && p < P) pc[p] = run > r ? (run - r + R - 1) / R : 0;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int p = 0; p < P; ++p) {
      offsets[p] = run;
      run += pc[p];
    }
    offsets[P] = run;
  }
}

__global__ __launch_bounds__(256) void k_permute(
    const int32_t* __restrict__ ids, const float* __restrict__ w, int T,
    int k, int e0, int L, int P, int max_rep, const int32_t* __restrict__ l2p,
    const int32_t* __restrict__ rep, const int32_t* __restrict__ block_base,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ row_token,
    float* __restrict__ row_weight, int32_t* __restrict__ pair_row) {
  extern __shared__ int32_t wave_cnt[];     // [4][L]
  const int t = blockIdx.x * kTokPerBlock + threadIdx.x;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int le[MOE_KMAX], rank[MOE_KMAX];
  load_local_ids(ids, t, T, k, e0, L, le);
  bool any_local = false;
#pragma unroll
  for (int j = 0; j < MOE_KMAX; ++j) {
    rank[j] = 0;
    any_local |= le[j] >= 0;
  }
  const bool wave_has = __ballot(any_local) != 0ull;
  const uint64_t lt = lanemask_lt();
  for (int e = 0; e < L; ++e) {
    int c = 0;
    if (wave_has) {
      bool has = false;
#pragma unroll
      for (int j = 0; j < MOE_KMAX; ++j) has |= le[j] == e;
      const uint64_t m = __ballot(has);
      c = __popcll(m);
      const int below = __popcll(m & lt);
#pragma unroll
      for (int j = 0; j < MOE_KMAX; ++j)
        if (le[j] == e) rank[j] = below;
    }
    if (lane == 0) wave_cnt[wv * L + e] = c;
  }
  __syncthreads();
  if (t >= T) return;
#pragma unroll
  for (int j = 0; j < MOE_KMAX; ++j) {
    if (j >= k) break;
    const size_t o = (size_t)t * k + j;
    const int e = le[j];
    if (e < 0) {
      pair_row[o] = -1;
      continue;
    }
    int n = block_base[(size_t)blockIdx.x * L + e] + rank[j];
    for (int v = 0; v < wv; ++v) n += wave_cnt[v * L + e];
    const int R = rep ? min(max(rep[e], 1), max_rep) : 1;
    const int p = l2p ? l2p[e * max_rep + (n % R)] : e;
    if (p < 0 || p >= P) {                   // a map entry out of range:
      pair_row[o] = -1;                      // the pair is dropped
      continue;
    }
    const int row = offsets[p] + n / R;
    pair_row[o] = row;
    row_token[row] = t;
    row_weight[row] = w[o];
  }
}

// ----------------------------------------- single-workgroup small batch
// For T <= 1024 one workgroup (one thread per token) does everything the
// three kernels above do, plus the expert counts over all E and, when asked,
// the expert FFN's tile list: fewer dependent launches on the decode path.
// Same positions as the multi-block path: the pair's rank inside its
// 64-token wavefront comes from a ballot, earlier wavefronts from LDS.
static constexpr int kSmallT = 1024, kSmallL = 256;

bool dispatch_small_ok(int T, int E, int L, int P) {
  return T <= kSmallT && L <= kSmallL && E <= MOE_EMAX && P <= MOE_LMAX;
}

__global__ __launch_bounds__(1024) void k_dispatch_small(DispatchArgs a,
                                                         SmallExtras x) {
  __shared__ int32_t cnt[MOE_EMAX];
  __shared__ int32_t pc[MOE_LMAX + 1];
  __shared__ int32_t tb[MOE_LMAX + 2];
  __shared__ int32_t wpre[16 * kSmallL];
  const int t = threadIdx.x, wv = t >> 6, lane = t & 63;
  const int T = a.T, k = a.k, L = a.num_local, P = a.P;
  for (int i = t; i < x.E; i += 1024) cnt[i] = 0;
  for (int i = t; i <= P; i += 1024) pc[i] = 0;
  __syncthreads();
  int le[MOE_KMAX], rank[MOE_KMAX];
  bool any_local = false;
#pragma unroll
  for (int j = 0; j < MOE_KMAX; ++j) {
    le[j] = -1;
    rank[j] = 0;
    if (j < k && t < T) {
      const int gid = a.ids[(size_t)t * k + j];
      atomicAdd(&cnt[gid], 1);
      const int e = gid - a.expert_begin;
      if (e >= 0 && e < L) {
        le[j] = e;
        any_local = true;
      }
    }
  }
  const bool wave_has = __ballot(any_local) != 0ull;
  const uint64_t lt = lanemask_lt();
  for (int e = 0; e < L; ++e) {
    int c = 0;
    if (wave_has) {
      bool has = false;
#pragma unroll
      for (int j = 0; j < MOE_KMAX; ++j) has |= le[j] == e;
      const uint64_t m = __ballot(has);
      c = __popcll(m);
      const int below = __popcll(m & lt);
#pragma unroll
      for (int j = 0; j < MOE_KMAX; ++j)
        if (le[j] == e) rank[j] = below;
    }
    if (lane == 0) wpre[wv * kSmallL + e] = c;
  }
  __syncthreads();
  if (x.counts)
    for (int i = t; i < x.E; i += 1024) x.counts[i] = cnt[i];
  if (t < L) {
    const int e = t;
    int run = 0;                           // exclusive prefix over wavefronts
    for (int v = 0; v < 16; ++v) {
      const int c = wpre[v * kSmallL + e];
      wpre[v * kSmallL + e] = run;
      run += c;
    }
    const int R = a.rep ? min(max(a.rep[e], 1), a.max_rep) : 1;
    for (int r = 0; r < R; ++r) {
      const int p = a.l2p ? a.l2p[e * a.max_rep + r] : e;
      if (p >= 0 && p < P) pc[p] = run > r ? (run - r + R - 1) / R : 0;
    }
  }
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int p = 0; p < P; ++p) {
      const int c = pc[p];
      pc[p] = run;
      a.offsets[p] = run;
      run += c;
    }
    pc[P] = run;
    a.offsets[P] = run;
    if (x.tiles) {                         // tile list of the expert FFN
      const int G = P + (x.has_shared ? 1 : 0);
      int nt = 0;
      for (int g = 0; g < G; ++g) {
        tb[g] = nt;
        const int rows = g < P ? pc[g + 1] - pc[g] : T;
        int per;
        nt += tile_split(rows, x.BM, x.balanced, &per);
      }
      tb[G] = nt;
      x.tile_count[0] = nt;
    }
  }
  __syncthreads();
  if (x.tiles) {
    const int G = P + (x.has_shared ? 1 : 0);
    for (int g = t; g < G; g += 1024) {
      const int start = g < P ? pc[g] : 0;
      const int rows = g < P ? pc[g + 1] - start : T;
      if (rows == 0) continue;
      int per;
      tile_split(rows, x.BM, x.balanced, &per);
      int i = tb[g];
      for (int r = 0; r < rows; r += per, ++i)
        x.tiles[i] = make_int4(g, start + r, min(per, rows - r), 0);
    }
  }
  if (t >= T) return;
#pragma unroll
  for (int j = 0; j < MOE_KMAX; ++j) {
    if (j >= k) break;
    const size_t o = (size_t)t * k + j;
    const int e = le[j];
    if (e < 0) {
      a.pair_row[o] = -1;
      continue;
    }
    const int n = wpre[wv * kSmallL + e] + rank[j];
    const int R = a.rep ? min(max(a.rep[e], 1), a.max_rep) : 1;
    const int p = a.l2p ? a.l2p[e * a.max_rep + (n % R)] : e;
    if (p < 0 || p >= P) {
      a.pair_row[o] = -1;
      continue;
    }
    const int row = pc[p] + n / R;
    a.pair_row[o] = row;
    a.row_token[row] = t;
    a.row_weight[row] = a.w[o];
  }
}

hipError_t launch_dispatch_small(const DispatchArgs& a, const SmallExtras& x,
                                 hipStream_t s) {
  k_dispatch_small<<<1, 1024, 0, s>>>(a, x);
  return hipGetLastError();
}

hipError_t launch_dispatch_index(const DispatchArgs& a, hipStream_t s) {
  const int nblk = dispatch_blocks(a.T);
  const size_t lds = sizeof(int32_t) * 4 * a.num_local;
  k_local_hist<<<nblk, 256, lds, s>>>(a.ids, a.T, a.k, a.expert_begin,
                                      a.num_local, a.block_counts);
  k_scan<<<1, 1024, 0, s>>>(a.block_counts, nblk, a.num_local, a.P,
                            a.max_rep, a.l2p, a.rep, a.block_base, a.offsets);
  k_permute<<<nblk, 256, lds, s>>>(a.ids, a.w, a.T, a.k, a.expert_begin,
                                   a.num_local, a.P, a.max_rep, a.l2p, a.rep,
                                   a.block_base, a.offsets, a.row_token,
                                   a.row_weight, a.pair_row);
  return hipGetLastError();
}

// ------------------------------------------------------------ row gather
// A persistent grid walks rows r < N (N read on the device); a workgroup
// copies one row with 16-byte loads and stores.
__global__ __launch_bounds__(256) void k_gather_rows(
    const u32x4_t* __restrict__ x, int row_vecs,
    const int32_t* __restrict__ row_token, const int32_t* __restrict__ n_rows,
    u32x4_t* __restrict__ out) {
  const int N = *n_rows;
  for (int r = blockIdx.x; r < N; r += gridDim.x) {
    const u32x4_t* src = x + (size_t)row_token[r] * row_vecs;
    u32x4_t* dst = out + (size_t)r * row_vecs;
    for (int c = threadIdx.x; c < row_vecs; c += blockDim.x) dst[c] = src[c];
  }
}

hipError_t launch_gather_rows(const void* x, size_t row_bytes,
                              const int32_t* row_token,
                              const int32_t* n_rows_dev, int cap, void* out,
                              hipStream_t s) {
  const int grid = cap < 4096 ? cap : 4096;
  if (grid <= 0) return hipSuccess;
  k_gather_rows<<<grid, 256, 0, s>>>((const u32x4_t*)x, (int)(row_bytes / 16),
                                     row_token, n_rows_dev, (u32x4_t*)out);
  return hipGetLastError();
}

// the same for rows of 4-byte words (fp8 scales: H/128 floats a row)
__global__ __launch_bounds__(256) void k_gather_words(
    const uint32_t* __restrict__ x, int row_words,
    const int32_t* __restrict__ row_token, const int32_t* __restrict__ n_rows,
    uint32_t* __restrict__ out) {
  const int N = *n_rows;
  const long total = (long)N * row_words;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (long)gridDim.x * blockDim.x) {
    const int r = (int)(i / row_words), c = (int)(i - (long)r * row_words);
    out[i] = x[(size_t)row_token[r] * row_words + c];
  }
}

hipError_t launch_gather_rows_words(const void* x, int row_words,
                                    const int32_t* row_token,
                                    const int32_t* n_rows_dev, int cap,
                                    void* out, hipStream_t s) {
  long work = (long)cap * row_words;
  long grid = (work + 255) / 256;
  if (grid > 2048) grid = 2048;
  if (grid <= 0) return hipSuccess;
  k_gather_words<<<(unsigned)grid, 256, 0, s>>>((const uint32_t*)x, row_words,
                                                row_token, n_rows_dev,
                                                (uint32_t*)out);
  return hipGetLastError();
}

// ----------------------------------------------------- FP8 quantisation
// One wavefront per (token, 128-channel group): amax over the group, scale
// amax/448 (1 if amax = 0), codes RNE(fl32(x / scale)) saturated.
__global__ __launch_bounds__(256) void k_quant_rows_fp8(
    const bf16_t* __restrict__ x, int T, int H, uint8_t* __restrict__ codes,
    float* __restrict__ scales) {
  const int G = H / 128;
  const long grp = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (grp >= (long)T * G) return;
  const long t = grp / G, g = grp % G;
  const bf16_t* src = x + t * H + g * 128;
  const uint32_t pair = *(const uint32_t*)(src + 2 * lane);
  const float v0 = bf16_to_f32((bf16_t)(pair & 0xFFFFu));
  const float v1 = bf16_to_f32((bf16_t)(pair >> 16));
  float amax = fmaxf(fabsf(v0), fabsf(v1));
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  const float sc = amax == 0.0f ? 1.0f : __fdiv_rn(amax, 448.0f);
  const uint8_t c0 = f32_to_e4m3(__fdiv_rn(v0, sc));
  const uint8_t c1 = f32_to_e4m3(__fdiv_rn(v1, sc));
  *(uint16_t*)(codes + t * H + g * 128 + 2 * lane) =
      (uint16_t)c0 | ((uint16_t)c1 << 8);
  if (lane == 0) scales[t * G + g] = sc;
}

hipError_t launch_quant_rows_fp8(const bf16_t* x, int T, int H,
                                 uint8_t* codes, float* scales,
                                 hipStream_t s) {
  const long groups = (long)T * (H / 128);
  if (groups == 0) return hipSuccess;
  k_quant_rows_fp8<<<(unsigned)((groups + 3) / 4), 256, 0, s>>>(x, T, H, codes,
                                                               scales);
  return hipGetLastError();
}

// One workgroup per 128x128 block of a float32 matrix.
__global__ __launch_bounds__(256) void k_quant_blocks_fp8(
    const float* __restrict__ w, int rows, int cols,
    uint8_t* __restrict__ codes, float* __restrict__ scales) {
  __shared__ float red[4];
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
  if (threadIdx.x == 0) scales[blockIdx.x] = sc;
}

hipError_t launch_quant_blocks_fp8(const float* w, int rows, int cols,
                                   uint8_t* codes, float* scales,
                                   hipStream_t s) {
  const int nb = (rows / 128) * (cols / 128);
  if (nb == 0) return hipSuccess;
  k_quant_blocks_fp8<<<nb, 256, 0, s>>>(w, rows, cols, codes, scales);
  return hipGetLastError();
}

__global__ void k_fill_i32(int32_t* p, int32_t v, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int32_t v, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t g = (n + 255) / 256;
  if (g > 1024) g = 1024;
  k_fill_i32<<<(unsigned)g, 256, 0, s>>>(p, v, n);
  return hipGetLastError();
}

}  // namespace moe
