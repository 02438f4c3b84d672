// Grouped SwiGLU expert FFN ("6.4 Data parallelism and expert parallelism",
// section 2.1: an expert is gate, up and down; section 3.1, step 3: each card
// runs its experts on the tokens it received).
//
// Work is described by a device-built tile list: every physical expert's
// segment [offsets[p], offsets[p+1]) is cut into tiles of at most BM rows,
// and the shared expert (group P) into tiles over its T token rows.  A
// persistent grid walks (tile, column block) items, so a hot expert with
// many rows simply owns more tiles and spreads over all CUs, and an expert
// with no rows owns none and its weights are never read.
//
// bf16 weights arrive in the packed operand layout written by
// moe_prepack_weights: a matrix stored output-major [R][C] (C = reduction) is
// cut into 16 x 32 blocks, block (r/16, c/32) stored at block index
// (r/16) * (C/32) + c/32, 1 KiB each, and inside a block lane
// L = r%16 + 16 * ((c%32)/8) holds the 8 consecutive values c%8 = 0..7.  A
// block is exactly one wavefront's operand of v_mfma_f32_16x16x32_bf16, so a
// 16-B load per lane reads 1 KiB of contiguous memory, and 16 output
// channels over the whole reduction are one contiguous run.
//
// bf16 kernels on the tile list:
//  * k_stream_bf16 (groups of a few rows, decode): each wavefront streams its
//    16 output channels' contiguous run straight into MFMA operand registers
//    with non-temporal loads, one 128-wide K chunk ahead; every weight byte
//    is read once per tile.
//  * k_gemm_bf16 (gemm_bf16.hip; groups of hundreds of rows, prefill): the
//    256 x 256 LDS-ring GEMM for gate/up and down.
//  * k_tile_bf16_down: 128 rows x 128 columns per workgroup, double-buffered LDS
//    holding operand blocks in lane order (conflict-free 16-B reads, no
//    padding), 2x2 wavefronts of 64 x 64; the down pass when H is not a
//    multiple of 256.
// The gate/up pass ends in the fused epilogue h = silu(g) * u rounded to
// bf16; the down pass writes y in float32.
//
// MFMA operand convention (16x16x32 bf16): lane l supplies row (A) or column
// (B) l % 16 and the 8 K-values of K-slot l / 16; the accumulator of lane l
// holds rows 4 * (l / 16) + i, i < 4, of column l % 16.
#include "common.h"

namespace moe {

enum { MODE_GATEUP = 0, MODE_DOWN = 1 };

struct KArgs {
  const int4* tiles;
  const int32_t* tile_count;
  int nb_per_tile;            // column blocks per tile
  int K, N;                   // reduction and output width
  int P, cap;
  const void* a_routed;       // rows of the routed groups ([cap][K], or [T][K]
  const int32_t* a_rows;      //   indexed through a_rows[r] when non-null)
  const void* a_shared;       // [T][K] rows of the shared expert
  const void* const* w0_arr;  // gate (or down) per physical expert
  const void* const* w1_arr;  // up per physical expert
  const void* w0_sh;
  const void* w1_sh;
  void* h_out;                // gate/up output [cap + T][N]
  float* y_routed;            // down output [cap][N]
  float* y_shared;            // down output [T][N]
};

// ------------------------------------------------------------ tile list
// One workgroup.  Group g < P has offsets[g+1]-offsets[g] rows starting at
// row offsets[g]; group P (shared) has T rows starting at 0.  Output:
// tiles[i] = {group, first row, rows, 0}, count[0] = number of tiles.
// Writes the tile list for tiles of BM rows (balanced: tile_split's
// near-equal tiles) and, when tiles2 is non-null, a second plain list for
// tiles of BM2 rows, each with its count.
__global__ __launch_bounds__(1024) void k_build_tiles(
    const int32_t* __restrict__ offsets, int P, int has_shared, int T, int BM,
    int balanced, int4* __restrict__ tiles, int32_t* __restrict__ count,
    int BM2, int4* __restrict__ tiles2, int32_t* __restrict__ count2) {
  __shared__ int32_t base[2][MOE_LMAX + 2];
  const int G = P + (has_shared ? 1 : 0);
  for (int g = threadIdx.x; g < G; g += blockDim.x) {
    const int rows = g < P ? offsets[g + 1] - offsets[g] : T;
    int per;
    base[0][g + 1] = tile_split(rows, BM, balanced, &per);
    base[1][g + 1] = (rows + BM2 - 1) / BM2;
  }
  __syncthreads();
  if (threadIdx.x < 2) {
    int32_t* b = base[threadIdx.x];
    b[0] = 0;
    for (int g = 0; g < G; ++g) b[g + 1] += b[g];
    if (threadIdx.x == 0) count[0] = b[G];
    else if (tiles2) count2[0] = b[G];
  }
  __syncthreads();
  for (int g = threadIdx.x; g < G; g += blockDim.x) {
    const int start = g < P ? offsets[g] : 0;
    const int rows = g < P ? offsets[g + 1] - start : T;
    int per;
    tile_split(rows, BM, balanced, &per);
    int i = base[0][g];
    for (int r = 0; r < rows; r += per, ++i)
      tiles[i] = make_int4(g, start + r, min(per, rows - r), 0);
    if (tiles2) {
      i = base[1][g];
      for (int r = 0; r < rows; r += BM2, ++i)
        tiles2[i] = make_int4(g, start + r, min(BM2, rows - r), 0);
    }
  }
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ u32x4_t load_nt(const u32x4_t* p) {
  return __builtin_nontemporal_load(p);
}

// Row of the A operand for tile row `row` of a group.
__device__ __forceinline__ const bf16_t* a_row(const KArgs& a, bool sh,
                                               int row) {
  if (sh) return (const bf16_t*)a.a_shared + (size_t)row * a.K;
  const int src = a.a_rows ? a.a_rows[row] : row;
  return (const bf16_t*)a.a_routed + (size_t)src * a.K;
}

// Store a 16x16 accumulator block (lane layout above).
template <int MODE>
__device__ __forceinline__ void store_block(const KArgs& a, bool sh, int row0,
                                            int nrows, int rbase, int n,
                                            f32x4_t g, f32x4_t u) {
  const int q = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = rbase + 4 * q + i;
    if (r >= nrows) continue;
    if (MODE == MODE_GATEUP) {
      const size_t hr = (size_t)(sh ? a.cap : 0) + row0 + r;
      ((bf16_t*)a.h_out)[hr * a.N + n] = f32_to_bf16(silu_f32(g[i]) * u[i]);
    } else {
      float* y = sh ? a.y_shared : a.y_routed;
      y[(size_t)(row0 + r) * a.N + n] = g[i];
    }
  }
}

// ---------------------------------------------- weight-streaming kernel
// Workgroup = 4 wavefronts; wavefront w streams two packed row blocks (16
// channels each) over the whole reduction: gate and up of block nb*4 + w
// (64 outputs an item), or down blocks nb*8 + w and nb*8 + w + 4 (128
// outputs an item), so every wavefront keeps two weight streams in flight.
// A tile has up to 16*NMB rows.  K chunk = 128 (4 MFMA steps), prefetched
// one chunk ahead.
template <int MODE, int NMB>
__global__ __launch_bounds__(256) void k_stream_bf16(KArgs a) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int c16 = lane & 15, q = lane >> 4;
  const int total = a.tile_count[0] * a.nb_per_tile;
  const int K = a.K, KB = K / 32;
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int tile = item / a.nb_per_tile;
    const int nb = item - tile * a.nb_per_tile;
    const int4 td = a.tiles[tile];
    const int g = td.x, row0 = td.y, nrows = td.z;
    const bool sh = g == a.P;
    const int nb16 = MODE == MODE_GATEUP ? nb * 4 + wv : nb * 8 + wv;
    const u32x4_t* b0p = (const u32x4_t*)(sh ? a.w0_sh : a.w0_arr[g]) +
                         (size_t)nb16 * KB * 64 + lane;
    const u32x4_t* b1p =
        MODE == MODE_GATEUP
            ? (const u32x4_t*)(sh ? a.w1_sh : a.w1_arr[g]) + (size_t)nb16 * KB * 64 + lane
            : b0p + (size_t)4 * KB * 64;        // down: the block 64 channels on
    const bf16_t* ap[NMB];
    bool av[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      const int r = mb * 16 + c16;
      av[mb] = r < nrows;
      ap[mb] = a_row(a, sh, row0 + (av[mb] ? r : 0)) + 8 * q;
    }
    const int nmb = (nrows + 15) >> 4;   // active row blocks (uniform)
    f32x4_t acc0[NMB], acc1[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      acc0[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      acc1[mb] = acc0[mb];
    }
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    u32x4_t b0c[4], b1c[4], acur[NMB][4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      b0c[s] = load_nt(b0p + s * 64);
      b1c[s] = load_nt(b1p + s * 64);
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
        acur[mb][s] = av[mb] ? *(const u32x4_t*)(ap[mb] + 32 * s) : zero;
    }
    for (int k0 = 0; k0 < K; k0 += 128) {
      u32x4_t b0n[4], b1n[4], anext[NMB][4];
      const bool more = k0 + 128 < K;
      if (more) {
        const int kb = (k0 + 128) / 32;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          b0n[s] = load_nt(b0p + (kb + s) * 64);
          b1n[s] = load_nt(b1p + (kb + s) * 64);
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb)
            anext[mb][s] = av[mb] ? *(const u32x4_t*)(ap[mb] + k0 + 128 + 32 * s) : zero;
        }
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
          if (mb < nmb) {
            acc0[mb] = mfma16(acur[mb][s], b0c[s], acc0[mb]);
            acc1[mb] = mfma16(acur[mb][s], b1c[s], acc1[mb]);
          }
        }
      }
      if (more) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          b0c[s] = b0n[s];
          b1c[s] = b1n[s];
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb) acur[mb][s] = anext[mb][s];
        }
      }
    }
    const int n = nb16 * 16 + c16;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      if (mb >= nmb) continue;
      store_block<MODE>(a, sh, row0, nrows, mb * 16, n, acc0[mb], acc1[mb]);
      if (MODE == MODE_DOWN)
        store_block<MODE>(a, sh, row0, nrows, mb * 16, n + 64, acc1[mb], acc1[mb]);
    }
  }
}

// ----------------------------------------------------- LDS-tiled kernel
// Down tile: 128 rows x 128 outputs, BK = 64 (two MFMA steps).  LDS holds,
// per stage, the A operand as 8 row blocks x 2 steps and the B operand as
// 8 column blocks x 2 steps, each a 1 KiB lane-ordered block, so every
// fragment read is one conflict-free ds_read_b128 at lane * 16 bytes.
// Wavefront (wm, wn) of a 2x2 grid owns 64 rows x 64 B-columns.
static constexpr int TBM = 128, TBK = 64;

__global__ __launch_bounds__(256) void k_tile_bf16_down(KArgs a) {
  __shared__ u32x4_t lds_a[2][16 * 64];
  __shared__ u32x4_t lds_b[2][16 * 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int K = a.K, KB = K / 32;
  const int total = a.tile_count[0] * a.nb_per_tile;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int tile = item / a.nb_per_tile;
    const int nb = item - tile * a.nb_per_tile;
    const int4 td = a.tiles[tile];
    const int g = td.x, row0 = td.y, nrows = td.z;
    const bool sh = g == a.P;
    // Staging: chunk c = tid + 256 j (j < 4) is block c/64 = 4j + wv,
    // lane c%64.  A block b = (row block b/2, step b%2); B block b = (column
    // block b/2, step b%2).
    const bf16_t* ga[4];
    const u32x4_t* gb[4];
    bool va[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int blk = 4 * j + wv;
      const int r = (blk >> 1) * 16 + (lane & 15);
      va[j] = r < nrows;
      ga[j] = a_row(a, sh, row0 + (va[j] ? r : 0)) + (blk & 1) * 32 + (lane >> 4) * 8;
      const int cb = blk >> 1;           // local column block 0..7
      const u32x4_t* W = (const u32x4_t*)(sh ? a.w0_sh : a.w0_arr[g]);
      const int nb16 = nb * 8 + cb;
      gb[j] = W + ((size_t)nb16 * KB + (blk & 1)) * 64 + lane;
    }
    u32x4_t ra[4], rb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ra[j] = va[j] ? *(const u32x4_t*)ga[j] : zero;
      rb[j] = gb[j][0];
    }
    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int nmb_valid = (nrows - wm * 64 + 15) >> 4;   // may be <= 0
    __syncthreads();   // the previous item's readers are done with LDS
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lds_a[0][tid + 256 * j] = ra[j];
      lds_b[0][tid + 256 * j] = rb[j];
    }
    __syncthreads();
    const int KT = K / TBK;
    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < KT;
      if (more) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ra[j] = va[j] ? *(const u32x4_t*)(ga[j] + (kt + 1) * TBK) : zero;
          rb[j] = gb[j][(size_t)(kt + 1) * 2 * 64];
        }
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        u32x4_t fa[4], fb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = lds_a[cur][((wm * 4 + i) * 2 + s) * 64 + lane];
#pragma unroll
        for (int j = 0; j < 4; ++j) fb[j] = lds_b[cur][((wn * 4 + j) * 2 + s) * 64 + lane];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i < nmb_valid)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(fa[i], fb[j], acc[i][j]);
      }
      if (more) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          lds_a[cur ^ 1][tid + 256 * j] = ra[j];
          lds_b[cur ^ 1][tid + 256 * j] = rb[j];
        }
      }
      __syncthreads();
    }
    const int c16 = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= nmb_valid) continue;
      const int rbase = wm * 64 + i * 16;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = nb * 128 + wn * 64 + j * 16 + c16;
        store_block<MODE_DOWN>(a, sh, row0, nrows, rbase, n, acc[i][j], acc[i][j]);
      }
    }
  }
}

// --------------------------------------------------------- fp32 recipe
// Plain float32 FMA kernels on natural output-major weights: one thread per
// (row, output channel).
template <int MODE>
__global__ __launch_bounds__(256) void k_f32(KArgs a) {
  const int total_tiles = a.tile_count[0];
  const long per_tile = (long)TBM * a.N;    // tiles of up to TBM rows
  const long total = (long)total_tiles * per_tile;
  for (long it = (long)blockIdx.x * blockDim.x + threadIdx.x; it < total;
       it += (long)gridDim.x * blockDim.x) {
    const int tile = (int)(it / per_tile);
    const int rem = (int)(it - (long)tile * per_tile);
    const int r = rem / a.N, n = rem - r * a.N;
    const int4 td = a.tiles[tile];
    if (r >= td.z) continue;
    const int g = td.x, row = td.y + r;
    const bool sh = g == a.P;
    const float* A;
    if (sh) A = (const float*)a.a_shared + (size_t)row * a.K;
    else A = (const float*)a.a_routed + (size_t)(a.a_rows ? a.a_rows[row] : row) * a.K;
    const float* W0 = (const float*)(sh ? a.w0_sh : a.w0_arr[g]) + (size_t)n * a.K;
    if (MODE == MODE_GATEUP) {
      const float* W1 = (const float*)(sh ? a.w1_sh : a.w1_arr[g]) + (size_t)n * a.K;
      float gs = 0.f, us = 0.f;
      for (int kk = 0; kk < a.K; ++kk) {
        gs = __builtin_fmaf(A[kk], W0[kk], gs);
        us = __builtin_fmaf(A[kk], W1[kk], us);
      }
      const size_t hr = (size_t)(sh ? a.cap : 0) + row;
      ((float*)a.h_out)[hr * a.N + n] = silu_f32(gs) * us;
    } else {
      float ys = 0.f;
      for (int kk = 0; kk < a.K; ++kk) ys = __builtin_fmaf(A[kk], W0[kk], ys);
      float* y = sh ? a.y_shared : a.y_routed;
      y[(size_t)row * a.N + n] = ys;
    }
  }
}

// ------------------------------------------------------- weight packing
// Natural output-major bf16 [R][C] -> packed 16 x 32 operand blocks (see the
// top of this file).  One thread per 16-byte output chunk.
__global__ __launch_bounds__(256) void k_pack_bf16(const bf16_t* __restrict__ src,
                                                   int R, int C,
                                                   u32x4_t* __restrict__ dst) {
  const size_t total = (size_t)R * C / 8;
  const int CB = C / 32;
  for (size_t gi = (size_t)blockIdx.x * 256 + threadIdx.x; gi < total;
       gi += (size_t)gridDim.x * 256) {
    const size_t blk = gi >> 6;
    const int lane = (int)(gi & 63);
    const size_t rb = blk / CB, cb = blk - rb * CB;
    const size_t r = rb * 16 + (lane & 15), c = cb * 32 + (lane >> 4) * 8;
    dst[gi] = *(const u32x4_t*)(src + r * C + c);
  }
}

hipError_t launch_pack_bf16(const bf16_t* src, int R, int C, void* dst,
                            hipStream_t s) {
  const size_t total = (size_t)R * C / 8;
  if (total == 0) return hipSuccess;
  size_t grid = (total + 255) / 256;
  if (grid > 8192) grid = 8192;
  k_pack_bf16<<<(unsigned)grid, 256, 0, s>>>(src, R, C, (u32x4_t*)dst);
  return hipGetLastError();
}

// -------------------------------------------------------------- driver
// Kernel choice for the bf16 recipe: the weight-streaming kernel for a few
// rows per group; for hundreds (prefill) the 256 x 256 LDS-ring GEMM on
// balanced tiles of up to 256 rows for gate/up and, when H % 256 == 0, for
// down (else the 128 x 128 tiled kernel on its own list of 128-row tiles).
static bool bf16_streaming(int rows_hint) { return rows_hint <= 32; }

int ffn_tile_rows(int act, int wdt, int rows_hint, int H, int I, int* balanced) {
  *balanced = 0;
  if (wdt == MOE_FP8_E4M3) return ffn_fp8_tile_rows(rows_hint, H, I, balanced);
  if (act == MOE_F32) return TBM;
  if (bf16_streaming(rows_hint)) return 32;
  *balanced = 1;
  return gemm_tile_rows();
}

hipError_t launch_build_tiles(const int32_t* offsets, int P, int has_shared,
                              int T, int BM, int balanced, int4* tiles,
                              int32_t* count, hipStream_t s) {
  k_build_tiles<<<1, 1024, 0, s>>>(offsets, P, has_shared, T, BM, balanced,
                                   tiles, count, BM, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_ffn(FfnArgs& f, hipStream_t s) {
  if (f.wdt == MOE_FP8_E4M3) return launch_ffn_fp8(f, s);
  const int G = f.P + (f.has_shared ? 1 : 0);
  if (G == 0) return hipSuccess;
  // The expected rows per routed group choose the kernel: a few rows per
  // expert (decode) stream the weights; hundreds (prefill) tile through LDS.
  const bool f32 = f.act == MOE_F32;
  int balanced;
  const int BM = ffn_tile_rows(f.act, f.wdt, f.rows_hint, f.H, f.I, &balanced);
  const bool stream = !f32 && BM == 32;
  const bool ring = !f32 && balanced;     // tiles of up to 256 rows
  // the ring GEMM's list (or the only list), plus down's 128-row list when
  // down runs the 128 x 128 tile kernel (H not a multiple of 256); a list
  // already written by the dispatch is the first one
  const bool down_list = ring && f.H % 256 != 0;
  if (!f.tiles_ready)
    k_build_tiles<<<1, 1024, 0, s>>>(f.offsets, f.P, f.has_shared, f.T, BM,
                                     balanced, f.tiles, f.tile_count, TBM,
                                     down_list ? f.tiles_down : nullptr,
                                     f.tile_count + 1);
  else if (down_list)
    k_build_tiles<<<1, 1024, 0, s>>>(f.offsets, f.P, f.has_shared, f.T, TBM, 0,
                                     f.tiles_down, f.tile_count + 1, TBM,
                                     nullptr, nullptr);
  if (f.events) hipEventRecord(f.events[0], s);
  // bound on the tile count for the grid size
  const long hrows = (long)f.cap + (f.has_shared ? f.T : 0);
  const long max_tiles = G + hrows / BM + 1;

  KArgs a{};
  a.tiles = f.tiles;
  a.tile_count = f.tile_count;
  a.P = f.P;
  a.cap = f.cap;
  const moe_weights* w = f.w;
  // ---- gate/up
  a.K = f.H;
  a.N = f.I;
  a.a_routed = f.a_routed;
  a.a_rows = f.a_rows;
  a.a_shared = f.a_shared;
  a.w0_arr = w->w_gate;
  a.w1_arr = w->w_up;
  a.w0_sh = w->sh_gate;
  a.w1_sh = w->sh_up;
  a.h_out = f.h;
  const int cu = 256;
  if (f32) {
    long work = max_tiles * TBM * (long)a.N;
    long grid = (work + 255) / 256;
    if (grid > cu * 8) grid = cu * 8;
    k_f32<MODE_GATEUP><<<(unsigned)grid, 256, 0, s>>>(a);
  } else if (stream) {
    a.nb_per_tile = a.N / 64;
    long items = max_tiles * a.nb_per_tile;
    // persistent: the two workgroups a CU holds at this kernel's registers
    long grid = items < cu * 2 ? items : cu * 2;
    k_stream_bf16<MODE_GATEUP, 2><<<(unsigned)grid, 256, 0, s>>>(a);
  } else {                                  // ring: bf16 beyond streaming
    hipError_t e = launch_gemm_bf16_gateup(f, s);
    if (e != hipSuccess) return e;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (f.events) hipEventRecord(f.events[1], s);
  // ---- down
  const size_t hb = f32 ? 4 : 2;
  a.K = f.I;
  a.N = f.H;
  a.a_routed = f.h;
  a.a_rows = nullptr;
  a.a_shared = (const char*)f.h + (size_t)f.cap * f.I * hb;
  a.w0_arr = w->w_down;
  a.w1_arr = nullptr;
  a.w0_sh = w->sh_down;
  a.w1_sh = nullptr;
  a.y_routed = f.y_routed;
  a.y_shared = f.y_shared;
  if (f32) {
    long work = max_tiles * TBM * (long)a.N;
    long grid = (work + 255) / 256;
    if (grid > cu * 8) grid = cu * 8;
    k_f32<MODE_DOWN><<<(unsigned)grid, 256, 0, s>>>(a);
  } else if (stream) {
    a.nb_per_tile = a.N / 128;                // two 64-apart blocks per wave
    long items = max_tiles * a.nb_per_tile;
    // persistent: the two workgroups a CU holds at this kernel's registers
    long grid = items < cu * 2 ? items : cu * 2;
    k_stream_bf16<MODE_DOWN, 2><<<(unsigned)grid, 256, 0, s>>>(a);
  } else if (ring && f.H % 256 == 0) {
    hipError_t e = launch_gemm_bf16_down(f, s);
    if (e != hipSuccess) return e;
  } else {
    if (ring) {
      a.tiles = f.tiles_down;
      a.tile_count = f.tile_count + 1;
    }
    a.nb_per_tile = a.N / 128;
    const long tiles_down = ring ? G + hrows / TBM + 1 : max_tiles;
    long items = tiles_down * a.nb_per_tile;
    long grid = items < cu * 2 ? items : cu * 2;
    k_tile_bf16_down<<<(unsigned)grid, 256, 0, s>>>(a);
  }
  if (f.events) hipEventRecord(f.events[2], s);
  return hipGetLastError();
}

}  // namespace moe
