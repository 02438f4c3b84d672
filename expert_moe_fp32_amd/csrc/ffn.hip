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
// Two bf16 kernels share the tile list:
//  * k_stream_bf16 (groups of a few rows, decode): weights go straight from
//    HBM into MFMA operand registers, each lane loading 64 contiguous bytes
//    of one output channel per 128-wide K chunk, one chunk ahead; every weight
//    byte is read once per tile.
//  * k_tile_bf16 (groups of hundreds of rows, prefill): 128-row x 128-column
//    tiles staged through double-buffered LDS, 2x2 wavefronts of 64x64.
// Both use v_mfma_f32_16x16x32_bf16 with fp32 accumulation; the gate/up pass
// ends in the fused epilogue h = silu(g) * u rounded to bf16, the down pass
// writes y in float32.
//
// MFMA operand convention: for one 16x16x32 step, lane l supplies row (or
// column) l % 16 and the 8 K-values of K-slot l / 16.  The K-values a lane
// carries are the same set for the A and the B operand, so the product sums
// every K index exactly once whatever order the slots take; this lets a lane
// read one contiguous run of K for several steps.  The accumulator of lane l
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
  const void* a_routed;       // [cap][K] rows of the routed groups
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
__global__ __launch_bounds__(1024) void k_build_tiles(
    const int32_t* __restrict__ offsets, int P, int has_shared, int T, int BM,
    int4* __restrict__ tiles, int32_t* __restrict__ count) {
  __shared__ int32_t base[MOE_LMAX + 2];
  const int G = P + (has_shared ? 1 : 0);
  for (int g = threadIdx.x; g < G; g += blockDim.x) {
    const int rows = g < P ? offsets[g + 1] - offsets[g] : T;
    base[g + 1] = (rows + BM - 1) / BM;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    base[0] = 0;
    for (int g = 0; g < G; ++g) base[g + 1] += base[g];
    count[0] = base[G];
  }
  __syncthreads();
  for (int g = threadIdx.x; g < G; g += blockDim.x) {
    const int start = g < P ? offsets[g] : 0;
    const int rows = g < P ? offsets[g + 1] - start : T;
    int i = base[g];
    for (int r = 0; r < rows; r += BM, ++i)
      tiles[i] = make_int4(g, start + r, min(BM, rows - r), 0);
  }
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c,
                                                 0, 0, 0);
}

// Epilogue helpers: store a 16x16 accumulator block (lane layout above).
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
// Workgroup = 4 wavefronts = 64 output columns; wavefront = 16 columns; a
// tile has up to 16*NMB rows.  K chunk = 128 (4 MFMA steps); lane (c, q)
// reads K range [k0 + 32q, k0 + 32q + 32) of its row / column.
template <int MODE, int NMB>
__global__ __launch_bounds__(256) void k_stream_bf16(KArgs a) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int c16 = lane & 15, q = lane >> 4;
  const int total = a.tile_count[0] * a.nb_per_tile;
  const int K = a.K;
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int tile = item / a.nb_per_tile;
    const int nb = item - tile * a.nb_per_tile;
    const int4 td = a.tiles[tile];
    const int g = td.x, row0 = td.y, nrows = td.z;
    const bool sh = g == a.P;
    const bf16_t* A = (const bf16_t*)(sh ? a.a_shared : a.a_routed);
    const bf16_t* W0 = (const bf16_t*)(sh ? a.w0_sh : a.w0_arr[g]);
    const bf16_t* W1 = nullptr;
    if (MODE == MODE_GATEUP) W1 = (const bf16_t*)(sh ? a.w1_sh : a.w1_arr[g]);
    const int n = nb * 64 + wv * 16 + c16;
    const u32x4_t* b0p = (const u32x4_t*)(W0 + (size_t)n * K + 32 * q);
    const u32x4_t* b1p = (const u32x4_t*)(W1 + (size_t)n * K + 32 * q);
    const u32x4_t* ap[NMB];
    bool av[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      const int r = mb * 16 + c16;
      av[mb] = r < nrows;
      ap[mb] = (const u32x4_t*)(A + (size_t)(row0 + (av[mb] ? r : 0)) * K + 32 * q);
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
      b0c[s] = b0p[s];
      if (MODE == MODE_GATEUP) b1c[s] = b1p[s];
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) acur[mb][s] = av[mb] ? ap[mb][s] : zero;
    }
    for (int k0 = 0; k0 < K; k0 += 128) {
      u32x4_t b0n[4], b1n[4], anext[NMB][4];
      const bool more = k0 + 128 < K;
      if (more) {
        const int o = (k0 + 128) / 8;     // in u32x4 units
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          b0n[s] = b0p[o + s];
          if (MODE == MODE_GATEUP) b1n[s] = b1p[o + s];
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb)
            anext[mb][s] = av[mb] ? ap[mb][o + s] : zero;
        }
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
          if (mb < nmb) {
            acc0[mb] = mfma16(acur[mb][s], b0c[s], acc0[mb]);
            if (MODE == MODE_GATEUP) acc1[mb] = mfma16(acur[mb][s], b1c[s], acc1[mb]);
          }
        }
      }
      if (more) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          b0c[s] = b0n[s];
          if (MODE == MODE_GATEUP) b1c[s] = b1n[s];
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb) acur[mb][s] = anext[mb][s];
        }
      }
    }
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      if (mb < nmb) store_block<MODE>(a, sh, row0, nrows, mb * 16, n, acc0[mb], acc1[mb]);
  }
}

// ----------------------------------------------------- LDS-tiled kernel
// Tile: BM = 128 rows x 128 B-columns (gate/up: 64 gate + 64 up channels of
// the same 64 outputs; down: 128 outputs), BK = 64, double-buffered LDS with
// rows padded to 72 elements (conflict-free 16-byte reads for 16 lanes).
// Wavefront (wm, wn) of a 2x2 grid owns 64 rows x 64 B-columns.
static constexpr int TBM = 128, TBN = 128, TBK = 64, TLD = 72;

template <int MODE>
__global__ __launch_bounds__(256) void k_tile_bf16(KArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t lds_a[2][TBM * TLD];
  __shared__ __attribute__((aligned(16))) bf16_t lds_b[2][TBN * TLD];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int c16 = lane & 15, q = lane >> 4;
  const int K = a.K;
  const int total = a.tile_count[0] * a.nb_per_tile;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int tile = item / a.nb_per_tile;
    const int nb = item - tile * a.nb_per_tile;
    const int4 td = a.tiles[tile];
    const int g = td.x, row0 = td.y, nrows = td.z;
    const bool sh = g == a.P;
    const bf16_t* A = (const bf16_t*)(sh ? a.a_shared : a.a_routed);
    const bf16_t* W0 = (const bf16_t*)(sh ? a.w0_sh : a.w0_arr[g]);
    const bf16_t* W1 = W0;
    if (MODE == MODE_GATEUP) W1 = (const bf16_t*)(sh ? a.w1_sh : a.w1_arr[g]);
    // global source of the 4 16-byte chunks this thread stages per operand:
    // chunk c = tid + 256 j covers row c / 8, columns 8 (c % 8) .. + 8
    const u32x4_t* ga[4];
    const u32x4_t* gb[4];
    bool va[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = tid + 256 * j;
      const int r = c >> 3, col = (c & 7) * 8;
      va[j] = r < nrows;
      ga[j] = (const u32x4_t*)(A + (size_t)(row0 + (va[j] ? r : 0)) * K + col);
      int wrow;
      const bf16_t* W;
      if (MODE == MODE_GATEUP) {       // rows 0..63 gate, 64..127 up
        W = r < 64 ? W0 : W1;
        wrow = nb * 64 + (r & 63);
      } else {
        W = W0;
        wrow = nb * 128 + r;
      }
      gb[j] = (const u32x4_t*)(W + (size_t)wrow * K + col);
    }
    u32x4_t ra[4], rb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ra[j] = va[j] ? ga[j][0] : zero;
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
      const int c = tid + 256 * j;
      *(u32x4_t*)&lds_a[0][(c >> 3) * TLD + (c & 7) * 8] = ra[j];
      *(u32x4_t*)&lds_b[0][(c >> 3) * TLD + (c & 7) * 8] = rb[j];
    }
    __syncthreads();
    const int KT = K / TBK;
    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < KT;
      if (more) {
        const int o = (kt + 1) * TBK / 8;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ra[j] = va[j] ? ga[j][o] : zero;
          rb[j] = gb[j][o];
        }
      }
      // two MFMA steps over BK = 64: lane reads 32 contiguous bytes per row
      u32x4_t fa[4][2], fb[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16_t* pa = &lds_a[cur][(wm * 64 + i * 16 + c16) * TLD + 16 * q];
        fa[i][0] = *(const u32x4_t*)pa;
        fa[i][1] = *(const u32x4_t*)(pa + 8);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int brow;
        if (MODE == MODE_GATEUP)          // j 0,1: gate; j 2,3: up
          brow = (j >> 1) * 64 + wn * 32 + (j & 1) * 16 + c16;
        else
          brow = wn * 64 + j * 16 + c16;
        const bf16_t* pb = &lds_b[cur][brow * TLD + 16 * q];
        fb[j][0] = *(const u32x4_t*)pb;
        fb[j][1] = *(const u32x4_t*)(pb + 8);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i < nmb_valid)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(fa[i][s], fb[j][s], acc[i][j]);
      if (more) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = tid + 256 * j;
          *(u32x4_t*)&lds_a[cur ^ 1][(c >> 3) * TLD + (c & 7) * 8] = ra[j];
          *(u32x4_t*)&lds_b[cur ^ 1][(c >> 3) * TLD + (c & 7) * 8] = rb[j];
        }
      }
      __syncthreads();
    }
    // epilogue
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= nmb_valid) continue;
      const int rbase = wm * 64 + i * 16;
      if (MODE == MODE_GATEUP) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = nb * 64 + wn * 32 + j * 16 + c16;
          store_block<MODE>(a, sh, row0, nrows, rbase, n, acc[i][j], acc[i][j + 2]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = nb * 128 + wn * 64 + j * 16 + c16;
          store_block<MODE>(a, sh, row0, nrows, rbase, n, acc[i][j], acc[i][j]);
        }
      }
    }
  }
}

// --------------------------------------------------------- fp32 recipe
// Plain float32 FMA kernels: one thread per (row, output channel).
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
    const float* A = (const float*)(sh ? a.a_shared : a.a_routed) + (size_t)row * a.K;
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

// -------------------------------------------------------------- driver
size_t ffn_scratch_bytes(int H, int I, int P, int T, int cap, int has_shared,
                         int act, int wdt) {
  const size_t hrows = (size_t)cap + (has_shared ? T : 0);
  size_t hb = act == MOE_F32 ? 4 : (wdt == MOE_FP8_E4M3 ? 1 : 2);
  size_t b = moe_align256(hrows * I * hb);
  if (wdt == MOE_FP8_E4M3) b += moe_align256(hrows * (I / 128) * sizeof(float));
  // tiles: at most one per group plus one per 16 rows
  const size_t max_tiles = (size_t)P + 1 + (hrows + 15) / 16 + 1;
  b += moe_align256(max_tiles * sizeof(int4));
  b += 256;
  return b;
}

hipError_t launch_ffn(FfnArgs& f, hipStream_t s) {
  const int G = f.P + (f.has_shared ? 1 : 0);
  if (G == 0) return hipSuccess;
  // The expected rows per routed group decide the kernel: a few rows per
  // expert (decode) stream the weights; hundreds (prefill) tile through LDS.
  const bool f32 = f.act == MOE_F32;
  int BM;
  bool stream = false;
  if (f32) {
    BM = TBM;
  } else if (f.rows_hint <= 32) {
    BM = 32;
    stream = true;
  } else {
    BM = TBM;
  }
  k_build_tiles<<<1, 1024, 0, s>>>(f.offsets, f.P, f.has_shared, f.T, BM,
                                   f.tiles, f.tile_count);
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
    long grid = items < cu * 12 ? items : cu * 12;
    k_stream_bf16<MODE_GATEUP, 2><<<(unsigned)grid, 256, 0, s>>>(a);
  } else {
    a.nb_per_tile = a.N / 64;
    long items = max_tiles * a.nb_per_tile;
    long grid = items < cu * 2 ? items : cu * 2;
    k_tile_bf16<MODE_GATEUP><<<(unsigned)grid, 256, 0, s>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (f.events) hipEventRecord(f.events[1], s);
  // ---- down
  const size_t hb = f32 ? 4 : 2;
  a.K = f.I;
  a.N = f.H;
  a.a_routed = f.h;
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
    a.nb_per_tile = a.N / 64;
    long items = max_tiles * a.nb_per_tile;
    long grid = items < cu * 12 ? items : cu * 12;
    k_stream_bf16<MODE_DOWN, 2><<<(unsigned)grid, 256, 0, s>>>(a);
  } else {
    a.nb_per_tile = a.N / 128;
    long items = max_tiles * a.nb_per_tile;
    long grid = items < cu * 2 ? items : cu * 2;
    k_tile_bf16<MODE_DOWN><<<(unsigned)grid, 256, 0, s>>>(a);
  }
  if (f.events) hipEventRecord(f.events[2], s);
  return hipGetLastError();
}

}  // namespace moe
