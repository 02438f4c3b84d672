// FP8 (OCP E4M3) recipe of the grouped expert FFN.
//
// The infra-guide page ("6.4 Data parallelism and expert parallelism",
// section 3.2) sends tokens in FP8 and stores expert weights in FP8 (section
// 2.3); the workload fixes the granularity: weights carry one float32 scale
// per 128 x 128 block, activations one per token per 128 channels, and the
// intermediate h is quantised the same way per row before the down
// projection.  Everything accumulates in float32.
//
// v_mfma_scale_f32_16x16x128_f8f6f4 reduces over K = 128, exactly one scale
// block, so each MFMA starts from zero and its block sum is folded into the
// float32 accumulator as acc += sum * s_act[row] * s_w[block] (the MFMA's own
// power-of-two scale inputs are left at 1).
//
// Packed FP8 weight layout (moe_prepack_weights with MOE_FP8_E4M3): a matrix
// [R][C] of codes (C = reduction) is cut into 16 x 128 blocks of 2 KiB, block
// (r/16, c/128) stored at block index (r/16) * (C/128) + c/128.  Lane
// L = r%16 + 16 * ((c%128)/32) owns the 32 codes of its K-slot; their first
// 16 bytes sit at byte L*16 of the block and the next 16 at 1024 + L*16, so
// each half of a wavefront's operand is 1 KiB of contiguous memory and a
// conflict-free 16-byte LDS read per lane.
#include "common.h"

namespace moe {

struct K8Args {
  const int4* tiles;
  const int32_t* tile_count;
  int nb_per_tile;
  int K, N;                   // reduction, output width
  int P, cap;
  const uint8_t* a_routed;    // codes of routed rows ([cap][K], or through a_rows)
  const float* as_routed;     // their scales [*][K/128]
  const int32_t* a_rows;
  const uint8_t* a_shared;    // [T][K] codes of the shared expert's rows
  const float* as_shared;
  const void* const* w0_arr;  // packed codes: gate (or down)
  const void* const* w1_arr;  // up
  const float* const* s0_arr; // block scales [N/128][K/128]
  const float* const* s1_arr;
  const void* w0_sh;
  const void* w1_sh;
  const float* s0_sh;
  const float* s1_sh;
  float* h_out;               // gate/up: float32 h [cap + T][N]
  float* y_routed;            // down: [cap][N]
  float* y_shared;            // down: [T][N]
};

enum { M8_GATEUP = 0, M8_DOWN = 1 };

__device__ __forceinline__ f32x4_t mfma_fp8(i32x8_t a, i32x8_t b) {
  const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
      a, b, z, 0, 0, 0, 0x7f7f7f7f, 0, 0x7f7f7f7f);
}

__device__ __forceinline__ i32x8_t join(u32x4_t lo, u32x4_t hi) {
  i32x8_t r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

// Tile: 128 rows x 128 B-columns (gate/up: 64 gate + 64 up channels of the
// same 64 outputs; down: 128 outputs), BK = 128, LDS double-buffered with
// 8 + 8 operand blocks of 2 KiB per stage and the stage's 128 row scales.
// Wavefront (wm, wn) of a 2x2 grid owns 64 rows x 64 B-columns.
template <int MODE>
__global__ __launch_bounds__(256) void k_tile_fp8(K8Args a) {
  __shared__ u32x4_t lds_a[2][8 * 128];
  __shared__ u32x4_t lds_b[2][8 * 128];
  __shared__ float lds_s[2][128];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int c16 = lane & 15, q = lane >> 4;
  const int K = a.K, KB = K / 128;
  const int total = a.tile_count[0] * a.nb_per_tile;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int tile = item / a.nb_per_tile;
    const int nb = item - tile * a.nb_per_tile;
    const int4 td = a.tiles[tile];
    const int g = td.x, row0 = td.y, nrows = td.z;
    const bool sh = g == a.P;
    // chunk c = tid + 256 j: block c >> 7, idx c & 127 = half * 64 + lane
    const uint8_t* ga[4];
    const u32x4_t* gb[4];
    bool va[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = tid + 256 * j;
      const int blk = c >> 7, idx = c & 127;
      const int L = idx & 63, half = idx >> 6;
      const int r = blk * 16 + (L & 15);
      va[j] = r < nrows;
      const int rr = row0 + (va[j] ? r : 0);
      const uint8_t* base;
      if (sh) base = a.a_shared + (size_t)rr * K;
      else base = a.a_routed + (size_t)(a.a_rows ? a.a_rows[rr] : rr) * K;
      ga[j] = base + 32 * (L >> 4) + 16 * half;
      const void* W;
      int nb16;
      if (MODE == M8_GATEUP) {
        W = blk < 4 ? (sh ? a.w0_sh : a.w0_arr[g]) : (sh ? a.w1_sh : a.w1_arr[g]);
        nb16 = nb * 4 + (blk & 3);
      } else {
        W = sh ? a.w0_sh : a.w0_arr[g];
        nb16 = nb * 8 + blk;
      }
      gb[j] = (const u32x4_t*)W + (size_t)nb16 * KB * 128 + idx;
    }
    // row scales: thread tid < 128 stages row tid's scale
    const float* srow = nullptr;
    if (tid < 128 && tid < nrows) {
      const int rr = row0 + tid;
      srow = sh ? a.as_shared + (size_t)rr * KB
                : a.as_routed + (size_t)(a.a_rows ? a.a_rows[rr] : rr) * KB;
    }
    // weight block scales: uniform per workgroup and stage
    const float* sw0;
    const float* sw1 = nullptr;
    if (MODE == M8_GATEUP) {
      sw0 = (sh ? a.s0_sh : a.s0_arr[g]) + (size_t)(nb >> 1) * KB;
      sw1 = (sh ? a.s1_sh : a.s1_arr[g]) + (size_t)(nb >> 1) * KB;
    } else {
      sw0 = (sh ? a.s0_sh : a.s0_arr[g]) + (size_t)nb * KB;
    }
    u32x4_t ra[4], rb[4];
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ra[j] = va[j] ? *(const u32x4_t*)ga[j] : zero;
      rb[j] = gb[j][0];
    }
    if (srow) rs = srow[0];
    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int nmb_valid = (nrows - wm * 64 + 15) >> 4;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lds_a[0][tid + 256 * j] = ra[j];
      lds_b[0][tid + 256 * j] = rb[j];
    }
    if (tid < 128) lds_s[0][tid] = rs;
    __syncthreads();
    for (int kt = 0; kt < KB; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < KB;
      if (more) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ra[j] = va[j] ? *(const u32x4_t*)(ga[j] + (size_t)(kt + 1) * 128) : zero;
          rb[j] = gb[j][(size_t)(kt + 1) * 128];
        }
        if (srow) rs = srow[kt + 1];
      }
      const float w0s = sw0[kt];
      const float w1s = MODE == M8_GATEUP ? sw1[kt] : w0s;
      i32x8_t fb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int cb;
        if (MODE == M8_GATEUP) cb = (j >> 1) * 4 + wn * 2 + (j & 1);
        else cb = wn * 4 + j;
        fb[j] = join(lds_b[cur][cb * 128 + lane], lds_b[cur][cb * 128 + 64 + lane]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < nmb_valid) {
          const int blk = wm * 4 + i;
          const i32x8_t fa = join(lds_a[cur][blk * 128 + lane],
                                  lds_a[cur][blk * 128 + 64 + lane]);
          f32x4_t sa;
#pragma unroll
          for (int r = 0; r < 4; ++r) sa[r] = lds_s[cur][blk * 16 + 4 * q + r];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4_t blk_sum = mfma_fp8(fa, fb[j]);
            const float ws = (MODE == M8_GATEUP && j >= 2) ? w1s : w0s;
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[i][j][r] = __builtin_fmaf(blk_sum[r], sa[r] * ws, acc[i][j][r]);
          }
        }
      }
      if (more) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          lds_a[cur ^ 1][tid + 256 * j] = ra[j];
          lds_b[cur ^ 1][tid + 256 * j] = rb[j];
        }
        if (tid < 128) lds_s[cur ^ 1][tid] = rs;
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= nmb_valid) continue;
      const int rbase = wm * 64 + i * 16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int lr = rbase + 4 * q + r;
        if (lr >= nrows) continue;
        if (MODE == M8_GATEUP) {
          const size_t hr = (size_t)(sh ? a.cap : 0) + row0 + lr;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int n = nb * 64 + wn * 32 + j * 16 + c16;
            a.h_out[hr * a.N + n] = silu_f32(acc[i][j][r]) * acc[i][j + 2][r];
          }
        } else {
          float* y = sh ? a.y_shared : a.y_routed;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int n = nb * 128 + wn * 64 + j * 16 + c16;
            y[(size_t)(row0 + lr) * a.N + n] = acc[i][j][r];
          }
        }
      }
    }
  }
}

// Quantise float32 h rows per 128 channels: routed rows [0, N) (N read on the
// device) and shared rows [cap, cap + T_sh).  One wavefront per group.
__global__ __launch_bounds__(256) void k_quant_h_fp8(
    const float* __restrict__ h, int I, const int32_t* __restrict__ n_routed,
    int cap, int T_sh, uint8_t* __restrict__ codes,
    float* __restrict__ scales) {
  const int GI = I / 128;
  const long rows = (long)(*n_routed) + T_sh;
  const long groups = rows * GI;
  const int lane = threadIdx.x & 63;
  for (long grp = (long)blockIdx.x * 4 + (threadIdx.x >> 6); grp < groups;
       grp += (long)gridDim.x * 4) {
    const long ri = grp / GI;
    const int gi = (int)(grp - ri * GI);
    const long hr = ri < *n_routed ? ri : cap + (ri - *n_routed);
    const float* src = h + hr * I + gi * 128;
    const float v0 = src[2 * lane], v1 = src[2 * lane + 1];
    float amax = fmaxf(fabsf(v0), fabsf(v1));
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
    const float sc = amax == 0.0f ? 1.0f : __fdiv_rn(amax, 448.0f);
    const uint8_t c0 = f32_to_e4m3(__fdiv_rn(v0, sc));
    const uint8_t c1 = f32_to_e4m3(__fdiv_rn(v1, sc));
    *(uint16_t*)(codes + hr * I + gi * 128 + 2 * lane) =
        (uint16_t)c0 | ((uint16_t)c1 << 8);
    if (lane == 0) scales[hr * GI + gi] = sc;
  }
}

// Natural E4M3 codes [R][C] -> packed blocks (top of this file).
__global__ __launch_bounds__(256) void k_pack_fp8(const uint8_t* __restrict__ src,
                                                  int R, int C,
                                                  u32x4_t* __restrict__ dst) {
  const size_t total = (size_t)R * C / 16;
  const int CB = C / 128;
  for (size_t gi = (size_t)blockIdx.x * 256 + threadIdx.x; gi < total;
       gi += (size_t)gridDim.x * 256) {
    const size_t blk = gi >> 7;
    const int idx = (int)(gi & 127);
    const int L = idx & 63, half = idx >> 6;
    const size_t rb = blk / CB, cb = blk - rb * CB;
    const size_t r = rb * 16 + (L & 15);
    const size_t c = cb * 128 + 32 * (L >> 4) + 16 * half;
    dst[gi] = *(const u32x4_t*)(src + r * C + c);
  }
}

hipError_t launch_pack_fp8(const uint8_t* src, int R, int C, void* dst,
                           hipStream_t s) {
  const size_t total = (size_t)R * C / 16;
  if (total == 0) return hipSuccess;
  size_t grid = (total + 255) / 256;
  if (grid > 8192) grid = 8192;
  k_pack_fp8<<<(unsigned)grid, 256, 0, s>>>(src, R, C, (u32x4_t*)dst);
  return hipGetLastError();
}

hipError_t launch_ffn_fp8(FfnArgs& f, hipStream_t s) {
  const int G = f.P + (f.has_shared ? 1 : 0);
  if (G == 0) return hipSuccess;
  const int BM = 128;
  if (!f.tiles_ready)
    launch_build_tiles(f.offsets, f.P, f.has_shared, f.T, BM, f.tiles,
                       f.tile_count, s);
  if (f.events) hipEventRecord(f.events[0], s);
  const long hrows = (long)f.cap + (f.has_shared ? f.T : 0);
  const long max_tiles = G + hrows / BM + 1;
  const int cu = 256;
  const moe_weights* w = f.w;
  K8Args a{};
  a.tiles = f.tiles;
  a.tile_count = f.tile_count;
  a.P = f.P;
  a.cap = f.cap;
  // ---- gate/up: float32 h
  a.K = f.H;
  a.N = f.I;
  a.a_routed = (const uint8_t*)f.a_routed;
  a.as_routed = f.a_routed_scales;
  a.a_rows = f.a_rows;
  a.a_shared = (const uint8_t*)f.a_shared;
  a.as_shared = f.a_shared_scales;
  a.w0_arr = w->w_gate;
  a.w1_arr = w->w_up;
  a.s0_arr = w->s_gate;
  a.s1_arr = w->s_up;
  a.w0_sh = w->sh_gate;
  a.w1_sh = w->sh_up;
  a.s0_sh = w->sh_s_gate;
  a.s1_sh = w->sh_s_up;
  a.h_out = f.h32;
  a.nb_per_tile = a.N / 64;
  long items = max_tiles * a.nb_per_tile;
  long grid = items < cu * 2 ? items : cu * 2;
  k_tile_fp8<M8_GATEUP><<<(unsigned)grid, 256, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // ---- h -> E4M3 per row per 128 channels
  {
    long groups = hrows * (f.I / 128);
    long qg = (groups + 3) / 4;
    if (qg > 8192) qg = 8192;
    if (qg < 1) qg = 1;
    k_quant_h_fp8<<<(unsigned)qg, 256, 0, s>>>(
        f.h32, f.I, f.offsets + f.P, f.cap, f.has_shared ? f.T : 0,
        (uint8_t*)f.h, f.h_scales);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (f.events) hipEventRecord(f.events[1], s);
  // ---- down
  a.K = f.I;
  a.N = f.H;
  a.a_routed = (const uint8_t*)f.h;
  a.as_routed = f.h_scales;
  a.a_rows = nullptr;
  a.a_shared = (const uint8_t*)f.h + (size_t)f.cap * f.I;
  a.as_shared = f.h_scales + (size_t)f.cap * (f.I / 128);
  a.w0_arr = w->w_down;
  a.w1_arr = nullptr;
  a.s0_arr = w->s_down;
  a.s1_arr = nullptr;
  a.w0_sh = w->sh_down;
  a.w1_sh = nullptr;
  a.s0_sh = w->sh_s_down;
  a.s1_sh = nullptr;
  a.y_routed = f.y_routed;
  a.y_shared = f.y_shared;
  a.nb_per_tile = a.N / 128;
  items = max_tiles * a.nb_per_tile;
  grid = items < cu * 2 ? items : cu * 2;
  k_tile_fp8<M8_DOWN><<<(unsigned)grid, 256, 0, s>>>(a);
  if (f.events) hipEventRecord(f.events[2], s);
  return hipGetLastError();
}

}  // namespace moe
