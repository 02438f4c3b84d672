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
// Packed FP8 weight layout (moe_prepack_weights with MOE_FP8_E4M3, in
// prepare.hip): a matrix of codes with reduction size K and N output
// channels is cut into blocks of 16 channels x 128 reduction values, 2 KiB,
// block (n/16, k/128) stored at block index (n/16) * (K/128) + k/128.  Lane
// L = n%16 + 16 * ((k%128)/32) owns the 32 codes of its K-slot; their first
// 16 bytes sit at byte L*16 of the block and the next 16 at 1024 + L*16, so
// each half of a wavefront's operand is 1 KiB of contiguous memory and a
// conflict-free 16-byte LDS read per lane.  Weight scales are
// [N/128][K/128].
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
  float* h_out;               // gate/up (128 x 128 tiles): float32 h [cap + T][N]
  uint8_t* hq_out;            // gate/up (streaming kernels): E4M3 codes of h
  float* hs_out;              //   [cap + T][N], scales [cap + T][N/128]
  float* y_routed;            // down: [cap][N]
  float* y_shared;            // down: [T][N]
};

enum { M8_GATEUP = 0, M8_DOWN = 1 };

// Weight-scale columns are copied to LDS per tile (a global load of one
// inside a K loop would sit behind that loop's prefetches on the in-order
// vector-memory counter); up to kMaxKB scale blocks, i.e. K <= 16384.
static constexpr int kMaxKB = 128;

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
  __shared__ float lds_w[2][kMaxKB];        // the tile's weight-scale columns
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
    for (int i = tid; i < KB; i += 256) {     // (the barrier above freed it)
      lds_w[0][i] = sw0[i];
      if (MODE == M8_GATEUP) lds_w[1][i] = sw1[i];
    }
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
      const float w0s = lds_w[0][kt];
      const float w1s = MODE == M8_GATEUP ? lds_w[1][kt] : w0s;
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

// ------------------------------------------------------ LDS-ring kernel
// Maximum over the 16 lanes of a DPP row (every lane gets it).
__device__ __forceinline__ float row16_max(float v) {
#define ROWF(ctrl)                                                            \
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(                    \
                   0, __float_as_int(v), ctrl, 0xF, 0xF, false)));
  ROWF(0x128) ROWF(0x124) ROWF(0x122) ROWF(0x121)
#undef ROWF
  return v;
}

// Gate/up epilogue of the streaming kernels, whose item covers one 128-
// channel group of h (= one quantisation group): h = silu(g) * u per element,
// then E4M3 per row over the group (scale = amax/448, 1 for an all-zero
// group; code = RNE of fl32(h / scale), saturated), the same float32 steps
// as k_quant_h_fp8.  A wavefront holds CW channels of each of its rows; the
// group's amax is the maximum of the partial maxima the item's wavefronts
// leave in LDS (pmax [NCW][rows]), and the codes are assembled in an LDS
// byte tile [rows][128] and stored 16 bytes a lane.  Called by the whole
// workgroup once every wavefront's transfers have landed; pmax and tile lie
// in ring slots no transfer writes any more.
struct HQuant {
  float* pmax;                // LDS [NCW * ROWS], then scale [ROWS]
  uint8_t* tile;              // LDS [ROWS * 128]
  int rows_cap;               // ROWS (rows of the tile, padded)
  float* scale;               // LDS [ROWS]: pmax + NCW * ROWS
};

// One thread per row: the group's amax from the NCW partial maxima, its
// scale into LDS and, for real rows, into the h scale rows.
__device__ __forceinline__ void hq_scales(const HQuant& q, const K8Args& a,
                                          bool sh, int row0, int nrows,
                                          int nb, int ncw, int nthreads) {
  float* out = a.hs_out + ((size_t)(sh ? a.cap : 0) + row0) * (a.N / 128) + nb;
  for (int lr = threadIdx.x; lr < q.rows_cap; lr += nthreads) {
    float amax = q.pmax[lr];
    for (int w = 1; w < ncw; ++w) amax = fmaxf(amax, q.pmax[w * q.rows_cap + lr]);
    const float sc = amax == 0.0f ? 1.0f : __fdiv_rn(amax, 448.0f);
    q.scale[lr] = sc;
    if (lr < nrows) out[(size_t)lr * (a.N / 128)] = sc;
  }
}

__device__ __forceinline__ void hq_store(const HQuant& q, const K8Args& a,
                                         bool sh, int row0, int nrows, int nb,
                                         int nthreads) {
  // codes of rows < nrows to the h code rows, 128 bytes a row
  const int N = a.N;
  uint8_t* dst = a.hq_out + ((size_t)(sh ? a.cap : 0) + row0) * N + nb * 128;
  for (int i = threadIdx.x; i < nrows * 8; i += nthreads) {
    const int r = i >> 3, c = i & 7;
    *(u32x4_t*)(dst + (size_t)r * N + 16 * c) =
        *(const u32x4_t*)(q.tile + r * 128 + 16 * c);
  }
}

// For groups of up to 16 * NMB = 160 rows (one tile per expert at
// prefill-like batches of ~130 rows per expert).  A workgroup of 8
// wavefronts owns one tile and a group of output channels; each wavefront
// owns two 16-channel weight columns -- gate and up of the same channels
// (128 channels an item), or two down columns 128 channels apart (256 an
// item) -- so each weight byte is read once per tile, the tile's activation
// rows are re-read once per 128 (256) channels, and the SiLU epilogue needs
// no exchange.  Operands come through a ring of 3 LDS stages of one 128-wide
// K block each (one scale block) that global_load_lds fills two stages ahead
// without holding registers.  A stage holds the tile's activation rows
// (2 NMB blocks of 8 rows x 128 bytes, each moved whole by one transfer and
// swizzled as described at the staging code), the 16 weight blocks (2 KiB
// each, lane order) and the tile rows' scales.  Every wavefront issues the
// same number of loads per stage (A_PER activation blocks -- ids past
// 2 NMB repeat the last one, writing identical bytes -- four weight halves
// and one 64-row scale slice;
// wavefronts past the last slice load 256 contiguous bytes into a dump
// slot), so "this stage has landed" is one fixed vmcnt.  The weight scales
// of the two columns sit one per lane (K <= 16384) and are read with
// readlane, so the loop issues no global load of its own.
template <int MODE, int NMB>
__global__ __launch_bounds__(512) void k_ring_fp8(K8Args a) {
  constexpr int NAB = 2 * NMB;                   // 8-row activation blocks
  constexpr int A_PER = (NAB + 7) / 8;
  constexpr int NRS = (16 * NMB + 63) / 64;      // 64-row scale slices
  constexpr int C = A_PER + 4 + 1;               // loads per stage per wave
  __shared__ u32x4_t la0[NMB * 128], la1[NMB * 128], la2[NMB * 128];
  __shared__ u32x4_t lb0[16 * 128], lb1[16 * 128], lb2[16 * 128];
  __shared__ __attribute__((aligned(16))) float ls0[(NRS + 1) * 64],
      ls1[(NRS + 1) * 64], ls2[(NRS + 1) * 64];  // slice NRS: dump slot
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, q = lane >> 4;
  const int K = a.K, KB = K / 128;
  const int total = a.tile_count[0] * a.nb_per_tile;
  // As many workgroups as make the rounds of the persistent loop equal (a
  // multiple of 8 for the XCD mapping); the rest exit at once.  A short last
  // round leaves the weight stream to a fraction of the CUs (low-latency
  // layer -2 %).
  const int rounds = (total + (int)gridDim.x - 1) / (int)gridDim.x;
  const int G = min((int)gridDim.x, (((total + rounds - 1) / max(rounds, 1)) + 7) & ~7);
  const int per_xcd = G >> 3;
  if ((int)blockIdx.x >= G) return;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  for (int base = 0; base < total; base += G) {
    const int item = base + xcd * per_xcd + slot;
    if (item >= total) continue;                 // uniform for the workgroup
    const int tile = item / a.nb_per_tile;
    const int nb = item - tile * a.nb_per_tile;
    const int4 td = a.tiles[tile];
    const int g = td.x, row0 = td.y, nrows = td.z;
    const bool sh = g == a.P;
    const int nmb = (nrows + 15) >> 4;
    const uint8_t* abase = sh ? a.a_shared : a.a_routed;
    const float* sbase = sh ? a.as_shared : a.as_routed;
    auto src_row = [&](int r) -> int {           // tile row -> source row
      if (r >= nrows) r = 0;                     // padded rows read row 0
      const int rr = row0 + r;
      return sh ? rr : (a.a_rows ? a.a_rows[rr] : rr);
    };
    // Activation staging: one transfer moves the whole 128-byte K block of
    // 8 rows (8-row block b = id, dealt round-robin, ids past the last
    // repeating it): lane i loads row 8 b + (i >> 3), 16-byte chunk
    // (i & 7) ^ (i >> 3) ^ (b & 1), landing in slot i & 7 of that row.
    int arow[A_PER], achunk[A_PER], aid[A_PER];
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      aid[i] = min(wv + 8 * i, NAB - 1);
      arow[i] = src_row(aid[i] * 8 + (lane >> 3));
      achunk[i] = 16 * ((lane & 7) ^ (lane >> 3) ^ (aid[i] & 1));
    }
    // MFMA operand of row block mb: lane l takes row l % 16 (8-row block
    // 2 mb + (l % 16) / 8), chunks 2 (l / 16) and 2 (l / 16) + 1, found at
    // slot chunk ^ (row % 8) ^ (block parity); the 16 lanes of a read hit 16
    // different bank groups.
    const int ab = (lane >> 3) & 1, ar = lane & 7;
    const int a_lo = ab * 64 + ar * 8 + ((2 * (lane >> 4)) ^ ar ^ ab);
    const int a_hi = ab * 64 + ar * 8 + ((2 * (lane >> 4) + 1) ^ ar ^ ab);
    // scale slice (rows 64 wv + lane) or the dump slot
    const bool sreal = wv < NRS;
    const int srow = src_row(64 * (sreal ? wv : 0) + lane);
    // the two weight columns of this wavefront
    int cb0, cb1;
    const void *W0, *W1;
    const float *S0, *S1;
    if (MODE == M8_GATEUP) {
      cb0 = cb1 = nb * 8 + wv;
      W0 = sh ? a.w0_sh : a.w0_arr[g];
      W1 = sh ? a.w1_sh : a.w1_arr[g];
      S0 = sh ? a.s0_sh : a.s0_arr[g];
      S1 = sh ? a.s1_sh : a.s1_arr[g];
    } else {
      cb0 = nb * 16 + wv;
      cb1 = cb0 + 8;
      W0 = W1 = sh ? a.w0_sh : a.w0_arr[g];
      S0 = S1 = sh ? a.s0_sh : a.s0_arr[g];
    }
    const u32x4_t* wp0 = (const u32x4_t*)W0 + (size_t)cb0 * KB * 128 + lane;
    const u32x4_t* wp1 = (const u32x4_t*)W1 + (size_t)cb1 * KB * 128 + lane;
    // dump-slot source: 256 contiguous bytes of the column's own block
    const float* sdump = (const float*)((const u32x4_t*)W0 + (size_t)cb0 * KB * 128) + lane;
    // Compute layout: wavefront (wr, wc) = (wv / 4, wv % 4) takes row blocks
    // [wr MH, wr MH + MH) and four of the stage's 16 weight blocks -- gate
    // and up of channel blocks 2 wc, 2 wc + 1, or down blocks 4 wc .. 4 wc + 3
    // -- so each activation fragment feeds 4 MFMAs and each weight fragment
    // MH.  Its weight scales (one 128-channel scale block per matrix), one K
    // block per lane (two registers cover KB <= 128):
    const int wr = wv >> 2, wc = wv & 3;
    const float* sc0 = MODE == M8_GATEUP ? S0 + (size_t)nb * KB
                                         : S0 + (size_t)(2 * nb + (wc >> 1)) * KB;
    const float* sc1 = MODE == M8_GATEUP ? S1 + (size_t)nb * KB : sc0;
    const float w0lo = lane < KB ? sc0[lane] : 0.f;
    const float w0hi = lane + 64 < KB ? sc0[lane + 64] : 0.f;
    const float w1lo = lane < KB ? sc1[lane] : 0.f;
    const float w1hi = lane + 64 < KB ? sc1[lane + 64] : 0.f;
    auto wscale = [&](float lo, float hi, int kb) -> float {
      const float v = kb < 64 ? lo : hi;
      return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kb & 63));
    };

    // transfer i of stage kb: the row scales first (a 4-byte gather over 64
    // rows, the slowest transfer for the address unit: first, it overlaps
    // the most; gate/up -4 %), then the A blocks, then the four weight
    // blocks.  Only whole stages are waited for, so the order inside one is
    // free.
    auto dma = [&](int i, int kb, u32x4_t* A, u32x4_t* B, float* S) {
      if (i == 0) {
        const float* sg = sreal ? sbase + (size_t)srow * KB + kb
                                : sdump + (size_t)kb * 512;
        __builtin_amdgcn_global_load_lds(sg, (lds_void*)(S + 64 * (sreal ? wv : NRS)),
                                         4, 0, 0);
      } else if (i <= A_PER) {
        lds_dma16(abase + (size_t)arow[i - 1] * K + kb * 128 + achunk[i - 1],
                  A + aid[i - 1] * 64);
      } else {
        const int b = i - 1 - A_PER;
        const u32x4_t* wp = b < 2 ? wp0 : wp1;
        const void* src = wp + (size_t)kb * 128 + 64 * (b & 1);
        lds_void* dst = (lds_void*)(B + ((b < 2 ? 0 : 8) + wv) * 128 + 64 * (b & 1));
        // gate/up weights streamed non-temporally: a routed expert's are
        // read once (its one tile), and they then do not displace the
        // activation rows the tile's other column items re-read (gate/up
        // -3 %; a branch on the group here, to exempt the shared expert,
        // broke the step's schedule).  Down keeps the default policy.
        __builtin_amdgcn_global_load_lds(src, dst, 16, 0, MODE == M8_GATEUP ? 2 : 0);
      }
    };
    constexpr int NT = A_PER + 5;                // transfers per stage
    auto issue = [&](int kb, u32x4_t* A, u32x4_t* B, float* S) {
#pragma unroll
      for (int i = 0; i < NT; ++i) dma(i, kb, A, B, S);
    };
    constexpr int MH = NMB / 2;                  // row blocks per wavefront
    // the stage's weight slot of this wavefront's block j (DMA order: slot s
    // < 8 gate / down block s, slot 8 + s up / down block 8 + s)
    auto bslot = [&](int j) -> int {
      return MODE == M8_GATEUP ? (j < 2 ? 2 * wc + j : 8 + 2 * wc + (j - 2)) : 4 * wc + j;
    };
    f32x4_t acc[MH][4];
#pragma unroll
    for (int m = 0; m < MH; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[m][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // All MH row blocks run, straight-line, whatever nrows is: the MFMAs
    // are cheap next to the weight stream, and a branch per block would
    // make every block wait out its own LDS latency.  Padded rows hold row
    // 0's data and are never stored.  The products of consecutive row blocks
    // alternate between two register sets and block m + 1's MFMAs issue
    // before block m's scaling: with one temporary, each MFMA waited for the
    // previous product's scaling and each scaling for its MFMA's result.
    auto compute = [&](int kb, const u32x4_t* A, const u32x4_t* B, const float* S,
                       auto&& xfer) {
      const float ws0 = wscale(w0lo, w0hi, kb);
      const float ws1 = MODE == M8_GATEUP ? wscale(w1lo, w1hi, kb) : ws0;
      i32x8_t fb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        fb[j] = join(B[bslot(j) * 128 + lane], B[bslot(j) * 128 + 64 + lane]);
      f32x4_t p[2][4];
      auto products = [&](int m) {
        const int mb = wr * MH + m;
        const i32x8_t fa = join(A[mb * 128 + a_lo], A[mb * 128 + a_hi]);
#pragma unroll
        for (int j = 0; j < 4; ++j) p[m & 1][j] = mfma_fp8(fa, fb[j]);
      };
      products(0);
#pragma unroll
      for (int m = 0; m < MH; ++m) {
        if (m + 1 < MH) products(m + 1);
        // the next stage's transfers, spread over the row blocks' MFMAs
#pragma unroll
        for (int i = m * NT / MH; i < (m + 1) * NT / MH; ++i) xfer(i);
        const f32x4_t sa = *(const f32x4_t*)(S + (wr * MH + m) * 16 + 4 * q);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float ws = (MODE == M8_GATEUP && j >= 2) ? ws1 : ws0;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[m][j][r] = __builtin_fmaf(p[m & 1][j][r], sa[r] * ws, acc[m][j][r]);
        }
      }
    };
    lds_barrier();                               // last item done with the ring
    issue(0, la0, lb0, ls0);
    issue(min(1, KB - 1), la1, lb1, ls1);
    // Three stages per trip; past the end a step re-issues the last K block
    // into a slot that is never read and computes nothing, so exactly one
    // later stage (C loads) is in flight at every wait.  A step's transfers
    // of the stage two ahead go out between its row blocks' MFMAs rather
    // than all at once after the barrier, where the wavefronts' 64 transfers
    // queued at the address unit and stalled their issue (gate/up -5 %).
    // Full trips run without conditions; the last partial trip computes only
    // its real stages.
    int kb = 0;
#define RING_STEP(J, AC, BC, SC, AN, BN, SN, TAIL)              \
      {                                                         \
        const int k = kb + J;                                   \
        const int kn = k + 2 < KB ? k + 2 : KB - 1;             \
        WAIT_VMCNT(C);                                          \
        lds_barrier();                                          \
        auto xf = [&](int i) { dma(i, kn, AN, BN, SN); };       \
        if (!TAIL || k < KB) compute(k, AC, BC, SC, xf);        \
        else issue(kn, AN, BN, SN);                             \
        __builtin_amdgcn_sched_barrier(0);                      \
      }
    for (; kb + 3 <= KB; kb += 3) {
      RING_STEP(0, la0, lb0, ls0, la2, lb2, ls2, false)
      RING_STEP(1, la1, lb1, ls1, la0, lb0, ls0, false)
      RING_STEP(2, la2, lb2, ls2, la1, lb1, ls1, false)
    }
    if (kb < KB) {
      RING_STEP(0, la0, lb0, ls0, la2, lb2, ls2, true)
      RING_STEP(1, la1, lb1, ls1, la0, lb0, ls0, true)
    }
#undef RING_STEP
    WAIT_VMCNT(0);                               // trailing re-reads landed
    // Epilogue from a wave-uniform 64-bit base and 32-bit offsets; N goes
    // through an opaque move so the offsets are formed here rather than
    // hoisted out of the item loop (hoisted, they held registers).
    int N;
    asm volatile("s_mov_b32 %0, %1" : "=s"(N) : "s"(a.N));
    float* out = MODE == M8_GATEUP
                     ? a.h_out + ((size_t)(sh ? a.cap : 0) + row0) * N + (nb * 8 + 2 * wc) * 16
                     : (sh ? a.y_shared : a.y_routed) + (size_t)row0 * N + (nb * 16 + 4 * wc) * 16;
#pragma unroll
    for (int m = 0; m < MH; ++m) {
      const int mb = wr * MH + m;
      if (mb >= nmb) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int lr = mb * 16 + 4 * q + r;
        if (lr >= nrows) continue;
        const int off = lr * N + c16;
        if (MODE == M8_GATEUP) {
#pragma unroll
          for (int j = 0; j < 2; ++j)
            out[off + j * 16] = silu_f32(acc[m][j][r]) * acc[m][2 + j][r];
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) out[off + j * 16] = acc[m][j][r];
        }
      }
    }
  }
}

// ------------------------------------------------- weight-streaming kernel
// For groups of a few rows (decode-sized tiles of up to 16 * NMB = 32 rows;
// in the down pass a larger group's tall tiles of up to 128 rows run with
// NMB = 8).  A workgroup of 8
// wavefronts owns one tile and a group of output channels; each wavefront
// owns two 16-channel weight columns -- gate and up of the same channels
// (128 channels an item), or two down columns 128 channels apart (256 an
// item) -- and all the tile's row blocks, so each weight byte is read once
// per tile, the tile's activation rows once per 128 (256) channels, and the
// SiLU epilogue needs no exchange.  The reduction runs in 128-wide K blocks
// (one scale block each).  Each wavefront streams its two weight columns
// straight into MFMA operand registers with non-temporal loads, three blocks
// ahead (four register sets), so about 96 KiB of weights per CU are in
// flight without LDS; the activation rows (2 NMB blocks of 8 rows x 128
// bytes, staged as in k_ring_fp8) and the tile rows' scales, which all
// wavefronts share, go through a ring of 4 LDS stages that global_load_lds
// fills three blocks ahead.  Every wavefront issues the same number of
// loads per block (A_PER activation blocks -- ids past 2 NMB repeat the
// last one, writing identical bytes -- one 64-row scale slice, wavefronts past the last slice loading
// 256 contiguous bytes into a dump slot, and four weight loads), so "this
// block has landed" is one fixed vmcnt.  The weight scales of the two
// columns sit one per lane (K <= 16384) and are read with readlane, so the
// loop issues no other load.
//
// One item (tile, nb) of k_wstream_fp8 with NMB row blocks; the LDS ring
// (4 stages of activation blocks la* and row scales ls*) is sized for the
// largest NMB the kernel runs.
template <int MODE, int NMB>
__device__ __forceinline__ void wstream_item(const K8Args& a, int4 td, int nb,
                                             u32x4_t* la0, u32x4_t* la1,
                                             u32x4_t* la2, u32x4_t* la3,
                                             float* ls0, float* ls1,
                                             float* ls2, float* ls3) {
  constexpr int NAB = 2 * NMB;                   // 8-row activation blocks
  constexpr int A_PER = (NAB + 7) / 8;
  constexpr int NRS = (16 * NMB + 63) / 64;      // 64-row scale slices
  constexpr int C = A_PER + 1 + 4;               // loads per block per wave
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, q = lane >> 4;
  const int K = a.K, KB = K / 128;
  {
    const int g = td.x, row0 = td.y, nrows = td.z;
    const bool sh = g == a.P;
    const int nmb = (nrows + 15) >> 4;
    const uint8_t* abase = sh ? a.a_shared : a.a_routed;
    const float* sbase = sh ? a.as_shared : a.as_routed;
    auto src_row = [&](int r) -> int {           // tile row -> source row
      if (r >= nrows) r = 0;                     // padded rows read row 0
      const int rr = row0 + r;
      return sh ? rr : (a.a_rows ? a.a_rows[rr] : rr);
    };
    // Activation staging: one transfer moves the whole 128-byte K block of
    // 8 rows (8-row block b = id, dealt round-robin, ids past the last
    // repeating it): lane i loads row 8 b + (i >> 3), 16-byte chunk
    // (i & 7) ^ (i >> 3) ^ (b & 1), landing in slot i & 7 of that row.
    int arow[A_PER], achunk[A_PER], aid[A_PER];
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      aid[i] = min(wv + 8 * i, NAB - 1);
      arow[i] = src_row(aid[i] * 8 + (lane >> 3));
      achunk[i] = 16 * ((lane & 7) ^ (lane >> 3) ^ (aid[i] & 1));
    }
    // MFMA operand of row block mb: lane l takes row l % 16 (8-row block
    // 2 mb + (l % 16) / 8), chunks 2 (l / 16) and 2 (l / 16) + 1, found at
    // slot chunk ^ (row % 8) ^ (block parity); the 16 lanes of a read hit 16
    // different bank groups.
    const int ab = (lane >> 3) & 1, ar = lane & 7;
    const int a_lo = ab * 64 + ar * 8 + ((2 * (lane >> 4)) ^ ar ^ ab);
    const int a_hi = ab * 64 + ar * 8 + ((2 * (lane >> 4) + 1) ^ ar ^ ab);
    // scale slice (rows 64 wv + lane) or the dump slot
    const bool sreal = wv < NRS;
    const int srow = src_row(64 * (sreal ? wv : 0) + lane);
    // the two weight columns of this wavefront and their scale blocks (one
    // 128-channel block per column)
    int cb0, cb1;
    const void *W0, *W1;
    const float *sc0, *sc1;
    if (MODE == M8_GATEUP) {
      cb0 = cb1 = nb * 8 + wv;
      W0 = sh ? a.w0_sh : a.w0_arr[g];
      W1 = sh ? a.w1_sh : a.w1_arr[g];
      sc0 = (sh ? a.s0_sh : a.s0_arr[g]) + (size_t)nb * KB;
      sc1 = (sh ? a.s1_sh : a.s1_arr[g]) + (size_t)nb * KB;
    } else {
      cb0 = nb * 16 + wv;
      cb1 = cb0 + 8;
      W0 = W1 = sh ? a.w0_sh : a.w0_arr[g];
      const float* S0 = sh ? a.s0_sh : a.s0_arr[g];
      sc0 = S0 + (size_t)(2 * nb) * KB;
      sc1 = S0 + (size_t)(2 * nb + 1) * KB;
    }
    const u32x4_t* wp0 = (const u32x4_t*)W0 + (size_t)cb0 * KB * 128 + lane;
    const u32x4_t* wp1 = (const u32x4_t*)W1 + (size_t)cb1 * KB * 128 + lane;
    // dump-slot source: 256 contiguous bytes of the column's own block
    const float* sdump = (const float*)((const u32x4_t*)W0 + (size_t)cb0 * KB * 128) + lane;
    const float w0lo = lane < KB ? sc0[lane] : 0.f;
    const float w0hi = lane + 64 < KB ? sc0[lane + 64] : 0.f;
    const float w1lo = lane < KB ? sc1[lane] : 0.f;
    const float w1hi = lane + 64 < KB ? sc1[lane + 64] : 0.f;
    auto wscale = [&](float lo, float hi, int kb) -> float {
      const float v = kb < 64 ? lo : hi;
      return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kb & 63));
    };

    auto issue_a = [&](int kb, u32x4_t* A, float* S) {
#pragma unroll
      for (int i = 0; i < A_PER; ++i) {
        lds_dma16(abase + (size_t)arow[i] * K + kb * 128 + achunk[i],
                  A + aid[i] * 64);
      }
      const float* sg = sreal ? sbase + (size_t)srow * KB + kb
                              : sdump + (size_t)kb * 512;
      __builtin_amdgcn_global_load_lds(sg, (lds_void*)(S + 64 * (sreal ? wv : NRS)),
                                       4, 0, 0);
    };
    // weight operand of one K block: lane l holds bytes 16 l and 1024 + 16 l
    // of the column's 2 KiB block
    auto load_b = [&](int kb, i32x8_t* B) {
      B[0] = join(load_global_nt(wp0 + (size_t)kb * 128),
                  load_global_nt(wp0 + (size_t)kb * 128 + 64));
      B[1] = join(load_global_nt(wp1 + (size_t)kb * 128),
                  load_global_nt(wp1 + (size_t)kb * 128 + 64));
    };
    f32x4_t acc[NMB][2];
#pragma unroll
    for (int m = 0; m < NMB; ++m)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[m][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // All NMB row blocks run, straight-line, whatever nrows is: the MFMAs
    // are cheap next to the weight stream, and a branch per block would
    // make every block wait out its own LDS latency.  Padded rows hold row
    // 0's data and are never stored.  The products of consecutive row blocks
    // alternate between two register sets and block m + 1's MFMAs issue
    // before block m's scaling, so MFMAs and scaling overlap.
    auto compute = [&](int kb, const u32x4_t* A, const float* S, const i32x8_t* B) {
      const float ws0 = wscale(w0lo, w0hi, kb);
      const float ws1 = wscale(w1lo, w1hi, kb);
      f32x4_t p[2][2];
      auto products = [&](int m) {
        const i32x8_t fa = join(A[m * 128 + a_lo], A[m * 128 + a_hi]);
        p[m & 1][0] = mfma_fp8(fa, B[0]);
        p[m & 1][1] = mfma_fp8(fa, B[1]);
      };
      products(0);
#pragma unroll
      for (int m = 0; m < NMB; ++m) {
        if (m + 1 < NMB) products(m + 1);
        const f32x4_t sa = *(const f32x4_t*)(S + m * 16 + 4 * q);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc[m][0][r] = __builtin_fmaf(p[m & 1][0][r], sa[r] * ws0, acc[m][0][r]);
          acc[m][1][r] = __builtin_fmaf(p[m & 1][1][r], sa[r] * ws1, acc[m][1][r]);
        }
      }
    };
    i32x8_t b0[2], b1[2], b2[2], b3[2];
    lds_barrier();                               // last item done with the ring
    issue_a(0, la0, ls0);
    load_b(0, b0);
    issue_a(min(1, KB - 1), la1, ls1);
    load_b(min(1, KB - 1), b1);
    issue_a(min(2, KB - 1), la2, ls2);
    load_b(min(2, KB - 1), b2);
    // Four blocks per trip; past the end a step re-issues the last K block
    // into a slot (and register set) that is never read and computes
    // nothing, so exactly two later blocks (C loads each) are in flight at
    // every wait.
    for (int kb = 0; kb < KB; kb += 4) {
#define RING_STEP(J, AC, SC, BC, AN, SN, BN)                    \
      {                                                         \
        const int k = kb + J;                                   \
        WAIT_VMCNT(2 * C);                                      \
        lds_barrier();                                          \
        const int kn = k + 3 < KB ? k + 3 : KB - 1;             \
        issue_a(kn, AN, SN);                                    \
        load_b(kn, BN);                                         \
        if (k < KB) compute(k, AC, SC, BC);                     \
        __builtin_amdgcn_sched_barrier(0);                      \
      }
      RING_STEP(0, la0, ls0, b0, la3, ls3, b3)
      RING_STEP(1, la1, ls1, b1, la0, ls0, b0)
      RING_STEP(2, la2, ls2, b2, la1, ls1, b1)
      RING_STEP(3, la3, ls3, b3, la2, ls2, b2)
#undef RING_STEP
    }
    WAIT_VMCNT(0);                               // trailing re-reads landed
    if (MODE == M8_GATEUP) {
      // h quantised here: wavefront wv holds channels 16 wv .. 16 wv + 15 of
      // the group for every row; partial maxima in la0, codes in la1
      HQuant hq{(float*)la0, (uint8_t*)la1, 16 * NMB, (float*)la0 + 8 * 16 * NMB};
      // h overwrites the gate accumulators (no registers beyond them)
#pragma unroll
      for (int m = 0; m < NMB; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[m][0][r] = silu_f32(acc[m][0][r]) * acc[m][1][r];
      auto hv = [&](int m, int r) -> float { return acc[m][0][r]; };
      lds_barrier();                             // every wavefront past the ring
#pragma unroll
      for (int m = 0; m < NMB; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = row16_max(fabsf(hv(m, r)));
          if (c16 == 0) hq.pmax[wv * hq.rows_cap + m * 16 + 4 * q + r] = v;
        }
      lds_barrier();
      hq_scales(hq, a, sh, row0, nrows, nb, 8, 512);
      lds_barrier();
#pragma unroll
      for (int m = 0; m < NMB; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int lr = m * 16 + 4 * q + r;
          hq.tile[lr * 128 + wv * 16 + c16] =
              f32_to_e4m3(__fdiv_rn(hv(m, r), hq.scale[lr]));
        }
      lds_barrier();
      hq_store(hq, a, sh, row0, nrows, nb, 512);
      return;
    }
    // Epilogue from a wave-uniform 64-bit base and 32-bit offsets; N goes
    // through an opaque move so the offsets are formed here rather than
    // hoisted out of the item loop (hoisted, they spilled).
    int N;
    asm volatile("s_mov_b32 %0, %1" : "=s"(N) : "s"(a.N));
    float* out = (sh ? a.y_shared : a.y_routed) + (size_t)row0 * N + cb0 * 16;
#pragma unroll
    for (int m = 0; m < NMB; ++m) {
      if (m >= nmb) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int lr = m * 16 + 4 * q + r;
        if (lr >= nrows) continue;
        const int off = lr * N + c16;
        out[off] = acc[m][0][r];
        out[off + (cb1 - cb0) * 16] = acc[m][1][r];
      }
    }
  }
}

// The down pass's tall tiles (a group of more than 32 rows in a
// decode-sized batch, listed once with the fourth descriptor field 1) run
// with eight row blocks, so a hot expert's down weights are streamed once
// per 128 rows instead of once per 32; every other tile, and every gate/up
// tile, with two.  (Gate/up keeps 32-row tiles: its eight-row-block items
// carry four times the MFMAs, scalings and fragment reads of a K block and
// were slower than the repeated stream.)
static constexpr int kWsRows = 2, kWsTallRows = 8;

template <int MODE>
__global__ __launch_bounds__(512) void k_wstream_fp8(K8Args a) {
  constexpr int NMAX = MODE == M8_DOWN ? kWsTallRows : kWsRows;
  constexpr int NS = ((16 * NMAX + 63) / 64 + 1) * 64;   // scale slices + dump
  __shared__ u32x4_t la0[NMAX * 128], la1[NMAX * 128], la2[NMAX * 128],
      la3[NMAX * 128];
  __shared__ __attribute__((aligned(16))) float ls0[NS], ls1[NS], ls2[NS], ls3[NS];
  const int total = a.tile_count[0] * a.nb_per_tile;
  // As many workgroups as make the rounds of the persistent loop equal (a
  // multiple of 8 for the XCD mapping); the rest exit at once.  A short last
  // round leaves the weight stream to a fraction of the CUs (low-latency
  // layer -2 %).
  const int rounds = (total + (int)gridDim.x - 1) / (int)gridDim.x;
  const int G = min((int)gridDim.x, (((total + rounds - 1) / max(rounds, 1)) + 7) & ~7);
  const int per_xcd = G >> 3;
  if ((int)blockIdx.x >= G) return;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  for (int base = 0; base < total; base += G) {
    const int item = base + xcd * per_xcd + slot;
    if (item >= total) continue;                 // uniform for the workgroup
    const int tile = item / a.nb_per_tile;
    const int nb = item - tile * a.nb_per_tile;
    const int4 td = a.tiles[tile];
    if (MODE == M8_DOWN && td.w)
      wstream_item<MODE, kWsTallRows>(a, td, nb, la0, la1, la2, la3, ls0, ls1, ls2, ls3);
    else
      wstream_item<MODE, kWsRows>(a, td, nb, la0, la1, la2, la3, ls0, ls1, ls2, ls3);
  }
}

// Quantise float32 h rows per 128 channels: routed rows [0, N) (N read on the
// device) and shared rows [cap, cap + T_sh).  A lane takes 8 channels (two
// 16-byte loads), the 16 lanes of a DPP row one 128-channel group.

__global__ __launch_bounds__(256) void k_quant_h_fp8(
    const float* __restrict__ h, int I, const int32_t* __restrict__ n_routed,
    int cap, int T_sh, uint8_t* __restrict__ codes,
    float* __restrict__ scales) {
  const int CI = I / 8;                          // chunks of 8 per row
  const long nr = *n_routed;
  const long total = (nr + T_sh) * CI;           // a multiple of 16
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (long)gridDim.x * 256) {
    const long ri = i / CI;
    const int ci = (int)(i - ri * CI);
    const long hr = ri < nr ? ri : cap + (ri - nr);
    const f32x4_t* src = (const f32x4_t*)(h + hr * I + 8 * ci);
    const f32x4_t v0 = src[0], v1 = src[1];
    float amax = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) amax = fmaxf(amax, fmaxf(fabsf(v0[r]), fabsf(v1[r])));
    amax = row16_max(amax);
    const float sc = amax == 0.0f ? 1.0f : __fdiv_rn(amax, 448.0f);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      lo |= (uint32_t)f32_to_e4m3(__fdiv_rn(v0[r], sc)) << (8 * r);
      hi |= (uint32_t)f32_to_e4m3(__fdiv_rn(v1[r], sc)) << (8 * r);
    }
    *(uint2*)(codes + hr * I + 8 * ci) = make_uint2(lo, hi);
    if ((threadIdx.x & 15) == 0) scales[hr * (I / 128) + ci / 16] = sc;
  }
}

// The FP8 streaming recipe's down pass runs a group of more than 32 rows in
// tall tiles of up to 128 rows, listed once, from a list of its own.
int ffn_down_tall_rows(int wdt, int BM) {
  return (wdt == MOE_FP8_E4M3 && BM == 32) ? -128 : 0;
}

// Tile rows of the FP8 recipe for an expected group size: the
// register weight-streaming kernel with 32-row tiles (a few rows per
// expert; the down pass puts a larger group in tall tiles) or the LDS-ring
// kernel with 160-row tiles (one tile per expert up to 160 rows), both
// balanced; else the 128 x 128 tiled kernel.  Both streaming kernels' down
// pass covers 256 channels an item, so they need H % 256 == 0.

int ffn_fp8_tile_rows(int rows_hint, int H, int I, int* balanced) {
  (void)I;
  *balanced = 0;
  if (H % 256 || rows_hint > 160) return 128;
  *balanced = 1;
  return rows_hint <= 24 ? 32 : 160;
}

template <int MODE>
static void launch_stream_fp8(const K8Args& a, int BM, hipStream_t s) {
  // one workgroup per CU (LDS); a multiple of 8 for the XCD-major order
  if (BM == 32)
    k_wstream_fp8<MODE><<<256, 512, 0, s>>>(a);
  else
    k_ring_fp8<MODE, 10><<<256, 512, 0, s>>>(a);
}

hipError_t launch_ffn_fp8(FfnArgs& f, hipStream_t s) {
  const int G = f.P + (f.has_shared ? 1 : 0);
  if (G == 0) return hipSuccess;
  int balanced;
  const int BM = ffn_fp8_tile_rows(f.rows_hint, f.H, f.I, &balanced);
  const bool stream = balanced != 0;
  if (!f.tiles_ready)
    launch_build_tiles(f.offsets, f.P, f.has_shared, f.T, BM, balanced, 0,
                       f.tiles, f.tile_count, ffn_down_tall_rows(f.wdt, BM),
                       ffn_down_tall_rows(f.wdt, BM) ? f.tiles_down : nullptr,
                       f.tile_count + 1, s);
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
  a.hq_out = (uint8_t*)f.h;
  a.hs_out = f.h_scales;
  a.nb_per_tile = a.N / (stream ? 128 : 64);
  long items = max_tiles * a.nb_per_tile;
  long grid = items < cu * 2 ? items : cu * 2;
  if (stream)
    launch_stream_fp8<M8_GATEUP>(a, BM, s);
  else
    k_tile_fp8<M8_GATEUP><<<(unsigned)grid, 256, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (f.events) hipEventRecord(f.events[1], s);   // gate/up kernel alone
  // ---- h -> E4M3 per row per 128 channels.  The register-streaming kernel
  // (32-row tiles) quantises in its epilogue.  The LDS ring (160-row tiles)
  // and the 128 x 128 tiles write float32 h for this pass: a fused epilogue
  // in the ring held its workgroup off the weight stream for four barriers
  // per item (FP8 layer 489 -> 502 us).
  if (BM != 32) {
    long qg = (hrows * (f.I / 8) + 255) / 256;
    if (qg > 8192) qg = 8192;
    if (qg < 1) qg = 1;
    k_quant_h_fp8<<<(unsigned)qg, 256, 0, s>>>(
        f.h32, f.I, f.offsets + f.P, f.cap, f.has_shared ? f.T : 0,
        (uint8_t*)f.h, f.h_scales);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
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
  if (ffn_down_tall_rows(f.wdt, BM)) {     // down's own list (tall tiles)
    a.tiles = f.tiles_down;
    a.tile_count = f.tile_count + 1;
  }
  a.nb_per_tile = a.N / (stream ? 256 : 128);
  items = max_tiles * a.nb_per_tile;
  grid = items < cu * 2 ? items : cu * 2;
  if (stream)
    launch_stream_fp8<M8_DOWN>(a, BM, s);
  else
    k_tile_fp8<M8_DOWN><<<(unsigned)grid, 256, 0, s>>>(a);
  if (f.events) hipEventRecord(f.events[2], s);
  return hipGetLastError();
}

}  // namespace moe
