// Internal helpers shared by the HIP kernels of the MoE layer (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

typedef uint16_t bf16_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(8))) int32_t i32x8_t;

#define MOE_WAVE 64
#define MOE_KMAX 16          // largest k the dispatch kernels hold in registers
#define MOE_EMAX 1024        // largest E the router handles (16 scores a lane)
#define MOE_LMAX 1024        // largest num_local / num_physical

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// round-to-nearest-even float32 -> bf16 (finite values; NaN stays NaN)
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (bf16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

// ---------------------------------------------------------------- OCP E4M3
// Round-to-nearest-even of a finite float32 to E4M3 ("e4m3fn": bias 7, no
// infinities, S.1111.111 = NaN, max 448), saturating to +-448; sign copied
// (also for results that round to zero).  gfx950's packed fp8 conversion
// produces exactly these codes once the input is clamped to [-448, 448]
// (the clamp is the saturation): it was compared bit for bit with a
// bit-level software rounding of the definition on every float32 pattern
// of magnitude below 1024, both signs, subnormals and zeros included.
__device__ __forceinline__ uint8_t f32_to_e4m3(float v) {
  const float c = __builtin_fminf(__builtin_fmaxf(v, -448.0f), 448.0f);
  return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFF);
}

__device__ __forceinline__ float e4m3_to_f32(uint8_t c) {
  uint32_t s = (uint32_t)(c & 0x80u) << 24;
  uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  float v;
  if (e == 0) v = (float)m * 0.001953125f;  // m * 2^-9
  else v = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return __uint_as_float(__float_as_uint(v) | s);
}

// Rows per tile and tile count for a group of `rows` rows: tiles of BM rows,
// or (balanced) ceil(rows / BM) near-equal tiles rounded up to 16 rows.
__device__ __forceinline__ int tile_split(int rows, int BM, int balanced,
                                          int* per) {
  int p = BM;
  if (balanced && rows > 0) {
    const int nt = (rows + BM - 1) / BM;
    p = (((rows + nt - 1) / nt) + 15) & ~15;
  }
  *per = p;
  return (rows + p - 1) / p;
}

// Tiles of one group under a per-group choice: a group of more than BM rows
// is cut into (balanced) tall tiles of up to |tallBM| rows instead of
// tile_split(rows, BM, balanced), so a streaming kernel reads each weight
// byte once per tall tile rather than once per BM rows.  tallBM > 0: each
// tall tile is listed four times, as quarters (the fourth descriptor field
// holds 1 + quarter; the bf16 streaming kernel); tallBM < 0: each is listed
// once with the fourth field 1 (the FP8 streaming kernel's down pass);
// tallBM = 0 keeps one tile height for every group.  Returns the number of
// descriptors; *tall is 0 (ordinary), 1 (quarters) or 2 (listed once).
__device__ __forceinline__ int group_tiles(int rows, int BM, int balanced,
                                           int tallBM, int* per, int* tall) {
  if (tallBM != 0 && rows > BM) {
    *tall = tallBM > 0 ? 1 : 2;
    const int n = tile_split(rows, tallBM > 0 ? tallBM : -tallBM, 1, per);
    return tallBM > 0 ? 4 * n : n;
  }
  *tall = 0;
  return tile_split(rows, BM, balanced, per);
}

// Writes the descriptors of one group from index i on (see group_tiles).
__device__ __forceinline__ void write_group_tiles(int4* tiles, int i, int g,
                                                  int start, int rows, int per,
                                                  int tall) {
  for (int r = 0; r < rows; r += per) {
    const int n = min(per, rows - r);
    if (tall == 1) {
      for (int qd = 0; qd < 4; ++qd) tiles[i++] = make_int4(g, start + r, n, 1 + qd);
    } else {
      tiles[i++] = make_int4(g, start + r, n, tall ? 1 : 0);
    }
  }
}

// ------------------------------------------------------ LDS ring helpers
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void lds_dma16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)l, 16, 0, 0);
}

// Non-temporal 16-byte load through the global address space.  Through a
// generic pointer the load becomes a FLAT access, which may read LDS, so the
// compiler waits for every outstanding LDS DMA before it.
__device__ __forceinline__ u32x4_t load_global_nt(const u32x4_t* p) {
  return __builtin_nontemporal_load(
      (const __attribute__((address_space(1))) u32x4_t*)p);
}

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8 left at maximum).
#define WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 0xF) | ((((n) >> 4) & 3) << 14) | (7 << 4) | (0xF << 8))

// Workgroup barrier for the LDS ring.  The stage about to be read was written
// by global_load_lds (tracked by vmcnt, waited for with WAIT_VMCNT by every
// wavefront before it arrives here); the stage about to be overwritten was
// read into registers that the MFMAs before this point consumed (lgkmcnt is
// drained here).  A memory-model fence would also drain the prefetches still
// in flight, so only the compiler is fenced.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);    // lgkmcnt(0), vmcnt/expcnt untouched
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

static inline size_t moe_align256(size_t b) { return (b + 255) & ~(size_t)255; }

static inline int moe_ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

// ------------------------------------------------------- launch functions
namespace moe {

hipError_t launch_route_topk(const float* logits, const float* bias, int T,
                             int E, int k, int32_t* ids, float* w,
                             int32_t* counts, hipStream_t s);

struct DispatchArgs {
  int T, k, expert_begin, num_local, P, max_rep, H;
  const int32_t* ids;
  const float* w;
  const int32_t* l2p;       // may be null (identity)
  const int32_t* rep;       // may be null
  int32_t* block_counts;    // [nblk][L]
  int32_t* block_base;      // [nblk][L]
  int32_t* block_ecounts;   // [nblk][E] partial expert counts (multi-block)
  int32_t* offsets;         // [P+1]
  int32_t* row_token;
  float* row_weight;
  int32_t* pair_row;
};
int dispatch_blocks(int T);

// Optional outputs of the dispatch's single-workgroup stage (the whole
// small-batch kernel, or the multi-block path's scan): the expert FFN's tile
// list and the expert counts over all E.
struct DispatchExtras {
  int E;
  int32_t* counts;        // [E] or null
  int4* tiles;            // or null
  int32_t* tile_count;
  int BM, has_shared;
  int balanced;           // near-equal tiles (multiples of 16 rows)
  int tallBM;             // != 0: groups of more than BM rows in tall
                          // tiles (see group_tiles)
  int4* tiles2;           // or null: a second list of the same BM and
  int32_t* count2;        //   balance with tallBM2 (the FP8 streaming
  int tallBM2;            //   recipe's down pass), count in count2[0]
};
bool dispatch_small_ok(int T, int E, int L, int P);
// FP8 layer: router top-k (E <= 256) and the activation quantiser in one
// launch (codes [T][H], scales [T][H/128])
hipError_t launch_route_quant_fp8(const float* logits, const float* bias,
                                  int T, int E, int k, int32_t* ids, float* w,
                                  const bf16_t* x, int H, uint8_t* codes,
                                  float* scales, hipStream_t s);
hipError_t launch_dispatch_small(const DispatchArgs& a, const DispatchExtras& x,
                                 hipStream_t s);
// multi-block dispatch index; x.tiles (optional) receives the FFN tile list
hipError_t launch_dispatch_index(const DispatchArgs& a, const DispatchExtras& x,
                                 hipStream_t s);

// x_perm[r] = x[row_token[r]] for r < offsets[P]; row_bytes % 16 == 0
hipError_t launch_gather_rows(const void* x, size_t row_bytes,
                              const int32_t* row_token,
                              const int32_t* n_rows_dev, int cap, void* out,
                              hipStream_t s);

hipError_t launch_gather_rows_words(const void* x, int row_words,
                                    const int32_t* row_token,
                                    const int32_t* n_rows_dev, int cap,
                                    void* out, hipStream_t s);

// per-token per-128 E4M3 quantisation of bf16 rows [T][H]
hipError_t launch_quant_rows_fp8(const bf16_t* x, int T, int H,
                                 uint8_t* codes, float* scales, hipStream_t s);

// FP8 block quantisation of a float32 matrix stored KN ([K][N]) or NK
// ([N][K]); codes in the source's order, scales [N/128][K/128]
hipError_t launch_quant_blocks_fp8(const float* w, int K, int N, int layout,
                                   uint8_t* codes, float* scales,
                                   hipStream_t s);

hipError_t launch_combine(const float* y_perm, const int32_t* pair_row,
                          const float* w, const float* y_shared, int T, int H,
                          int k, int out_dtype, void* out, hipStream_t s);

hipError_t launch_fill_i32(int32_t* p, int32_t v, size_t n, hipStream_t s);

// ------------------------------------------------------------- the FFN
// One "group list" describes all the work of a grouped FFN call: the P
// routed physical experts (rows from offsets) and optionally the shared
// expert (group index P, rows 0..T-1 of its own input).
struct FfnArgs {
  int H, I, P, T, cap, has_shared;
  int rows_hint;                      // expected rows per routed group
  int act, wdt;                       // moe_dtype
  const int32_t* offsets;             // [P+1] device
  const void* a_routed;               // [cap][H], or [T][H] through a_rows
  const int32_t* a_rows;              // row_token of each routed row, or null
  const float* a_routed_scales;       // fp8: [cap][H/128]
  const void* a_shared;               // [T][H]
  const float* a_shared_scales;
  const moe_weights* w;               // host copy of the struct
  void* h;                            // [cap + T][I] intermediate
  float* h_scales;                    // fp8: [cap + T][I/128]
  float* h32;                         // fp8: float32 h before quantisation
  float* y_routed;                    // [cap][H]
  float* y_shared;                    // [T][H]
  int4* tiles;                        // tile list scratch
  int4* tiles_down;                   // second list: 128-row tiles for the
                                      // bf16 down pass when H % 256 != 0, or
                                      // the FP8 streaming down pass's tiles
  int32_t* tile_count;                // [2] scratch: counts of the lists
  int max_tiles;
  bool tiles_ready;                   // tile list already written
  hipEvent_t* events;                 // optional: after tiles, gate/up, down
};
hipError_t launch_ffn(FfnArgs& a, hipStream_t s);
hipError_t launch_ffn_fp8(FfnArgs& a, hipStream_t s);
// rows per tile the FFN uses for this recipe and expected group size; sets
// *balanced when a group's tiles are near-equal multiples of 16 rows
int ffn_tile_rows(int act, int wdt, int rows_hint, int H, int I, int* balanced);
// rows of the tall tiles that groups larger than a tile get (0: none)
int ffn_tall_rows(int act, int wdt, int BM);
// tall rows of the down pass's own tile list (0: down uses the first list)
int ffn_down_tall_rows(int wdt, int BM);
int ffn_fp8_tile_rows(int rows_hint, int H, int I, int* balanced);
// gate/up LDS-ring GEMM over a list of tiles of up to gemm_tile_rows() rows
hipError_t launch_gemm_bf16_gateup(const FfnArgs& f, hipStream_t s);
hipError_t launch_gemm_bf16_down(const FfnArgs& f, hipStream_t s);
int gemm_tile_rows();
// tile list of BM-row tiles (see group_tiles), and when tiles2 is non-null
// a second list of the same tiles but tallBM2
hipError_t launch_build_tiles(const int32_t* offsets, int P, int has_shared,
                              int T, int BM, int balanced, int tallBM,
                              int4* tiles, int32_t* count, int tallBM2,
                              int4* tiles2, int32_t* count2, hipStream_t s);

// a K x N matrix stored KN or NK -> its prepared form for `dtype` (float32
// [K][N]; bf16 16x32 or fp8 16x128 packed operand blocks)
hipError_t launch_prepack(const void* src, int K, int N, int dtype, int layout,
                          void* dst, hipStream_t s);

}  // namespace moe
