// Prefill-shaped grouped bf16 GEMM for the expert FFN -- gate/up with the
// fused SiLU epilogue, and down -- on the packed operand layout of ffn.hip.
//
// Work item = (tile of <= 256 rows of one group, 128 gate + 128 up columns,
// or 256 down columns).
// A workgroup of 8 wavefronts (2 x 4) computes 256 x 256 B-columns:
// wavefront (wm, wn) owns 128 rows x 64 columns = 4 x 2 MFMA blocks of
// 32 x 32 (128 fp32 accumulators per lane, two wavefronts per SIMD).  The
// reduction runs in 32-wide stages through LDS filled by
// global_load_lds_dwordx4 (each lane's 16 bytes land at the transfer's base
// + 16 * lane, so no registers stage the copy): B in a ring of 4 stages of 16
// column blocks of 1 KiB, A in 2 slots of a stage pair, where one transfer
// moves 8 whole 128-byte row segments (64 K), each read by 8 consecutive
// lanes, so every group of 8 lanes touches one cache line (lanes spread over
// 8 lines per group ran gate/up 6 % slower, 16 rows x 64 bytes slower
// still).  Every fragment read is one conflict-free ds_read_b128.  One
// barrier per stage; the DMA runs two to three stages ahead, and the
// fragments one stage ahead in registers, so after its barrier a stage's
// MFMAs start at once while its transfers and the next stage's reads are
// issued between them (gate/up 6 %, down 7 % faster than reading each
// stage's fragments after its barrier).
//
// Placement: workgroups are dealt round-robin to the 8 XCDs (workgroup b on
// XCD b % 8), and a round of the persistent loop gives each XCD a chunk of
// 32 items that run together and share operands through that XCD's L2: TG
// consecutive tiles x CB column blocks (TG x CB = 32).  A tile's A rows and
// a column block's weights are about the same size at these shapes (256
// rows or 256 columns over the same K), so a squarer chunk misses less:
// gate/up 4 tiles x 8 blocks, down 8 tiles x 4 blocks (prefill down 524 ->
// 488 us and 24 % fewer L2 misses than one tile's 28 blocks a chunk; gate/up,
// 7 % fewer misses at the same time, is bound by its issue rate rather than
// by these misses).
#include <type_traits>

#include "common.h"

namespace moe {

struct GArgs {
  const int4* tiles;
  const int32_t* tile_count;
  int nb_per_tile;
  int chunk_cols;             // column blocks per XCD chunk (divides nb_per_tile)
  int K, N;
  int P, cap;
  const bf16_t* a_routed;
  const int32_t* a_rows;
  const bf16_t* a_shared;
  const void* const* w0_arr;
  const void* const* w1_arr;
  const void* w0_sh;
  const void* w1_sh;
  bf16_t* h_out;              // gate/up output [cap + T][N]
  float* y_routed;            // down output [cap][N]
  float* y_shared;            // down output [T][N]
};

enum { G_GATEUP = 0, G_DOWN = 1 };

__device__ __forceinline__ f32x4_t mfma16b(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t mfma32b(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

// Issue order of one ring step, pinned for the scheduler: each of the NV
// DMA transfers after an MFMA, then the next stage's twelve fragment reads
// two per MFMA, then the remaining MFMAs -- so the address unit (whose
// queue stalled the issuing wavefront for hundreds of cycles when all
// transfers of a stage went out at once after the barrier) and the LDS
// work while the MFMAs run.
// NM MFMAs, NV DMA transfers and NR fragment reads in the step.
template <int NV, int NM, int NR>
__device__ __forceinline__ void interleave() {
  constexpr int MD = NV < NM ? NV : NM;          // MFMAs paired with a DMA
  constexpr int PR = (NR + 1) / 2;               // read pairs
  constexpr int MR = PR < NM - MD ? PR : NM - MD;  // MFMAs paired with reads
#pragma unroll
  for (int i = 0; i < MD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
  if (NV > MD) __builtin_amdgcn_sched_group_barrier(0x020, NV - MD, 0);
#pragma unroll
  for (int i = 0; i < MR; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  if (NR > 2 * MR) __builtin_amdgcn_sched_group_barrier(0x100, NR - 2 * MR, 0);
  if (NM > MD + MR) __builtin_amdgcn_sched_group_barrier(0x008, NM - MD - MR, 0);
}

// Workgroup = WM x WN wavefronts; wavefront (wm, wn) owns TM x TN blocks of
// 32 x 32 computed with v_mfma_f32_32x32x16_bf16 (on gfx950 this instruction
// sustains about 1.6x the rate of the 16x16x32 form), so a tile is
// 32*TM*WM rows x 32*TN*WN B-columns.  B stages hold the tile's 16-column x
// 32-K blocks (1 KiB, lane order): a 16 x 32 B operand is read from two
// adjacent blocks, lane l taking column l % 32 (block (l % 32) / 16, its
// column l % 16) and K-slot 2s + l / 32 of the stage (substep s = 0, 1), so
// 16 lanes read 256 contiguous bytes.  A pair slots hold 8-row blocks laid
// out as described at the staging code; lane l reads row l % 32 and the same
// K-slot.  The accumulator of lane l holds column l % 32 and rows
// 8 * (r / 4) + 4 * (l / 32) + r % 4, r < 16.
template <int MODE, int TM, int TN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void k_gemm_bf16(GArgs a) {
  constexpr int NW = WM * WN;                      // wavefronts
  constexpr int NR8 = 4 * TM * WM;                 // 8-row A blocks per tile
  constexpr int NB = 2 * TN * WN;                  // 16-column B blocks per stage
  constexpr int HA = NR8 / NW, HB = NB / NW;       // DMA per wavefront: A per pair, B per stage
  __shared__ u32x4_t pa0[NR8 * 64], pa1[NR8 * 64];   // A: two slots of a stage pair
  __shared__ u32x4_t lb0[NB * 64], lb1[NB * 64], lb2[NB * 64], lb3[NB * 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w / WN, wn = w % WN;
  const int c16 = lane & 15;
  const int c32 = lane & 31, hi = (lane >> 4) & 1, ks = lane >> 5;
  const int K = a.K, KB = K / 32, KT = K / 32;
  const int ntiles = a.tile_count[0];
  const int G = gridDim.x, per_xcd = G >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  // index idx -> (tile, column block): groups of TG tiles x all blocks, each
  // cut into chunks of TG tiles x CB blocks; indices of tiles past the last
  // are skipped
  const int CB = a.chunk_cols, TG = max(1, per_xcd / CB);  // CB | nb_per_tile
  const int grp_items = TG * a.nb_per_tile;
  const int total = (ntiles + TG - 1) / TG * grp_items;
  for (int base = 0; base < total; base += G) {
    const int idx = base + xcd * per_xcd + slot;
    if (idx >= total) continue;            // uniform for the workgroup
    const int grp = idx / grp_items;
    const int r = idx - grp * grp_items;
    const int part = r / (TG * CB), j = r - part * (TG * CB);
    const int tile = grp * TG + j / CB;
    if (tile >= ntiles) continue;
    const int nb = part * CB + j % CB;
    const int4 td = a.tiles[tile];
    const int g = td.x, row0 = td.y, nrows = td.z;
    const bool sh = g == a.P;
    // This wavefront stages A blocks w + NW h (8 rows of a stage pair) and
    // B column blocks w + NW h.  An A transfer takes 128 contiguous bytes
    // (64 K, 8 chunks of 8 elements: chunks 0-3 the pair's first stage,
    // 4-7 its second) of each of 8 rows: lane i loads row 8b + i / 8, chunk
    // (i % 8) ^ z with z = 4 (b & 1) + i / 16 (the row's index inside its
    // 32-row block, halved, mod 8), and lands at 16 i, so a block is
    // [row][chunk slot].
    // A: the operand's base and a byte offset per lane; B: a wave-uniform
    // base per column block and the lane's 16 bytes
    const char* abase = (const char*)(sh ? a.a_shared : a.a_routed);
    size_t aoff[HA];
    const char* gbb[HB];
#pragma unroll
    for (int h = 0; h < HA; ++h) {
      const int b8 = w + NW * h;
      int r = b8 * 8 + (lane >> 3);
      if (r >= nrows) r = 0;               // padded rows read row 0, unused
      const int rr = row0 + r;
      const size_t srow = sh ? rr : (a.a_rows ? a.a_rows[rr] : rr);
      aoff[h] = srow * (size_t)K * 2u +
                (size_t)(((lane & 7) ^ ((b8 & 1) * 4 + (lane >> 4))) * 16);
    }
#pragma unroll
    for (int h = 0; h < HB; ++h) {
      const int cb = w + NW * h;
      const void* W;
      int nb16;
      if (MODE == G_GATEUP) {   // blocks [0, NB/2) gate, the rest up, same outputs
        W = cb < NB / 2 ? (sh ? a.w0_sh : a.w0_arr[g]) : (sh ? a.w1_sh : a.w1_arr[g]);
        nb16 = nb * (NB / 2) + (cb < NB / 2 ? cb : cb - NB / 2);
      } else {
        W = sh ? a.w0_sh : a.w0_arr[g];
        nb16 = nb * NB + cb;
      }
      gbb[h] = (const char*)W + (size_t)nb16 * KB * 1024;
    }
    const uint32_t loff = (uint32_t)lane * 16u;
    auto issue_a = [&](int kp, u32x4_t* A) {     // stages 2 kp and 2 kp + 1
      const char* base = abase + (size_t)kp * 128;
#pragma unroll
      for (int h = 0; h < HA; ++h) lds_dma16(base + aoff[h], A + (w + NW * h) * 64);
    };
    auto issue_b = [&](int kt, u32x4_t* B) {
#pragma unroll
      for (int h = 0; h < HB; ++h)
        lds_dma16(gbb[h] + (size_t)kt * 1024 + loff, B + (w + NW * h) * 64);
    };
    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x16_t{};
    // Fragments of one stage (all twelve reads) in two register sets: a
    // stage's MFMAs run from one set while the next stage is read into the
    // other.  Stage HH of the pair in slot A: lane l reads row r = l % 32 of
    // a 32-row block (8-row block r / 8, its row r % 8), chunk
    // c = 4 HH + 2 s + l / 32 at chunk slot c ^ ((r / 2) % 8); the 16 lanes
    // of a read take 16 distinct 16-byte bank groups (row parity x slot).
    // A wavefront whose rows are all padding multiplies them too (its
    // stores are skipped), which keeps the step one basic block.
    // Only the wavefront's first NMB row blocks hold tile rows (the rest
    // are padding of a partial tile): their fragments are read and
    // multiplied, the others skipped.
    auto load = [&](auto nmb_c, const u32x4_t* A, int HH, const u32x4_t* B,
                    u32x4_t (&fa)[2][TM], u32x4_t (&fb)[2][TN]) {
      constexpr int NMB = decltype(nmb_c)::value;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int pos = c16 + 16 * (2 * s + ks);   // lane slot inside a B block
        const int apos = ((lane & 31) >> 3) * 64 + (lane & 7) * 8 +
                         ((HH * 4 + 2 * s + ks) ^ (((lane & 31) >> 1) & 7));
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int cb32 = MODE == G_DOWN ? wn * TN + j
                           : (j < TN / 2) ? wn * (TN / 2) + j
                                          : NB / 4 + wn * (TN / 2) + (j - TN / 2);
          fb[s][j] = B[(2 * cb32 + hi) * 64 + pos];
        }
#pragma unroll
        for (int i = 0; i < NMB; ++i) fa[s][i] = A[(wm * TM + i) * 4 * 64 + apos];
      }
    };
    auto mma = [&](auto nmb_c, const u32x4_t (&fa)[2][TM],
                   const u32x4_t (&fb)[2][TN]) {
      constexpr int NMB = decltype(nmb_c)::value;
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < NMB; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = mfma32b(fa[s][i], fb[s][j], acc[i][j]);
    };
    u32x4_t fa0[2][TM], fb0[2][TN], fa1[2][TM], fb1[2][TN];
    lds_barrier();                       // previous item done with the ring
    // Ring: B stage k in slot k % 4, A pair k / 2 in slot (k / 2) % 2.
    // Step k: wait for this wavefront's part of stage k + 1, barrier (stage
    // k + 1 complete; stage k, read during step k - 1, free), issue B stage
    // k + 4 into stage k's slot and, on odd k, A pair (k + 3) / 2 into the
    // pair slot of stages k - 1, k; then the MFMAs of stage k from registers
    // and the reads of stage k + 1 into the other register set.  In-order
    // completion makes the waits fixed counts: an even step needs the B
    // stage issued three steps back (2 HB + HA younger transfers), an odd
    // step the A pair issued two steps back (HB younger).  Past the end the
    // last stage / pair is re-read into slots that are never read again, and
    // the last step's reads of the stage after the last fetch that complete
    // re-read data into registers that go unused.
    issue_b(0, lb0);
    issue_a(0, pa0);
    issue_b(1, lb1);
    issue_b(2, lb2);
    issue_a(1, pa1);
    issue_b(3, lb3);
    WAIT_VMCNT(3 * HB + HA);             // stage 0
    lds_barrier();
    const int last_pair = KT / 2 - 1;
    // The K loop for a wavefront with NMB row blocks of tile rows (a
    // wave-uniform choice per item; a wavefront without any still issues
    // its share of the transfers and meets every barrier).  Written out
    // once per NMB by a macro rather than as a lambda: through a lambda the
    // fragment reads lost track of which LDS slots the transfers write, and
    // the compiler waited for all transfers before every read.
#define GEMM_STEP(NMB, S, PA1, HH1, BC1, PN, BN_, FC_A, FC_B, FN_A, FN_B)     \
    {                                                                        \
      const int k = kt + S;                                                  \
      if (S % 2 == 0) WAIT_VMCNT(2 * HB + HA);                               \
      else WAIT_VMCNT(HB);                                                   \
      lds_barrier();                                                         \
      __builtin_amdgcn_sched_barrier(0);                                     \
      issue_b(k + 4 < KT ? k + 4 : KT - 1, BN_);                             \
      if (S % 2 == 1) issue_a((k + 3) / 2 < last_pair ? (k + 3) / 2 : last_pair, PN); \
      if ((NMB) > 0) {                                                       \
        load(std::integral_constant<int, (NMB)>{}, PA1, HH1, BC1, FN_A, FN_B); \
        mma(std::integral_constant<int, (NMB)>{}, FC_A, FC_B);                 \
      }                                                                      \
      interleave<(S % 2 == 1 ? HB + HA : HB), (2 * (NMB) * TN),               \
                 ((NMB) > 0 ? 2 * ((NMB) + TN) : 0)>();                      \
      __builtin_amdgcn_sched_barrier(0);                                     \
    }
#define GEMM_K_LOOP(NMB)                                                     \
    {                                                                        \
      if ((NMB) > 0) load(std::integral_constant<int, (NMB)>{}, pa0, 0, lb0, fa0, fb0); \
      for (int kt = 0; kt < KT; kt += 4) {                                   \
        GEMM_STEP(NMB, 0, pa0, 1, lb1, pa0, lb0, fa0, fb0, fa1, fb1)         \
        GEMM_STEP(NMB, 1, pa1, 0, lb2, pa0, lb1, fa1, fb1, fa0, fb0)         \
        GEMM_STEP(NMB, 2, pa1, 1, lb3, pa1, lb2, fa0, fb0, fa1, fb1)         \
        GEMM_STEP(NMB, 3, pa0, 0, lb0, pa1, lb3, fa1, fb1, fa0, fb0)         \
      }                                                                      \
    }
    {
      int nmb = (nrows - wm * TM * 32 + 31) / 32;   // wave-uniform
      nmb = nmb < 0 ? 0 : (nmb > TM ? TM : nmb);
      nmb = __builtin_amdgcn_readfirstlane(nmb);
      if (nmb == TM) GEMM_K_LOOP(TM)
      else if (nmb == 0) GEMM_K_LOOP(0)
      else if (nmb == 1) GEMM_K_LOOP(1)
      else if (nmb == 2) GEMM_K_LOOP((TM > 2 ? 2 : 1))
      else GEMM_K_LOOP((TM > 3 ? 3 : 1))
    }
#undef GEMM_K_LOOP
#undef GEMM_STEP
    WAIT_VMCNT(0);                       // the trailing re-reads have landed
    // Epilogue, one row block at a time: a wave-uniform 64-bit base per
    // block and 32-bit lane offsets.  N and the lane's row half are read
    // through opaque moves so the offsets and row indices are formed here
    // rather than hoisted out of the item loop (hoisted, they held about 80
    // registers through the MFMA loop, which then read one fragment per
    // MFMA pair and waited for each: gate/up 2 % slower).
    int N, kse;
    asm volatile("s_mov_b32 %0, %1" : "=s"(N) : "s"(a.N));
    asm volatile("v_mov_b32 %0, %1" : "=v"(kse) : "v"(ks));
    const int lane_off = 4 * kse * N + c32;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      const int rb = wm * TM * 32 + i * 32;      // the block's first row
      if (rb >= nrows) break;
      if (MODE == G_GATEUP) {
        bf16_t* base = a.h_out + ((size_t)(sh ? a.cap : 0) + row0 + rb) * N +
                       nb * (NB / 2) * 16 + wn * (TN / 2) * 32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = 8 * (r >> 2) + 4 * kse + (r & 3);
          if (rb + lr >= nrows) continue;
          const int off = lane_off + (8 * (r >> 2) + (r & 3)) * N;
#pragma unroll
          for (int jj = 0; jj < TN / 2; ++jj)
            base[off + jj * 32] =
                f32_to_bf16(silu_f32(acc[i][jj][r]) * acc[i][TN / 2 + jj][r]);
        }
      } else {
        float* base = (sh ? a.y_shared : a.y_routed) + (size_t)(row0 + rb) * N +
                      nb * NB * 16 + wn * TN * 32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = 8 * (r >> 2) + 4 * kse + (r & 3);
          if (rb + lr >= nrows) continue;
          const int off = lane_off + (8 * (r >> 2) + (r & 3)) * N;
#pragma unroll
          for (int j = 0; j < TN; ++j) base[off + j * 32] = acc[i][j][r];
        }
      }
    }
  }
}

// 256 x 256 tiles from 2 x 4 wavefronts of 4 x 2 blocks: two wavefronts per
// SIMD, so one's barrier or LDS wait is covered by the other's MFMAs (one
// wavefront per SIMD with 4 x 4 blocks each ran gate/up 17 % slower).
static constexpr int kGemmWM = 2, kGemmWN = 4;
static constexpr int kGemmTM = 4, kGemmTN = 2;
static constexpr int kGemmRows = 32 * kGemmTM * kGemmWM;
int gemm_tile_rows() { return kGemmRows; }

// Column blocks per XCD chunk: the largest divisor of nb_per_tile up to want.
static int chunk_cols(int nb_per_tile, int want) {
  for (int c = want < nb_per_tile ? want : nb_per_tile; c > 1; --c)
    if (nb_per_tile % c == 0) return c;
  return 1;
}

hipError_t launch_gemm_bf16_gateup(const FfnArgs& f, hipStream_t s) {
  const moe_weights* w = f.w;
  GArgs a{};
  a.tiles = f.tiles;
  a.tile_count = f.tile_count;
  a.P = f.P;
  a.cap = f.cap;
  a.K = f.H;
  a.N = f.I;
  a.a_routed = (const bf16_t*)f.a_routed;
  a.a_rows = f.a_rows;
  a.a_shared = (const bf16_t*)f.a_shared;
  a.w0_arr = w->w_gate;
  a.w1_arr = w->w_up;
  a.w0_sh = w->sh_gate;
  a.w1_sh = w->sh_up;
  a.h_out = (bf16_t*)f.h;
  a.nb_per_tile = a.N / (16 * kGemmTN * kGemmWN);  // 32 TN WN B-columns
  a.chunk_cols = chunk_cols(a.nb_per_tile, 8);     // 4 tiles x 8 blocks
  // persistent: one workgroup per CU (128 KiB of LDS)
  k_gemm_bf16<G_GATEUP, kGemmTM, kGemmTN, kGemmWM, kGemmWN>
      <<<256, 64 * kGemmWM * kGemmWN, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16_down(const FfnArgs& f, hipStream_t s) {
  const moe_weights* w = f.w;
  GArgs a{};
  a.tiles = f.tiles;
  a.tile_count = f.tile_count;
  a.P = f.P;
  a.cap = f.cap;
  a.K = f.I;
  a.N = f.H;
  a.a_routed = (const bf16_t*)f.h;
  a.a_rows = nullptr;
  a.a_shared = (const bf16_t*)f.h + (size_t)f.cap * f.I;
  a.w0_arr = w->w_down;
  a.w1_arr = nullptr;
  a.w0_sh = w->sh_down;
  a.w1_sh = nullptr;
  a.y_routed = f.y_routed;
  a.y_shared = f.y_shared;
  a.nb_per_tile = a.N / (32 * kGemmTN * kGemmWN);  // 32 TN WN outputs
  a.chunk_cols = chunk_cols(a.nb_per_tile, 4);     // 8 tiles x 4 blocks
  k_gemm_bf16<G_DOWN, kGemmTM, kGemmTN, kGemmWM, kGemmWN>
      <<<256, 64 * kGemmWM * kGemmWN, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
