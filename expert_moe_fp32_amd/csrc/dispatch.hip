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
#include "route_row.h"

namespace moe {

static constexpr int kTokPerBlock = 256;

int dispatch_blocks(int T) { return (T + kTokPerBlock - 1) / kTokPerBlock; }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Each thread loads its token's local expert ids (-1 where not local).
// Exclusive prefix sum over the 64 lanes of a wavefront; *total gets the sum.
__device__ __forceinline__ int wave_excl_scan(int v, int* total) {
  const int lane = threadIdx.x & 63;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  *total = __shfl(incl, 63, 64);
  return incl - v;
}

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

// For every local expert e < L calls store(e, m), with m = the ballot of the
// lanes whose token picked e (a token picks an expert at most once), on one
// lane.  With L <= 256 each lane first folds its picks into a 256-bit mask,
// so an expert costs one shift-and-ballot; the ballots are gathered into
// the registers of lane e % 64 (a select, no branch per expert) and stored
// from there, every lane at most four times.  Beyond 256 every expert is
// compared against every slot and stored from lane 0.
template <class Store>
__device__ __forceinline__ void for_each_expert_ballot(
    const int (&le)[MOE_KMAX], int L, Store store) {
  const int lane = threadIdx.x & 63;
  if (L <= 256) {
    uint64_t m0 = 0, m1 = 0, m2 = 0, m3 = 0;
#pragma unroll
    for (int j = 0; j < MOE_KMAX; ++j) {
      const int e = le[j];
      const uint64_t bit = e >= 0 ? 1ull << (e & 63) : 0ull;
      const int w = e >> 6;
      m0 |= w == 0 ? bit : 0ull;
      m1 |= w == 1 ? bit : 0ull;
      m2 |= w == 2 ? bit : 0ull;
      m3 |= w == 3 ? bit : 0ull;
    }
    uint64_t mine[4] = {0ull, 0ull, 0ull, 0ull};
    auto word = [&](uint64_t mw, int base, uint64_t& dst) {
      const int n = min(64, L - base);
      for (int b = 0; b < n; ++b) {
        const uint64_t m = __ballot((mw >> b) & 1ull);
        dst = lane == b ? m : dst;
      }
    };
    word(m0, 0, mine[0]);
    if (L > 64) word(m1, 64, mine[1]);
    if (L > 128) word(m2, 128, mine[2]);
    if (L > 192) word(m3, 192, mine[3]);
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (64 * w + lane < L) store(64 * w + lane, mine[w]);
  } else {
    for (int e = 0; e < L; ++e) {
      bool has = false;
#pragma unroll
      for (int j = 0; j < MOE_KMAX; ++j) has |= le[j] == e;
      const uint64_t m = __ballot(has);
      if (lane == 0) store(e, m);
    }
  }
}

// Per block of tokens: the rows of each local expert, and (block_ecounts
// non-null) the block's pairs of every one of the E experts, counted in an
// LDS histogram and stored for the scan to sum.
__global__ __launch_bounds__(256) void k_local_hist(
    const int32_t* __restrict__ ids, int T, int k, int e0, int L,
    int32_t* __restrict__ block_counts, int E,
    int32_t* __restrict__ block_ecounts) {
  extern __shared__ int32_t wave_cnt[];     // [4][L], then [E]
  int32_t* ehist = wave_cnt + 4 * L;
  const int t = blockIdx.x * kTokPerBlock + threadIdx.x;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (block_ecounts) {                      // uniform
    for (int e = threadIdx.x; e < E; e += blockDim.x) ehist[e] = 0;
    __syncthreads();
    if (t < T)
      for (int j = 0; j < k; ++j) {       // ids outside [0, E): not counted
        const int gid = ids[(size_t)t * k + j];
        if ((unsigned)gid < (unsigned)E) atomicAdd(&ehist[gid], 1);
      }
  }
  int le[MOE_KMAX];
  load_local_ids(ids, t, T, k, e0, L, le);
  for_each_expert_ballot(le, L, [&](int e, uint64_t m) {
    wave_cnt[wv * L + e] = __popcll(m);
  });
  __syncthreads();
  for (int e = threadIdx.x; e < L; e += blockDim.x)
    block_counts[(size_t)blockIdx.x * L + e] =
        wave_cnt[e] + wave_cnt[L + e] + wave_cnt[2 * L + e] + wave_cnt[3 * L + e];
  if (block_ecounts)
    for (int e = threadIdx.x; e < E; e += blockDim.x)
      block_ecounts[(size_t)blockIdx.x * E + e] = ehist[e];
}

// FFN tile lists (tiles of BM rows, see group_tiles) from the segment
// offsets held in LDS (off[0 .. P]) by a single workgroup: x.tiles, and
// x.tiles2 (the same tiles with x.tallBM2) when set.  Wavefront 0 counts
// each group's tiles and scans them into tb (and tb2; G + 1 entries each,
// G = P + shared), the workgroup barrier follows, then every thread writes
// its groups' tiles.  Called by all threads.
__device__ void tile_list_from_offsets(const int32_t* off, int P, int T,
                                       const DispatchExtras& x, int32_t* tb,
                                       int32_t* tb2) {
  const int G = P + (x.has_shared ? 1 : 0);
  const bool two = x.tiles2 != nullptr;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int carry = 0, carry2 = 0;
    for (int base = 0; base < G; base += 64) {
      const int g = base + lane;
      int nt = 0, nt2 = 0;
      if (g < G) {
        const int rows = g < P ? off[g + 1] - off[g] : T;
        int per, tall;
        nt = group_tiles(rows, x.BM, x.balanced, x.tallBM, &per, &tall);
        if (two) nt2 = group_tiles(rows, x.BM, x.balanced, x.tallBM2, &per, &tall);
      }
      int tot, tot2 = 0;
      const int ex = wave_excl_scan(nt, &tot);
      const int ex2 = two ? wave_excl_scan(nt2, &tot2) : 0;
      if (g < G) {
        tb[g] = carry + ex;
        if (two) tb2[g] = carry2 + ex2;
      }
      carry += tot;
      carry2 += tot2;
    }
    if (lane == 0) {
      x.tile_count[0] = carry;
      if (two) x.count2[0] = carry2;
    }
  }
  __syncthreads();
  for (int g = threadIdx.x; g < G; g += blockDim.x) {
    const int start = g < P ? off[g] : 0;
    const int rows = g < P ? off[g + 1] - start : T;
    if (rows == 0) continue;
    int per, tall;
    group_tiles(rows, x.BM, x.balanced, x.tallBM, &per, &tall);
    write_group_tiles(x.tiles, tb[g], g, start, rows, per, tall);
    if (two) {
      group_tiles(rows, x.BM, x.balanced, x.tallBM2, &per, &tall);
      write_group_tiles(x.tiles2, tb2[g], g, start, rows, per, tall);
    }
  }
}

__global__ __launch_bounds__(1024) void k_scan(
    const int32_t* __restrict__ block_counts, int nblk, int L, int P,
    int max_rep, const int32_t* __restrict__ l2p,
    const int32_t* __restrict__ rep, int32_t* __restrict__ block_base,
    int32_t* __restrict__ offsets, int T, DispatchExtras x,
    const int32_t* __restrict__ block_ecounts) {
  __shared__ int32_t pc[MOE_LMAX + 1];
  __shared__ int32_t tb[MOE_LMAX + 2], tb2[MOE_LMAX + 2];
  if (x.counts) {                          // expert counts: sum the block rows
    for (int e = threadIdx.x; e < x.E; e += blockDim.x) {
      int c = 0;
      for (int b0 = 0; b0 < nblk; b0 += 8) {   // eight loads in flight
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          v[u] = b0 + u < nblk ? block_ecounts[(size_t)(b0 + u) * x.E + e] : 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) c += v[u];
      }
      x.counts[e] = c;
    }
  }
  for (int p = threadIdx.x; p < P; p += blockDim.x) pc[p] = 0;
  __syncthreads();
  for (int e = threadIdx.x; e < L; e += blockDim.x) {
    int run = 0;
    for (int b0 = 0; b0 < nblk; b0 += 8) {     // eight loads in flight
      int c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        c[u] = b0 + u < nblk ? block_counts[(size_t)(b0 + u) * L + e] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (b0 + u < nblk) block_base[(size_t)(b0 + u) * L + e] = run;
        run += c[u];
      }
    }
    const int R = rep ? min(max(rep[e], 1), max_rep) : 1;
    for (int r = 0; r < R; ++r) {
      const int p = l2p ? l2p[e * max_rep + r] : e;
      if (p >= 0 && p < P) pc[p] = run > r ? (run - r + R - 1) / R : 0;
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) {                  // one wavefront scans pc
    const int lane = threadIdx.x;
    int carry = 0;
    for (int base = 0; base <= P; base += 64) {
      const int p = base + lane;
      int tot;
      const int ex = wave_excl_scan(p < P ? pc[p] : 0, &tot);
      if (p <= P) {
        offsets[p] = carry + ex;
        pc[p] = carry + ex;                // offsets stay in LDS for the tiles
      }
      carry += tot;
    }
  }
  if (x.tiles) {                           // uniform
    __syncthreads();
    tile_list_from_offsets(pc, P, T, x, tb, tb2);
  }
}

__global__ __launch_bounds__(256) void k_permute(
    const int32_t* __restrict__ ids, const float* __restrict__ w, int T,
    int k, int e0, int L, int P, int max_rep, const int32_t* __restrict__ l2p,
    const int32_t* __restrict__ rep, const int32_t* __restrict__ block_base,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ row_token,
    float* __restrict__ row_weight, int32_t* __restrict__ pair_row) {
  extern __shared__ uint64_t dyn[];        // bal [4][L], then wave_cnt [4][L]
  uint64_t* bal = dyn;
  int32_t* wave_cnt = (int32_t*)(dyn + 4 * L);
  const int t = blockIdx.x * kTokPerBlock + threadIdx.x;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int le[MOE_KMAX];
  load_local_ids(ids, t, T, k, e0, L, le);
  for_each_expert_ballot(le, L, [&](int e, uint64_t m) {
    bal[wv * L + e] = m;
    wave_cnt[wv * L + e] = __popcll(m);
  });
  __syncthreads();
  if (t >= T) return;
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int j = 0; j < MOE_KMAX; ++j) {
    if (j >= k) break;
    const size_t o = (size_t)t * k + j;
    const int e = le[j];
    if (e < 0) {
      pair_row[o] = -1;
      continue;
    }
    int n = block_base[(size_t)blockIdx.x * L + e] +
            __popcll(bal[wv * L + e] & lt);  // earlier lanes of this wave
    for (int v = 0; v < wv; ++v) n += wave_cnt[v * L + e];
    const int R = rep ? min(max(rep[e], 1), max_rep) : 1;
    const int nq = R == 1 ? n : n / R;       // one replica: no division
    const int p = l2p ? l2p[e * max_rep + (n - nq * R)] : e;
    if (p < 0 || p >= P) {                   // a map entry out of range:
      pair_row[o] = -1;                      // the pair is dropped
      continue;
    }
    const int row = offsets[p] + nq;
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
static constexpr int kSmallT = 1024, kSmallL = 256, kSmallMap = 2048;


bool dispatch_small_ok(int T, int E, int L, int P) {
  return T <= kSmallT && L <= kSmallL && E <= MOE_EMAX && P <= MOE_LMAX;
}

__global__ __launch_bounds__(1024) void k_dispatch_small(DispatchArgs a,
                                                         DispatchExtras x) {
  __shared__ int32_t cnt[MOE_EMAX];
  __shared__ int32_t pc[MOE_LMAX + 1];
  __shared__ int32_t tb[MOE_LMAX + 2], tb2[MOE_LMAX + 2];
  __shared__ int32_t wpre[16 * kSmallL];
  __shared__ uint64_t bal[16 * kSmallL];    // per wavefront: ballot per expert
  __shared__ int32_t reps[kSmallL];         // replica counts (clamped)
  __shared__ int32_t maps[kSmallMap];       // the replica map when it fits
  const int t = threadIdx.x, wv = t >> 6, lane = t & 63;
  const int T = a.T, k = a.k, L = a.num_local, P = a.P;
  // The replica counts and map are loaded into LDS here, alongside the
  // ids, rather than read from global memory where they are needed: two
  // dependent round trips fewer on this single-workgroup path.
  const bool map_lds = a.l2p && L * a.max_rep <= kSmallMap;
  // the token's ids and route weights are requested first: their latency
  // overlaps the LDS set-up below
  int gid[MOE_KMAX];
  float wj[MOE_KMAX];
#pragma unroll
  for (int j = 0; j < MOE_KMAX; ++j) {
    gid[j] = -1;
    wj[j] = 0.0f;
    if (j < k && t < T) {
      gid[j] = a.ids[(size_t)t * k + j];
      wj[j] = a.w[(size_t)t * k + j];
    }
  }
  for (int i = t; i < L; i += 1024)
    reps[i] = a.rep ? min(max(a.rep[i], 1), a.max_rep) : 1;
  if (map_lds)
    for (int i = t; i < L * a.max_rep; i += 1024) maps[i] = a.l2p[i];
  for (int i = t; i < x.E; i += 1024) cnt[i] = 0;
  for (int i = t; i <= P; i += 1024) pc[i] = 0;
  __syncthreads();
  int le[MOE_KMAX];
#pragma unroll
  for (int j = 0; j < MOE_KMAX; ++j) {
    le[j] = -1;
    if (j < k && t < T) {
      // expert counts only when asked for, and only of ids in [0, E)
      if (x.counts && (unsigned)gid[j] < (unsigned)x.E) atomicAdd(&cnt[gid[j]], 1);
      const int e = gid[j] - a.expert_begin;
      if (e >= 0 && e < L) le[j] = e;
    }
  }
  const uint64_t lt = lanemask_lt();
  for_each_expert_ballot(le, L, [&](int e, uint64_t m) {
    bal[wv * kSmallL + e] = m;
    wpre[wv * kSmallL + e] = __popcll(m);
  });
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
    const int R = reps[e];
    for (int r = 0; r < R; ++r) {
      const int p = !a.l2p ? e : map_lds ? maps[e * a.max_rep + r] : a.l2p[e * a.max_rep + r];
      if (p >= 0 && p < P) pc[p] = run > r ? (run - r + R - 1) / R : 0;
    }
  }
  __syncthreads();
  if (wv == 0) {
    // segment offsets: exclusive scan of the rows per physical expert,
    // 64 entries at a time (pc[p] becomes offsets[p] in place; pc[P] = N)
    int carry = 0;
    for (int base = 0; base <= P; base += 64) {
      const int p = base + lane;
      const int c = p < P ? pc[p] : 0;
      int tot;
      const int ex = wave_excl_scan(c, &tot);
      if (p <= P) {
        pc[p] = carry + ex;
        a.offsets[p] = carry + ex;
      }
      carry += tot;
    }
  }
  __syncthreads();
  if (x.tiles) tile_list_from_offsets(pc, P, T, x, tb, tb2);   // uniform
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
    const int n = wpre[wv * kSmallL + e] + __popcll(bal[wv * kSmallL + e] & lt);
    const int R = reps[e];
    const int nq = R == 1 ? n : n / R;       // one replica: no division
    const int mi = e * a.max_rep + (n - nq * R);
    const int p = !a.l2p ? e : map_lds ? maps[mi] : a.l2p[mi];
    if (p < 0 || p >= P) {
      a.pair_row[o] = -1;
      continue;
    }
    const int row = pc[p] + nq;
    a.pair_row[o] = row;
    a.row_token[row] = t;
    a.row_weight[row] = wj[j];
  }
}

hipError_t launch_dispatch_small(const DispatchArgs& a, const DispatchExtras& x,
                                 hipStream_t s) {
  k_dispatch_small<<<1, 1024, 0, s>>>(a, x);
  return hipGetLastError();
}

hipError_t launch_dispatch_index(const DispatchArgs& a, const DispatchExtras& x,
                                 hipStream_t s) {
  const int nblk = dispatch_blocks(a.T);
  int32_t* ecounts = x.counts ? a.block_ecounts : nullptr;
  const size_t lds = sizeof(int32_t) * (4 * a.num_local + (ecounts ? x.E : 0));
  k_local_hist<<<nblk, 256, lds, s>>>(a.ids, a.T, a.k, a.expert_begin,
                                      a.num_local, a.block_counts, x.E, ecounts);
  k_scan<<<1, 1024, 0, s>>>(a.block_counts, nblk, a.num_local, a.P,
                            a.max_rep, a.l2p, a.rep, a.block_base, a.offsets,
                            a.T, x, ecounts);
  const size_t lds_perm = (sizeof(uint64_t) + sizeof(int32_t)) * 4 * a.num_local;
  k_permute<<<nblk, 256, lds_perm, s>>>(a.ids, a.w, a.T, a.k, a.expert_begin,
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
// Per-token, per-128-channel E4M3 quantisation: amax over the group, scale
// amax/448 (1 if amax = 0), codes RNE(fl32(x / scale)) saturated.  A lane
// takes 8 consecutive channels (one 16-byte load), the 16 lanes of a DPP row
// one 128-channel group, whose amax is a 4-step row rotation.
__device__ __forceinline__ float row_max_f32(float v) {
#define ROWF(ctrl)                                                            \
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(                    \
                   0, __float_as_int(v), ctrl, 0xF, 0xF, false)));
  ROWF(0x128) ROWF(0x124) ROWF(0x122) ROWF(0x121)
#undef ROWF
  return v;
}

// Chunk i (8 values) of the row-major activation rows; n8 chunks in all.
__device__ __forceinline__ void quant_chunk_fp8(const bf16_t* __restrict__ x,
                                                long i, long n8,
                                                uint8_t* __restrict__ codes,
                                                float* __restrict__ scales) {
  const bool valid = i < n8;               // whole rows of 16 lanes agree
  u32x4_t raw = {0u, 0u, 0u, 0u};
  if (valid) raw = *(const u32x4_t*)(x + 8 * i);
  float v[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[2 * q] = bf16_to_f32((bf16_t)(raw[q] & 0xFFFFu));
    v[2 * q + 1] = bf16_to_f32((bf16_t)(raw[q] >> 16));
  }
  float amax = 0.0f;
#pragma unroll
  for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(v[q]));
  amax = row_max_f32(amax);
  const float sc = amax == 0.0f ? 1.0f : __fdiv_rn(amax, 448.0f);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    lo |= (uint32_t)f32_to_e4m3(__fdiv_rn(v[q], sc)) << (8 * q);
    hi |= (uint32_t)f32_to_e4m3(__fdiv_rn(v[q + 4], sc)) << (8 * q);
  }
  if (!valid) return;
  *(uint2*)(codes + 8 * i) = make_uint2(lo, hi);
  if ((threadIdx.x & 15) == 0) scales[i >> 4] = sc;
}

__global__ __launch_bounds__(256) void k_quant_rows_fp8(
    const bf16_t* __restrict__ x, long n8, uint8_t* __restrict__ codes,
    float* __restrict__ scales) {
  quant_chunk_fp8(x, (long)blockIdx.x * 256 + threadIdx.x, n8, codes, scales);
}

// The FP8 layer's router and activation quantiser in one launch: the first
// nroute workgroups route 16 tokens each (route_row.h), the rest quantise,
// so the router's latency hides under the quantiser's stream instead of
// preceding it (the two read different inputs and write different outputs).
template <int KPL, bool BIAS>
__global__ __launch_bounds__(256) void k_route_quant_fp8(
    const float* __restrict__ logits, const float* __restrict__ bias, int T,
    int E, int k, int32_t* __restrict__ ids, float* __restrict__ w,
    int nroute, const bf16_t* __restrict__ x, long n8,
    uint8_t* __restrict__ codes, float* __restrict__ scales) {
  if ((int)blockIdx.x < nroute)
    route_rows_block<KPL, BIAS>(logits, bias, T, E, k, ids, w, blockIdx.x);
  else
    quant_chunk_fp8(x, (long)(blockIdx.x - nroute) * 256 + threadIdx.x, n8,
                    codes, scales);
}

hipError_t launch_route_quant_fp8(const float* logits, const float* bias,
                                  int T, int E, int k, int32_t* ids, float* w,
                                  const bf16_t* x, int H, uint8_t* codes,
                                  float* scales, hipStream_t s) {
  const int nroute = (T + 15) / 16;
  const long n8 = (long)T * H / 8;          // H % 128 == 0
  const unsigned grid = (unsigned)(nroute + (n8 + 255) / 256);
#define ROUTE_QUANT(KPL)                                                      \
  (bias ? k_route_quant_fp8<KPL, true><<<grid, 256, 0, s>>>(logits, bias, T, E, k, ids, w, nroute, x, n8, codes, scales) \
        : k_route_quant_fp8<KPL, false><<<grid, 256, 0, s>>>(logits, bias, T, E, k, ids, w, nroute, x, n8, codes, scales))
  if (E <= 16) ROUTE_QUANT(1);
  else if (E <= 32) ROUTE_QUANT(2);
  else if (E <= 64) ROUTE_QUANT(4);
  else if (E <= 128) ROUTE_QUANT(8);
  else ROUTE_QUANT(16);
#undef ROUTE_QUANT
  return hipGetLastError();
}

hipError_t launch_quant_rows_fp8(const bf16_t* x, int T, int H,
                                 uint8_t* codes, float* scales,
                                 hipStream_t s) {
  const long n8 = (long)T * H / 8;         // H % 128 == 0
  if (n8 == 0) return hipSuccess;
  k_quant_rows_fp8<<<(unsigned)((n8 + 255) / 256), 256, 0, s>>>(x, n8, codes,
                                                               scales);
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
