/*
 * moe.h -- C ABI of the expert-parallel MoE layer on one EP rank's share of
 * experts, for AMD Instinct MI355X (gfx950).
 *
 * The layer (pages as titled; see each entry point for its passage):
 *   route   -> each token's top-k experts and weights
 *   dispatch-> the rank keeps the pairs whose expert it owns and permutes the
 *              token rows into expert-contiguous order (on one GPU this is the
 *              local stand-in for the dispatch all-to-all)
 *   experts -> each physical expert's SwiGLU FFN on its rows (grouped GEMM)
 *   combine -> un-permute and sum each token's expert outputs weighted by its
 *              route weights, plus the optional shared expert
 * "6.4 Data parallelism and expert parallelism" (infra-guide), section 3.1,
 * lists these four steps; section 2.1 gives the expert as three matrices
 * gate, up, down and one shared expert per layer; "How Expert Parallelism
 * Works for Mixture-of-Experts Models in vLLM" (instagit), "MoE Layer
 * Construction", gives physical experts = logical + redundant replicas.
 *
 * Conventions for every entry point:
 *  - All arrays are device memory owned by the caller, except where an
 *    argument is marked "host".  The library allocates and frees nothing,
 *    never synchronises, and enqueues all work on `stream` (a hipStream_t;
 *    NULL means the null stream).  Calls return once work is enqueued.
 *  - Row-major layouts throughout.  bf16 data is passed as 16-bit patterns,
 *    fp8 data as one byte per element (OCP E4M3, "e4m3fn").
 *  - Activation and output row arrays (x, x_perm, x_shared, y_perm,
 *    y_shared, out) are 16-byte aligned, as any device allocator returns
 *    them: the kernels move rows with 16-byte loads and stores.  A
 *    misaligned one is INVALID_ARGUMENT.
 *  - Data-dependent sizes stay on the device: the number of local rows is
 *    offsets[P].  Row buffers are sized for the capacity
 *    cap = T * min(k, num_local) rows.
 *  - Errors are reported only through the returned status; nothing is
 *    printed and nothing aborts.  Argument errors are detected on the host
 *    before any work is enqueued.  Device-data preconditions (finite logits;
 *    topk_ids entries in [0, E); map entries in [0, P) or -1; each physical
 *    id used by exactly one (expert, replica)) are not checked beyond this:
 *    an id outside [0, E) is neither counted nor local (its pair_row is -1),
 *    and a map entry outside [0, P) drops its pair (pair_row -1).
 *  - T = 0 is valid: the call enqueues nothing and succeeds (an idle rank's
 *    dummy forward, infra-guide page, section 4.3).
 *  - Re-entrant; no global mutable state, except the per-device scratch of
 *    moe_layer_forward_noalloc (see there).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size or range          */
  MOE_ERR_UNSUPPORTED = 2,      /* dtype combination or shape not built     */
  MOE_ERR_WORKSPACE = 3,        /* workspace smaller than required          */
  MOE_ERR_HIP = 4               /* a HIP launch failed                       */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;

/* Shape of one call.  Supported dtype recipes:
 *   act F32,  weight F32,      out F32      (float32 arithmetic)
 *   act BF16, weight BF16,     out BF16|F32 (bf16 MFMA, fp32 accumulate)
 *   act BF16, weight FP8_E4M3, out BF16|F32 (activations quantised to E4M3
 *        per token per quant_block channels; fp8 MFMA, fp32 accumulate)
 * The FP8 recipe needs H and I to be multiples of quant_block (= 128) and at
 * most 16384. */
typedef struct {
  int32_t T;            /* tokens on this rank                               */
  int32_t H;            /* hidden size                                       */
  int32_t I;            /* expert intermediate size                          */
  int32_t E;            /* global logical experts                            */
  int32_t k;            /* experts per token, 1 <= k <= E                    */
  int32_t expert_begin; /* this rank owns logical experts                    */
  int32_t num_local;    /*   [expert_begin, expert_begin + num_local)        */
  int32_t num_physical; /* P >= 1 physical experts held here: num_local plus
                           local replicas, or a group-wide placement's S */
  int32_t max_replicas; /* columns of the logical-to-physical map (>= 1)     */
  int32_t has_shared;   /* 1: one always-on shared expert, weight 1          */
  int32_t act_dtype;    /* moe_dtype of x                                    */
  int32_t weight_dtype; /* moe_dtype of the expert weights                   */
  int32_t out_dtype;    /* moe_dtype of out                                  */
  int32_t quant_block;  /* fp8 block / group size; must be 128 for FP8      */
} moe_problem;

/* Storage order of a weight matrix handed to the one-time preparation calls.
 * An expert is three matrices ("6.4 Data parallelism and expert
 * parallelism", section 2.1: gate, up, down): W_gate and W_up with H rows and
 * I columns, W_down with I rows and H columns, so that
 *   h = silu(x W_gate) * (x W_up)   (x a row of H values)
 *   y = h W_down.
 * For a matrix with reduction size K and N output channels (gate/up: K = H,
 * N = I; down: K = I, N = H):
 *   MOE_LAYOUT_KN  the logical layout above, row-major [K][N]
 *   MOE_LAYOUT_NK  its transpose, row-major [N][K] (output-major, the way a
 *                  linear layer stores its weight) */
typedef enum { MOE_LAYOUT_KN = 0, MOE_LAYOUT_NK = 1 } moe_layout;

/* Expert weights, in the library's prepared form (made once, off the layer's
 * path, by moe_prepack_weights from either storage order):
 *   F32   the logical layout [K][N] itself (W_gate, W_up [H][I]; W_down
 *         [I][H]); a MOE_LAYOUT_KN source needs no preparation;
 *   BF16  packed operand blocks (see moe_prepack_weights);
 *   FP8   packed operand blocks of the E4M3 codes from
 *         moe_quantize_fp8_blocks, with float32 block scales (one per
 *         128 x 128 block) in output-block-major order [N/128][K/128]: gate
 *         and up [I/128][H/128], down [H/128][I/128], whatever the source's
 *         storage order was; scales are NULL for the other recipes.
 * w_gate, w_up, w_down and s_gate, s_up, s_down are DEVICE arrays of P
 * device pointers, one per physical expert (replicas may alias).  The sh_*
 * members are plain device pointers for the shared expert (NULL when
 * has_shared = 0).  Element type = weight_dtype. */
typedef struct {
  const void* const* w_gate;
  const void* const* w_up;
  const void* const* w_down;
  const float* const* s_gate;
  const float* const* s_up;
  const float* const* s_down;
  const void* sh_gate;
  const void* sh_up;
  const void* sh_down;
  const float* sh_s_gate;
  const float* sh_s_up;
  const float* sh_s_down;
} moe_weights;

/* Human-readable name of a status code (static storage). */
MOE_API const char* moe_status_string(moe_status s);

/* Validate a problem description (host only). */
MOE_API moe_status moe_check_problem(const moe_problem* p);

/* Bytes of scratch each entry point needs (host only).  Workspaces must be
 * 256-byte aligned device memory; their contents need not be initialised.
 * moe_workspace_size gives one size that serves every entry point of the
 * problem (the largest of the three below); the others give what
 * moe_dispatch, moe_grouped_ffn and moe_layer_forward need alone. */
MOE_API moe_status moe_workspace_size(const moe_problem* p, size_t* bytes);
MOE_API moe_status moe_dispatch_workspace_size(const moe_problem* p, size_t* bytes);
MOE_API moe_status moe_ffn_workspace_size(const moe_problem* p, size_t* bytes);
MOE_API moe_status moe_layer_workspace_size(const moe_problem* p, size_t* bytes);

/* Router top-k ("6.4 Data parallelism and expert parallelism", section 3.1,
 * step 1: each token gets its top-k experts and weights).
 *   logits        [T][E] float32
 *   bias          [E] float32 added to every token's logits, or NULL
 *   topk_ids      [T][k] int32 out: slot j holds the j-th largest score
 *                 s = fl32(logit + bias); equal scores keep the lower expert
 *                 id first (+0.0 and -0.0 are equal)
 *   topk_w        [T][k] float32 out: softmax over all E renormalised over
 *                 the k chosen = exp(s_j - s_0) / sum_i exp(s_i - s_0)
 *   expert_counts [E] int32 out (overwritten): pairs per logical expert over
 *                 all T tokens -- the per-expert load an EPLB records
 *                 (infra-guide page, section 5.3).  May be NULL. */
MOE_API moe_status moe_route_topk(const moe_problem* p, const float* logits,
                          const float* bias, int32_t* topk_ids,
                          float* topk_w, int32_t* expert_counts,
                          void* stream);

/* Dispatch: local filter, replica remap and expert-contiguous permutation
 * (infra-guide page, section 3.1, step 2, and section 5.3 for replicas).
 *   x             [T][H] activations (act_dtype)
 *   topk_ids/_w   from moe_route_topk
 *   l2p           [num_local][max_replicas] int32 logical-to-physical map;
 *                 column r < replica_count[e] holds the physical id of
 *                 replica r of local expert e, or -1 when that replica is
 *                 placed on another rank (section 5.2's placement spreads an
 *                 expert's replicas over cards): such pairs count in n below
 *                 but are not local here.  NULL = identity (P must equal
 *                 num_local and replica_count must be NULL).
 *   replica_count [num_local] int32, each in [1, max_replicas], or NULL
 * A local pair is (t, j) with topk_ids[t][j] in the rank's range.  Walking
 * pairs in token order, the n-th pair of local expert e goes to physical
 * expert l2p[e][n mod R_e] at position floor(n / R_e) of its segment;
 * segments follow physical-id order.  Outputs (capacity cap rows):
 *   x_perm        [cap][H] the token rows in permuted order: act_dtype, or,
 *                 for the FP8 recipe, E4M3 codes of the token quantised per
 *                 quant_block channels (scale = amax/448, code = RNE of
 *                 fl32(x/scale), saturated)
 *   x_perm_scales [cap][H/quant_block] float32 scales (FP8 recipe; else NULL)
 *   offsets       [P+1] int32: segment starts, offsets[P] = local rows N
 *   row_token     [cap] int32 token of each row (rows >= N untouched)
 *   row_weight    [cap] float32 route weight of each row
 *   pair_row      [T][k] int32 row of each pair, -1 for non-local pairs
 * Identical inputs give bit-identical outputs (no atomics decide order). */
MOE_API moe_status moe_dispatch(const moe_problem* p, const void* x,
                        const int32_t* topk_ids, const float* topk_w,
                        const int32_t* l2p, const int32_t* replica_count,
                        void* x_perm, float* x_perm_scales, int32_t* offsets,
                        int32_t* row_token, float* row_weight,
                        int32_t* pair_row, void* workspace, size_t ws_bytes,
                        void* stream);

/* Grouped expert FFN (infra-guide page, section 2.1: gate, up, down; section
 * 3.1, step 3: each card runs its experts on the tokens it received).
 * For every physical expert p and every row r in [offsets[p],
 * offsets[p+1]):  h = silu(x_perm[r] Wg_p) * (x_perm[r] Wu_p), rounded to
 * bf16 (BF16 recipe), to E4M3 per row per 128 channels (FP8 recipe) or to
 * float32; y_perm[r] = h Wd_p in float32.  With has_shared, the same for the
 * shared expert on every token row of x_shared into y_shared.
 *   x_perm, x_perm_scales, offsets   as produced by moe_dispatch
 *   x_shared      [T][H] rows for the shared expert in the same encoding as
 *                 x_perm (FP8: codes), with x_shared_scales [T][H/128]; NULL
 *                 when has_shared = 0
 *   y_perm        [cap][H] float32 out;  y_shared [T][H] float32 out */
MOE_API moe_status moe_grouped_ffn(const moe_problem* p, const void* x_perm,
                           const float* x_perm_scales, const int32_t* offsets,
                           const void* x_shared, const float* x_shared_scales,
                           const moe_weights* w, float* y_perm,
                           float* y_shared, void* workspace, size_t ws_bytes,
                           void* stream);

/* Where moe_grouped_ffn left the expert intermediate h inside `workspace`
 * (host only; the workspace passed to that call).  Once the call's work has
 * completed on its stream, the device arrays hold
 *   h         [cap + T][I]: routed row r (r < offsets[P], the permuted
 *             order of moe_dispatch) in row r, the shared expert's row of
 *             token t in row cap + t; element type bf16 (BF16 recipe), E4M3
 *             codes (FP8 recipe, the value is code * scale) or float32
 *   h_scales  [cap + T][I/128] float32 scales of the FP8 recipe (one per row
 *             per 128 channels), set to NULL for the other recipes
 * h is the value the down projection multiplies: silu(x W_gate) * (x W_up)
 * after its rounding (infra-guide page, section 2.1).  WORKSPACE when
 * ws_bytes is below moe_ffn_workspace_size. */
MOE_API moe_status moe_ffn_intermediate(const moe_problem* p, void* workspace,
                                        size_t ws_bytes, void** h,
                                        float** h_scales);

/* Combine (infra-guide page, section 3.1, step 4: results return to the
 * token and are summed weighted by the route weights).
 *   out[t] = sum over slots j ascending with pair_row[t][j] >= 0 of
 *            topk_w[t][j] * y_perm[pair_row[t][j]]  (+ y_shared[t])
 * accumulated in float32 and rounded once to out_dtype.  Tokens with no
 * local pair and no shared expert get zero rows.
 *   y_shared may be NULL (then has_shared is ignored). */
MOE_API moe_status moe_combine(const moe_problem* p, const float* y_perm,
                       const int32_t* pair_row, const float* topk_w,
                       const float* y_shared, void* out, void* stream);

/* The whole layer: route -> dispatch -> grouped FFN -> combine, all on
 * `stream`, with intermediates in `workspace`.
 *   out           [T][H] out_dtype
 *   expert_counts [E] int32 out, or NULL
 * Other arguments as in the single steps. */
MOE_API moe_status moe_layer_forward(const moe_problem* p, const float* logits,
                             const float* bias, const void* x,
                             const moe_weights* w, const int32_t* l2p,
                             const int32_t* replica_count, void* out,
                             int32_t* expert_counts, void* workspace,
                             size_t ws_bytes, void* stream);

/* Profiling variant of moe_layer_forward: the same work, plus hipEventRecord
 * on `stream` at the stage boundaries, so a caller can time each stage with
 * hipEventElapsedTime.  events: HOST array of MOE_STAGE_EVENTS hipEvent_t
 * handles created by the caller; recorded in order
 *   [0] start  [1] route done  [2] dispatch index done  [3] row gather done
 *   [4] FFN tile list built  [5] gate/up done  [6] down done  [7] combine done
 * (on the T = 0 path nothing is recorded).  The layer writes no permuted
 * copy of the rows (the expert kernels read token rows through the
 * dispatch's row index), so [2, 3] holds only the FP8 activation quantiser
 * when it runs on its own (E > 256); with E <= 256 it shares the router's
 * launch and falls in [0, 1].  The quantisation of h to E4M3 falls in the
 * down interval [5, 6] except where the gate/up kernel does it itself
 * (groups of a few rows). */
#define MOE_STAGE_EVENTS 8
MOE_API moe_status moe_layer_forward_timed(const moe_problem* p,
                                   const float* logits, const float* bias,
                                   const void* x, const moe_weights* w,
                                   const int32_t* l2p,
                                   const int32_t* replica_count, void* out,
                                   int32_t* expert_counts, void* workspace,
                                   size_t ws_bytes, void* stream,
                                   void* const* events);

/* moe_layer_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same work, with the workspace taken from a device array
 * the library holds, MOE_NOALLOC_SCRATCH_BYTES on each GPU it runs on (kept
 * until the process ends), instead of a caller's buffer.  The call itself
 * allocates nothing.  WORKSPACE when the problem needs more than that
 * (moe_layer_workspace_size; e.g. a 256-token decode batch at H = 6144,
 * I = 2048, 32 local experts needs 56 MiB).  Every call on one GPU shares
 * its array and the array keeps the last call's contents (the layer needs
 * none of them: whatever must start at zero is cleared by its kernels), so
 * calls that overlap on one GPU -- on different streams, or from different
 * threads -- race; calls one after another on one stream do not.  The
 * array's address on each device is looked up once, on that device's first
 * call (the device of `stream`, or the current device for the null
 * stream). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
MOE_API moe_status moe_layer_forward_noalloc(const moe_problem* p,
                                             const float* logits,
                                             const float* bias, const void* x,
                                             const moe_weights* w,
                                             const int32_t* l2p,
                                             const int32_t* replica_count,
                                             void* out, int32_t* expert_counts,
                                             void* stream);

/* One-time weight preparation (not on the layer's path): a matrix with
 * reduction size K and N output channels, stored as `layout` says (see
 * moe_layout: gate/up K = H, N = I; down K = I, N = H), into the prepared
 * form that moe_weights holds for `dtype`:
 *   MOE_F32       dst = the logical layout [K][N] (a copy, or the transpose
 *                 of a MOE_LAYOUT_NK source)
 *   MOE_BF16      packed operand blocks: the matrix is cut into blocks of 16
 *                 output channels x 32 reduction values; block (n/16, k/32)
 *                 is stored at block index (n/16) * (K/32) + k/32, 1 KiB per
 *                 block; inside a block, 16-byte lane L = n%16 + 16*((k%32)/8)
 *                 holds the 8 values k%8 = 0..7.  16 output channels over the
 *                 whole reduction form one contiguous run and each 1 KiB block
 *                 is one wavefront's matrix-core operand.  Needs N % 16 == 0,
 *                 K % 32 == 0.
 *   MOE_FP8_E4M3  src holds E4M3 codes (from moe_quantize_fp8_blocks);
 *                 blocks of 16 output channels x 128 reduction values, 2 KiB,
 *                 block (n/16, k/128) at block index (n/16) * (K/128) + k/128;
 *                 lane L = n%16 + 16*((k%128)/32) owns 32 codes, the first 16
 *                 at byte L*16 of the block and the rest at 1024 + L*16.
 *                 Needs N % 16 == 0, K % 128 == 0.
 * src and dst are distinct device buffers of K*N elements.  UNSUPPORTED for
 * another dtype, INVALID_ARGUMENT for a bad layout or shape. */
MOE_API moe_status moe_prepack_weights(const void* src, int32_t K, int32_t N,
                                       int32_t dtype, int32_t layout,
                                       void* dst, void* stream);

/* One-time weight preparation for the FP8 recipe (not on the layer's path):
 * quantise a float32 matrix (reduction size K, N outputs, stored as `layout`
 * says) to E4M3 with one float32 scale per block x block tile (block = 128):
 * scale = amax/448 over the tile (1 for an all-zero tile), code = RNE of
 * fl32(w/scale) saturated to +-448.
 *   w      float32 [K][N] (MOE_LAYOUT_KN) or [N][K] (MOE_LAYOUT_NK)
 *   codes  uint8 out, in the same storage order as w (to be packed by
 *          moe_prepack_weights with the same layout)
 *   scales float32 out, [N/128][K/128] whatever the layout (the order
 *          moe_weights takes).
 * K and N must be multiples of block. */
MOE_API moe_status moe_quantize_fp8_blocks(const float* w, int32_t K, int32_t N,
                                   int32_t block, int32_t layout,
                                   uint8_t* codes, float* scales,
                                   void* stream);

/* Host-side replica map for a skewed rank (infra-guide page, section 5.3:
 * redundant experts replicate hot experts so their load splits).  The
 * `redundant` local experts with the most pairs (lower id on ties) get one
 * extra replica each; physical id num_local + i is the second replica of
 * the i-th hottest.  All arrays are HOST memory.
 *   local_counts [num_local] pairs per local expert (e.g. from
 *                expert_counts[expert_begin ...])
 *   l2p          [num_local][2] out (-1 padded); replica_count [num_local]
 *   num_physical out: num_local + redundant */
MOE_API moe_status moe_eplb_hottest_map(const int32_t* local_counts,
                                int32_t num_local, int32_t redundant,
                                int32_t* l2p, int32_t* replica_count,
                                int32_t* num_physical);

/* Replica plan and placement over an EP group (infra-guide page, section
 * 5.2: redundant slots go one at a time to the expert with the highest load
 * per replica; replicas are then placed heaviest first onto the currently
 * lightest rank that still has a free slot; section 5.3: every rank holds
 * (E + redundant) / ep physical experts).  All arrays are HOST memory.
 *   load         [E] int64 load per logical expert (e.g. a window sum from
 *                moe_eplb_record_load), each >= 0
 *   replicas     [E] out: replica count per expert (sums to E + redundant)
 *   slot_expert  [ep][S] out, S = (E + redundant) / ep: rank g's physical
 *                expert s is a replica of expert slot_expert[g][s]; a rank's
 *                slots are in (expert, replica) order
 *   slot_replica [ep][S] out: which replica of that expert
 *   rank_load    [ep] out: sum over the rank's replicas of load / replicas,
 *                added in placement order
 * Ties: the lower expert id gets a redundant slot; equal per-replica loads
 * are placed in (expert, replica) order; the lower rank wins among equally
 * light ranks.  INVALID_ARGUMENT when (E + redundant) % ep != 0 or a load
 * is negative. */
MOE_API moe_status moe_eplb_plan(const int64_t* load, int32_t E, int32_t ep,
                         int32_t redundant, int32_t* replicas,
                         int32_t* slot_expert, int32_t* slot_replica,
                         double* rank_load);

/* One rank's dispatch map under a plan from moe_eplb_plan, for a problem
 * with expert_begin = 0, num_local = E, num_physical = S and max_replicas
 * columns.  All arrays are HOST memory.
 *   l2p           [E][max_replicas] out: physical id on this rank of replica
 *                 r of expert e, -1 when it is placed on another rank
 *   replica_count [E] out: the expert's replica count over the whole group
 *   num_physical  out: S
 * INVALID_ARGUMENT when a replica count exceeds max_replicas or the plan's
 * entries are out of range. */
MOE_API moe_status moe_eplb_rank_map(const int32_t* replicas,
                             const int32_t* slot_expert,
                             const int32_t* slot_replica, int32_t E,
                             int32_t ep, int32_t redundant, int32_t rank,
                             int32_t max_replicas, int32_t* l2p,
                             int32_t* replica_count, int32_t* num_physical);

/* Sliding-window load record (section 5.3: the balancer records per-expert
 * load every forward and plans from the most recent window of steps).
 * Enqueued on `stream`; no synchronisation.
 *   expert_counts [E] int32 device: this step's pairs per expert (the
 *                 expert_counts output of moe_route_topk/moe_layer_forward)
 *   history       [window][E] int32 device ring, zeroed by the caller
 *                 before step 0
 *   window_load   [E] int64 device, zeroed with the history: after the call
 *                 for step s it holds the sum of the counts of steps
 *                 max(0, s - window + 1) .. s
 * Calls must come in step order 0, 1, 2, ... on one stream; step selects the
 * ring slot step % window. */
MOE_API moe_status moe_eplb_record_load(const int32_t* expert_counts,
                                int32_t E, int32_t window, int64_t step,
                                int32_t* history, int64_t* window_load,
                                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
