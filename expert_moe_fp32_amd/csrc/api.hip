// C ABI of the MoE layer: argument validation, workspace layout and the
// launch sequence of each step.  No allocation, no synchronisation.
#include <algorithm>
#include <numeric>
#include <vector>

#include "common.h"

using namespace moe;

namespace {

struct Carver {  // hands out 256-byte aligned pieces of a workspace
  char* base;
  size_t used = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <class T>
  T* take(size_t count) {
    T* p = base ? (T*)(base + used) : nullptr;
    used += moe_align256(count * sizeof(T));
    return p;
  }
};

inline size_t dtype_bytes(int d) {
  return d == MOE_F32 ? 4 : (d == MOE_BF16 ? 2 : 1);
}

inline long cap_rows(const moe_problem* p) {
  return (long)p->T * std::min(p->k, p->num_local);
}

inline hipStream_t S(void* s) { return (hipStream_t)s; }

inline moe_status hip_status(hipError_t e) {
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// scratch of the dispatch step (also used by the layer)
struct DispatchScratch {
  int32_t* block_counts;
  int32_t* block_base;
  int32_t* block_ecounts;  // [nblk][E] partial expert counts
  uint8_t* xq;     // fp8: [T][H] codes of every token
  float* xs;       // fp8: [T][H/128]
};

DispatchScratch carve_dispatch(Carver& c, const moe_problem* p) {
  DispatchScratch d{};
  const size_t nb = (size_t)dispatch_blocks(p->T) * p->num_local;
  d.block_counts = c.take<int32_t>(nb);
  d.block_base = c.take<int32_t>(nb);
  d.block_ecounts = c.take<int32_t>((size_t)dispatch_blocks(p->T) * p->E);
  if (p->weight_dtype == MOE_FP8_E4M3) {
    d.xq = c.take<uint8_t>((size_t)p->T * p->H);
    d.xs = c.take<float>((size_t)p->T * (p->H / 128));
  }
  return d;
}

// Expected rows per physical expert: the local pairs over the physical
// experts, where a rank with fewer physical than logical experts (a
// group-wide placement whose other replicas sit on other ranks) expects
// about one logical expert's pairs per physical expert.
int rows_hint(const moe_problem* p) {
  const double pairs = (double)p->T * p->k * p->num_local / p->E;
  return (int)(pairs / std::max(p->num_physical, p->num_local) + 0.5);
}

struct FfnScratch {
  void* h;
  float* h_scales;
  float* h32;
  int4* tiles;
  int4* tiles_down;
  int32_t* tile_count;
  int max_tiles;
};

FfnScratch carve_ffn(Carver& c, const moe_problem* p) {
  FfnScratch f{};
  const long cap = cap_rows(p);
  const size_t hrows = (size_t)cap + (p->has_shared ? p->T : 0);
  const size_t hb = p->act_dtype == MOE_F32 ? 4
                    : (p->weight_dtype == MOE_FP8_E4M3 ? 1 : 2);
  f.h = c.take<char>(hrows * p->I * hb);
  if (p->weight_dtype == MOE_FP8_E4M3) {
    f.h_scales = c.take<float>(hrows * (p->I / 128));
    // float32 h only for the kernels that leave quantisation to a pass of
    // its own (the 32-row register-streaming kernel quantises in place)
    int balanced;
    if (ffn_fp8_tile_rows(rows_hint(p), p->H, p->I, &balanced) != 32)
      f.h32 = c.take<float>(hrows * p->I);
  }
  // descriptors: at most one per 16 rows plus one per group, and the four
  // quarters of a tall tile (groups of more than 32 rows) at most one per 8
  // rows of their group
  f.max_tiles = (int)(p->num_physical + 2 + (hrows + 15) / 16 + (hrows + 7) / 8);
  f.tiles = c.take<int4>((size_t)f.max_tiles);
  // 128-row tiles (or the FP8 streaming down pass's tiles: one per group of
  // up to 32 rows, tall tiles of up to 128 beyond): at most one partial tile
  // per group
  f.tiles_down = c.take<int4>((size_t)p->num_physical + 2 + hrows / 128);
  f.tile_count = c.take<int32_t>(4);
  return f;
}

moe_status launch_ffn_common(const moe_problem* p, const void* x_perm,
                             const float* x_perm_scales,
                             const int32_t* offsets, const void* x_shared,
                             const float* x_shared_scales,
                             const moe_weights* w, float* y_perm,
                             float* y_shared, const FfnScratch& fs,
                             hipStream_t s, hipEvent_t* events = nullptr,
                             const int32_t* a_rows = nullptr,
                             bool tiles_ready = false) {
  FfnArgs a{};
  a.a_rows = a_rows;
  a.tiles_ready = tiles_ready;
  a.H = p->H;
  a.I = p->I;
  a.P = p->num_physical;
  a.T = p->T;
  a.cap = (int)cap_rows(p);
  a.has_shared = p->has_shared;
  a.rows_hint = rows_hint(p);
  a.act = p->act_dtype;
  a.wdt = p->weight_dtype;
  a.offsets = offsets;
  a.a_routed = x_perm;
  a.a_routed_scales = x_perm_scales;
  a.a_shared = x_shared;
  a.a_shared_scales = x_shared_scales;
  a.w = w;
  a.h = fs.h;
  a.h_scales = fs.h_scales;
  a.h32 = fs.h32;
  a.y_routed = y_perm;
  a.y_shared = y_shared;
  a.tiles = fs.tiles;
  a.tiles_down = fs.tiles_down;
  a.tile_count = fs.tile_count;
  a.max_tiles = fs.max_tiles;
  a.events = events;
  return hip_status(launch_ffn(a, s));
}

moe_status check_weights(const moe_problem* p, const moe_weights* w) {
  if (!w || !w->w_gate || !w->w_up || !w->w_down)
    return MOE_ERR_INVALID_ARGUMENT;
  if (p->weight_dtype == MOE_FP8_E4M3 && (!w->s_gate || !w->s_up || !w->s_down))
    return MOE_ERR_INVALID_ARGUMENT;
  if (p->has_shared) {
    if (!w->sh_gate || !w->sh_up || !w->sh_down) return MOE_ERR_INVALID_ARGUMENT;
    if (p->weight_dtype == MOE_FP8_E4M3 &&
        (!w->sh_s_gate || !w->sh_s_up || !w->sh_s_down))
      return MOE_ERR_INVALID_ARGUMENT;
  }
  return MOE_OK;
}

moe_status dispatch_impl(const moe_problem* p, const void* x,
                         const int32_t* ids, const float* tw,
                         const int32_t* l2p, const int32_t* rep,
                         void* x_perm, float* x_perm_scales, int32_t* offsets,
                         int32_t* row_token, float* row_weight,
                         int32_t* pair_row, const DispatchScratch& d,
                         hipStream_t s, hipEvent_t ev_index = nullptr,
                         bool materialize = true,
                         const DispatchExtras* extras = nullptr,
                         bool x_quantised = false) {
  DispatchArgs a{};
  a.T = p->T;
  a.k = p->k;
  a.expert_begin = p->expert_begin;
  a.num_local = p->num_local;
  a.P = p->num_physical;
  a.max_rep = l2p ? p->max_replicas : 1;
  a.H = p->H;
  a.ids = ids;
  a.w = tw;
  a.l2p = l2p;
  a.rep = rep;
  a.block_counts = d.block_counts;
  a.block_base = d.block_base;
  a.block_ecounts = d.block_ecounts;
  a.offsets = offsets;
  a.row_token = row_token;
  a.row_weight = row_weight;
  a.pair_row = pair_row;
  hipError_t e;
  DispatchExtras xt{};
  xt.E = p->E;
  if (extras) xt = *extras;
  if (dispatch_small_ok(p->T, p->E, p->num_local, p->num_physical))
    e = launch_dispatch_small(a, xt, s);
  else
    e = launch_dispatch_index(a, xt, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (ev_index) hipEventRecord(ev_index, s);
  const int cap = (int)cap_rows(p);
  const int32_t* nrows = offsets + p->num_physical;
  if (p->weight_dtype == MOE_FP8_E4M3) {
    if (!x_quantised)     // else done with the router (launch_route_quant_fp8)
      e = launch_quant_rows_fp8((const bf16_t*)x, p->T, p->H, d.xq, d.xs, s);
    if (e != hipSuccess || !materialize) return hip_status(e);
    e = launch_gather_rows(d.xq, (size_t)p->H, row_token, nrows, cap, x_perm, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
    // scales: H/128 floats per row, gathered 4 bytes at a time
    e = launch_gather_rows_words(d.xs, p->H / 128, row_token, nrows, cap,
                                 x_perm_scales, s);
    return hip_status(e);
  }
  if (!materialize) return MOE_OK;
  e = launch_gather_rows(x, (size_t)p->H * dtype_bytes(p->act_dtype),
                         row_token, nrows, cap, x_perm, s);
  return hip_status(e);
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported dtype or shape";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

moe_status moe_check_problem(const moe_problem* p) {
  if (!p) return MOE_ERR_INVALID_ARGUMENT;
  if (p->T < 0 || p->H <= 0 || p->I <= 0 || p->E <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if (p->k < 1 || p->k > p->E) return MOE_ERR_INVALID_ARGUMENT;
  if (p->expert_begin < 0 || p->num_local < 1 ||
      (long)p->expert_begin + p->num_local > p->E)
    return MOE_ERR_INVALID_ARGUMENT;
  if (p->num_physical < 1 || p->max_replicas < 1)
    return MOE_ERR_INVALID_ARGUMENT;
  if (p->has_shared != 0 && p->has_shared != 1) return MOE_ERR_INVALID_ARGUMENT;
  const int a = p->act_dtype, w = p->weight_dtype, o = p->out_dtype;
  if (a < 0 || a > 2 || w < 0 || w > 2 || o < 0 || o > 2) return MOE_ERR_INVALID_ARGUMENT;
  if (p->k > MOE_KMAX || p->E > MOE_EMAX || p->num_physical > MOE_LMAX)
    return MOE_ERR_UNSUPPORTED;
  if (o == MOE_FP8_E4M3) return MOE_ERR_UNSUPPORTED;
  if (a == MOE_F32 && w == MOE_F32) {
    if (p->H % 4) return MOE_ERR_UNSUPPORTED;
  } else if (a == MOE_BF16 && w == MOE_BF16) {
    if (p->H % 128 || p->I % 128) return MOE_ERR_UNSUPPORTED;
  } else if (a == MOE_BF16 && w == MOE_FP8_E4M3) {
    // reductions of at most 128 scale blocks (the kernels keep a tile's
    // weight-scale column in LDS)
    if (p->quant_block != 128 || p->H % 128 || p->I % 128 || p->H > 16384 ||
        p->I > 16384)
      return MOE_ERR_UNSUPPORTED;
  } else {
    return MOE_ERR_UNSUPPORTED;
  }
  // row indices are 32-bit
  if ((double)p->T * p->k >= 2147483647.0) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status moe_dispatch_workspace_size(const moe_problem* p, size_t* bytes) {
  moe_status st = moe_check_problem(p);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARGUMENT;
  Carver c(nullptr);
  carve_dispatch(c, p);
  *bytes = c.used;
  return MOE_OK;
}

moe_status moe_ffn_workspace_size(const moe_problem* p, size_t* bytes) {
  moe_status st = moe_check_problem(p);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARGUMENT;
  Carver c(nullptr);
  carve_ffn(c, p);
  *bytes = c.used;
  return MOE_OK;
}

namespace {
struct LayerScratch {
  int32_t* ids;
  float* tw;
  int32_t* counts;
  int32_t* offsets;
  int32_t* row_token;
  float* row_weight;
  int32_t* pair_row;
  void* x_perm;
  float* x_perm_scales;
  float* y_perm;
  float* y_shared;
  DispatchScratch d;
  FfnScratch f;
};

LayerScratch carve_layer(Carver& c, const moe_problem* p) {
  LayerScratch L{};
  const size_t Tk = (size_t)p->T * p->k;
  const size_t cap = (size_t)cap_rows(p);
  L.ids = c.take<int32_t>(Tk);
  L.tw = c.take<float>(Tk);
  L.counts = c.take<int32_t>((size_t)p->E);
  L.offsets = c.take<int32_t>((size_t)p->num_physical + 1);
  L.row_token = c.take<int32_t>(cap);
  L.row_weight = c.take<float>(cap);
  L.pair_row = c.take<int32_t>(Tk);
  // no permuted activation copy: the expert kernels gather rows themselves
  L.y_perm = c.take<float>(cap * p->H);
  if (p->has_shared) L.y_shared = c.take<float>((size_t)p->T * p->H);
  L.d = carve_dispatch(c, p);
  L.f = carve_ffn(c, p);
  return L;
}
}  // namespace

moe_status moe_layer_workspace_size(const moe_problem* p, size_t* bytes) {
  moe_status st = moe_check_problem(p);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARGUMENT;
  Carver c(nullptr);
  carve_layer(c, p);
  *bytes = c.used;
  return MOE_OK;
}

moe_status moe_workspace_size(const moe_problem* p, size_t* bytes) {
  moe_status st = moe_check_problem(p);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARGUMENT;
  size_t d = 0, f = 0, l = 0;
  moe_dispatch_workspace_size(p, &d);
  moe_ffn_workspace_size(p, &f);
  moe_layer_workspace_size(p, &l);
  *bytes = std::max(d, std::max(f, l));
  return MOE_OK;
}

moe_status moe_ffn_intermediate(const moe_problem* p, void* workspace,
                                size_t ws_bytes, void** h, float** h_scales) {
  moe_status st = moe_check_problem(p);
  if (st != MOE_OK) return st;
  if (!h || !h_scales) return MOE_ERR_INVALID_ARGUMENT;
  size_t need;
  moe_ffn_workspace_size(p, &need);
  if (!workspace || ws_bytes < need) return MOE_ERR_WORKSPACE;
  Carver c(workspace);
  FfnScratch fs = carve_ffn(c, p);
  *h = fs.h;
  *h_scales = p->weight_dtype == MOE_FP8_E4M3 ? fs.h_scales : nullptr;
  return MOE_OK;
}

moe_status moe_route_topk(const moe_problem* p, const float* logits,
                          const float* bias, int32_t* topk_ids, float* topk_w,
                          int32_t* expert_counts, void* stream) {
  moe_status st = moe_check_problem(p);
  if (st != MOE_OK) return st;
  if (p->T == 0) {
    if (expert_counts)
      return hip_status(launch_fill_i32(expert_counts, 0, (size_t)p->E, S(stream)));
    return MOE_OK;
  }
  if (!logits || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARGUMENT;
  return hip_status(launch_route_topk(logits, bias, p->T, p->E, p->k, topk_ids,
                                      topk_w, expert_counts, S(stream)));
}

// 16-byte vector loads and stores touch the row arrays
static inline bool al16(const void* q) { return ((uintptr_t)q & 15) == 0; }

static moe_status check_map(const moe_problem* p, const int32_t* l2p,
                            const int32_t* rep) {
  if (!l2p) {
    if (rep || p->num_physical != p->num_local) return MOE_ERR_INVALID_ARGUMENT;
  } else if (!rep) {
    return MOE_ERR_INVALID_ARGUMENT;
  }
  return MOE_OK;
}

moe_status moe_dispatch(const moe_problem* p, const void* x,
                        const int32_t* topk_ids, const float* topk_w,
                        const int32_t* l2p, const int32_t* replica_count,
                        void* x_perm, float* x_perm_scales, int32_t* offsets,
                        int32_t* row_token, float* row_weight,
                        int32_t* pair_row, void* workspace, size_t ws_bytes,
                        void* stream) {
  moe_status st = moe_check_problem(p);
  if (st != MOE_OK) return st;
  if ((st = check_map(p, l2p, replica_count)) != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;
  if (!x || !topk_ids || !topk_w || !x_perm || !offsets || !row_token ||
      !row_weight || !pair_row)
    return MOE_ERR_INVALID_ARGUMENT;
  if (p->weight_dtype == MOE_FP8_E4M3 && !x_perm_scales) return MOE_ERR_INVALID_ARGUMENT;
  if (!al16(x) || !al16(x_perm)) return MOE_ERR_INVALID_ARGUMENT;
  size_t need;
  moe_dispatch_workspace_size(p, &need);
  if (need && (!workspace || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  Carver c(workspace);
  DispatchScratch d = carve_dispatch(c, p);
  return dispatch_impl(p, x, topk_ids, topk_w, l2p, replica_count, x_perm,
                       x_perm_scales, offsets, row_token, row_weight, pair_row,
                       d, S(stream));
}

moe_status moe_grouped_ffn(const moe_problem* p, const void* x_perm,
                           const float* x_perm_scales, const int32_t* offsets,
                           const void* x_shared, const float* x_shared_scales,
                           const moe_weights* w, float* y_perm,
                           float* y_shared, void* workspace, size_t ws_bytes,
                           void* stream) {
  moe_status st = moe_check_problem(p);
  if (st != MOE_OK) return st;
  if ((st = check_weights(p, w)) != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;
  if (!x_perm || !offsets || !y_perm) return MOE_ERR_INVALID_ARGUMENT;
  const bool fp8 = p->weight_dtype == MOE_FP8_E4M3;
  if (fp8 && !x_perm_scales) return MOE_ERR_INVALID_ARGUMENT;
  if (p->has_shared && (!x_shared || !y_shared || (fp8 && !x_shared_scales)))
    return MOE_ERR_INVALID_ARGUMENT;
  if (!al16(x_perm) || !al16(x_shared) || !al16(y_perm) || !al16(y_shared))
    return MOE_ERR_INVALID_ARGUMENT;
  size_t need;
  moe_ffn_workspace_size(p, &need);
  if (!workspace || ws_bytes < need) return MOE_ERR_WORKSPACE;
  Carver c(workspace);
  FfnScratch fs = carve_ffn(c, p);
  return launch_ffn_common(p, x_perm, x_perm_scales, offsets, x_shared,
                           x_shared_scales, w, y_perm, y_shared, fs, S(stream));
}

moe_status moe_combine(const moe_problem* p, const float* y_perm,
                       const int32_t* pair_row, const float* topk_w,
                       const float* y_shared, void* out, void* stream) {
  moe_status st = moe_check_problem(p);
  if (st != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;
  if (!y_perm || !pair_row || !topk_w || !out) return MOE_ERR_INVALID_ARGUMENT;
  if (!al16(y_perm) || !al16(y_shared) || !al16(out)) return MOE_ERR_INVALID_ARGUMENT;
  return hip_status(launch_combine(y_perm, pair_row, topk_w, y_shared, p->T,
                                   p->H, p->k, p->out_dtype, out, S(stream)));
}

static moe_status layer_impl(const moe_problem* p, const float* logits,
                             const float* bias, const void* x,
                             const moe_weights* w, const int32_t* l2p,
                             const int32_t* replica_count, void* out,
                             int32_t* expert_counts, void* workspace,
                             size_t ws_bytes, void* stream, hipEvent_t* ev) {
  moe_status st = moe_check_problem(p);
  if (st != MOE_OK) return st;
  if ((st = check_map(p, l2p, replica_count)) != MOE_OK) return st;
  if ((st = check_weights(p, w)) != MOE_OK) return st;
  hipStream_t s = S(stream);
  if (p->T == 0) {
    if (expert_counts)
      return hip_status(launch_fill_i32(expert_counts, 0, (size_t)p->E, s));
    return MOE_OK;
  }
  if (!logits || !x || !out) return MOE_ERR_INVALID_ARGUMENT;
  if (!al16(x) || !al16(out)) return MOE_ERR_INVALID_ARGUMENT;
  size_t need;
  moe_layer_workspace_size(p, &need);
  if (!workspace || ws_bytes < need) return MOE_ERR_WORKSPACE;
  Carver c(workspace);
  LayerScratch L = carve_layer(c, p);
  if (ev) hipEventRecord(ev[0], s);
  int32_t* counts = expert_counts ? expert_counts : L.counts;
  // The dispatch's single-workgroup stage counts the experts and writes the
  // FFN tile list, so neither needs a launch of its own.
  DispatchExtras extras{};
  extras.E = p->E;
  extras.counts = counts;
  extras.tiles = L.f.tiles;
  extras.tile_count = L.f.tile_count;
  extras.BM = ffn_tile_rows(p->act_dtype, p->weight_dtype, rows_hint(p),
                            p->H, p->I, &extras.balanced);
  extras.tallBM = ffn_tall_rows(p->act_dtype, p->weight_dtype, extras.BM);
  extras.tallBM2 = ffn_down_tall_rows(p->weight_dtype, extras.BM);
  if (extras.tallBM2) {           // the down pass's own list
    extras.tiles2 = L.f.tiles_down;
    extras.count2 = L.f.tile_count + 1;
  }
  extras.has_shared = p->has_shared;
  // FP8 recipe: the router and the activation quantiser share one launch
  // (the quantiser reads only x), so the router's latency hides under the
  // quantiser's stream; the route stage then holds both.
  const bool fp8_q = p->weight_dtype == MOE_FP8_E4M3 && p->E <= 256;
  const hipError_t re =
      fp8_q ? launch_route_quant_fp8(logits, bias, p->T, p->E, p->k, L.ids,
                                     L.tw, (const bf16_t*)x, p->H, L.d.xq,
                                     L.d.xs, s)
            : launch_route_topk(logits, bias, p->T, p->E, p->k, L.ids, L.tw,
                                nullptr, s);
  if (re != hipSuccess) return MOE_ERR_HIP;
  if (ev) hipEventRecord(ev[1], s);
  st = dispatch_impl(p, x, L.ids, L.tw, l2p, replica_count, L.x_perm,
                     L.x_perm_scales, L.offsets, L.row_token, L.row_weight,
                     L.pair_row, L.d, s, ev ? ev[2] : nullptr,
                     /*materialize=*/false, &extras, /*x_quantised=*/fp8_q);
  if (st != MOE_OK) return st;
  if (ev) hipEventRecord(ev[3], s);
  // The expert kernels read each routed row straight from the token rows
  // through row_token (the permuted copy is never written); the shared
  // expert reads the same token rows in order.
  const bool fp8 = p->weight_dtype == MOE_FP8_E4M3;
  const void* xs = fp8 ? (const void*)L.d.xq : x;
  st = launch_ffn_common(p, xs, fp8 ? L.d.xs : nullptr, L.offsets,
                         p->has_shared ? xs : nullptr,
                         p->has_shared && fp8 ? L.d.xs : nullptr, w, L.y_perm,
                         L.y_shared, L.f, s, ev ? ev + 4 : nullptr,
                         L.row_token, /*tiles_ready=*/true);
  if (st != MOE_OK) return st;
  st = hip_status(launch_combine(L.y_perm, L.pair_row, L.tw,
                                 p->has_shared ? L.y_shared : nullptr, p->T,
                                 p->H, p->k, p->out_dtype, out, s));
  if (ev) hipEventRecord(ev[7], s);
  return st;
}

moe_status moe_layer_forward(const moe_problem* p, const float* logits,
                             const float* bias, const void* x,
                             const moe_weights* w, const int32_t* l2p,
                             const int32_t* replica_count, void* out,
                             int32_t* expert_counts, void* workspace,
                             size_t ws_bytes, void* stream) {
  return layer_impl(p, logits, bias, x, w, l2p, replica_count, out,
                    expert_counts, workspace, ws_bytes, stream, nullptr);
}

moe_status moe_layer_forward_timed(const moe_problem* p, const float* logits,
                                   const float* bias, const void* x,
                                   const moe_weights* w, const int32_t* l2p,
                                   const int32_t* replica_count, void* out,
                                   int32_t* expert_counts, void* workspace,
                                   size_t ws_bytes, void* stream,
                                   void* const* events) {
  if (!events) return MOE_ERR_INVALID_ARGUMENT;
  hipEvent_t ev[MOE_STAGE_EVENTS];
  for (int i = 0; i < MOE_STAGE_EVENTS; ++i) {
    if (!events[i]) return MOE_ERR_INVALID_ARGUMENT;
    ev[i] = (hipEvent_t)events[i];
  }
  return layer_impl(p, logits, bias, x, w, l2p, replica_count, out,
                    expert_counts, workspace, ws_bytes, stream, ev);
}

moe_status moe_prepack_weights(const void* src, int32_t K, int32_t N,
                               int32_t dtype, int32_t layout, void* dst,
                               void* stream) {
  if (dtype != MOE_F32 && dtype != MOE_BF16 && dtype != MOE_FP8_E4M3)
    return MOE_ERR_UNSUPPORTED;
  if (layout != MOE_LAYOUT_KN && layout != MOE_LAYOUT_NK)
    return MOE_ERR_INVALID_ARGUMENT;
  if (K < 0 || N < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (dtype == MOE_BF16 && (N % 16 || K % 32)) return MOE_ERR_INVALID_ARGUMENT;
  if (dtype == MOE_FP8_E4M3 && (N % 16 || K % 128))
    return MOE_ERR_INVALID_ARGUMENT;
  if (K == 0 || N == 0) return MOE_OK;
  if (!src || !dst || src == dst) return MOE_ERR_INVALID_ARGUMENT;
  return hip_status(launch_prepack(src, K, N, dtype, layout, dst, S(stream)));
}

moe_status moe_quantize_fp8_blocks(const float* w, int32_t K, int32_t N,
                                   int32_t block, int32_t layout,
                                   uint8_t* codes, float* scales,
                                   void* stream) {
  if (block != 128) return MOE_ERR_UNSUPPORTED;
  if (layout != MOE_LAYOUT_KN && layout != MOE_LAYOUT_NK)
    return MOE_ERR_INVALID_ARGUMENT;
  if (K < 0 || N < 0 || K % block || N % block) return MOE_ERR_INVALID_ARGUMENT;
  if (K == 0 || N == 0) return MOE_OK;
  if (!w || !codes || !scales) return MOE_ERR_INVALID_ARGUMENT;
  return hip_status(
      launch_quant_blocks_fp8(w, K, N, layout, codes, scales, S(stream)));
}

}  // extern "C"
