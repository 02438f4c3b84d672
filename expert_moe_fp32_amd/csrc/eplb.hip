// Expert-parallel load balancing: where the physical experts go.
//
// "6.4 Data parallelism and expert parallelism" (infra-guide), section 5.2:
// with a load per expert, each redundant slot goes to the expert with the
// highest load per replica, and the replicas are then placed heaviest first
// onto the currently lightest rank that still has a free slot; every rank
// holds (experts + redundant) / EP physical experts (section 5.3).  Section
// 5.3 also has the balancer record per-expert load every forward and plan
// from the load over a window of recent steps.
//
// The plan and the per-rank map are host code (a rebalance runs every few
// thousand steps on a few hundred experts).  Recording the load is a device
// kernel on the layer's stream, so the per-step history never forces a
// synchronisation; the host reads the window's sum only when it plans.
#include <algorithm>
#include <numeric>
#include <vector>

#include "common.h"

namespace {

// load[a] / rep[a] > load[b] / rep[b], exactly
inline bool heavier(int64_t la, int64_t ra, int64_t lb, int64_t rb) {
  return (__int128)la * rb > (__int128)lb * ra;
}

// Sliding window of per-expert load: slot step % window of the history is
// replaced by this step's counts and the window sum follows.
__global__ __launch_bounds__(256) void k_record_load(
    const int32_t* __restrict__ counts, int E, int slot,
    int32_t* __restrict__ history, int64_t* __restrict__ window_load) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  int32_t* h = history + (size_t)slot * E + e;
  const int32_t old = *h, now = counts[e];
  *h = now;
  window_load[e] += (int64_t)now - old;
}

}  // namespace

extern "C" {

moe_status moe_eplb_plan(const int64_t* load, int32_t E, int32_t ep,
                         int32_t redundant, int32_t* replicas,
                         int32_t* slot_expert, int32_t* slot_replica,
                         double* rank_load) {
  if (!load || !replicas || !slot_expert || !slot_replica || !rank_load)
    return MOE_ERR_INVALID_ARGUMENT;
  if (E < 1 || ep < 1 || redundant < 0 || (E + redundant) % ep != 0)
    return MOE_ERR_INVALID_ARGUMENT;
  for (int e = 0; e < E; ++e)
    if (load[e] < 0) return MOE_ERR_INVALID_ARGUMENT;
  // replicas: the expert with the highest load per replica (lower id on ties)
  for (int e = 0; e < E; ++e) replicas[e] = 1;
  for (int i = 0; i < redundant; ++i) {
    int best = 0;
    for (int e = 1; e < E; ++e)
      if (heavier(load[e], replicas[e], load[best], replicas[best])) best = e;
    ++replicas[best];
  }
  // copies heaviest first; equal loads in (expert, replica) order
  struct Copy { int e, r; };
  std::vector<Copy> copies;
  copies.reserve((size_t)E + redundant);
  for (int e = 0; e < E; ++e)
    for (int r = 0; r < replicas[e]; ++r) copies.push_back({e, r});
  std::stable_sort(copies.begin(), copies.end(), [&](const Copy& a, const Copy& b) {
    return heavier(load[a.e], replicas[a.e], load[b.e], replicas[b.e]);
  });
  const int slots = (E + redundant) / ep;
  std::vector<int> used(ep, 0);
  std::vector<std::vector<Copy>> held(ep);
  for (int g = 0; g < ep; ++g) rank_load[g] = 0.0;
  for (const Copy& c : copies) {
    int g = -1;                           // lightest rank with a free slot
    for (int q = 0; q < ep; ++q)
      if (used[q] < slots && (g < 0 || rank_load[q] < rank_load[g])) g = q;
    rank_load[g] += (double)load[c.e] / (double)replicas[c.e];
    ++used[g];
    held[g].push_back(c);
  }
  // a rank's slots in (expert, replica) order: slot s is its physical id s
  for (int g = 0; g < ep; ++g) {
    std::sort(held[g].begin(), held[g].end(), [](const Copy& a, const Copy& b) {
      return a.e != b.e ? a.e < b.e : a.r < b.r;
    });
    for (int s = 0; s < slots; ++s) {
      slot_expert[(size_t)g * slots + s] = held[g][s].e;
      slot_replica[(size_t)g * slots + s] = held[g][s].r;
    }
  }
  return MOE_OK;
}

moe_status moe_eplb_rank_map(const int32_t* replicas, const int32_t* slot_expert,
                             const int32_t* slot_replica, int32_t E,
                             int32_t ep, int32_t redundant, int32_t rank,
                             int32_t max_replicas, int32_t* l2p,
                             int32_t* replica_count, int32_t* num_physical) {
  if (!replicas || !slot_expert || !slot_replica || !l2p || !replica_count ||
      !num_physical)
    return MOE_ERR_INVALID_ARGUMENT;
  if (E < 1 || ep < 1 || redundant < 0 || (E + redundant) % ep != 0 ||
      rank < 0 || rank >= ep || max_replicas < 1)
    return MOE_ERR_INVALID_ARGUMENT;
  const int slots = (E + redundant) / ep;
  for (int e = 0; e < E; ++e) {
    if (replicas[e] < 1 || replicas[e] > max_replicas)
      return MOE_ERR_INVALID_ARGUMENT;
  }
  for (int s = 0; s < slots; ++s) {
    const int e = slot_expert[(size_t)rank * slots + s];
    const int r = slot_replica[(size_t)rank * slots + s];
    if (e < 0 || e >= E || r < 0 || r >= replicas[e])
      return MOE_ERR_INVALID_ARGUMENT;
  }
  for (int e = 0; e < E; ++e) {
    replica_count[e] = replicas[e];
    for (int r = 0; r < max_replicas; ++r) l2p[(size_t)e * max_replicas + r] = -1;
  }
  for (int s = 0; s < slots; ++s) {
    const int e = slot_expert[(size_t)rank * slots + s];
    const int r = slot_replica[(size_t)rank * slots + s];
    l2p[(size_t)e * max_replicas + r] = s;
  }
  *num_physical = slots;
  return MOE_OK;
}

moe_status moe_eplb_record_load(const int32_t* expert_counts, int32_t E,
                                int32_t window, int64_t step,
                                int32_t* history, int64_t* window_load,
                                void* stream) {
  if (!expert_counts || !history || !window_load)
    return MOE_ERR_INVALID_ARGUMENT;
  if (E < 1 || E > MOE_EMAX || window < 1 || step < 0)
    return MOE_ERR_INVALID_ARGUMENT;
  const int slot = (int)(step % window);
  k_record_load<<<(E + 255) / 256, 256, 0, (hipStream_t)stream>>>(
      expert_counts, E, slot, history, window_load);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_eplb_hottest_map(const int32_t* local_counts, int32_t num_local,
                                int32_t redundant, int32_t* l2p,
                                int32_t* replica_count,
                                int32_t* num_physical) {
  if (!local_counts || !l2p || !replica_count || !num_physical)
    return MOE_ERR_INVALID_ARGUMENT;
  if (num_local < 1 || num_local > MOE_LMAX || redundant < 0 ||
      redundant > num_local || num_local + redundant > MOE_LMAX)
    return MOE_ERR_INVALID_ARGUMENT;
  std::vector<int> order(num_local);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
    return local_counts[a] > local_counts[b];
  });
  for (int e = 0; e < num_local; ++e) {
    l2p[2 * e] = e;
    l2p[2 * e + 1] = -1;
    replica_count[e] = 1;
  }
  for (int i = 0; i < redundant; ++i) {
    const int e = order[i];
    l2p[2 * e + 1] = num_local + i;
    replica_count[e] = 2;
  }
  *num_physical = num_local + redundant;
  return MOE_OK;
}

}  // extern "C"
