// The layer handle behind the C ABI's opaque coli_moe_t, shared by the
// library's host files (coli_moe.hip, expert_cache.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "coli_moe.h"

// Byte offsets of the workspace regions.
struct Layout {
  size_t wrP, logits, xq, xs, idx, w, offsets, sorted_ids, inv, active, n_active, mq, ms, midf, y;
  size_t dcnt;                      // per-workgroup key counts of the many-workgroup dispatch
  size_t xb, xexp, xn2, midb, pstats, tiles, n_tiles;  // prefill path
  size_t queues;                    // row queues of the small-batch gate/up launch
  size_t status;                    // device error word (coli_moe_status)
  size_t total;
};

struct ProfRecord {
  int kernel;
  hipEvent_t start, stop;
};

struct coli_moe {
  coli_moe_config_t cfg;
  coli_moe_weights_t w;
  char *ws;
  Layout L;
  int last_T;
  // profiling
  int prof_calls_left;
  int prof_calls_done;
  std::vector<ProfRecord> prof;
  size_t prof_used;
  // routed expert e's tables sit at index slot_of[e] of the stacked tables
  // (device array; NULL: at index e)
  const int32_t *slot_of;
  // run-time routing limits (k_use = top_k, top_p = 1: none)
  int32_t k_use;
  float top_p;
  int32_t spin_limit;  // bound of the one-token gate/up launch's LDS-flag wait, in polls
  int32_t batch_mfma;  // larger int4 batches: 2 = by size (default), 1 = int8 MFMA kernels, 0 = v_dot8 GEMV kernels
};

namespace coli {

// Phases of a forward: the router, selection and dispatch; the experts and
// the combine.  A routing-only call leaves idx, w, offsets, sorted_ids,
// inv, active and n_active in the workspace; an experts-only call after it
// (same hidden, same T) finishes the forward.
constexpr int kPhaseRoute = 1, kPhaseExperts = 2, kPhaseAll = 3;
int forward_phases(coli_moe_t *m, const float *hidden, float *out, int32_t T, hipStream_t s, int phase);

// Checks shared by the entry points (COLI_MOE_* codes).
int config_check(const coli_moe_config_t &c);
int weights_check(const coli_moe_config_t &cfg, const coli_moe_weights_t &w);
Layout workspace_layout(const coli_moe_config_t &c);
// A handle over workspace ws (host fields only), then its device state.
void handle_set_up(coli_moe_t *m, const coli_moe_config_t &cfg, const coli_moe_weights_t &w, char *ws,
                   const Layout &L);
hipError_t handle_stage(coli_moe_t *m, hipStream_t s);
// Sets the handle's run-time routing limits (COLI_MOE_* code).
int set_route_limits(coli_moe_t *m, int32_t k_use, float top_p);

}  // namespace coli
