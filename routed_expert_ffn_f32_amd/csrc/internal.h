// Internal declarations of the gfx950 routed-MoE library (not part of the
// C ABI).  Every kernel here is launched by coli_moe.hip on the caller's
// stream; launchers return hipError_t.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace coli {

constexpr int kWave = 64;           // CDNA wavefront width
constexpr int kMaxExperts = 512;    // dispatch keeps per-wave histograms of E bins in LDS
constexpr int kMaxTopK = 32;
constexpr int kDispatchThreads = 1024;

// ---------------------------------------------------------------------------
// Routing (router.hip)
// ---------------------------------------------------------------------------

// wrT[e][i] = wr[i][e]: the router stored expert-major so that lane l of a
// wave reads element l + 64m of expert e with a coalesced load.
hipError_t launch_router_transpose(const float *wr, float *wrT, int h, int E, hipStream_t s);

// logits[t][e] = sum_i x[t][i] wr[i][e] in the fixed float32 order: lane l of
// the wave owning (t, e) keeps p_l = fma(x[l+64m], w[l+64m], p_l) over
// m = 0..h/64-1, then the 64 partials meet in an xor butterfly (32,16,..,1).
hipError_t launch_router_logits(const float *x, const float *wrT, int T, int h, int E, float *logits,
                                hipStream_t s);

// One wave per token: sigmoid scores, biased key, top-k (key desc, index
// asc), renormalised weights times rsf.
hipError_t launch_router_select(const float *logits, const float *bias, int T, int E, int k, float rsf,
                                int32_t *idx, float *w, hipStream_t s);

// ---------------------------------------------------------------------------
// Dispatch (dispatch.hip): stable counting sort of assignments by expert.
// ---------------------------------------------------------------------------
hipError_t launch_dispatch(const int32_t *idx, int n, int E, int32_t *offsets, int32_t *sorted_ids,
                           int32_t *inv, int32_t *active, int32_t *n_active, hipStream_t s);

// ---------------------------------------------------------------------------
// Expert GEMV path (expert_gemv.hip), decode-sized batches.
// ---------------------------------------------------------------------------
struct ExpertTables {
  const uint8_t *q;  // [rows][cols/2] per expert, experts stacked with stride rows*cols/2
  const float *s;    // [rows][cols/64] per expert
};

struct GemvProblem {
  // Matrix A (gate in gate/up mode, down in down mode) and B (up; gate/up mode only).
  ExpertTables a, b;          // routed, stacked over experts
  ExpertTables sh_a, sh_b;    // shared expert (used when has_shared)
  int rows, cols;             // of each matrix
  const float *x;             // gate/up: hidden [T][h]; down: mid [P][I]
  float *out;                 // gate/up: mid [P][I]; down: y [P][h]
  const int32_t *offsets;     // [E+1]
  const int32_t *sorted_ids;  // [T*k]
  const int32_t *active;      // [E]
  const int32_t *n_active;    // [1]
  int T, k, E;
  int n_routed_slots;         // min(E, T*k): grid slots for routed experts
  int has_shared;
};

// gate/up: mid[p][i] = silu(g) * u for every assignment position p (routed:
// p = sorted position; shared: p = T*k + t).  down: y[p][r] = Wd[r] . mid[p].
hipError_t launch_gemv_gate_up(const GemvProblem &P, hipStream_t s);
hipError_t launch_gemv_down(const GemvProblem &P, hipStream_t s);

// out[t] = sum_j w[t*k+j] y[inv[t*k+j]] + (shared ? y[T*k + t] : 0)
hipError_t launch_combine(const float *y, const float *w, const int32_t *inv, int T, int k, int h,
                          int has_shared, float *out, hipStream_t s);

}  // namespace coli
