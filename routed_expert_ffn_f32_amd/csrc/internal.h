// Internal declarations of the gfx950 routed-MoE library (not part of the
// C ABI).  Every kernel here is launched by coli_moe.hip on the caller's
// stream; launchers return hipError_t.
#pragma once

#include <hip/hip_bf16.h>
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace coli {

// Kernel launch.  When the library's profiling wrapper has set an event pair,
// the launch records it at the kernel's own start and end (AMD's extended
// launch), so that the measured time is the kernel's duration alone.  A step
// of two launches splits the pair (split_launch_events): the start event on
// the first, the stop event on the second.
struct LaunchEvents {
  hipEvent_t start, stop;
};
extern thread_local LaunchEvents launch_events;

template <typename... KArgs, typename... Args>
hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t s, Args &&...args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  if (launch_events.start || launch_events.stop) {
    const LaunchEvents ev = launch_events;
    launch_events = LaunchEvents{nullptr, nullptr};
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, ev.start, ev.stop, 0u, static_cast<KArgs>(args)...);
  } else {
    kernel<<<grid, block, shmem, s>>>(static_cast<KArgs>(args)...);
  }
  return hipGetLastError();
}

// The pending event pair, taken for a step of two launches: the caller sets
// launch_events to {first.start, nullptr} and then {nullptr, first.stop}.
inline LaunchEvents split_launch_events() {
  const LaunchEvents ev = launch_events;
  launch_events = LaunchEvents{nullptr, nullptr};
  return ev;
}

constexpr int kWave = 64;              // CDNA wavefront width
constexpr int kMaxExperts = 512;       // dispatch keeps per-wave histograms of E bins in LDS
constexpr int kMaxTopK = 32;
constexpr int kDispatchThreads = 1024;
constexpr int kFusedDispatchMax = 4096;  // T*k up to which selection and dispatch share a launch
constexpr int kSmallT = 4;               // small batches: routing computed inside each gate/up block
constexpr int kSmallAssign = 64;         // and T*k at most one wave of assignments

// ---------------------------------------------------------------------------
// Routing (router.hip)
// ---------------------------------------------------------------------------

// Run-time routing limits, two lossy overrides of the routing named as
// engine knobs in the knob table of "Colibri 调优与运行时旋钮实战指南"
// (Colibri tuning and runtime knobs guide): an explicit smaller k and
// adaptive expert top-p.  With k_use <= k and 0 < top_p <= 1:
//  - the k_use experts first in the order (c desc, e asc) are the
//    candidates, in slots 0..k_use-1, and den sums their scores in slot
//    order;
//  - top_p < 1: cum_j = ((s_0 + s_1) + ...) + s_(j-1) is the score of the
//    candidates before slot j; slot 0 is kept, slot j >= 1 while
//    cum_j < top_p * den (cum never decreases, so the kept slots are a
//    prefix of m slots: the shortest one reaching the share top_p);
//  - the kept slots are renormalised over themselves, w_j = (s_j / cum_m)
//    * rsf; every other slot of the k is dropped: expert -1, weight 0.
// k_use = k, top_p = 1 is the plain selection.
struct RouteLimits {
  int k_use;
  float top_p;
};


// Floats of the lane-permuted router copy for (h, E).
size_t router_permuted_floats(int h, int E);

// wrP[e][b][l][i] = wr[l + 64(4b + i)][e]: the router stored so that lane l
// of a wave reads its four consecutive chain elements as one float4.
hipError_t launch_router_permute(const float *wr, float *wrP, int h, int E, hipStream_t s);

// logits[t][e] = sum_i x[t][i] wr[i][e] in the fixed float32 order: lane l of
// the wave owning (t, e) keeps p_l = fma(x[l+64m], w[l+64m], p_l) over
// m = 0..h/64-1, then the 64 partials meet in an xor butterfly (32,16,..,1).
// The same launch writes the digit-plane form of x (xq, xs) for the experts
// (xq == NULL: no planes), in the form plane_mode names: the int4 digit
// planes of the GEMV kernels, the byte planes of int8 tables, or the byte
// planes of the matrix-core batch kernels (byte_planes.h).  One token with h
// in {2048, 4096, 6144} takes a launch that issues every load of a chain
// before its first fma.
constexpr int kPlanesInt4 = 0, kPlanesInt8 = 1, kPlanesMatrixCore = 2;
hipError_t launch_router_logits(const float *x, const float *wrP, int T, int h, int E, float *logits,
                                uint32_t *xq, float *xs, int plane_mode, hipStream_t s);  // xq == NULL: no planes

// One wave per token: sigmoid scores, biased key, top-k (key desc, index
// asc), renormalised weights times rsf.
// Routing limits as in RouteLimits; idx and w keep their [T][k] layout.
hipError_t launch_router_select(const float *logits, const float *bias, int T, int E, int k, float rsf,
                                RouteLimits lim, int32_t *idx, float *w, hipStream_t s);

// Selection of T tokens and the dispatch in one workgroup (T*k <= kFusedDispatchMax).
hipError_t launch_select_dispatch(const float *logits, const float *bias, int T, int E, int k, float rsf,
                                  RouteLimits lim, int32_t *idx, float *w, int32_t *offsets, int32_t *sorted_ids,
                                  int32_t *inv, int32_t *active, int32_t *n_active, hipStream_t s);

// ---------------------------------------------------------------------------
// Dispatch (dispatch.hip): stable counting sort of assignments by expert;
// negative ids (dropped slots) follow every expert's group.  Batches of more
// than one workgroup's assignments are sorted over many workgroups when a
// count array of dispatch_count_ints(n, E) ints is given (else by one).
// ---------------------------------------------------------------------------
size_t dispatch_count_ints(int n, int E);
hipError_t launch_dispatch(const int32_t *idx, int n, int E, int32_t *offsets, int32_t *sorted_ids,
                           int32_t *inv, int32_t *active, int32_t *n_active, int32_t *cnt, hipStream_t s);

// ---------------------------------------------------------------------------
// Expert GEMV path (expert_gemv.hip), decode-sized batches.
// ---------------------------------------------------------------------------
struct ExpertTables {
  const uint8_t *q;  // [rows][cols/2] per expert, experts stacked with stride rows*cols/2
  const float *s;    // [rows][cols/64] per expert
};

// Index of routed expert e's tables in the stacked arrays: e itself, or its
// cache slot when the tables are the slots of an expert cache (slot_of[e],
// valid for every expert a call routes to).
// The map is read through the constant address space: with a wave-uniform
// e that is a scalar load, whose wait counts scalar and LDS operations only
// (a vector load here made the kernels wait for every row load in flight at
// each routed row or slot).  The map is written before the launch and never
// during it.
typedef const __attribute__((address_space(4))) int32_t *SlotMapPtr;
__device__ __forceinline__ size_t table_index(const int32_t *slot_of, int e) {
  if (!slot_of) return (size_t)e;
  return (size_t)((SlotMapPtr)slot_of)[e];
}

struct DecodeProblem {
  ExpertTables gate, up, down;           // routed experts, stacked
  ExpertTables sh_gate, sh_up, sh_down;  // shared expert
  int h, I, T, k, E;
  int n_routed_slots;  // min(E, T*k): grid slots for routed experts
  int has_shared;
  int int8;             // tables are int8 with a scale per row (else int4 gs64)
  float rsf;
  RouteLimits lim;      // run-time routing limits (small batches route in the gate/up launch)
  const float *logits;  // [T][E] router logits (small batches route from them)
  const float *bias;    // [E] selection bias or NULL
  const uint32_t *xq;   // hidden rows as digit planes [T][6][h/8]
  const float *xs;      // and block scales [T][h/32]
  uint32_t *mq;         // expert intermediates as digit planes [P][6][I/8], P = T*k + T*has_shared
  float *ms;            // and block scales [P][I/32] (larger batches)
  float *midf;          // expert intermediates as float32 [P][I]
  float *y;             // expert outputs [P][h] (larger batches)
  // routing and dispatch: written by the gate/up launch for small batches,
  // read by it otherwise
  int32_t *idx, *sorted_ids, *inv, *offsets, *active, *n_active;
  float *wsel;
  // small batches: row queues of the gate/up launch (kRowQueueWords int32,
  // zero when it starts; the down launch clears them again)
  int32_t *queues;
  const int32_t *slot_of;  // expert -> table index (NULL: identity)
  // error word: a launch that gave up a bounded wait stores 1 (read and
  // cleared by coli_moe_status); the bound of that wait in polls
  int32_t *status;
  int32_t spin_limit;
};
constexpr int32_t kSpinLimit = 1 << 22;  // polls of about 64 cycles: about 0.1 s
constexpr int kRowQueueWords = 64 * 64;

// True when the batch takes the small-batch launch structure (router and
// routing in one launch, gate/up, then down fused with the combine).  int8
// tables run only there.
bool small_batch(int T, int k, int h, int I, bool int8);
// Fill n int32 values.
hipError_t launch_fill_i32(int32_t *p, int n, int32_t v, hipStream_t s);

// gate/up: mid = silu(Wg x) * (Wu x) for every assignment position p
// (routed: p = sorted position; shared: p = T*k + t), written as digit planes.
hipError_t launch_gemv_gate_up(const DecodeProblem &P, hipStream_t s);
// Read probe: the gate and up rows of n experts (device ids, -1 = shared;
// h <= 8192) with pure loads and the small-batch gate/up launch shape; sink
// receives at most one word.
// Measurement probes (probes.hip): XOR of every word of a device buffer
// (bytes a multiple of 16) into *sink; back-to-back bf16 MFMAs, `blocks`
// blocks of 4 waves, each wave adding 1 to *sink when its results check.
constexpr int kProbeStreamBlocks = 256 * 8;
constexpr int kMfmaChains = 8;  // MFMAs per round of the MFMA probe
hipError_t launch_stream_probe(const void *buf, size_t bytes, uint32_t *sink, hipStream_t s);
hipError_t launch_mfma_probe(int iters, int blocks, uint32_t *sink, hipStream_t s);
hipError_t launch_mfma_probe_f16(int iters, int blocks, uint32_t seed, uint32_t *sink, hipStream_t s);
hipError_t launch_read_probe(const DecodeProblem &P, const int32_t *experts, int n, uint32_t *sink,
                             hipStream_t s);
hipError_t launch_read_probe_down(const DecodeProblem &P, const int32_t *experts, int n, uint32_t *sink,
                                  hipStream_t s);
// Small batches: out[t] = sum_j w[t,j] Wd_e mid[inv(t,j)] + Wd_sh mid[T*k + t].
hipError_t launch_down_combine(const DecodeProblem &P, float *out, hipStream_t s);
// Larger batches: y[p] = Wd mid[p] ...
hipError_t launch_gemv_down(const DecodeProblem &P, hipStream_t s);
// ... then out[t] = sum_j w[t*k+j] y[inv[t*k+j]] + (shared ? y[T*k + t] : 0),
// the sum over the slots j with idx[t*k+j] >= 0 (dropped slots add nothing).
hipError_t launch_combine(const float *y, const float *w, const int32_t *idx, const int32_t *inv, int T, int k,
                          int h, int has_shared, float *out, hipStream_t s);

// ---------------------------------------------------------------------------
// Prefill path (expert_mfma.hip): grouped GEMMs on fp16 MFMA.
// ---------------------------------------------------------------------------
// Power-of-two prescaling of one expert's tables (index E: the shared expert):
// weights w' = w * 2^ew[m] (m: 0 gate, 1 up, 2 down), and the largest squared
// row norm of the prescaled gate and up scales.
struct PrefillStats {
  int32_t ew[3];
  float n2[2];
  int32_t pad[3];
};

struct PrefillProblem {
  ExpertTables gate, up, down;
  ExpertTables sh_gate, sh_up, sh_down;
  int h, I, T, k, E, has_shared;
  const _Float16 *xb;    // [T][h] hidden rows x * 2^-xexp[t] in half, columns permuted in 8s
  int32_t *xexp;         // [T] per-token exponents
  float *xn2;            // [T] squared norms of the scaled rows
  _Float16 *mid;         // [P][I] intermediate (scaled), half, columns permuted in 8s
  float *y;              // [P][h] expert outputs
  PrefillStats *stats;   // [E + has_shared]
  const int32_t *offsets, *sorted_ids, *active, *n_active;
  int2 *tiles;           // (slot or -1 for the shared expert, first token)
  int32_t *n_tiles;
};

// Shapes the prefill path takes (h and I multiples of 256).
bool prefill_shape_ok(int h, int I);
// Largest tile count of a call (grid size of the GEMM launches).
int prefill_max_tiles(int T, int k, int E, int has_shared);
// x [T][h] float -> scaled half rows (P.xb), P.xexp, P.xn2.
hipError_t launch_prefill_prep(const float *x, int T, int h, PrefillProblem &P, hipStream_t s);
// P.stats from the scale tables (once per set of tables).
hipError_t launch_prefill_stats(const PrefillProblem &P, hipStream_t s);
hipError_t launch_build_tiles(const PrefillProblem &P, hipStream_t s);
// mid = silu(x Wg^T) * (x Wu^T) per expert tile, half (scaled).
hipError_t launch_gate_up_mfma(const PrefillProblem &P, hipStream_t s);
// y = mid Wd^T per expert tile, float32.
hipError_t launch_down_mfma(const PrefillProblem &P, hipStream_t s);

}  // namespace coli
