// Host side of the C ABI declared in include/coli_moe.h: argument checks,
// workspace layout, and the launch sequence of one layer forward.
//
// API shape (init / forward / free, negative error codes, dry run for zero
// tokens, capacity fixed at init): trdm.cn article "Colibri: a pure-C
// lightweight inference engine built for MoE models", sections 3.2 (buffers
// sized once from the maximum batch), 4.2 (return codes), 5.1 (batch above
// the maximum is an error; one handle per thread) and 5.2 (batch size 0
// checks the setup without computing).  The per-handle device state (router
// copy, expert offsets) follows the opaque context of the cf-1.com Colibri
// article, section 3.2.
#include <algorithm>
#include <atomic>
#include <new>
#include <vector>

#include "coli_moe.h"
#include "expert_batch.h"
#include "handle.h"
#include "internal.h"

namespace {

enum Kernel {
  K_ROUTER_LOGITS = 0,
  K_ROUTER_SELECT = 1,
  K_DISPATCH = 2,
  K_GATE_UP = 3,
  K_DOWN = 4,
  K_COMBINE = 5,
  K_MFMA_GATE_UP = 6,
  K_MFMA_DOWN = 7,
  K_PREFILL_PREP = 8,
  K_BUILD_TILES = 9,
};

const char *const kKernelNames[COLI_MOE_N_KERNELS] = {
    "router_logits",    "router_select_dispatch", "dispatch",            "expert_gemv_gate_up",
    "expert_gemv_down", "combine",                "expert_mfma_gate_up", "expert_mfma_down",
    "prefill_to_half",  "build_tiles"};
// (small batches: "expert_gemv_down" is the down projection fused with the combine)

constexpr size_t kAlign = 256;
constexpr int kBatchMfmaMinTokens = 16;  // larger int4 batches: the int8 matrix-core kernels from here
size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

// The prefill (MFMA) path takes h and I multiples of 256, and half
// activation buffers ([max_tokens][h] and [P][I]) under 4 GiB, since its
// copies address them with 32-bit offsets; T below the threshold, or other
// shapes, take the GEMV path.
bool prefill_shape(const coli_moe_config_t &c) {
  const uint64_t T = (uint64_t)c.max_tokens, P = T * (uint64_t)(c.top_k + (c.n_shared ? 1 : 0));
  return coli::prefill_shape_ok(c.hidden, c.inter) && T * (uint64_t)c.hidden * 2 < (1ull << 32) &&
         P * (uint64_t)c.inter * 2 < (1ull << 32);
}

bool int8_tables(const coli_moe_config_t &c) { return c.weight_format == COLI_MOE_WEIGHTS_INT8_ROW; }

// True when the handle's workspace holds the prefill buffers (int4 tables).
bool prefill_enabled(const coli_moe_config_t &c) {
  return !int8_tables(c) && prefill_shape(c) && (c.prefill_threshold == 0 ? 256 : c.prefill_threshold) <= c.max_tokens;
}

// Tokens per group of an int8 forward: the most (up to the small-batch
// limits) that take the small-batch launches; 0 if not even one does.
int int8_group(const coli_moe_config_t &c) {
  for (int g = coli::kSmallT; g >= 1; --g)
    if (coli::small_batch(g, c.top_k, c.hidden, c.inter, true)) return g;
  return 0;
}

bool config_ok(const coli_moe_config_t &c, int *code) {
  if (c.hidden < 64 || c.hidden > 16384 || c.hidden % 64 || c.inter < 64 || c.inter > 16384 ||
      c.inter % 64 || c.n_experts < 1 || c.n_experts > coli::kMaxExperts || c.max_tokens < 1 ||
      (c.n_shared != 0 && c.n_shared != 1) || c.prefill_threshold < 0) {
    *code = COLI_MOE_EARG;
    return false;
  }
  if (c.weight_format != COLI_MOE_WEIGHTS_INT4_GS64 && c.weight_format != COLI_MOE_WEIGHTS_INT8_ROW) {
    *code = COLI_MOE_EARG;
    return false;
  }
  if (c.top_k < 1 || c.top_k > c.n_experts || c.top_k > coli::kMaxTopK || c.n_group != 1 ||
      c.group_size != (int8_tables(c) ? 0 : 64)) {
    *code = COLI_MOE_EROUTING;
    return false;
  }
  if (int8_tables(c) && int8_group(c) == 0) {
    *code = COLI_MOE_EARG;
    return false;
  }
  if ((int64_t)c.max_tokens * c.top_k > (1 << 20)) {
    *code = COLI_MOE_EARG;
    return false;
  }
  return true;
}

Layout layout_of(const coli_moe_config_t &c) {
  Layout L{};
  const size_t T = (size_t)c.max_tokens, E = (size_t)c.n_experts, k = (size_t)c.top_k;
  const size_t h = (size_t)c.hidden, I = (size_t)c.inter;
  const size_t P = T * k + (c.n_shared ? T : 0);  // expert-output rows
  const size_t planes = 6;  // digit planes per activation row
  size_t o = 0;
  L.wrP = o;        o = align_up(o + coli::router_permuted_floats(c.hidden, c.n_experts) * 4);
  L.logits = o;     o = align_up(o + T * E * 4);
  L.xq = o;         o = align_up(o + T * planes * (h / 8) * 4);
  L.xs = o;         o = align_up(o + T * (h / 32) * 4);
  L.idx = o;        o = align_up(o + T * k * 4);
  L.w = o;          o = align_up(o + T * k * 4);
  L.offsets = o;    o = align_up(o + (E + 1) * 4);
  L.sorted_ids = o; o = align_up(o + T * k * 4);
  L.inv = o;        o = align_up(o + T * k * 4);
  L.active = o;     o = align_up(o + E * 4);
  L.n_active = o;   o = align_up(o + 4);
  L.dcnt = o;       o = align_up(o + coli::dispatch_count_ints((int)(T * k), (int)E) * 4);
  L.mq = o;         o = align_up(o + P * planes * (I / 8) * 4);
  L.ms = o;         o = align_up(o + P * (I / 32) * 4);
  L.midf = o;       o = align_up(o + P * I * 4);
  L.y = o;          o = align_up(o + P * h * 4);
  const bool pre = prefill_enabled(c);
  const size_t tiles = pre ? (size_t)coli::prefill_max_tiles(c.max_tokens, c.top_k, c.n_experts, c.n_shared) : 0;
  L.xb = o;         o = align_up(o + (pre ? T * h * 2 : 0));
  L.xexp = o;       o = align_up(o + (pre ? T * 4 : 0));
  L.xn2 = o;        o = align_up(o + (pre ? T * 4 : 0));
  L.midb = o;       o = align_up(o + (pre ? P * I * 2 : 0));
  L.pstats = o;     o = align_up(o + (pre ? (E + 1) * sizeof(coli::PrefillStats) : 0));
  L.tiles = o;      o = align_up(o + tiles * 8);
  L.n_tiles = o;    o = align_up(o + 4);
  L.queues = o;     o = align_up(o + coli::kRowQueueWords * 4);
  L.status = o;     o = align_up(o + 4);
  L.total = o;
  return L;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }


}  // namespace


namespace coli {
thread_local LaunchEvents launch_events = {nullptr, nullptr};
}

namespace {

// Runs `launch` (one kernel launch); while profiling, that kernel records the
// next event pair of the handle at its start and end.
template <class F>
hipError_t timed(coli_moe_t *m, int kernel, hipStream_t s, F &&launch) {
  if (m->prof_calls_left <= 0 || m->prof_used >= m->prof.size()) return launch();
  ProfRecord &r = m->prof[m->prof_used++];
  r.kernel = kernel;
  coli::launch_events = coli::LaunchEvents{r.start, r.stop};  // taken by the launch
  const hipError_t e = launch();
  coli::launch_events = coli::LaunchEvents{nullptr, nullptr};
  return e;
}

template <class T>
T *at(coli_moe_t *m, size_t off) {
  return reinterpret_cast<T *>(m->ws + off);
}

coli::PrefillProblem prefill_problem(coli_moe_t *m, int T) {
  const coli_moe_config_t &c = m->cfg;
  const Layout &L = m->L;
  coli::PrefillProblem Q{};
  Q.gate = {m->w.gate_q, m->w.gate_s};
  Q.up = {m->w.up_q, m->w.up_s};
  Q.down = {m->w.down_q, m->w.down_s};
  Q.sh_gate = {m->w.sh_gate_q, m->w.sh_gate_s};
  Q.sh_up = {m->w.sh_up_q, m->w.sh_up_s};
  Q.sh_down = {m->w.sh_down_q, m->w.sh_down_s};
  Q.h = c.hidden;
  Q.I = c.inter;
  Q.T = T;
  Q.k = c.top_k;
  Q.E = c.n_experts;
  Q.has_shared = c.n_shared;
  Q.xb = at<_Float16>(m, L.xb);
  Q.xexp = at<int32_t>(m, L.xexp);
  Q.xn2 = at<float>(m, L.xn2);
  Q.mid = at<_Float16>(m, L.midb);
  Q.y = at<float>(m, L.y);
  Q.stats = at<coli::PrefillStats>(m, L.pstats);
  Q.offsets = at<int32_t>(m, L.offsets);
  Q.sorted_ids = at<int32_t>(m, L.sorted_ids);
  Q.active = at<int32_t>(m, L.active);
  Q.n_active = at<int32_t>(m, L.n_active);
  Q.tiles = at<int2>(m, L.tiles);
  Q.n_tiles = at<int32_t>(m, L.n_tiles);
  return Q;
}


int weights_ok(const coli_moe_config_t &cfg, const coli_moe_weights_t &w) {
  const void *tabs[] = {w.gate_q, w.gate_s, w.up_q, w.up_s, w.down_q, w.down_s};
  for (const void *p : tabs)
    if (!p || !aligned(p, 16)) return COLI_MOE_EARG;
  if (!w.router_w || !aligned(w.router_w, 4) || (w.sel_bias && !aligned(w.sel_bias, 4))) return COLI_MOE_EARG;
  if (cfg.n_shared) {
    const void *sh[] = {w.sh_gate_q, w.sh_gate_s, w.sh_up_q, w.sh_up_s, w.sh_down_q, w.sh_down_s};
    for (const void *p : sh)
      if (!p || !aligned(p, 16)) return COLI_MOE_EARG;
  }
  return COLI_MOE_OK;
}

// Host fields of a handle over the workspace ws (no allocation).
void set_up(coli_moe_t *m, const coli_moe_config_t &cfg, const coli_moe_weights_t &w, char *ws, const Layout &L) {
  m->cfg = cfg;
  if (m->cfg.prefill_threshold == 0) m->cfg.prefill_threshold = 256;
  m->w = w;
  m->ws = ws;
  m->L = L;
  m->last_T = 0;
  m->prof_calls_left = 0;
  m->prof_calls_done = 0;
  m->prof_used = 0;
  m->slot_of = nullptr;
  m->k_use = cfg.top_k;
  m->top_p = 1.0f;
  m->spin_limit = coli::kSpinLimit;
  m->batch_mfma = 2;
}

// The workspace state every forward starts from: the lane-permuted router,
// cleared row queues, and the prefill prescale statistics.
hipError_t stage(coli_moe_t *m, hipStream_t s) {
  hipError_t e = coli::launch_router_permute(m->w.router_w, at<float>(m, m->L.wrP), m->cfg.hidden,
                                             m->cfg.n_experts, s);
  if (e == hipSuccess) e = coli::launch_fill_i32(at<int32_t>(m, m->L.queues), coli::kRowQueueWords, 0, s);
  if (e == hipSuccess) e = coli::launch_fill_i32(at<int32_t>(m, m->L.status), 1, 0, s);
  if (e == hipSuccess && prefill_enabled(m->cfg)) e = coli::launch_prefill_stats(prefill_problem(m, 0), s);
  return e;
}

// ---------------------------------------------------------------------------
// Workspace of coli_moe_forward_noalloc: one file-scope device array (each
// device the library runs on holds its own copy until the process ends).
// Host code never passes the array's name to a kernel: it is a host-side
// stand-in, not a device address.  The device address is taken once per
// device with hipGetSymbolAddress and used everywhere instead.
// ---------------------------------------------------------------------------
static __device__ __attribute__((aligned(256))) char scratch[COLI_MOE_STATIC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::atomic<char *> scratch_ptr[kMaxDevices];

hipError_t scratch_of_current_device(char **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  char *p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    void *addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    p = static_cast<char *>(addr);
    scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

namespace coli {

int forward_phases(coli_moe_t *m, const float *hidden, float *out, int32_t T, hipStream_t s, int phase) {
  if (!m || T < 0) return COLI_MOE_EARG;
  if (T > m->cfg.max_tokens) return COLI_MOE_ECAPACITY;
  if (T == 0) return COLI_MOE_OK;
  if (!hidden || !aligned(hidden, 16)) return COLI_MOE_EARG;
  if ((phase & kPhaseExperts) && (!out || !aligned(out, 16))) return COLI_MOE_EARG;
  const coli_moe_config_t &c = m->cfg;
  const Layout &L = m->L;
  const int E = c.n_experts, k = c.top_k, h = c.hidden, I = c.inter;
  float *logits = at<float>(m, L.logits);
  uint32_t *xq = at<uint32_t>(m, L.xq);
  float *xs = at<float>(m, L.xs);
  int32_t *idx = at<int32_t>(m, L.idx);
  float *wsel = at<float>(m, L.w);
  int32_t *offsets = at<int32_t>(m, L.offsets), *sorted_ids = at<int32_t>(m, L.sorted_ids);
  int32_t *inv = at<int32_t>(m, L.inv), *active = at<int32_t>(m, L.active);
  int32_t *n_active = at<int32_t>(m, L.n_active);
  float *y = at<float>(m, L.y);
  const float *bias = m->w.sel_bias;
  const float rsf = c.routed_scaling_factor;
  const coli::RouteLimits lim{m->k_use, m->top_p};

  const bool int8 = int8_tables(c);
  const bool prefill = !int8 && T >= c.prefill_threshold && prefill_shape(c);
  const bool small = !prefill && coli::small_batch(T, k, h, I, int8);
  // larger batches of int4 experts: int8 matrix cores on byte planes
  // (by size: from 16 tokens; measured on the GLM-like and OLMoE-like
  // layers, the GEMV kernels are as fast or faster below, the matrix cores
  // 1.15x (GLM-like) and 1.45x (OLMoE-like) faster at 64 tokens)
  const bool batch = !prefill && !small && !int8 && coli::batch_mfma_fits(T, k, c.n_shared, h, I) &&
                     (m->batch_mfma == 1 || (m->batch_mfma == 2 && T >= kBatchMfmaMinTokens));
  hipError_t e;
  // 1. router logits and, for every path but prefill, the hidden rows in
  // the plane form of the expert kernels (the batch path's byte planes go in
  // the digit-plane buffers, which it does not otherwise use)
  if (phase & kPhaseRoute) {
    const int planes = batch ? kPlanesMatrixCore : int8 ? kPlanesInt8 : kPlanesInt4;
    e = timed(m, K_ROUTER_LOGITS, s, [&] {
      return launch_router_logits(hidden, at<float>(m, L.wrP), T, h, E, logits, prefill ? nullptr : xq, xs, planes,
                                  s);
    });
    if (e != hipSuccess) return COLI_MOE_EDEVICE;
  }
  // Selection and dispatch: one workgroup does both while each of its waves
  // selects at most one token (its counting sort then reads the choices from
  // LDS); larger batches select one token per wave over many workgroups,
  // then sort in a launch of their own.
  auto select_and_dispatch = [&]() -> hipError_t {
    if (T <= coli::kDispatchThreads / coli::kWave) {
      static_assert(coli::kDispatchThreads / coli::kWave * coli::kMaxTopK <= coli::kFusedDispatchMax,
                    "the fused launch's LDS holds every choice");
      return timed(m, K_ROUTER_SELECT, s, [&] {
        return launch_select_dispatch(logits, bias, T, E, k, rsf, lim, idx, wsel, offsets, sorted_ids, inv,
                                            active, n_active, s);
      });
    }
    hipError_t err = timed(m, K_ROUTER_SELECT, s,
                           [&] { return launch_router_select(logits, bias, T, E, k, rsf, lim, idx, wsel, s); });
    if (err != hipSuccess) return err;
    return timed(m, K_DISPATCH, s, [&] {
      return launch_dispatch(idx, T * k, E, offsets, sorted_ids, inv, active, n_active, at<int32_t>(m, L.dcnt), s);
    });
  };
  // Routing alone (phase kPhaseRoute without kPhaseExperts): selection and
  // dispatch written to the workspace, for the host to read.
  if (!(phase & kPhaseExperts)) {
    if (select_and_dispatch() != hipSuccess) return COLI_MOE_EDEVICE;
    m->last_T = T;
    return COLI_MOE_OK;
  }
  const bool routed = !(phase & kPhaseRoute);  // selection and dispatch already in the workspace
  if (prefill) {
    // 2. selection and dispatch, 3. half activations and the tile list,
    // 4. grouped GEMMs on MFMA, 5. weighted combine
    if (!routed && select_and_dispatch() != hipSuccess) return COLI_MOE_EDEVICE;
    coli::PrefillProblem Q = prefill_problem(m, T);
    e = timed(m, K_PREFILL_PREP, s, [&] { return launch_prefill_prep(hidden, T, h, Q, s); });
    if (e != hipSuccess) return COLI_MOE_EDEVICE;
    e = timed(m, K_BUILD_TILES, s, [&] { return launch_build_tiles(Q, s); });
    if (e != hipSuccess) return COLI_MOE_EDEVICE;
    e = timed(m, K_MFMA_GATE_UP, s, [&] { return launch_gate_up_mfma(Q, s); });
    if (e != hipSuccess) return COLI_MOE_EDEVICE;
    e = timed(m, K_MFMA_DOWN, s, [&] { return launch_down_mfma(Q, s); });
    if (e != hipSuccess) return COLI_MOE_EDEVICE;
    e = timed(m, K_COMBINE, s,
              [&] { return launch_combine(y, wsel, idx, inv, T, k, h, c.n_shared, out, s); });
    if (e != hipSuccess) return COLI_MOE_EDEVICE;
    m->last_T = T;
    if (m->prof_calls_left > 0) {
      --m->prof_calls_left;
      ++m->prof_calls_done;
    }
    return COLI_MOE_OK;
  }
  coli::DecodeProblem P{};
  P.gate = {m->w.gate_q, m->w.gate_s};
  P.up = {m->w.up_q, m->w.up_s};
  P.down = {m->w.down_q, m->w.down_s};
  P.sh_gate = {m->w.sh_gate_q, m->w.sh_gate_s};
  P.sh_up = {m->w.sh_up_q, m->w.sh_up_s};
  P.sh_down = {m->w.sh_down_q, m->w.sh_down_s};
  P.h = h;
  P.I = I;
  P.T = T;
  P.k = k;
  P.E = E;
  P.n_routed_slots = E < T * k ? E : T * k;
  P.has_shared = c.n_shared;
  P.int8 = int8 ? 1 : 0;
  P.rsf = rsf;
  P.lim = lim;
  P.logits = logits;
  P.bias = bias;
  P.xq = xq;
  P.xs = xs;
  P.mq = at<uint32_t>(m, L.mq);
  P.ms = at<float>(m, L.ms);
  P.midf = at<float>(m, L.midf);
  P.y = y;
  P.idx = idx;
  P.wsel = wsel;
  P.sorted_ids = sorted_ids;
  P.inv = inv;
  P.offsets = offsets;
  P.active = active;
  P.n_active = n_active;
  P.queues = at<int32_t>(m, L.queues);
  P.slot_of = m->slot_of;
  P.status = at<int32_t>(m, L.status);
  P.spin_limit = m->spin_limit;

  if (small) {
    // 2. gate/up (each block routes the batch itself), 3. down + combine
    e = timed(m, K_GATE_UP, s, [&] { return launch_gemv_gate_up(P, s); });
    if (e != hipSuccess) return COLI_MOE_EDEVICE;
    e = timed(m, K_DOWN, s, [&] { return launch_down_combine(P, out, s); });
    if (e != hipSuccess) return COLI_MOE_EDEVICE;
  } else if (int8) {
    // int8 tables: consecutive groups of G tokens through the small-batch
    // launches (each group routes itself; the router launch above covered
    // every token), then the selection and dispatch of the whole batch, so
    // that the routing arrays describe the call
    const int G = int8_group(c);
    for (int t0 = 0; t0 < T; t0 += G) {
      coli::DecodeProblem Pg = P;
      Pg.T = std::min(G, T - t0);
      Pg.n_routed_slots = std::min(E, Pg.T * k);
      Pg.logits = logits + (size_t)t0 * E;
      Pg.xq = xq + (size_t)t0 * (3 * (h / 4));
      Pg.xs = xs + (size_t)t0 * (h / 32);
      e = timed(m, K_GATE_UP, s, [&] { return launch_gemv_gate_up(Pg, s); });
      if (e != hipSuccess) return COLI_MOE_EDEVICE;
      e = timed(m, K_DOWN, s, [&] { return launch_down_combine(Pg, out + (size_t)t0 * h, s); });
      if (e != hipSuccess) return COLI_MOE_EDEVICE;
    }
    if (select_and_dispatch() != hipSuccess) return COLI_MOE_EDEVICE;
  } else {
    // 2. selection and dispatch
    if (!routed && select_and_dispatch() != hipSuccess) return COLI_MOE_EDEVICE;
    // 3. gate/up, down, weighted combine
    if (batch) {
      // the hidden rows' byte planes come from the router launch, the
      // intermediates' from the gate/up launch's epilogue
      e = timed(m, K_GATE_UP, s, [&] { return coli::launch_batch_gate_up(P, s); });
      if (e != hipSuccess) return COLI_MOE_EDEVICE;
      e = timed(m, K_DOWN, s, [&] { return coli::launch_batch_down(P, s); });
    } else {
      e = timed(m, K_GATE_UP, s, [&] { return launch_gemv_gate_up(P, s); });
      if (e != hipSuccess) return COLI_MOE_EDEVICE;
      e = timed(m, K_DOWN, s, [&] { return launch_gemv_down(P, s); });
    }
    if (e != hipSuccess) return COLI_MOE_EDEVICE;
    e = timed(m, K_COMBINE, s,
              [&] { return launch_combine(y, wsel, idx, inv, T, k, h, c.n_shared, out, s); });
    if (e != hipSuccess) return COLI_MOE_EDEVICE;
  }

  m->last_T = T;
  if (m->prof_calls_left > 0) {
    --m->prof_calls_left;
    ++m->prof_calls_done;
  }
  return COLI_MOE_OK;
}

int config_check(const coli_moe_config_t &c) {
  int code = COLI_MOE_OK;
  return config_ok(c, &code) ? COLI_MOE_OK : code;
}
int weights_check(const coli_moe_config_t &cfg, const coli_moe_weights_t &w) { return weights_ok(cfg, w); }
Layout workspace_layout(const coli_moe_config_t &c) { return layout_of(c); }
void handle_set_up(coli_moe_t *m, const coli_moe_config_t &cfg, const coli_moe_weights_t &w, char *ws,
                   const Layout &L) {
  set_up(m, cfg, w, ws, L);
}
hipError_t handle_stage(coli_moe_t *m, hipStream_t s) { return stage(m, s); }

int set_route_limits(coli_moe_t *m, int32_t k_use, float top_p) {
  if (!m) return COLI_MOE_EARG;
  if (k_use < 1 || k_use > m->cfg.top_k || !(top_p > 0.0f && top_p <= 1.0f)) return COLI_MOE_EROUTING;
  m->k_use = k_use;
  m->top_p = top_p;
  return COLI_MOE_OK;
}

}  // namespace coli

extern "C" {

size_t coli_moe_workspace_bytes(const coli_moe_config_t *cfg) {
  int code;
  if (!cfg || !config_ok(*cfg, &code)) return 0;
  return layout_of(*cfg).total;
}

int coli_moe_init(coli_moe_t **out, const coli_moe_config_t *cfg, const coli_moe_weights_t *w,
                  void *workspace, size_t workspace_bytes, void *stream) {
  if (!out || !cfg || !w || !workspace) return COLI_MOE_EARG;
  *out = nullptr;
  int code = COLI_MOE_OK;
  if (!config_ok(*cfg, &code)) return code;
  if ((code = weights_ok(*cfg, *w)) != COLI_MOE_OK) return code;
  if (!aligned(workspace, kAlign)) return COLI_MOE_EARG;
  const Layout L = layout_of(*cfg);
  if (workspace_bytes < L.total) return COLI_MOE_ECAPACITY;

  coli_moe_t *m = new (std::nothrow) coli_moe_t();
  if (!m) return COLI_MOE_EARG;
  set_up(m, *cfg, *w, static_cast<char *>(workspace), L);
  if (stage(m, static_cast<hipStream_t>(stream)) != hipSuccess) {
    delete m;
    return COLI_MOE_EDEVICE;
  }
  *out = m;
  return COLI_MOE_OK;
}

int coli_moe_forward(coli_moe_t *m, const float *hidden, float *out, int32_t T, void *stream) {
  return coli::forward_phases(m, hidden, out, T, static_cast<hipStream_t>(stream), coli::kPhaseAll);
}

int coli_moe_forward_noalloc(const coli_moe_config_t *cfg, const coli_moe_weights_t *w, const float *hidden,
                             float *out, int32_t T, void *stream) {
  if (!cfg || !w || T < 0) return COLI_MOE_EARG;
  int code = COLI_MOE_OK;
  if (!config_ok(*cfg, &code)) return code;
  if ((code = weights_ok(*cfg, *w)) != COLI_MOE_OK) return code;
  if (T > cfg->max_tokens) return COLI_MOE_ECAPACITY;
  const Layout L = layout_of(*cfg);
  if (L.total > (size_t)COLI_MOE_STATIC_SCRATCH_BYTES) return COLI_MOE_ECAPACITY;
  if (T == 0) return COLI_MOE_OK;
  if (!hidden || !out || !aligned(hidden, 16) || !aligned(out, 16)) return COLI_MOE_EARG;
  char *ws = nullptr;
  if (scratch_of_current_device(&ws) != hipSuccess) return COLI_MOE_EDEVICE;
  coli_moe_t m;  // on the stack: no host allocation either
  set_up(&m, *cfg, *w, ws, L);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (stage(&m, s) != hipSuccess) return COLI_MOE_EDEVICE;
  return coli_moe_forward(&m, hidden, out, T, stream);
}

int coli_moe_set_routing(coli_moe_t *m, int32_t k_use, float top_p) { return coli::set_route_limits(m, k_use, top_p); }

void coli_moe_free(coli_moe_t *m) {
  if (!m) return;
  for (ProfRecord &r : m->prof) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  delete m;
}

int coli_moe_last_routing(const coli_moe_t *mc, int32_t *idx, float *w, int32_t *offsets,
                          int32_t *sorted_ids, int32_t *inv, int32_t *active, int32_t *n_active,
                          void *stream) {
  if (!mc) return COLI_MOE_EARG;
  coli_moe_t *m = const_cast<coli_moe_t *>(mc);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t n = (size_t)m->last_T * m->cfg.top_k, E = (size_t)m->cfg.n_experts;
  struct Copy {
    void *dst;
    size_t off, bytes;
  } copies[] = {{idx, m->L.idx, n * 4},         {w, m->L.w, n * 4},
                {offsets, m->L.offsets, (E + 1) * 4}, {sorted_ids, m->L.sorted_ids, n * 4},
                {inv, m->L.inv, n * 4},         {active, m->L.active, E * 4},
                {n_active, m->L.n_active, 4}};
  for (const Copy &c : copies) {
    if (!c.dst || c.bytes == 0) continue;
    if (hipMemcpyAsync(c.dst, m->ws + c.off, c.bytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
      return COLI_MOE_EDEVICE;
  }
  return m->last_T;
}

static_assert(coli::kSpinLimit == COLI_MOE_DEFAULT_SPIN_LIMIT, "one default bound");

int coli_moe_status(coli_moe_t *m, void *stream) {
  if (!m) return COLI_MOE_EARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t word = 0;
  if (hipMemcpyAsync(&word, m->ws + m->L.status, 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return COLI_MOE_EDEVICE;
  if (word == 0) return COLI_MOE_OK;
  if (coli::launch_fill_i32(at<int32_t>(m, m->L.status), 1, 0, s) != hipSuccess) return COLI_MOE_EDEVICE;
  return COLI_MOE_EDEVICE;
}

int coli_moe_test_spin_limit(coli_moe_t *m, int32_t polls) {
  if (!m || polls < 0) return COLI_MOE_EARG;
  m->spin_limit = polls;
  return COLI_MOE_OK;
}

int coli_moe_test_batch_kernels(coli_moe_t *m, int32_t mfma) {
  if (!m || mfma < 0 || mfma > 2) return COLI_MOE_EARG;
  m->batch_mfma = mfma;
  return COLI_MOE_OK;
}

int coli_moe_test_dispatch(const int32_t *idx, int32_t T, int32_t k, int32_t E, int32_t *offsets,
                           int32_t *sorted_ids, int32_t *inv, int32_t *active, int32_t *n_active,
                           void *stream) {
  if (T < 0 || k < 1 || k > coli::kMaxTopK || E < 1 || E > coli::kMaxExperts ||
      (int64_t)T * k > (1 << 20))
    return COLI_MOE_EARG;
  if (!offsets || !active || !n_active || (T > 0 && (!idx || !sorted_ids || !inv))) return COLI_MOE_EARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // the many-workgroup sort's count array, stream-ordered
  const size_t cnt_bytes = coli::dispatch_count_ints(T * k, E) * 4;
  int32_t *cnt = nullptr;
  if (cnt_bytes && hipMallocAsync(reinterpret_cast<void **>(&cnt), cnt_bytes, s) != hipSuccess)
    return COLI_MOE_EDEVICE;
  const hipError_t e = coli::launch_dispatch(idx, T * k, E, offsets, sorted_ids, inv, active, n_active, cnt, s);
  if (cnt && hipFreeAsync(cnt, s) != hipSuccess) return COLI_MOE_EDEVICE;
  return e == hipSuccess ? COLI_MOE_OK : COLI_MOE_EDEVICE;
}

int coli_moe_probe_read(const coli_moe_t *mc, const int32_t *experts, int32_t n, void *stream) {
  if (!mc || !experts || n < 1 || n > 64 || mc->cfg.hidden > 8192 ||
      mc->cfg.weight_format != COLI_MOE_WEIGHTS_INT4_GS64)
    return COLI_MOE_EARG;
  coli_moe_t *m = const_cast<coli_moe_t *>(mc);
  coli::DecodeProblem P{};
  P.gate = {m->w.gate_q, m->w.gate_s};
  P.up = {m->w.up_q, m->w.up_s};
  P.sh_gate = {m->w.sh_gate_q, m->w.sh_gate_s};
  P.sh_up = {m->w.sh_up_q, m->w.sh_up_s};
  P.h = m->cfg.hidden;
  P.I = m->cfg.inter;
  P.E = m->cfg.n_experts;
  P.has_shared = m->cfg.n_shared;
  if (coli::launch_read_probe(P, experts, n, at<uint32_t>(m, m->L.logits), static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return COLI_MOE_EDEVICE;
  return COLI_MOE_OK;
}

int coli_moe_probe_read_down(const coli_moe_t *mc, const int32_t *experts, int32_t n, void *stream) {
  if (!mc || !experts || n < 1 || n > 64 || mc->cfg.inter > 8192 ||
      mc->cfg.weight_format != COLI_MOE_WEIGHTS_INT4_GS64)
    return COLI_MOE_EARG;
  coli_moe_t *m = const_cast<coli_moe_t *>(mc);
  coli::DecodeProblem P{};
  P.down = {m->w.down_q, m->w.down_s};
  P.sh_down = {m->w.sh_down_q, m->w.sh_down_s};
  P.h = m->cfg.hidden;
  P.I = m->cfg.inter;
  P.E = m->cfg.n_experts;
  P.has_shared = m->cfg.n_shared;
  if (coli::launch_read_probe_down(P, experts, n, at<uint32_t>(m, m->L.logits), static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return COLI_MOE_EDEVICE;
  return COLI_MOE_OK;
}

int coli_moe_probe_stream(const void *buf, size_t bytes, uint32_t *sink, void *stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 || !aligned(buf, 16) || !aligned(sink, 4)) return COLI_MOE_EARG;
  return coli::launch_stream_probe(buf, bytes, sink, static_cast<hipStream_t>(stream)) == hipSuccess
             ? COLI_MOE_OK
             : COLI_MOE_EDEVICE;
}

int coli_moe_probe_mfma(int32_t iters, int32_t blocks, uint32_t *sink, void *stream) {
  if (!sink || !aligned(sink, 4) || iters < 1 || iters >= (1 << 20) || blocks < 1 || blocks > (1 << 20))
    return COLI_MOE_EARG;
  return coli::launch_mfma_probe(iters, blocks, sink, static_cast<hipStream_t>(stream)) == hipSuccess
             ? COLI_MOE_OK
             : COLI_MOE_EDEVICE;
}

int coli_moe_probe_mfma_f16(int32_t iters, int32_t blocks, uint32_t seed, uint32_t *sink, void *stream) {
  if (!sink || !aligned(sink, 4) || iters < 1 || iters >= (1 << 20) || blocks < 1 || blocks > (1 << 20))
    return COLI_MOE_EARG;
  return coli::launch_mfma_probe_f16(iters, blocks, seed, sink, static_cast<hipStream_t>(stream)) == hipSuccess
             ? COLI_MOE_OK
             : COLI_MOE_EDEVICE;
}

int coli_moe_profile_begin(coli_moe_t *m, int32_t max_calls) {
  if (!m || max_calls < 0) return COLI_MOE_EARG;
  const size_t need = (size_t)max_calls * COLI_MOE_N_KERNELS;
  while (m->prof.size() < need) {
    ProfRecord r{};
    if (hipEventCreate(&r.start) != hipSuccess) return COLI_MOE_EDEVICE;
    if (hipEventCreate(&r.stop) != hipSuccess) {
      (void)hipEventDestroy(r.start);
      return COLI_MOE_EDEVICE;
    }
    m->prof.push_back(r);
  }
  m->prof_used = 0;
  m->prof_calls_left = max_calls;
  m->prof_calls_done = 0;
  return COLI_MOE_OK;
}

int coli_moe_profile_end(coli_moe_t *m, float *kernel_ms, int32_t *kernel_launches) {
  if (!m) return COLI_MOE_EARG;
  float ms[COLI_MOE_N_KERNELS] = {0};
  int32_t cnt[COLI_MOE_N_KERNELS] = {0};
  for (size_t i = 0; i < m->prof_used; ++i) {
    ProfRecord &r = m->prof[i];
    if (hipEventSynchronize(r.stop) != hipSuccess) return COLI_MOE_EDEVICE;
    float t = 0.0f;
    if (hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess) return COLI_MOE_EDEVICE;
    ms[r.kernel] += t;
    cnt[r.kernel] += 1;
  }
  if (kernel_ms)
    for (int i = 0; i < COLI_MOE_N_KERNELS; ++i) kernel_ms[i] = ms[i];
  if (kernel_launches)
    for (int i = 0; i < COLI_MOE_N_KERNELS; ++i) kernel_launches[i] = cnt[i];
  const int done = m->prof_calls_done;
  m->prof_calls_left = 0;
  m->prof_calls_done = 0;
  m->prof_used = 0;
  return done;
}

const char *coli_moe_kernel_name(int32_t i) {
  return (i >= 0 && i < COLI_MOE_N_KERNELS) ? kKernelNames[i] : "";
}

const char *coli_moe_error_string(int32_t code) {
  switch (code) {
    case COLI_MOE_OK: return "ok";
    case COLI_MOE_ECAPACITY: return "capacity: more tokens than max_tokens, or workspace too small";
    case COLI_MOE_EROUTING: return "routing configuration: top_k, n_group or group_size unsupported";
    case COLI_MOE_EDEVICE: return "HIP launch or runtime error";
    case COLI_MOE_EARG: return "bad argument: NULL or misaligned pointer, unsupported dimension";
    default: return "unknown error code";
  }
}

}  // extern "C"
