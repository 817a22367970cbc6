// HBM expert cache with host-RAM backing, router look-ahead prefetch, and
// the usage history file: the C ABI functions coli_moe_cache_* and
// coli_moe_usage_* of include/coli_moe.h.
//
// Source: "Colibri 调优与运行时旋钮实战指南" (Colibri tuning and runtime
// knobs guide): hot / warm / cold tiers with a per-layer expert LRU, LFRU
// re-pinning with hysteresis, the learning cache (.coli_usage: per-expert
// routing counts, text records), and router look-ahead prefetch (PILOT:
// layer L+1's router applied to layer L's state predicts its experts, which
// are read ahead on an I/O thread while layer L computes; prefetched experts
// are guarded from eviction until used).  "colibrì 引擎拆解" (engine
// teardown), "System map": routed experts streamed on demand through a
// per-layer LRU; "Task flow example": a miss loads while the next layer's
// experts are already being fetched.
//
// On MI355X the tiers are HBM slots (this cache) over pinned host memory
// (the caller's tables).  A forward runs the router, selection and dispatch
// on the device, reads the call's expert list back (one host
// synchronisation per call), copies the misses from pinned host memory into
// their slots on the cache's own copy stream (default priority), updates the
// device slot map, makes the compute stream wait for the copies, and runs
// the expert kernels with the slot map as the expert -> table indirection.
// The math is the uncached layer's, on the same bytes: outputs are bit for
// bit those of coli_moe_forward on fully resident tables.
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <vector>

#include "cache_policy.h"
#include "coli_moe.h"
#include "handle.h"
#include "internal.h"

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }
constexpr int kMapRing = 8;  // staging copies of the slot map in flight

// Byte offsets of the slot memory regions for S slots: the stacked tables of
// the six matrices, then the slot map [E] int32.
struct SlotLayout {
  size_t gq, gs, uq, us, dq, ds, map, total;
  size_t gq_e, gs_e, dq_e, ds_e;  // bytes of one expert's matrix
};

SlotLayout slot_layout(const coli_moe_config_t &c, int S) {
  SlotLayout L{};
  const size_t h = (size_t)c.hidden, I = (size_t)c.inter;
  L.gq_e = I * h / 2;
  L.gs_e = I * (h / 64) * 4;
  L.dq_e = h * I / 2;
  L.ds_e = h * (I / 64) * 4;
  size_t o = 0;
  L.gq = o; o = align_up(o + S * L.gq_e);
  L.gs = o; o = align_up(o + S * L.gs_e);
  L.uq = o; o = align_up(o + S * L.gq_e);
  L.us = o; o = align_up(o + S * L.gs_e);
  L.dq = o; o = align_up(o + S * L.dq_e);
  L.ds = o; o = align_up(o + S * L.ds_e);
  L.map = o; o = align_up(o + (size_t)c.n_experts * 4);
  L.total = o;
  return L;
}

}  // namespace

struct coli_moe_cache {
  coli_moe_t inner;                 // the layer over the slots
  coli_moe_config_t cfg;            // as given (the inner handle has prefill off)
  coli_moe_host_experts_t host;
  char *slots;
  SlotLayout SL;
  coli::CachePolicy *policy;
  hipStream_t copy_stream;
  hipEvent_t copy_done;             // last copy enqueued on copy_stream
  hipEvent_t map_event[kMapRing];
  int32_t *map_stage[kMapRing];     // pinned staging of the slot map
  int map_next;
  int32_t *rt_stage;                // pinned: n_active, active[E], offsets[E+1], idx[T*k]
  std::vector<char> guard;          // prefetched, not yet used
  coli_moe_cache_stats_t st;
  std::vector<coli::CacheLoad> loads;
};

namespace {

size_t expert_bytes(const SlotLayout &L) { return 2 * (L.gq_e + L.gs_e) + L.dq_e + L.ds_e; }

// Enqueue the copies of one load (expert -> slot) on the copy stream.
hipError_t copy_expert(coli_moe_cache_t *c, const coli::CacheLoad &ld) {
  const SlotLayout &L = c->SL;
  const size_t e = (size_t)ld.expert, s = (size_t)ld.slot;
  struct Part {
    size_t dst, per;
    const void *src;
  } parts[] = {{L.gq, L.gq_e, c->host.gate_q}, {L.gs, L.gs_e, c->host.gate_s}, {L.uq, L.gq_e, c->host.up_q},
               {L.us, L.gs_e, c->host.up_s},   {L.dq, L.dq_e, c->host.down_q}, {L.ds, L.ds_e, c->host.down_s}};
  for (const Part &p : parts) {
    const hipError_t err = hipMemcpyAsync(c->slots + p.dst + s * p.per, static_cast<const char *>(p.src) + e * p.per,
                                          p.per, hipMemcpyHostToDevice, c->copy_stream);
    if (err != hipSuccess) return err;
  }
  c->st.bytes_copied += (int64_t)expert_bytes(L);
  if (ld.evicted >= 0) ++c->st.evictions;
  return hipSuccess;
}

// Enqueue the slot map (from the policy) on the copy stream, through a
// staging buffer whose previous copy has completed.
hipError_t push_map(coli_moe_cache_t *c) {
  const int i = c->map_next;
  c->map_next = (c->map_next + 1) % kMapRing;
  hipError_t err = hipEventSynchronize(c->map_event[i]);
  if (err != hipSuccess) return err;
  const int E = c->cfg.n_experts;
  for (int e = 0; e < E; ++e) c->map_stage[i][e] = c->policy->slot_of(e);
  err = hipMemcpyAsync(c->slots + c->SL.map, c->map_stage[i], (size_t)E * 4, hipMemcpyHostToDevice, c->copy_stream);
  if (err != hipSuccess) return err;
  return hipEventRecord(c->map_event[i], c->copy_stream);
}

// Read back n_active, active and offsets (and, when idx_n > 0, the first
// idx_n entries of idx) of the inner handle's last routing; waits for stream.
hipError_t read_routing(coli_moe_cache_t *c, hipStream_t s, int idx_n) {
  coli_moe_t *m = &c->inner;
  const int E = c->cfg.n_experts;
  int32_t *st = c->rt_stage;
  hipError_t err = hipMemcpyAsync(st, m->ws + m->L.n_active, 4, hipMemcpyDeviceToHost, s);
  if (err == hipSuccess) err = hipMemcpyAsync(st + 1, m->ws + m->L.active, (size_t)E * 4, hipMemcpyDeviceToHost, s);
  if (err == hipSuccess)
    err = hipMemcpyAsync(st + 1 + E, m->ws + m->L.offsets, (size_t)(E + 1) * 4, hipMemcpyDeviceToHost, s);
  if (err == hipSuccess && idx_n > 0)
    err = hipMemcpyAsync(st + 2 + 2 * E, m->ws + m->L.idx, (size_t)idx_n * 4, hipMemcpyDeviceToHost, s);
  if (err == hipSuccess) err = hipStreamSynchronize(s);
  return err;
}

void free_cache(coli_moe_cache_t *c) {
  if (!c) return;
  if (c->copy_stream) {
    (void)hipStreamSynchronize(c->copy_stream);
    (void)hipStreamDestroy(c->copy_stream);
  }
  if (c->copy_done) (void)hipEventDestroy(c->copy_done);
  for (int i = 0; i < kMapRing; ++i) {
    if (c->map_event[i]) (void)hipEventDestroy(c->map_event[i]);
    if (c->map_stage[i]) (void)hipHostFree(c->map_stage[i]);
  }
  if (c->rt_stage) (void)hipHostFree(c->rt_stage);
  for (ProfRecord &r : c->inner.prof) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  delete c->policy;
  delete c;
}

// Distinct experts one call can need.
int call_reserve(const coli_moe_config_t &cfg) {
  const int64_t n = (int64_t)cfg.top_k * cfg.max_tokens;
  return (int)(n < cfg.n_experts ? n : cfg.n_experts);
}

}  // namespace

extern "C" {

size_t coli_moe_cache_slot_bytes(const coli_moe_config_t *cfg, int32_t n_slots) {
  if (!cfg || coli::config_check(*cfg) != COLI_MOE_OK || n_slots < 1 || n_slots > cfg->n_experts ||
      cfg->weight_format != COLI_MOE_WEIGHTS_INT4_GS64)
    return 0;
  return slot_layout(*cfg, n_slots).total;
}

int coli_moe_cache_init(coli_moe_cache_t **out, const coli_moe_config_t *cfg, const coli_moe_cache_config_t *cc,
                        const coli_moe_weights_t *resident, const coli_moe_host_experts_t *host, void *slots,
                        size_t slot_bytes, void *workspace, size_t workspace_bytes, void *stream) {
  if (!out || !cfg || !cc || !resident || !host || !slots || !workspace) return COLI_MOE_EARG;
  *out = nullptr;
  int code = coli::config_check(*cfg);
  if (code != COLI_MOE_OK) return code;
  if (cfg->weight_format != COLI_MOE_WEIGHTS_INT4_GS64) return COLI_MOE_EARG;  // slots hold int4 gs64 tables
  const int S = cc->n_slots;
  if (S < 1 || S > cfg->n_experts) return COLI_MOE_EARG;
  if (S < call_reserve(*cfg)) return COLI_MOE_ECAPACITY;
  const float decay = cc->decay == 0.0f ? 0.9f : cc->decay;
  if (!(decay > 0.0f && decay <= 1.0f) || cc->repin_every < 0) return COLI_MOE_EARG;
  const void *h6[] = {host->gate_q, host->gate_s, host->up_q, host->up_s, host->down_q, host->down_s};
  for (const void *p : h6)
    if (!p || ((uintptr_t)p % 16)) return COLI_MOE_EARG;
  if ((uintptr_t)slots % kAlign || (uintptr_t)workspace % kAlign) return COLI_MOE_EARG;
  const SlotLayout SL = slot_layout(*cfg, S);
  if (slot_bytes < SL.total) return COLI_MOE_ECAPACITY;
  // the inner layer: every call on the GEMV path (its prefill statistics
  // would be per table, and the tables move)
  coli_moe_config_t icfg = *cfg;
  icfg.prefill_threshold = cfg->max_tokens + 1;
  const Layout L = coli::workspace_layout(icfg);
  if (workspace_bytes < L.total) return COLI_MOE_ECAPACITY;
  char *sb = static_cast<char *>(slots);
  coli_moe_weights_t w = *resident;
  w.gate_q = reinterpret_cast<const uint8_t *>(sb + SL.gq);
  w.gate_s = reinterpret_cast<const float *>(sb + SL.gs);
  w.up_q = reinterpret_cast<const uint8_t *>(sb + SL.uq);
  w.up_s = reinterpret_cast<const float *>(sb + SL.us);
  w.down_q = reinterpret_cast<const uint8_t *>(sb + SL.dq);
  w.down_s = reinterpret_cast<const float *>(sb + SL.ds);
  if ((code = coli::weights_check(icfg, w)) != COLI_MOE_OK) return code;

  coli_moe_cache_t *c = new (std::nothrow) coli_moe_cache_t();
  if (!c) return COLI_MOE_EARG;
  c->cfg = *cfg;
  c->host = *host;
  c->slots = sb;
  c->SL = SL;
  c->policy = new (std::nothrow) coli::CachePolicy(cfg->n_experts, S, call_reserve(*cfg), decay, cc->repin_every);
  c->guard.assign(cfg->n_experts, 0);
  memset(&c->st, 0, sizeof(c->st));
  hipStream_t s = static_cast<hipStream_t>(stream);
  bool ok = c->policy != nullptr;
  ok = ok && hipStreamCreateWithFlags(&c->copy_stream, hipStreamNonBlocking) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&c->copy_done, hipEventDisableTiming) == hipSuccess;
  for (int i = 0; ok && i < kMapRing; ++i) {
    ok = hipEventCreateWithFlags(&c->map_event[i], hipEventDisableTiming) == hipSuccess;
    ok = ok && hipHostMalloc(reinterpret_cast<void **>(&c->map_stage[i]), (size_t)cfg->n_experts * 4) == hipSuccess;
  }
  const size_t rt = (size_t)(2 + 2 * cfg->n_experts + cfg->max_tokens * cfg->top_k) * 4;
  ok = ok && hipHostMalloc(reinterpret_cast<void **>(&c->rt_stage), rt) == hipSuccess;
  if (!ok) {
    free_cache(c);
    return COLI_MOE_EDEVICE;
  }
  coli::handle_set_up(&c->inner, icfg, w, static_cast<char *>(workspace), L);
  c->inner.slot_of = reinterpret_cast<const int32_t *>(sb + SL.map);
  if (coli::handle_stage(&c->inner, s) != hipSuccess || push_map(c) != hipSuccess ||
      hipEventRecord(c->copy_done, c->copy_stream) != hipSuccess || hipStreamWaitEvent(s, c->copy_done, 0) != hipSuccess) {
    free_cache(c);
    return COLI_MOE_EDEVICE;
  }
  *out = c;
  return COLI_MOE_OK;
}

int coli_moe_cache_forward(coli_moe_cache_t *c, const float *hidden, float *out, int32_t T, void *stream) {
  if (!c || T < 0) return COLI_MOE_EARG;
  if (T > c->cfg.max_tokens) return COLI_MOE_ECAPACITY;
  if (T == 0) return COLI_MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int rc = coli::forward_phases(&c->inner, hidden, out, T, s, coli::kPhaseRoute);
  if (rc != COLI_MOE_OK) return rc;
  if (read_routing(c, s, 0) != hipSuccess) return COLI_MOE_EDEVICE;
  const int E = c->cfg.n_experts;
  const int na = c->rt_stage[0];
  if (na < 0 || na > E) return COLI_MOE_EDEVICE;
  const int32_t *active = c->rt_stage + 1, *offsets = c->rt_stage + 1 + E;
  std::vector<int64_t> counts(na);
  for (int i = 0; i < na; ++i) counts[i] = offsets[active[i] + 1] - offsets[active[i]];
  int resident_before = 0;
  for (int i = 0; i < na; ++i) {
    const int e = active[i];
    if (c->policy->slot_of(e) >= 0) ++resident_before;
    if (c->guard[e]) {
      ++c->st.prefetch_hits;
      c->guard[e] = 0;
    }
  }
  // misses avoid the slots of experts prefetched for this call; such
  // guards expire with it
  if (!c->policy->plan_call(active, counts.data(), na, c->loads, &c->guard)) return COLI_MOE_ECAPACITY;
  std::fill(c->guard.begin(), c->guard.end(), 0);
  for (const coli::CacheLoad &ld : c->loads)
    if (copy_expert(c, ld) != hipSuccess) return COLI_MOE_EDEVICE;
  if (!c->loads.empty() && push_map(c) != hipSuccess) return COLI_MOE_EDEVICE;
  if (hipEventRecord(c->copy_done, c->copy_stream) != hipSuccess || hipStreamWaitEvent(s, c->copy_done, 0) != hipSuccess)
    return COLI_MOE_EDEVICE;
  c->st.calls += 1;
  c->st.needed += na;
  c->st.hits += resident_before;
  c->st.misses += (int64_t)c->loads.size();
  return coli::forward_phases(&c->inner, hidden, out, T, s, coli::kPhaseExperts);
}

int coli_moe_cache_prefetch(coli_moe_cache_t *c, const float *hidden, int32_t T, int32_t n_predict, void *stream) {
  if (!c || !hidden || T < 1 || n_predict < 1 || n_predict > c->cfg.top_k) return COLI_MOE_EARG;
  if (T > c->cfg.max_tokens) return COLI_MOE_ECAPACITY;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int k = c->cfg.top_k, E = c->cfg.n_experts;
  const int rc = coli::forward_phases(&c->inner, hidden, nullptr, T, s, coli::kPhaseRoute);
  if (rc != COLI_MOE_OK) return rc;
  if (read_routing(c, s, T * k) != hipSuccess) return COLI_MOE_EDEVICE;
  const int32_t *idx = c->rt_stage + 2 + 2 * E;
  bool any = false;
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < n_predict; ++j) {
      const int e = idx[t * k + j];
      if (e < 0) continue;  // a slot the routing limits dropped
      if (e >= E) return COLI_MOE_EDEVICE;
      if (c->policy->slot_of(e) >= 0) continue;
      coli::CacheLoad ld;
      if (c->policy->prefetch(e, c->guard, ld) < 0) continue;  // no slot free of pins and guards
      c->guard[e] = 1;
      if (ld.evicted >= 0) c->guard[ld.evicted] = 0;
      ++c->st.prefetched;
      if (copy_expert(c, ld) != hipSuccess) return COLI_MOE_EDEVICE;
      any = true;
    }
  if (any && push_map(c) != hipSuccess) return COLI_MOE_EDEVICE;
  return COLI_MOE_OK;
}

int coli_moe_cache_pin(coli_moe_cache_t *c, const int32_t *experts, int32_t n, void *stream) {
  if (!c || n < 0 || (n > 0 && !experts)) return COLI_MOE_EARG;
  int pinned = 0;
  bool any = false;
  for (int i = 0; i < n; ++i) {
    coli::CacheLoad ld;
    if (!c->policy->pin(experts[i], ld)) break;
    ++pinned;
    if (ld.expert >= 0) {
      c->guard[ld.expert] = 0;
      if (ld.evicted >= 0) c->guard[ld.evicted] = 0;
      if (copy_expert(c, ld) != hipSuccess) return COLI_MOE_EDEVICE;
      any = true;
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (any && push_map(c) != hipSuccess) return COLI_MOE_EDEVICE;
  if (hipEventRecord(c->copy_done, c->copy_stream) != hipSuccess || hipStreamWaitEvent(s, c->copy_done, 0) != hipSuccess)
    return COLI_MOE_EDEVICE;
  return pinned;
}

int coli_moe_cache_stats(const coli_moe_cache_t *c, coli_moe_cache_stats_t *st) {
  if (!c || !st) return COLI_MOE_EARG;
  *st = c->st;
  st->repin_swaps = c->policy->repin_swaps();
  st->pinned = c->policy->n_pinned();
  int res = 0;
  for (int s = 0; s < c->policy->n_slots(); ++s) res += c->policy->expert_in(s) >= 0;
  st->resident = res;
  return COLI_MOE_OK;
}

int coli_moe_cache_usage(const coli_moe_cache_t *c, int64_t *counts) {
  if (!c || !counts) return COLI_MOE_EARG;
  for (int e = 0; e < c->cfg.n_experts; ++e) counts[e] = c->policy->usage(e);
  return COLI_MOE_OK;
}

int coli_moe_cache_slots(const coli_moe_cache_t *c, int32_t *slot_of) {
  if (!c || !slot_of) return COLI_MOE_EARG;
  for (int e = 0; e < c->cfg.n_experts; ++e) slot_of[e] = c->policy->slot_of(e);
  return COLI_MOE_OK;
}

coli_moe_t *coli_moe_cache_layer(coli_moe_cache_t *c) { return c ? &c->inner : nullptr; }

void coli_moe_cache_free(coli_moe_cache_t *c) { free_cache(c); }

// ---------------------------------------------------------------------------
// Usage history file.
// ---------------------------------------------------------------------------

// FNV-1a, 32 bits, of the engine name: the writer's identity in the file.
uint32_t coli_moe_usage_engine_id(void) {
  uint32_t h = 2166136261u;
  for (const char *p = "coli_moe_gfx950"; *p; ++p) h = (h ^ (uint8_t)*p) * 16777619u;
  return h;
}

int coli_moe_usage_write(const char *path, int32_t n_layers, int32_t n_experts, const int64_t *counts) {
  if (!path || n_layers < 1 || n_experts < 1 || !counts) return COLI_MOE_EARG;
  FILE *f = fopen(path, "w");
  if (!f) return COLI_MOE_EARG;
  bool any = false;
  for (int64_t i = 0; i < (int64_t)n_layers * n_experts; ++i) any = any || counts[i] != 0;
  // an empty history is an empty file (no header either)
  if (any) {
    fprintf(f, "-1 %d %d\n-2 %d %u\n", n_layers, n_experts, 1, coli_moe_usage_engine_id());
    for (int l = 0; l < n_layers; ++l)
      for (int e = 0; e < n_experts; ++e) {
        const int64_t v = counts[(int64_t)l * n_experts + e];
        if (v != 0) fprintf(f, "%d %d %lld\n", l, e, (long long)v);
      }
  }
  return fclose(f) == 0 ? COLI_MOE_OK : COLI_MOE_EARG;
}

int coli_moe_usage_read(const char *path, int32_t n_layers, int32_t n_experts, int64_t *counts) {
  if (!path || n_layers < 1 || n_experts < 1 || !counts) return COLI_MOE_EARG;
  FILE *f = fopen(path, "r");
  if (!f) return COLI_MOE_EARG;
  for (int64_t i = 0; i < (int64_t)n_layers * n_experts; ++i) counts[i] = 0;
  long long a, b, c;
  int records = 0, rc = COLI_MOE_OK;
  while (fscanf(f, "%lld %lld %lld", &a, &b, &c) == 3) {
    if (a == -1) {  // dimensions
      if (b != n_layers || c != n_experts) {
        rc = COLI_MOE_EROUTING;
        break;
      }
      continue;
    }
    if (a == -2) {  // format version, engine id
      if ((uint32_t)c != coli_moe_usage_engine_id()) {
        rc = COLI_MOE_EROUTING;
        break;
      }
      continue;
    }
    if (a < 0) continue;  // header records of later versions
    if (a >= n_layers || b < 0 || b >= n_experts || c < 0) {
      rc = COLI_MOE_EARG;
      break;
    }
    counts[a * n_experts + b] += c;
    ++records;
  }
  fclose(f);
  return rc == COLI_MOE_OK ? records : rc;
}

// ---------------------------------------------------------------------------
// Host logic test: the policy alone over a request sequence.
// ---------------------------------------------------------------------------
int coli_moe_test_cache_policy(int32_t n_experts, int32_t n_slots, int32_t reserve, float decay, int32_t repin_every,
                               const int32_t *pins, int32_t n_pins, const int32_t *calls, const int32_t *call_len,
                               int32_t n_calls, int32_t *miss_out, int32_t *slot_out) {
  if (n_experts < 1 || n_slots < 1 || n_slots > n_experts || reserve < 0 || n_calls < 0 || !(decay > 0.0f) ||
      decay > 1.0f || (n_calls > 0 && (!calls || !call_len || !miss_out)) || (n_pins > 0 && !pins))
    return COLI_MOE_EARG;
  coli::CachePolicy P(n_experts, n_slots, reserve, decay, repin_every);
  coli::CacheLoad ld;
  for (int i = 0; i < n_pins; ++i)
    if (!P.pin(pins[i], ld)) return COLI_MOE_ECAPACITY;
  std::vector<coli::CacheLoad> loads;
  int64_t o = 0;
  for (int k = 0; k < n_calls; ++k) {
    if (!P.plan_call(calls + o, nullptr, call_len[k], loads)) return COLI_MOE_ECAPACITY;
    miss_out[k] = (int32_t)loads.size();
    o += call_len[k];
  }
  if (slot_out)
    for (int e = 0; e < n_experts; ++e) slot_out[e] = P.slot_of(e);
  return P.repin_swaps();
}

}  // extern "C"
