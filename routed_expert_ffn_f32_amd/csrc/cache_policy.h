// Residency policy of the HBM expert cache: which routed experts of one
// layer occupy the cache's slots, which miss and where a miss goes.  Plain
// C++ (host only, no HIP), driven by expert_cache.hip and by the host-logic
// test entry point.
//
// Source: "Colibri 调优与运行时旋钮实战指南" (Colibri tuning and runtime
// knobs guide), sections on the resource plan (hot / warm / cold tiers, a
// per-layer expert LRU in the warm tier), online re-pinning (REPIN: at safe
// boundaries, a per-layer LFRU score combining decayed session frequency and
// recent access; at most four swaps, 25% hysteresis against thrashing) and
// the learning cache (per-expert routing counts kept across sessions, the
// hottest experts pinned at start-up); "colibrì 引擎拆解" (engine teardown),
// "System map" (per-layer LRU cache of routed experts).
//
// Here the slots are HBM and the backing store is pinned host memory.  The
// policy, as implemented:
//  - score(e) = f(e) * decay^(now - last(e)): f is the expert's frequency,
//    decayed by `decay` per call and raised by 1 for every call that routes
//    a token to it; now is the call counter, last(e) the last call that
//    used e.  Recently and often used experts score high.
//  - A call's needed experts are pinned against eviction for that call.  A
//    miss takes an empty slot if there is one, else the unpinned, not
//    needed slot of lowest score (ties: least recently used, then lowest
//    slot index).
//  - Pinned experts are never evicted by misses.  At most S - reserve
//    experts are pinned (reserve = the most distinct experts one call can
//    need), so every call's misses fit.
//  - Re-pinning (every repin_every calls, 0 = never): while the hottest
//    resident unpinned expert scores more than 1.25 times the coldest pinned
//    one, they swap roles (no data moves: both are resident), at most 4
//    swaps per round.
#pragma once

#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <vector>

namespace coli {

struct CacheLoad {
  int expert, slot, evicted;  // evicted: the expert that held the slot, or -1
};

class CachePolicy {
 public:
  CachePolicy(int n_experts, int n_slots, int reserve, double decay, int repin_every)
      : E_(n_experts), S_(n_slots), reserve_(std::min(reserve, n_slots)), decay_(decay),
        repin_every_(repin_every), slot_expert_(n_slots, -1), expert_slot_(n_experts, -1),
        freq_(n_experts, 0.0), last_(n_experts, -1), pinned_(n_experts, 0), usage_(n_experts, 0) {}

  int n_experts() const { return E_; }
  int n_slots() const { return S_; }
  int slot_of(int e) const { return expert_slot_[e]; }
  int expert_in(int s) const { return slot_expert_[s]; }
  bool pinned(int e) const { return pinned_[e] != 0; }
  int n_pinned() const { return n_pinned_; }
  int max_pinned() const { return S_ - reserve_; }
  int64_t usage(int e) const { return usage_[e]; }
  int64_t calls() const { return now_; }

  double score(int e) const {
    if (last_[e] < 0) return 0.0;
    return freq_[e] * std::pow(decay_, (double)(now_ - last_[e]));
  }

  // One call that routes tokens to `needed` (distinct experts, counts[i]
  // tokens each).  Returns the loads to make (miss -> slot) in `loads`;
  // every needed expert is resident afterwards.  Misses avoid the slots of
  // `guard` experts (prefetched ones) while other slots can take them.
  // False if the needed experts cannot all fit (more than the unpinned
  // slots plus the resident needed ones).
  bool plan_call(const int *needed, const int64_t *counts, int n, std::vector<CacheLoad> &loads,
                 const std::vector<char> *guard = nullptr) {
    loads.clear();
    ++now_;
    for (int e = 0; e < E_; ++e) freq_[e] *= decay_;
    std::vector<char> need(E_, 0);
    for (int i = 0; i < n; ++i) {
      const int e = needed[i];
      if (e < 0 || e >= E_ || need[e]) return false;
      need[e] = 1;
      freq_[e] += 1.0;
      last_[e] = now_;
      usage_[e] += counts ? counts[i] : 1;
    }
    std::vector<char> keep;
    if (guard) {
      keep = need;
      for (int e = 0; e < E_; ++e) keep[e] = keep[e] || (*guard)[e];
    }
    for (int i = 0; i < n; ++i) {
      const int e = needed[i];
      if (expert_slot_[e] >= 0) continue;
      int s = guard ? victim(keep) : -1;
      if (s < 0) s = victim(need);
      if (s < 0) return false;
      const int old = slot_expert_[s];
      if (old >= 0) expert_slot_[old] = -1;
      slot_expert_[s] = e;
      expert_slot_[e] = s;
      loads.push_back(CacheLoad{e, s, old});
    }
    if (repin_every_ > 0 && now_ % repin_every_ == 0) repin();
    return true;
  }

  // Makes `e` resident ahead of a call (a prefetch) without counting a use;
  // -1 if no slot can take it (all pinned, or all holding `guard` experts).
  int prefetch(int e, const std::vector<char> &guard, CacheLoad &load) {
    if (e < 0 || e >= E_) return -1;
    if (expert_slot_[e] >= 0) return -2;  // already resident
    const int s = victim(guard);
    if (s < 0) return -1;
    const int old = slot_expert_[s];
    if (old >= 0) expert_slot_[old] = -1;
    slot_expert_[s] = e;
    expert_slot_[e] = s;
    load = CacheLoad{e, s, old};
    return s;
  }

  // Pins e (loading it if needed: the load is returned in `load`, expert
  // -1 when none).  False when the pin budget is full.
  bool pin(int e, CacheLoad &load) {
    load = CacheLoad{-1, -1, -1};
    if (e < 0 || e >= E_) return false;
    if (pinned_[e]) return true;
    if (n_pinned_ >= max_pinned()) return false;
    if (expert_slot_[e] < 0) {
      std::vector<char> none(E_, 0);
      const int s = victim(none);
      if (s < 0) return false;
      const int old = slot_expert_[s];
      if (old >= 0) expert_slot_[old] = -1;
      slot_expert_[s] = e;
      expert_slot_[e] = s;
      load = CacheLoad{e, s, old};
    }
    pinned_[e] = 1;
    ++n_pinned_;
    return true;
  }

  void unpin_all() {
    std::fill(pinned_.begin(), pinned_.end(), 0);
    n_pinned_ = 0;
  }

  int repin_swaps() const { return repin_swaps_; }

 private:
  // Slot for a miss: an empty slot, else the unpinned slot not in `keep` of
  // lowest score (ties: least recently used, then lowest slot).
  int victim(const std::vector<char> &keep) const {
    for (int s = 0; s < S_; ++s)
      if (slot_expert_[s] < 0) return s;
    int best = -1;
    double bs = 0.0;
    int64_t bl = 0;
    for (int s = 0; s < S_; ++s) {
      const int e = slot_expert_[s];
      if (pinned_[e] || keep[e]) continue;
      const double sc = score(e);
      if (best < 0 || sc < bs || (sc == bs && last_[e] < bl)) {
        best = s;
        bs = sc;
        bl = last_[e];
      }
    }
    return best;
  }

  void repin() {
    for (int round = 0; round < kMaxSwaps; ++round) {
      int hot = -1, cold = -1;
      for (int s = 0; s < S_; ++s) {
        const int e = slot_expert_[s];
        if (e < 0) continue;
        if (!pinned_[e]) {
          if (hot < 0 || score(e) > score(hot)) hot = e;
        } else if (cold < 0 || score(e) < score(cold)) {
          cold = e;
        }
      }
      if (hot < 0 || cold < 0 || !(score(hot) > kHysteresis * score(cold))) return;
      pinned_[hot] = 1;
      pinned_[cold] = 0;
      ++repin_swaps_;
    }
  }

  static constexpr int kMaxSwaps = 4;
  static constexpr double kHysteresis = 1.25;
  int E_, S_, reserve_;
  double decay_;
  int repin_every_;
  std::vector<int> slot_expert_, expert_slot_;
  std::vector<double> freq_;
  std::vector<int64_t> last_;
  std::vector<char> pinned_;
  std::vector<int64_t> usage_;
  int64_t now_ = 0;
  int n_pinned_ = 0;
  int repin_swaps_ = 0;
};

}  // namespace coli
