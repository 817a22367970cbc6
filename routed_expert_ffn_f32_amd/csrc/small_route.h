// Routing of a small batch (T <= kSmallT tokens, T*k <= kSmallAssign) by one
// workgroup: expert selection of every token, then the stable counting sort
// of the assignments by expert, in LDS.
//
// Sources: "colibri engine teardown" page, "Three key engineering
// decisions", item 1 (sigmoid router, noaux_tc top-k, n_group = 1,
// routed_scaling_factor); cf-1.com Colibri article, section 3.3, step 3
// (per-expert counts, prefix sum into expert offsets, scatter by expert).
#pragma once

#include "internal.h"
#include "select.h"

namespace coli {

struct SmallRouting {
  int32_t idx[kSmallAssign];
  float w[kSmallAssign];
  int32_t sorted_ids[kSmallAssign];
  int32_t inv[kSmallAssign];
  int32_t active[kSmallAssign];
  int32_t seg_begin[kSmallAssign + 1];
  int32_t n_active;
  // selection candidates per token: key image, expert, score; merge scratch
  alignas(16) uint32_t cu[kSmallT][64];
  int32_t ce[kSmallT][64];
  float cs[kSmallT][64];
  uint32_t scratch[kSmallT][kMaxTopK];
  int32_t slot_of[kSmallT][kMaxTopK];
};

// How the block's waves share the selection: each token gets WT = waves / T
// waves (WT * k <= 64), wave w working on token w / WT, part w % WT of the
// experts (a chunk of ceil(E / WT)).
struct SmallSelectPlan {
  int wt, chunk, t, part, e_lo, ne;
};

__device__ __forceinline__ SmallSelectPlan small_select_plan(int T, int E, int k) {
  // the wave index as a scalar: the buffer resources built from the plan
  // must be wave-uniform values
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), waves = blockDim.x >> 6;
  SmallSelectPlan p;
  p.wt = waves / T;
  if (p.wt * k > 64) p.wt = max(1, 64 / k);
  p.chunk = (E + p.wt - 1) / p.wt;
  p.t = wave / p.wt;
  p.part = wave % p.wt;
  p.e_lo = p.part * p.chunk;
  p.ne = p.t < T ? max(0, min(p.chunk, E - p.e_lo)) : 0;
  return p;
}

// This wave's selection inputs (issue before other loads: the routing is the
// first thing the block waits for).
__device__ __forceinline__ void route_small_load(const float *__restrict__ logits, const float *__restrict__ bias,
                                                 int T, int E, int k, SelectInput &in) {
  const SmallSelectPlan p = small_select_plan(T, E, k);
  select_part_load(logits + (size_t)min(p.t, T - 1) * E, bias, p.e_lo, p.ne, in);
}

// Routing of the batch by the whole block (waves >= T), from the inputs of
// route_small_load, in two calls: route_small_a (phase A over E / WT experts
// per wave, candidates into LDS, block barrier), then route_small_b (phase B
// by wave t for token t, select.h, then the sort).  A part's k best contain
// every expert of the token's k best that falls in the part, so phase B sees
// all of them.  Wave 0 then sorts the
// n = T*k assignments by expert, stably (position = smaller keys + equal keys
// of lower a), and lists the segments (an assignment with no equal key before
// it starts one).  Ends with the block synchronised for LDS (global loads in
// flight are not waited for).
__device__ __forceinline__ void route_small_a(const SelectInput &in, int T, int E, int k, SmallRouting &R) {
  const SmallSelectPlan p = small_select_plan(T, E, k);
  if (p.t < T) {
    uint32_t *cu = R.cu[p.t] + p.part * k;
    int32_t *ce = R.ce[p.t] + p.part * k;
    float *cs = R.cs[p.t] + p.part * k;
    const int nk = (p.ne + 63) >> 6;
    if (nk <= 1)
      select_part<1>(in, p.e_lo, p.ne, k, cu, ce, cs);
    else if (nk <= 2)
      select_part<2>(in, p.e_lo, p.ne, k, cu, ce, cs);
    else if (nk <= 4)
      select_part<4>(in, p.e_lo, p.ne, k, cu, ce, cs);
    else
      select_part<8>(in, p.e_lo, p.ne, k, cu, ce, cs);
  }
  block_barrier();
}

// One token: the merge lists the kept experts in ascending order, each with
// exactly one assignment (its slot), and the dropped slots are the slots
// m..k-1 (a suffix), which follow every expert's group in ascending order.
__device__ __forceinline__ void route_small_one_token(int k, int m, SmallRouting &R) {
  const int lane = threadIdx.x & 63;
  if (lane < m) {
    const int sl = R.slot_of[0][lane];
    R.sorted_ids[lane] = sl;
    R.inv[sl] = lane;
    R.active[lane] = R.idx[sl];
    R.seg_begin[lane] = lane;
  } else if (lane < k) {
    R.sorted_ids[lane] = lane;
    R.inv[lane] = lane;
  }
  if (lane == 0) {
    R.n_active = m;
    R.seg_begin[m] = m;
  }
}

// Phase B and the sort (after route_small_a).  Dropped slots (expert -1,
// routing limits) take the positions after every expert's group, in
// ascending order, and start no group.
__device__ __forceinline__ void route_small_b(int T, int E, int k, float rsf, const RouteLimits &lim,
                                              SmallRouting &R) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wt = small_select_plan(T, E, k).wt;
  int m = 0;
  if (wave < T)
    m = select_merge(R.cu[wave], R.ce[wave], R.cs[wave], wt * k, k, rsf, lim, R.idx + wave * k, R.w + wave * k,
                     R.scratch[wave], R.slot_of[wave]);
  if (T == 1) {
    if (wave == 0) route_small_one_token(k, m, R);
    block_barrier();
    return;
  }
  block_barrier();
  const int n = T * k;
  if (wave == 0) {
    const bool valid = lane < n;
    const int id = valid ? R.idx[lane] : -1;
    const bool kept = valid && id >= 0;
    const int key = kept ? id : 0x7fffffff;
    int lt = 0, eq_before = 0;
    uint64_t m_lt = 0;
    for (int b = 0; b < n; ++b) {
      const int kb = __builtin_amdgcn_readlane(key, b);
      lt += kb < key;
      eq_before += kb == key && b < lane;
      m_lt |= (uint64_t)(kb < key) << b;
    }
    const bool start = kept && eq_before == 0;
    const uint64_t starts = __ballot(start);
    const int n_kept = __popcll(__ballot(kept));
    if (valid) {
      R.sorted_ids[lt + eq_before] = lane;
      R.inv[lane] = lt + eq_before;
    }
    if (start) {
      const int slot = __popcll(starts & m_lt);
      R.active[slot] = key;
      R.seg_begin[slot] = lt;
    }
    if (lane == 0) {
      R.n_active = __popcll(starts);
      R.seg_begin[__popcll(starts)] = n_kept;
    }
  }
  block_barrier();
}

// Phase B for one token, by the calling wave alone and without a block
// barrier (after route_small_a): the merge, then the assignments in expert
// order.
__device__ __forceinline__ void route_small_b1(int E, int k, float rsf, const RouteLimits &lim, SmallRouting &R) {
  const int wt = small_select_plan(1, E, k).wt;
  const int m = select_merge(R.cu[0], R.ce[0], R.cs[0], wt * k, k, rsf, lim, R.idx, R.w, R.scratch[0], R.slot_of[0]);
  route_small_one_token(k, m, R);
}

// Where the routing of a call goes (device arrays of the C ABI's layout).
struct RoutingOut {
  int32_t *idx;
  float *w;
  int32_t *sorted_ids, *inv, *offsets, *active, *n_active;
};

// The routing of the batch from LDS to the arrays of `o`, by one block.
__device__ __forceinline__ void publish_routing(const SmallRouting &R, int T, int k, int E, const RoutingOut &o) {
  const int n = T * k;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    o.idx[i] = R.idx[i];
    o.w[i] = R.w[i];
    o.sorted_ids[i] = R.sorted_ids[i];
    o.inv[i] = R.inv[i];
  }
  for (int e = threadIdx.x; e <= E; e += blockDim.x) {
    int c = 0;
    for (int a = 0; a < n; ++a) c += R.idx[a] >= 0 && R.idx[a] < e;  // dropped slots (-1) in no group
    o.offsets[e] = c;
  }
  for (int s = threadIdx.x; s < R.n_active; s += blockDim.x) o.active[s] = R.active[s];
  if (threadIdx.x == 0) *o.n_active = R.n_active;
}

}  // namespace coli
