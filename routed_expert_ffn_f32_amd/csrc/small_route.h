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
};

// Waves 0..T-1 select one token each (their logits already loaded into
// `in`); wave 0 then sorts the n = T*k assignments by expert, stably
// (position = smaller keys + equal keys of lower a), and lists the segments
// (an assignment with no equal key before it starts one).  Ends with the
// block synchronised.
__device__ __forceinline__ void route_small(const SelectInput &in, int T, int E, int k, float rsf,
                                            SmallRouting &R) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave < T) {
    int e;
    float w;
    select_token_regs(in, E, k, rsf, e, w);
    if (lane < k) {
      R.idx[wave * k + lane] = e;
      R.w[wave * k + lane] = w;
    }
  }
  __syncthreads();
  const int n = T * k;
  if (wave == 0) {
    const bool valid = lane < n;
    const int key = valid ? R.idx[lane] : 0x7fffffff;
    int lt = 0, eq_before = 0;
    uint64_t m_lt = 0;
    for (int b = 0; b < n; ++b) {
      const int kb = __builtin_amdgcn_readlane(key, b);
      lt += kb < key;
      eq_before += kb == key && b < lane;
      m_lt |= (uint64_t)(kb < key) << b;
    }
    const bool start = valid && eq_before == 0;
    const uint64_t starts = __ballot(start);
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
      R.seg_begin[__popcll(starts)] = n;
    }
  }
  __syncthreads();
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
    for (int a = 0; a < n; ++a) c += R.idx[a] < e;
    o.offsets[e] = c;
  }
  for (int s = threadIdx.x; s < R.n_active; s += blockDim.x) o.active[s] = R.active[s];
  if (threadIdx.x == 0) *o.n_active = R.n_active;
}

}  // namespace coli
