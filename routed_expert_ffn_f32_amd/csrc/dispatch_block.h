// Stable counting sort of (token, slot) assignments by expert, as a device
// function run by one whole workgroup of kDispatchThreads threads.
//
// Source: cf-1.com Colibri article, section 3.3, colibri_forward step 3 --
// per-expert counts, a prefix sum into per-expert offsets, then a scatter of
// the tokens by expert id; section 2.2 shows the grouping on six tokens.
//
// Output (assignment a = t*k + j, n = T*k):
//   offsets[E+1]   exclusive prefix sum of the per-expert counts
//   sorted_ids[n]  assignments grouped by expert ascending, a ascending inside
//   inv[n]         position of assignment a in sorted_ids
//   active[E]      experts with at least one assignment, ascending
//   n_active[1]    how many
// A negative id is a dropped slot (run-time routing limits): it sorts as an
// extra key E after every expert, so the dropped assignments fill
// sorted_ids from offsets[E] on (a ascending) and offsets[E] counts the kept
// ones.
//
// Wave w owns a contiguous range of assignments.  Within a 64-assignment
// chunk, lanes with equal keys are found with ballots over the key bits; the
// rank of a lane among its equals is the popcount of the lower lanes of its
// match mask.  Pass 1 builds one histogram per wave in LDS; the workgroup
// then turns them into per-(wave, expert) start positions; pass 2 repeats
// the chunk walk and scatters.  Positions depend only on the data, so the
// result is identical on every run.
#pragma once

#include "internal.h"

namespace coli {

// Lanes of this wave holding the same (valid) key as the calling lane.
__device__ __forceinline__ uint64_t match_mask(int key, bool valid, int key_bits) {
  uint64_t m = __ballot(valid);
  for (int b = 0; b < key_bits; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t ones = __ballot(valid && bit);
    m &= bit ? ones : ~ones;
  }
  return m;
}

// The key of an id: the id, a negative one E (dropped), one past the
// experts clamped to E - 1 (unspecified but in-bounds result).
__device__ __forceinline__ int dispatch_key(int id, int E) { return id < 0 ? E : min(id, E - 1); }

// Exclusive scan of per-key counts over a block of KW waves (thread t holds
// the count of key t; threads past the keys hold 0; NK = E + 1 <= 64 KW).
// Returns key t's start, offsets[t].  With `write`, also stores offsets[0..E]
// (offsets[E] = the kept assignments), the active experts in ascending
// order and their number.  Ends with the block synchronised.
template <int KW>
__device__ __forceinline__ int key_scan(int count, int E, bool write, int32_t *__restrict__ offsets,
                                        int32_t *__restrict__ active, int32_t *__restrict__ n_active,
                                        int32_t *wave_sum, int32_t *wave_act) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int flag = (tid < E && count > 0) ? 1 : 0;  // the dropped key is no active expert
  int incl = count, incl_f = flag;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d), vf = __shfl_up(incl_f, d);
    if (lane >= d) {
      incl += v;
      incl_f += vf;
    }
  }
  if (lane == 63) {
    wave_sum[wave] = incl;
    wave_act[wave] = incl_f;
  }
  __syncthreads();
  int before = 0, before_f = 0;
  for (int w = 0; w < wave; ++w) {
    before += wave_sum[w];
    before_f += wave_act[w];
  }
  const int start = before + incl - count;
  const int act_pos = before_f + incl_f - flag;
  if (write) {
    if (tid <= E) offsets[tid] = start;
    if (flag) active[act_pos] = tid;
    if (tid == E) *n_active = act_pos;
  }
  __syncthreads();
  return start;
}

// `idx` may point to global or shared memory.
__device__ __forceinline__ void dispatch_block(const int32_t *idx, int n, int E, int32_t *__restrict__ offsets,
                                               int32_t *__restrict__ sorted_ids, int32_t *__restrict__ inv,
                                               int32_t *__restrict__ active, int32_t *__restrict__ n_active) {
  constexpr int kWaves = kDispatchThreads / kWave;      // 16
  static_assert(kMaxExperts < kDispatchThreads, "one thread per key");
  __shared__ int32_t hist[kWaves][kMaxExperts + 1];     // counts, then start positions (key E: dropped)
  __shared__ int32_t wave_sum[kWaves];
  __shared__ int32_t wave_act[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NK = E + 1;  // keys
  int key_bits = 0;
  while ((1 << key_bits) < NK) ++key_bits;

  for (int e = lane; e < NK; e += 64) hist[wave][e] = 0;
  const int per_wave = ((n + kWaves - 1) / kWaves + 63) & ~63;
  const int lo = min(n, wave * per_wave), hi = min(n, lo + per_wave);
  __syncthreads();

  // pass 1: per-wave histograms
  for (int base = lo; base < hi; base += 64) {
    const int a = base + lane;
    const bool valid = a < hi;
    const int key = valid ? dispatch_key(idx[a], E) : 0;
    const uint64_t m = match_mask(key, valid, key_bits);
    const bool leader = valid && ((m & ((1ull << lane) - 1)) == 0);
    if (leader) hist[wave][key] += __popcll(m);
  }
  __syncthreads();

  // per key: start of each wave's share (exclusive over waves), total count
  int count = 0;
  if (tid < NK) {
    for (int w = 0; w < kWaves; ++w) {
      const int v = hist[w][tid];
      hist[w][tid] = count;
      count += v;
    }
  }
  const int start = key_scan<kWaves>(count, E, true, offsets, active, n_active, wave_sum, wave_act);
  if (tid < NK)
    for (int w = 0; w < kWaves; ++w) hist[w][tid] += start;
  __syncthreads();

  // pass 2: scatter; equal keys of a chunk take consecutive positions in lane
  // order, chunks in order, waves in order
  for (int base = lo; base < hi; base += 64) {
    const int a = base + lane;
    const bool valid = a < hi;
    const int key = valid ? dispatch_key(idx[a], E) : 0;
    const uint64_t m = match_mask(key, valid, key_bits);
    const int rank = __popcll(m & ((1ull << lane) - 1));
    const int pos = hist[wave][key] + rank;
    if (valid) {
      sorted_ids[pos] = a;
      inv[a] = pos;
    }
    // every lane has read its start before the leader moves it on
    __builtin_amdgcn_wave_barrier();
    if (valid && rank == 0) hist[wave][key] = pos + __popcll(m);
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace coli

namespace coli {

// ---------------------------------------------------------------------------
// The same sort over many workgroups, for large batches: blocks of
// kDispatchThreads threads, block b taking assignments [b B, (b + 1) B),
// B = kDispatchThreads (one per thread, wave w the 64 from b B + 64 w).
//  - count launch: block b writes the histogram of its keys, cnt[b][0..E];
//  - scatter launch: every block sums the histograms (key e: the blocks
//    before it, and all of them), scans the totals over the keys into the
//    offsets (block 0 stores them with the active list), and scatters its
//    assignments: positions offsets[e] + (key e in earlier blocks) + (key e
//    in earlier waves of the block) + (equal keys in lower lanes).
// Every position is the one the one-workgroup sort gives.
// ---------------------------------------------------------------------------
constexpr int kDispatchPerBlock = kDispatchThreads;

__device__ __forceinline__ void dispatch_count_block(const int32_t *__restrict__ idx, int n, int E,
                                                     int32_t *__restrict__ cnt) {
  __shared__ int32_t c[kMaxExperts + 1];
  const int tid = threadIdx.x, NK = E + 1;
  const int a = blockIdx.x * kDispatchPerBlock + tid;
  const int key = a < n ? dispatch_key(idx[a], E) : -1;
  for (int e = tid; e < NK; e += blockDim.x) c[e] = 0;
  __syncthreads();
  if (key >= 0) atomicAdd(&c[key], 1);
  __syncthreads();
  for (int e = tid; e < NK; e += blockDim.x) cnt[(size_t)blockIdx.x * NK + e] = c[e];
}

__device__ __forceinline__ void dispatch_scatter_block(const int32_t *__restrict__ idx, int n, int E,
                                                       const int32_t *__restrict__ cnt, int32_t *__restrict__ offsets,
                                                       int32_t *__restrict__ sorted_ids, int32_t *__restrict__ inv,
                                                       int32_t *__restrict__ active, int32_t *__restrict__ n_active) {
  constexpr int kWaves = kDispatchThreads / kWave;
  static_assert(kMaxExperts < kDispatchThreads, "one thread per key");
  __shared__ int32_t whist[kWaves][kMaxExperts + 1];  // per-wave counts, then start positions
  __shared__ int32_t wave_sum[kWaves];
  __shared__ int32_t wave_act[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NK = E + 1, nb = (int)gridDim.x, b = (int)blockIdx.x;
  int key_bits = 0;
  while ((1 << key_bits) < NK) ++key_bits;
  const int a = b * kDispatchPerBlock + tid;
  const bool valid = a < n;
  const int key = valid ? dispatch_key(idx[a], E) : 0;
  // key tid over the blocks: before this one, and in all
  int below = 0, total = 0;
  if (tid < NK) {
    constexpr int kU = 8;
    int bb = 0;
    for (; bb + kU <= nb; bb += kU) {
      int v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) v[u] = cnt[(size_t)(bb + u) * NK + tid];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        below += bb + u < b ? v[u] : 0;
        total += v[u];
      }
    }
    for (; bb < nb; ++bb) {
      const int v = cnt[(size_t)bb * NK + tid];
      below += bb < b ? v : 0;
      total += v;
    }
  }
  for (int i = tid; i < kWaves * NK; i += blockDim.x) whist[i / NK][i % NK] = 0;
  const int start = key_scan<kWaves>(total, E, b == 0, offsets, active, n_active, wave_sum, wave_act);
  // this wave's chunk: counts by key (one leader per key), ranks
  const uint64_t m = match_mask(key, valid, key_bits);
  const int rank = __popcll(m & ((1ull << lane) - 1));
  if (valid && rank == 0) whist[wave][key] = __popcll(m);
  __syncthreads();
  if (tid < NK) {
    int p = start + below;
    for (int w = 0; w < kWaves; ++w) {
      const int v = whist[w][tid];
      whist[w][tid] = p;
      p += v;
    }
  }
  __syncthreads();
  if (valid) {
    const int pos = whist[wave][key] + rank;
    sorted_ids[pos] = a;
    inv[a] = pos;
  }
}

}  // namespace coli
