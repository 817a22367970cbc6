// Expert selection of one token by one wave: the exact float32 sigmoid of
// the router logits, the biased key, noaux_tc top-k with n_group = 1 and the
// renormalised weights.
//
// Source: "colibri engine teardown" page, "Three key engineering decisions",
// item 1 -- sigmoid router with noaux_tc top-k (n_group = 1) and a
// routed_scaling_factor; router and bias stay float32.  The float32 program
// is exact (IEEE operations in a fixed order, correctly rounded division, no
// contraction) so expert choices are reproducible bit for bit.
#pragma once

#include "internal.h"
#include "wave.h"

namespace coli {

__device__ __forceinline__ float pow2i(int n) { return __int_as_float((n + 127) << 23); }

// e^y in float32: y = n ln2 + r, n = rint(y log2e), r by two fma steps with
// ln 2 split into a 16-bit head (exact products n * head) and its float tail;
// e^r = sum_{i<=7} r^i / i! in Horner form; scale by 2^n through the exponent
// field, in two steps outside the normal range.
__device__ __forceinline__ float exp_spec(float y) {
  const float kLog2e = 0x1.715476p+0f;
  const float kLn2Hi = 0x1.62e4p-1f;
  const float kLn2Lo = 0x1.7f7d1cp-20f;
  const float kInv2 = 0x1p-1f;
  const float kInv6 = 0x1.555556p-3f;
  const float kInv24 = 0x1.555556p-5f;
  const float kInv120 = 0x1.111112p-7f;
  const float kInv720 = 0x1.6c16c2p-10f;
  const float kInv5040 = 0x1.a01a02p-13f;
  if (y != y) return y;
  if (y > 89.0f) return __int_as_float(0x7f800000);
  if (y < -104.0f) return 0.0f;
  const float n = __builtin_rintf(y * kLog2e);
  float r = __builtin_fmaf(-n, kLn2Hi, y);
  r = __builtin_fmaf(-n, kLn2Lo, r);
  float p = kInv5040;
  p = __builtin_fmaf(p, r, kInv720);
  p = __builtin_fmaf(p, r, kInv120);
  p = __builtin_fmaf(p, r, kInv24);
  p = __builtin_fmaf(p, r, kInv6);
  p = __builtin_fmaf(p, r, kInv2);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  const int ni = (int)n;
  if (ni > 127) return (p * pow2i(127)) * pow2i(ni - 127);
  if (ni < -126) return (p * pow2i(ni + 64)) * pow2i(-64);
  return p * pow2i(ni);
}

__device__ __forceinline__ float sigmoid_spec(float z) { return 1.0f / (1.0f + exp_spec(-z)); }

// ---------------------------------------------------------------------------
// Selection.  The float key c = s + b is mapped to an unsigned integer with
// the same order (c is never -0: s >= +0); ties on c go to the lower expert
// index.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ordered_bits(float c) {
  const uint32_t u = __float_as_uint(c);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One wave selects the experts of one token (logits row l[0..E)): sigmoid
// scores, biased keys c = s + b, then the k best under (c desc, e asc), then
// den = sum of the selected s in slot order and w_j = (s_j / den) * rsf.
// Lane j < k returns slot j in (e_out, w_out).
//
// Top-k by ballots: with the order-preserving integer image u(c), the k-th
// largest value th is found bit by bit from the top (th grows while at least
// k keys are >= th | bit), 32 compare + popcount steps on SGPR lane masks.
// Keys above th are taken, and of the keys equal to th the lowest expert
// indices fill the remaining places.  The k chosen keys are then ranked among
// themselves (slot = number of chosen keys that beat it) through LDS.
template <int R>
__device__ __forceinline__ void select_token_r(const float *__restrict__ l, const float *__restrict__ bias, int E,
                                               int k, float rsf, int &e_out, float &w_out, uint32_t *lds_key,
                                               int32_t *lds_e, float *lds_s) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt = (1ull << lane) - 1;
  float s[R], lv[R], bv[R];
  uint32_t u[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int e = min(lane + 64 * r, E - 1);
    lv[r] = l[e];
    bv[r] = bias ? bias[e] : 0.0f;
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool valid = lane + 64 * r < E;
    s[r] = valid ? sigmoid_spec(lv[r]) : 0.0f;
    u[r] = valid ? ordered_bits(s[r] + bv[r]) : 0u;  // invalid keys sort below every real key
  }
  // threshold: the k-th largest u
  uint32_t th = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = th | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) cnt += __popcll(__ballot(u[r] >= cand));
    if (cnt >= k) th = cand;
  }
  // keys above th, then the lowest-index keys equal to th
  int n_above = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) n_above += __popcll(__ballot(u[r] > th && lane + 64 * r < E));
  const int need = k - n_above;
  int eq_before = 0, sel_before = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool valid = lane + 64 * r < E;
    const uint64_t eq = __ballot(valid && u[r] == th);
    const bool pick_eq = valid && u[r] == th && eq_before + __popcll(eq & lt) < need;
    const bool pick = (valid && u[r] > th) || pick_eq;
    const uint64_t sel = __ballot(pick);
    if (pick) {
      const int pos = sel_before + __popcll(sel & lt);  // position in expert order
      lds_key[pos] = u[r];
      lds_e[pos] = lane + 64 * r;
      lds_s[pos] = s[r];
    }
    eq_before += __popcll(eq);
    sel_before += __popcll(sel);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // slot of chosen entry i: how many chosen entries beat it
  int my_slot = k, my_e = 0;
  float my_s = 0.0f;
  if (lane < k) {
    const uint32_t ku = lds_key[lane];
    my_e = lds_e[lane];
    my_s = lds_s[lane];
    int beat = 0;
    for (int j = 0; j < k; ++j) {
      const uint32_t kj = lds_key[j];
      beat += (kj > ku) || (kj == ku && lds_e[j] < my_e);
    }
    my_slot = beat;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lane < k) {
    lds_e[k + my_slot] = my_e;
    lds_s[k + my_slot] = my_s;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // den = ((s_0 + s_1) + s_2) + ... in slot order, identical in every lane
  float den = 0.0f;
  for (int j = 0; j < k; ++j) den = den + lds_s[k + j];
  e_out = lane < k ? lds_e[k + lane] : 0;
  w_out = lane < k ? (lds_s[k + lane] / den) * rsf : 0.0f;
}

// Per-wave LDS scratch of the selection: keys, experts and scores of the k
// chosen entries in expert order, then in slot order.
struct SelectScratch {
  uint32_t key[kMaxTopK];
  int32_t e[2 * kMaxTopK];
  float s[2 * kMaxTopK];
};

__device__ __forceinline__ void select_token(const float *__restrict__ l, const float *__restrict__ bias, int E,
                                             int k, float rsf, int &e_out, float &w_out, SelectScratch &sc) {
  if (E <= 64)
    select_token_r<1>(l, bias, E, k, rsf, e_out, w_out, sc.key, sc.e, sc.s);
  else if (E <= 128)
    select_token_r<2>(l, bias, E, k, rsf, e_out, w_out, sc.key, sc.e, sc.s);
  else if (E <= 256)
    select_token_r<4>(l, bias, E, k, rsf, e_out, w_out, sc.key, sc.e, sc.s);
  else
    select_token_r<8>(l, bias, E, k, rsf, e_out, w_out, sc.key, sc.e, sc.s);
}

}  // namespace coli
