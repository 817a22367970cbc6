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

constexpr int kSelMaxKeys = kMaxExperts / kWave;  // keys per lane

// The logits and selection biases of one token, lane l holding experts
// l + 64 i (i < kSelMaxKeys; zeros past E).  Issued early by callers that
// want the loads in flight while they do other work.
struct SelectInput {
  float l[kSelMaxKeys], b[kSelMaxKeys];
};

__device__ __forceinline__ void select_load(const float *__restrict__ l, const float *__restrict__ bias, int E,
                                            SelectInput &in) {
  const int lane = threadIdx.x & 63, nk = (E + 63) >> 6;
  const Rsrc rl = make_rsrc(l, (uint32_t)E * 4), rb = make_rsrc(bias, bias ? (uint32_t)E * 4 : 0u);
#pragma unroll
  for (int i = 0; i < kSelMaxKeys; ++i) {
    if (i >= nk) break;  // uniform
    const uint32_t off = (uint32_t)(lane + 64 * i) * 4;
    in.l[i] = bloadf(rl, off, 0);
    in.b[i] = bloadf(rb, off, 0);  // no bias: zeros
  }
}

// Largest unsigned value over the 64 lanes, returned uniformly.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)dpp_i<kDppQuadXor1>((int)v));
  v = max(v, (uint32_t)dpp_i<kDppQuadXor2>((int)v));
  v = max(v, (uint32_t)dpp_i<kDppRowRor4>((int)v));
  v = max(v, (uint32_t)dpp_i<kDppRowRor8>((int)v));           // every lane: its row's max
  v = max(v, (uint32_t)dpp_i<kDppRowBcast15, 0xA>((int)v));   // rows 1, 3 take rows 0, 2
  v = max(v, (uint32_t)dpp_i<kDppRowBcast31, 0xC>((int)v));   // rows 2, 3 take lane 31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// One wave selects the experts of one token: sigmoid scores s, biased keys
// c = s + b, then the k best under (c desc, e asc), then den = sum of the
// selected s in slot order and w_j = (s_j / den) * rsf.  Lane j < k returns
// slot j in (e_out, w_out).
//
// Tournament on the order-preserving integer image u(c): every lane keeps
// its best remaining key (ties to its lower expert, e = lane + 64 i rises
// with i), round j takes the largest over the lanes (wave max; ties to the
// lowest expert among the lanes holding it) and removes it from its lane, so
// the rounds yield the slots in rank order.  Every real key is >= 0x00800000
// (the image of -FLT_MAX), removed or invalid keys count as 0.
__device__ __forceinline__ void select_token_regs(const SelectInput &in, int E, int k, float rsf, int &e_out,
                                                  float &w_out) {
  const int lane = threadIdx.x & 63, nk = (E + 63) >> 6;
  float s[kSelMaxKeys];
  uint32_t u[kSelMaxKeys];
#pragma unroll
  for (int i = 0; i < kSelMaxKeys; ++i) {
    s[i] = 0.0f;
    u[i] = 0u;
    if (i >= nk) continue;  // uniform
    const bool valid = lane + 64 * i < E;
    s[i] = valid ? sigmoid_spec(in.l[i]) : 0.0f;
    u[i] = valid ? ordered_bits(s[i] + in.b[i]) : 0u;
  }
  float den = 0.0f, my_s = 0.0f;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t bu = 0u;
    int bi = 0;
    float bs = 0.0f;
#pragma unroll
    for (int i = 0; i < kSelMaxKeys; ++i)
      if (i < nk && u[i] > bu) {  // strict: the lower expert of equal keys stays
        bu = u[i];
        bi = i;
        bs = s[i];
      }
    const uint32_t m = wave_max_u32(bu);
    uint64_t cand = __ballot(bu == m);
    int wl = __builtin_ctzll(cand);
    int e_win = __builtin_amdgcn_readlane(lane + 64 * bi, wl);
    if (__popcll(cand) > 1) {  // equal keys on several lanes: the lowest expert wins
      cand &= cand - 1;
      while (cand) {
        const int l2 = __builtin_ctzll(cand);
        const int e2 = __builtin_amdgcn_readlane(lane + 64 * bi, l2);
        if (e2 < e_win) {
          e_win = e2;
          wl = l2;
        }
        cand &= cand - 1;
      }
    }
    const float s_win = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bs), wl));
    den = den + s_win;
    if (lane == j) {
      my_e = e_win;
      my_s = s_win;
    }
    if (lane == wl) {
#pragma unroll
      for (int i = 0; i < kSelMaxKeys; ++i)
        if (i == bi) u[i] = 0u;
    }
  }
  e_out = lane < k ? my_e : 0;
  w_out = lane < k ? (my_s / den) * rsf : 0.0f;
}

__device__ __forceinline__ void select_token(const float *__restrict__ l, const float *__restrict__ bias, int E,
                                             int k, float rsf, int &e_out, float &w_out) {
  SelectInput in;
  select_load(l, bias, E, in);
  select_token_regs(in, E, k, rsf, e_out, w_out);
}

}  // namespace coli
