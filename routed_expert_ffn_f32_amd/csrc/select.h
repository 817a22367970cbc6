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
//
// Routing limits (lim): the tournament runs k_use rounds; lane j also keeps
// cum_j (den before its slot was added), from which the kept prefix and
// its denominator follow; dropped slots j < k return (-1, 0).
__device__ __forceinline__ void select_token_regs(const SelectInput &in, int E, int k, float rsf,
                                                  const RouteLimits &lim, int &e_out, float &w_out) {
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
  float den = 0.0f, my_s = 0.0f, my_cum = 0.0f;
  int my_e = 0;
  for (int j = 0; j < lim.k_use; ++j) {
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
    if (lane == j) {
      my_e = e_win;
      my_s = s_win;
      my_cum = den;
    }
    den = den + s_win;
    if (lane == wl) {
#pragma unroll
      for (int i = 0; i < kSelMaxKeys; ++i)
        if (i == bi) u[i] = 0u;
    }
  }
  bool keep = lane < lim.k_use;
  if (lim.top_p < 1.0f) {
    const float thr = lim.top_p * den;
    keep = keep && (lane == 0 || my_cum < thr);
    const int m = __popcll(__ballot(keep));
    // cum_m: the same float32 sum as den after round m - 1
    den = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_cum + my_s), m - 1));
  }
  e_out = lane < k ? (keep ? my_e : -1) : 0;
  w_out = keep ? (my_s / den) * rsf : 0.0f;
}

// ---------------------------------------------------------------------------
// Selection spread over several waves (small batches, one block).
//
// Phase A: wave p of a token's WT waves takes experts [p c, p c + c) (c =
// ceil(E / WT)), lane l holding expert p c + l + 64 i, finds the k-th largest
// key by a bitwise search over ballot counts and writes the part's k best
// under (key desc, expert asc) to LDS in ascending expert order.  The
// token's k best overall are among these WT k candidates.  Phase B: one wave
// holds the candidates, one per lane (ascending expert order, so the lowest
// lane is the lowest expert), takes the k best of them the same way, ranks
// them into slot order and sums den in slot order.
// ---------------------------------------------------------------------------

// Phase A inputs: this lane's logits and biases of experts
// e_lo + lane + 64 i, i < kSelMaxKeys (zeros past ne); loaded early.
__device__ __forceinline__ void select_part_load(const float *__restrict__ l, const float *__restrict__ bias,
                                                 int e_lo, int ne, SelectInput &in) {
  // buffer loads (reads past ne give zeros), only for the keys that exist
  const int lane = threadIdx.x & 63, nk = (ne + 63) >> 6;
  const Rsrc rl = make_rsrc(l + e_lo, (uint32_t)ne * 4);
  const Rsrc rb = make_rsrc(bias ? bias + e_lo : l, bias ? (uint32_t)ne * 4 : 0u);
#pragma unroll
  for (int i = 0; i < kSelMaxKeys; ++i) {
    in.l[i] = in.b[i] = 0.0f;
    if (i < nk) {  // uniform
      const uint32_t off = (uint32_t)(lane + 64 * i) * 4;
      in.l[i] = bloadf(rl, off, 0);
      in.b[i] = bloadf(rb, off, 0);
    }
  }
}

// The k-th largest of the keys u[] over the wave (NK per lane; absent keys
// 0): the largest th with #{u >= th} >= k, found bit by bit from the top.
template <int NK>
__device__ __forceinline__ uint32_t wave_kth_key(const uint32_t (&u)[NK], int k) {
  uint32_t th = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = th | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < NK; ++i) cnt += __popcll(__ballot(u[i] >= cand));
    if (cnt >= k) th = cand;
  }
  return th;
}

// Positions, in ascending expert order (key i of lane l is expert
// l + 64 i), of the k keys that the order (key desc, expert asc) puts first:
// every key above the k-th largest, then the lowest experts among the keys
// equal to it.  pos[i] = -1 for keys not taken.
template <int NK>
__device__ __forceinline__ void wave_take_k(const uint32_t (&u)[NK], int k, uint32_t th, int (&pos)[NK]) {
  int n_above = 0;
#pragma unroll
  for (int i = 0; i < NK; ++i) n_above += __popcll(__ballot(u[i] > th));
  const int need = k - n_above;
  const int below = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));  // lanes under this one
  const uint64_t lt_mask = below == 0 ? 0ull : (~0ull >> (64 - below));
  int eq_before = 0, taken_before = 0;
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const uint64_t eq = __ballot(u[i] == th);
    const bool take = u[i] > th || (u[i] == th && eq_before + __popcll(eq & lt_mask) < need);
    const uint64_t tk = __ballot(take);
    pos[i] = take ? taken_before + __popcll(tk & lt_mask) : -1;
    eq_before += __popcll(eq);
    taken_before += __popcll(tk);
  }
}

// Phase A for experts [e_lo, e_lo + ne) of one token (inputs from
// select_part_load): the part's k best, in ascending expert order, into
// cu/ce/cs[0..k) (key image, expert, score).
template <int NK>
__device__ __forceinline__ void select_part(const SelectInput &in, int e_lo, int ne, int k, uint32_t *cu, int32_t *ce,
                                            float *cs) {
  const int lane = threadIdx.x & 63;
  uint32_t u[NK];
  float s[NK];
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const bool valid = lane + 64 * i < ne;
    s[i] = valid ? sigmoid_spec(in.l[i]) : 0.0f;
    u[i] = valid ? ordered_bits(s[i] + in.b[i]) : 0u;
  }
  const uint32_t th = wave_kth_key<NK>(u, k);
  int pos[NK];
  wave_take_k<NK>(u, k, th, pos);
#pragma unroll
  for (int i = 0; i < NK; ++i)
    if (pos[i] >= 0) {
      cu[pos[i]] = u[i];
      ce[pos[i]] = e_lo + lane + 64 * i;
      cs[pos[i]] = s[i];
    }
}

// LDS writes of this wave done and ordered before its later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Phase B: n <= 64 candidates (cu, ce, cs in LDS, ascending expert order)
// -> slot j (j < k) of the token in se[j], sw[j] = (s_j / den) * rsf with
// den = ((s_0 + s_1) + s_2) + ... in slot order, and slot_of[p] = the slot
// of the p-th kept expert in ascending expert order.  One wave: lane c
// holds candidate c and counts the candidates the order (key desc, expert
// asc) puts before it -- its slot when that count is below k_use (equal
// keys: the lower lane is the lower expert).  Routing limits as in
// select_token_regs: slots past the kept prefix get (-1, 0).  Returns the
// number of kept slots (uniform); se, sw and slot_of are readable by the
// calling wave on return.  `scratch` holds kMaxTopK words of LDS.
__device__ __forceinline__ int select_merge(const uint32_t *cu, const int32_t *ce, const float *cs, int n, int k,
                                            float rsf, const RouteLimits &lim, int32_t *se, float *sw,
                                            uint32_t *scratch, int32_t *slot_of) {
  const int lane = threadIdx.x & 63;
  const bool valid = lane < n;
  const uint32_t u = valid ? cu[lane] : 0u;
  const int e = valid ? ce[lane] : 0;
  const float sv = valid ? cs[lane] : 0.0f;
  // every lane reads the candidate keys from LDS (same addresses in all
  // lanes: broadcasts), four at a time
  int rank = 0;
  const uint4 *cu4 = reinterpret_cast<const uint4 *>(cu);
  for (int j4 = 0; j4 < n; j4 += 4) {
    const uint4 q = cu4[j4 >> 2];
    const uint32_t uj[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j4 + i;
      rank += j < n && (uj[i] > u || (uj[i] == u && j < lane));
    }
  }
  const bool win = valid && rank < lim.k_use;
  const int below = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const uint64_t lt_mask = below == 0 ? 0ull : (~0ull >> (64 - below));
  float *ss = reinterpret_cast<float *>(scratch);  // scores in slot order
  if (win) ss[rank] = sv;
  wave_lds_sync();
  float den = 0.0f, my_cum = 0.0f;
  for (int j = 0; j < lim.k_use; ++j) {
    if (j == rank) my_cum = den;
    den = den + ss[j];
  }
  bool keep = win;
  int m = lim.k_use;
  if (lim.top_p < 1.0f) {
    const float thr = lim.top_p * den;
    keep = win && (rank == 0 || my_cum < thr);
    m = __popcll(__ballot(keep));
    den = 0.0f;
    for (int j = 0; j < m; ++j) den = den + ss[j];
  }
  const uint64_t keeps = __ballot(keep);
  if (keep) {
    se[rank] = e;
    sw[rank] = (sv / den) * rsf;
    slot_of[__popcll(keeps & lt_mask)] = rank;
  }
  if (lane >= m && lane < k) {  // dropped slots
    se[lane] = -1;
    sw[lane] = 0.0f;
  }
  wave_lds_sync();  // se, sw, slot_of readable by the whole wave
  return m;
}

__device__ __forceinline__ void select_token(const float *__restrict__ l, const float *__restrict__ bias, int E,
                                             int k, float rsf, const RouteLimits &lim, int &e_out, float &w_out) {
  SelectInput in;
  select_load(l, bias, E, in);
  select_token_regs(in, E, k, rsf, lim, e_out, w_out);
}

}  // namespace coli
