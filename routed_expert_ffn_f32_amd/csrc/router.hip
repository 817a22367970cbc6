// Router kernels: float32 logits, sigmoid scores with a selection bias,
// noaux_tc top-k with n_group = 1, renormalised weights x routed scaling.
//
// Source: "colibri engine teardown" page, "Three key engineering decisions",
// item 1 -- the engine's router is a sigmoid with noaux_tc top-k (n_group = 1)
// and a routed_scaling_factor, and router and bias stay float32.  The exact
// float32 program below (fixed summation order, exp by Cody-Waite reduction
// and a degree-7 Taylor polynomial, IEEE division) makes expert choices
// reproducible bit for bit: near-ties between the k-th and (k+1)-th key are
// decided identically on every run and by any conforming implementation of
// the same program.
//
// Compiled with -ffp-contract=off and correctly rounded float32 division, so
// the only fused multiply-adds are the explicit __builtin_fmaf calls.
#include "internal.h"

namespace coli {
namespace {

__device__ __forceinline__ float pow2i(int n) { return __int_as_float((n + 127) << 23); }

// e^y in float32: y = n ln2 + r, n = rint(y log2e), r by two fma steps with
// ln 2 split into a 16-bit head (exact products n * head) and its float tail;
// e^r = sum_{i<=7} r^i / i! in Horner form; scale by 2^n through the exponent
// field, in two steps outside the normal range.
__device__ float exp_spec(float y) {
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

__global__ __launch_bounds__(256) void router_transpose_kernel(const float *__restrict__ wr,
                                                               float *__restrict__ wrT, int h, int E) {
  __shared__ float tile[32][33];
  const int e0 = blockIdx.x * 32, i0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int r = ty; r < 32; r += 8) {
    const int i = i0 + r, e = e0 + tx;
    tile[r][tx] = (i < h && e < E) ? wr[(size_t)i * E + e] : 0.0f;
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int e = e0 + r, i = i0 + tx;
    if (e < E && i < h) wrT[(size_t)e * h + i] = tile[tx][r];
  }
}

// One wave computes TPW tokens x EPW experts.  Lane l owns the chain of
// elements l + 64m; after the chains, the xor butterfly leaves the full sum
// in every lane.
template <int EPW, int TPW>
__global__ __launch_bounds__(256) void router_logits_kernel(const float *__restrict__ x,
                                                            const float *__restrict__ wrT, int T, int h,
                                                            int E, float *__restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int e0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * EPW;
  const int t0 = blockIdx.y * TPW;
  if (e0 >= E) return;  // uniform over the wave
  const int M = h >> 6;
  const float *xp[TPW];
  const float *wp[EPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) xp[t] = x + (size_t)min(t0 + t, T - 1) * h + lane;
#pragma unroll
  for (int e = 0; e < EPW; ++e) wp[e] = wrT + (size_t)min(e0 + e, E - 1) * h + lane;
  float acc[TPW][EPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int e = 0; e < EPW; ++e) acc[t][e] = 0.0f;
  for (int m = 0; m < M; ++m) {
    float xv[TPW], wv[EPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) xv[t] = xp[t][m * 64];
#pragma unroll
    for (int e = 0; e < EPW; ++e) wv[e] = wp[e][m * 64];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int e = 0; e < EPW; ++e) acc[t][e] = __builtin_fmaf(xv[t], wv[e], acc[t][e]);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1)
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int e = 0; e < EPW; ++e) acc[t][e] = acc[t][e] + __shfl_xor(acc[t][e], d);
  if (lane == 0) {
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int e = 0; e < EPW; ++e)
        if (t0 + t < T && e0 + e < E) logits[(size_t)(t0 + t) * E + e0 + e] = acc[t][e];
  }
}

// (c, e) beats (oc, oe) when c is larger, or equal with a smaller index.
__device__ __forceinline__ bool beats(float c, int e, float oc, int oe) {
  return c > oc || (c == oc && e < oe);
}

// One wave per token.  Lane l holds experts l + 64r.  k rounds of a wave-wide
// arg-max under (key desc, index asc); the winner's lane marks it taken.
__global__ __launch_bounds__(256) void router_select_kernel(const float *__restrict__ logits,
                                                            const float *__restrict__ bias, int T, int E,
                                                            int k, float rsf, int32_t *__restrict__ idx,
                                                            float *__restrict__ wout) {
  constexpr int R = kMaxExperts / kWave;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float s[R], c[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int e = lane + 64 * r;
    if (e < E) {
      s[r] = sigmoid_spec(logits[(size_t)t * E + e]);
      c[r] = s[r] + (bias ? bias[e] : 0.0f);
    } else {
      s[r] = 0.0f;
      c[r] = -__int_as_float(0x7f800000);
    }
  }
  uint32_t taken = 0;
  int my_e = 0;
  float my_s = 0.0f;
  for (int j = 0; j < k; ++j) {
    float bc = -__int_as_float(0x7f800000), bs = 0.0f;
    int be = 0x7fffffff;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int e = lane + 64 * r;
      if (e < E && !((taken >> r) & 1u) && beats(c[r], e, bc, be)) {
        bc = c[r];
        be = e;
        bs = s[r];
      }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      const float oc = __shfl_xor(bc, d);
      const int oe = __shfl_xor(be, d);
      const float os = __shfl_xor(bs, d);
      if (beats(oc, oe, bc, be)) {
        bc = oc;
        be = oe;
        bs = os;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == j) {
      my_e = be;
      my_s = bs;
    }
  }
  // den = ((s_0 + s_1) + s_2) + ... in slot order, identical in every lane
  float den = 0.0f;
  for (int j = 0; j < k; ++j) den = den + __shfl(my_s, j);
  if (lane < k) {
    idx[(size_t)t * k + lane] = my_e;
    wout[(size_t)t * k + lane] = (my_s / den) * rsf;
  }
}

}  // namespace

hipError_t launch_router_transpose(const float *wr, float *wrT, int h, int E, hipStream_t s) {
  dim3 grid((E + 31) / 32, (h + 31) / 32);
  router_transpose_kernel<<<grid, 256, 0, s>>>(wr, wrT, h, E);
  return hipGetLastError();
}

hipError_t launch_router_logits(const float *x, const float *wrT, int T, int h, int E, float *logits,
                                hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (T < 4) {
    dim3 grid((E + 3) / 4, T);
    router_logits_kernel<1, 1><<<grid, 256, 0, s>>>(x, wrT, T, h, E, logits);
  } else if (T < 64) {
    dim3 grid((E + 7) / 8, (T + 3) / 4);
    router_logits_kernel<2, 4><<<grid, 256, 0, s>>>(x, wrT, T, h, E, logits);
  } else {
    dim3 grid((E + 15) / 16, (T + 3) / 4);
    router_logits_kernel<4, 4><<<grid, 256, 0, s>>>(x, wrT, T, h, E, logits);
  }
  return hipGetLastError();
}

hipError_t launch_router_select(const float *logits, const float *bias, int T, int E, int k, float rsf,
                                int32_t *idx, float *w, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  router_select_kernel<<<(T + 3) / 4, 256, 0, s>>>(logits, bias, T, E, k, rsf, idx, w);
  return hipGetLastError();
}

}  // namespace coli
