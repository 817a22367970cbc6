// Router logits of a tile of (token, expert) pairs by one wave, as an exact
// float32 program.
//
// Source: "colibri engine teardown" page, "Three key engineering decisions",
// item 1 -- the router stays float32.  The summation order is fixed so that
// the expert choice that follows is reproducible bit for bit: lane l of the
// wave owning (t, e) keeps p_l = fma(x[l + 64m], w[l + 64m], p_l) over m
// ascending, then the 64 partials meet in an xor butterfly (32, 16, ..., 1).
// The router is read from its lane-permuted copy
// wrP[e][b][l][i] = wr[l + 64(4b + i)][e], so a lane's four consecutive chain
// elements come as one float4.
#pragma once

#include "internal.h"

namespace coli {

// Logits.  One wave computes TPW tokens x EPW experts.  Lane l owns the chain
// of elements l + 64m, m ascending; the xor butterfly (32, 16, ..., 1) then
// leaves the full sum in every lane.
template <int EPW, int TPW>
__device__ __forceinline__ void logits_tile(const float *__restrict__ x, const float *__restrict__ wrP, int T,
                                            int h, int E, int t0, int e0, float *__restrict__ logits) {
  // blocks of 4 chain steps per float4; CH blocks are loaded before any is used
  constexpr int CH = (EPW * TPW <= 2) ? 8 : 2;
  const int lane = threadIdx.x & 63;
  const int M = h >> 6, MB = (M + 3) >> 2, MBfull = M >> 2;
  const float *xp[TPW];
  const float4 *wp[EPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) xp[t] = x + (size_t)min(t0 + t, T - 1) * h + lane;
#pragma unroll
  for (int e = 0; e < EPW; ++e)
    wp[e] = reinterpret_cast<const float4 *>(wrP) + ((size_t)min(e0 + e, E - 1) * MB) * 64 + lane;
  float acc[TPW][EPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int e = 0; e < EPW; ++e) acc[t][e] = 0.0f;
  int b0 = 0;
  for (; b0 + CH <= MBfull; b0 += CH) {
    float4 wv[CH][EPW];
    float xv[CH][4][TPW];
#pragma unroll
    for (int u = 0; u < CH; ++u)
#pragma unroll
      for (int e = 0; e < EPW; ++e) wv[u][e] = wp[e][(size_t)(b0 + u) * 64];
#pragma unroll
    for (int u = 0; u < CH; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < TPW; ++t) xv[u][i][t] = xp[t][(4 * (b0 + u) + i) * 64];
#pragma unroll
    for (int u = 0; u < CH; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
          for (int e = 0; e < EPW; ++e) {
            const float w = i == 0 ? wv[u][e].x : i == 1 ? wv[u][e].y : i == 2 ? wv[u][e].z : wv[u][e].w;
            acc[t][e] = __builtin_fmaf(xv[u][i][t], w, acc[t][e]);
          }
  }
  // remaining chain steps one at a time, in order
  for (int m = 4 * b0; m < M; ++m) {
    const int b = m >> 2, i = m & 3;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const float xv = xp[t][m * 64];
#pragma unroll
      for (int e = 0; e < EPW; ++e) {
        const float *w4 = reinterpret_cast<const float *>(wp[e] + (size_t)b * 64);
        acc[t][e] = __builtin_fmaf(xv, w4[i], acc[t][e]);
      }
    }
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

// One (token, expert) logit by one wave, the same float32 program as
// logits_tile: the first PRE float4 blocks of this lane's chain come from
// registers (wv, loaded early by the caller from wp; blocks past the chain
// are never added), the rest from wp; the
// token's row is xrow (LDS).  Returns the sum in every lane.
template <int PRE>
__device__ __forceinline__ float logit_chain(const float4 (&wv)[PRE], const float4 *__restrict__ wp,
                                             const float *xrow, int h) {
  const int lane = threadIdx.x & 63;
  const int M = h >> 6, MB = (M + 3) >> 2;
  float acc = 0.0f;
#pragma unroll
  for (int b = 0; b < PRE; ++b) {
    const float w[4] = {wv[b].x, wv[b].y, wv[b].z, wv[b].w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * b + i < M) acc = __builtin_fmaf(xrow[lane + 64 * (4 * b + i)], w[i], acc);
  }
  for (int b = PRE; b < MB; ++b) {
    const float4 v = wp[(size_t)b * 64];
    const float w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * b + i < M) acc = __builtin_fmaf(xrow[lane + 64 * (4 * b + i)], w[i], acc);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) acc = acc + __shfl_xor(acc, d);
  return acc;
}

// One token, one expert per wave (lane l of the wave owning expert e): every
// load of the chain (MB float4 blocks of the permuted router, the token's
// h/64 values for this lane) is issued before the first fma, so the wave
// costs one memory round trip; the arithmetic is logits_tile's, element for
// element.  Returns the logit in every lane.
template <int MB>
__device__ __forceinline__ float logit_t1(const float *__restrict__ x, const float *__restrict__ wrP, int e) {
  constexpr int M = 4 * MB;  // chain length h / 64
  const int lane = threadIdx.x & 63;
  const float4 *wp = reinterpret_cast<const float4 *>(wrP) + (size_t)e * MB * 64 + lane;
  float4 wv[MB];
  float xv[M];
#pragma unroll
  for (int b = 0; b < MB; ++b) wv[b] = wp[(size_t)b * 64];
#pragma unroll
  for (int m = 0; m < M; ++m) xv[m] = x[lane + 64 * m];
  float acc = 0.0f;
#pragma unroll
  for (int b = 0; b < MB; ++b) {
    acc = __builtin_fmaf(xv[4 * b + 0], wv[b].x, acc);
    acc = __builtin_fmaf(xv[4 * b + 1], wv[b].y, acc);
    acc = __builtin_fmaf(xv[4 * b + 2], wv[b].z, acc);
    acc = __builtin_fmaf(xv[4 * b + 3], wv[b].w, acc);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) acc = acc + __shfl_xor(acc, d);
  return acc;
}

}  // namespace coli
