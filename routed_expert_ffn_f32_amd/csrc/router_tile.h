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

#include <type_traits>

#include "internal.h"
#include "wave.h"

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
  // left to itself the scheduler keeps about a quarter of these loads in
  // flight (for occupancy the launch does not need: one wave per block, a
  // block per expert) and issues the rest between the fmas.  Measured: the
  // same 4.1 us either way at h = 6144, E = 256 (the launch is bound by its
  // dispatch and one round trip, not by the loads' issue).
  __builtin_amdgcn_sched_barrier(0);
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

// The xor butterfly (32, 16, 8, 4, 2, 1) of 64 values at once, transposed:
// each step pairs value i with value i + N/2 (N values left) and every lane
// keeps the one its lane bit selects, adding the partner lane's partial of
// it -- the same two partials the butterfly adds, so every sum is the
// butterfly's, bit for bit.  Lane l ends with the full sum of value l.
// Partners: the 32- and 16-lane swaps (each pairs two registers at once),
// row_ror:8 (= xor 8 within a 16-lane row), the xor-4 swizzle, quad
// permutations for xor 2 and 1.
template <int CTRL>
__device__ __forceinline__ float dpp_xf(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float butterfly64_transposed(float (&v)[64]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + 32]), false, false);
    v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + 16]), false, false);
    v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  const bool b3 = lane & 8, b2 = lane & 4, b1 = lane & 2, b0 = lane & 1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float keep = b3 ? v[i + 8] : v[i], send = b3 ? v[i] : v[i + 8];
    v[i] = keep + dpp_xf<0x128>(send);  // row_ror:8
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float keep = b2 ? v[i + 4] : v[i], send = b2 ? v[i] : v[i + 4];
    v[i] = keep + __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, send), 0x101F));
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float keep = b1 ? v[i + 2] : v[i], send = b1 ? v[i] : v[i + 2];
    v[i] = keep + dpp_xf<0x4E>(send);  // quad_perm [2,3,0,1]
  }
  const float keep = b0 ? v[1] : v[0], send = b0 ? v[0] : v[1];
  return keep + dpp_xf<0xB1>(send);  // quad_perm [1,0,3,2]
}

// Large batches: a block of kWideWaves waves computes kWideT tokens x kWideE
// experts (kWideT * kWideE = 64 kWideWaves), wave w the 8 x 8 pairs of token
// group w / (kWideE / 8) and expert group w % (kWideE / 8); every lane holds its
// chain partial of all 64 pairs.  Per block of 4 chain steps
// the block stages the 32 token rows and the 16 router columns in LDS in
// the lane-permuted order (a lane's 4 consecutive chain elements are one
// 16-byte read), double-buffered, the next block's global loads in flight
// during the current block's fmas.  Each fma is logits_tile's, element for
// element, and the final butterfly runs transposed.
constexpr int kWideT = 32, kWideE = 16;
constexpr int kWideWaves = kWideT * kWideE / 64;
static_assert(kWideT % 8 == 0 && kWideE % 8 == 0 && kWideT % kWideWaves == 0 && kWideE % kWideWaves == 0,
              "waves of 8 x 8 pairs; every thread stages the same number of rows");

__device__ __forceinline__ void logits_wide_tile(const float *__restrict__ x, const float *__restrict__ wrP, int T,
                                                 int h, int E, int t0, int e0, float *__restrict__ logits,
                                                 float4 (*xs)[kWideT][64], float4 (*ws)[kWideE][64]) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int NW = kWideWaves, XK = kWideT / NW, WK = kWideE / NW;  // staged rows per thread
  const int tw = wave / WK, ew = wave % WK;
  const int M = h >> 6, MB = (M + 3) >> 2;
  // staging: this thread copies lane `lane` of tokens wave + NW k (k < XK)
  // and of experts wave + NW k (k < WK); a token row's descriptor ends at its
  // h columns, so chain steps past M read zeros without a branch
  Rsrc xr[XK];
  const float4 *wr[WK];
#pragma unroll
  for (int k = 0; k < XK; ++k) xr[k] = make_rsrc(x + (size_t)min(t0 + wave + NW * k, T - 1) * h, (uint32_t)h * 4);
#pragma unroll
  for (int k = 0; k < WK; ++k)
    wr[k] = reinterpret_cast<const float4 *>(wrP) + (size_t)min(e0 + wave + NW * k, E - 1) * MB * 64 + lane;
  // two register sets: block b + 2's loads are issued while block b is
  // computed (one block of fmas is shorter than a load's latency here);
  // past the last block they re-read it (unused)
  // The set index is a compile-time constant at every use (passed as an
  // integral_constant): indexed at run time, the compiler moves the sets to
  // LDS, with an LDS round trip per step and a wait for every load.
  float4 xv[2][XK], wv[2][WK];
  auto load = [&](int b, auto setc) {
    constexpr int set = decltype(setc)::value;
    b = min(b, MB - 1);
#pragma unroll
    for (int k = 0; k < XK; ++k) {
      float f[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) f[i] = bloadf(xr[k], (uint32_t)(lane + 64 * (4 * b + i)) * 4, 0);
      xv[set][k] = make_float4(f[0], f[1], f[2], f[3]);
    }
#pragma unroll
    for (int k = 0; k < WK; ++k) {
      const float4 v = wr[k][(size_t)b * 64];
      wv[set][k] = make_float4(v.x, v.y, v.z, v.w);
    }
  };
  float acc[64];
#pragma unroll
  for (int j = 0; j < 64; ++j) acc[j] = 0.0f;
  auto step = [&](int b, auto setc) {
    constexpr int set = decltype(setc)::value;
#pragma unroll
    for (int k = 0; k < XK; ++k) xs[set][wave + NW * k][lane] = xv[set][k];
#pragma unroll
    for (int k = 0; k < WK; ++k) ws[set][wave + NW * k][lane] = wv[set][k];
    // block b staged; every wave past block b - 1's reads of the other
    // buffer.  An LDS-only barrier: the next block's global loads stay in
    // flight across it (__syncthreads would wait for them too).
    block_barrier();
    load(b + 2, setc);
    float4 a[8], c[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) a[t] = xs[set][8 * tw + t][lane];
#pragma unroll
    for (int e = 0; e < 8; ++e) c[e] = ws[set][8 * ew + e][lane];
    auto fmas = [&](int i) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float xa = i == 0 ? a[t].x : i == 1 ? a[t].y : i == 2 ? a[t].z : a[t].w;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float wc = i == 0 ? c[e].x : i == 1 ? c[e].y : i == 2 ? c[e].z : c[e].w;
          acc[8 * t + e] = __builtin_fmaf(xa, wc, acc[8 * t + e]);
        }
      }
    };
    if (4 * b + 4 <= M) {  // a full block: no per-step guard, so the reads are hoisted
#pragma unroll
      for (int i = 0; i < 4; ++i) fmas(i);
    } else {  // the chain's last, partial block: its steps past M are skipped
#pragma unroll
      for (int i = 0; i < 3; ++i)
        if (4 * b + i < M) fmas(i);
    }
  };
  const std::integral_constant<int, 0> set0;
  const std::integral_constant<int, 1> set1;
  load(0, set0);
  load(1, set1);
  // straight-line pairs (a skippable second step would leave the compiler's
  // count of loads in flight unknown at the loop head, and it would wait
  // for all of them there), then an odd last block
  int b = 0;
  for (; b + 1 < MB; b += 2) {
    step(b, set0);
    step(b + 1, set1);
  }
  if (b < MB) step(b, set0);
  const float sum = butterfly64_transposed(acc);
  const int t = t0 + 8 * tw + (lane >> 3), e = e0 + 8 * ew + (lane & 7);
  if (t < T && e < E) logits[(size_t)t * E + e] = sum;
}

}  // namespace coli
