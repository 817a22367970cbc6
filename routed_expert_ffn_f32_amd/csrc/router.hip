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
#include "byte_planes.h"
#include "dispatch_block.h"
#include "internal.h"
#include "router_tile.h"
#include "select.h"
#include "wave.h"

namespace coli {
namespace {


// wrP[e][b][l][i] = wr[l + 64 (4b + i)][e] (0 where 4b + i >= h/64): lane l's
// four consecutive chain elements form one float4.
__global__ __launch_bounds__(256) void router_permute_kernel(const float *__restrict__ wr,
                                                             float *__restrict__ wrP, int h, int E) {
  const int M = h >> 6, MB = (M + 3) >> 2;
  const size_t n = (size_t)E * MB * 256;
  for (size_t o = (size_t)blockIdx.x * 256 + threadIdx.x; o < n; o += (size_t)gridDim.x * 256) {
    const int i = (int)(o & 3), l = (int)((o >> 2) & 63);
    const size_t eb = o >> 8;
    const int b = (int)(eb % MB), e = (int)(eb / MB);
    const int m = 4 * b + i;
    wrP[o] = m < M ? wr[(size_t)(l + 64 * m) * E + e] : 0.0f;
  }
}

// One launch: blocks [0, n_logit_blocks) compute logits (4 waves, one tile
// each); the remaining blocks write the digit-plane form of the hidden rows
// (256 words of 8 columns per block) for the expert kernels.
template <int EPW, int TPW>
__global__ __launch_bounds__(256) void router_logits_kernel(const float *__restrict__ x,
                                                            const float *__restrict__ wrP, int T, int h, int E,
                                                            float *__restrict__ logits, int n_logit_blocks,
                                                            uint32_t *__restrict__ xq, float *__restrict__ xs,
                                                            int plane_mode) {
  const int bid = blockIdx.x;
  if (bid < n_logit_blocks) {
    const int egroups = (E + 4 * EPW - 1) / (4 * EPW);
    const int tg = bid / egroups, eg = bid % egroups;
    const int e0 = (eg * 4 + (threadIdx.x >> 6)) * EPW;
    if (e0 >= E) return;  // uniform over the wave
    logits_tile<EPW, TPW>(x, wrP, T, h, E, tg * TPW, e0, logits);
    return;
  }
  const int words = h >> 3;
  const size_t wg = (size_t)(bid - n_logit_blocks) * 256 + threadIdx.x;  // word over all rows
  const bool valid = wg < (size_t)T * words;
  const size_t t = valid ? wg / words : 0;
  const int w = valid ? (int)(wg % words) : 0;
  float v[8];
  if (valid) {
    const float4 a = *reinterpret_cast<const float4 *>(x + t * h + 8 * w);
    const float4 b = *reinterpret_cast<const float4 *>(x + t * h + 8 * w + 4);
    v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
  // a 32-column block is 4 words and never straddles a row (words % 8 == 0),
  // so the four lanes of a quad share the row and the block; either plane
  // form takes 3 h / 4 words per row
  uint32_t *row = xq + t * (size_t)(3 * (h >> 2));
  float *sb = xs + t * (words >> 2) + (w >> 2);
  if (plane_mode == kPlanesMatrixCore)
    byte_planes_word(v, valid, t, w, h, reinterpret_cast<uint8_t *>(xq), xs);
  else if (plane_mode == kPlanesInt8)
    FmtI8::quantize(v, (w & 3) == 0, valid, row, h, w, sb);
  else
    FmtI4::quantize(v, (w & 3) == 0, valid, row, h, w, sb);
}

__global__ __launch_bounds__(256) void router_select_kernel(const float *__restrict__ logits,
                                                            const float *__restrict__ bias, int T, int E,
                                                            int k, float rsf, RouteLimits lim,
                                                            int32_t *__restrict__ idx, float *__restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + uniform(threadIdx.x >> 6);  // scalar: the loads' buffer resources
  if (t >= T) return;
  int e;
  float w;
  select_token(logits + (size_t)t * E, bias, E, k, rsf, lim, e, w);
  if (lane < k) {
    idx[(size_t)t * k + lane] = e;
    wout[(size_t)t * k + lane] = w;
  }
}

// Small batches: selection of every token and the dispatch in one workgroup
// (16 waves); the selected ids go through LDS to the counting sort.
__global__ __launch_bounds__(kDispatchThreads) void select_dispatch_kernel(
    const float *__restrict__ logits, const float *__restrict__ bias, int T, int E, int k, float rsf,
    RouteLimits lim, int32_t *__restrict__ idx, float *__restrict__ wout, int32_t *__restrict__ offsets,
    int32_t *__restrict__ sorted_ids, int32_t *__restrict__ inv, int32_t *__restrict__ active,
    int32_t *__restrict__ n_active) {
  __shared__ int32_t sel[kFusedDispatchMax];
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  for (int t = wave; t < T; t += kDispatchThreads / kWave) {
    int e;
    float w;
    select_token(logits + (size_t)t * E, bias, E, k, rsf, lim, e, w);
    if (lane < k) {
      idx[(size_t)t * k + lane] = e;
      wout[(size_t)t * k + lane] = w;
      sel[t * k + lane] = e;
    }
  }
  __syncthreads();
  dispatch_block(sel, T * k, E, offsets, sorted_ids, inv, active, n_active);
}

// Large batches: grid = ceil(T / kWideT) x ceil(E / kWideE) blocks (token
// groups major) of kWideWaves waves, logits only.
__global__ __launch_bounds__(kWideWaves * 64) void router_logits_wide_kernel(const float *__restrict__ x,
                                                                 const float *__restrict__ wrP, int T, int h, int E,
                                                                 float *__restrict__ logits) {
  __shared__ float4 xs[2][kWideT][64];
  __shared__ float4 ws[2][kWideE][64];
  const int egroups = (E + kWideE - 1) / kWideE;
  logits_wide_tile(x, wrP, T, h, E, (blockIdx.x / egroups) * kWideT, (blockIdx.x % egroups) * kWideE, logits, xs, ws);
}

// One token: grid = E blocks of one wave, block e owning expert e (one wave
// per block spreads the table's read over every CU: 4-wave blocks on a
// quarter of the CUs took 8% longer), then the digit-plane blocks.  Every
// load of its chain (MB float4 blocks of the permuted router, the token's
// h/64 values for this lane) is issued before the first fma, so the launch
// costs one memory round trip; the arithmetic is logits_tile's, element for
// element.
template <int MB>
__global__ __launch_bounds__(64) void router_logits_t1_kernel(const float *__restrict__ x,
                                                               const float *__restrict__ wrP, int E,
                                                               float *__restrict__ logits, int n_logit_blocks,
                                                               uint32_t *__restrict__ xq, float *__restrict__ xs,
                                                               int plane_mode) {
  constexpr int M = 4 * MB;  // chain length h / 64
  const int lane = threadIdx.x & 63;
  if ((int)blockIdx.x >= n_logit_blocks) {  // the token's digit planes, 64 words per block
    const int words = M * 8;  // h / 8
    const int w = (blockIdx.x - n_logit_blocks) * 64 + threadIdx.x;
    const bool valid = w < words;
    float v[8];
    if (valid) {
      const float4 a = *reinterpret_cast<const float4 *>(x + 8 * w);
      const float4 b = *reinterpret_cast<const float4 *>(x + 8 * w + 4);
      v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    const int wq = valid ? w : 0;
    if (plane_mode == kPlanesMatrixCore)
      byte_planes_word(v, valid, 0, wq, M * 64, reinterpret_cast<uint8_t *>(xq), xs);
    else if (plane_mode == kPlanesInt8)
      FmtI8::quantize(v, (w & 3) == 0, valid, xq, M * 64, wq, xs + (wq >> 2));
    else
      FmtI4::quantize(v, (w & 3) == 0, valid, xq, M * 64, wq, xs + (wq >> 2));
    return;
  }
  const int e = blockIdx.x;
  const float acc = logit_t1<MB>(x, wrP, e);
  if (lane == 0) logits[e] = acc;
}

}  // namespace

hipError_t launch_router_permute(const float *wr, float *wrP, int h, int E, hipStream_t s) {
  const int MB = ((h >> 6) + 3) >> 2;
  const size_t n = (size_t)E * MB * 256;
  const size_t want = (n + 255) / 256;
  const int blocks = (int)(want < 4096 ? want : 4096);
  return launch(router_permute_kernel, blocks, 256, 0, s, wr, wrP, h, E);
}

size_t router_permuted_floats(int h, int E) { return (size_t)E * ((((h >> 6) + 3) >> 2)) * 256; }

// Batches from this size on take the wide tiles (enough blocks to fill the chip).
constexpr int kWideMinT = 256;

hipError_t launch_router_logits(const float *x, const float *wrP, int T, int h, int E, float *logits, uint32_t *xq,
                                float *xs, int plane_mode, hipStream_t s) {
  const int bp = plane_mode;
  if (T <= 0) return hipSuccess;
  const int qblocks = xq ? (int)(((size_t)T * (h >> 3) + 255) / 256) : 0;
  if (T == 1 && (h == 2048 || h == 4096 || h == 6144)) {
    const int qb = xq ? (h / 8 + 63) / 64 : 0;  // 64 plane words per block
    if (h == 2048) return launch(router_logits_t1_kernel<8>, E + qb, 64, 0, s, x, wrP, E, logits, E, xq, xs, bp);
    if (h == 4096) return launch(router_logits_t1_kernel<16>, E + qb, 64, 0, s, x, wrP, E, logits, E, xq, xs, bp);
    return launch(router_logits_t1_kernel<24>, E + qb, 64, 0, s, x, wrP, E, logits, E, xq, xs, bp);
  }
  // tiles per wave (experts x tokens) by batch size, measured on the GLM-like
  // layer (h = 6144, E = 256): the smallest tiles while they give the chip
  // enough waves, larger ones as the batch grows
  if (T < 12) {
    const int nlb = T * ((E + 3) / 4);
    return launch(router_logits_kernel<1, 1>, nlb + qblocks, 256, 0, s, x, wrP, T, h, E, logits, nlb, xq, xs, bp);
  } else if (T < 24) {
    const int nlb = ((T + 1) / 2) * ((E + 3) / 4);
    return launch(router_logits_kernel<1, 2>, nlb + qblocks, 256, 0, s, x, wrP, T, h, E, logits, nlb, xq, xs, bp);
  } else if (T < 48) {
    const int nlb = ((T + 1) / 2) * ((E + 7) / 8);
    return launch(router_logits_kernel<2, 2>, nlb + qblocks, 256, 0, s, x, wrP, T, h, E, logits, nlb, xq, xs, bp);
  } else if (T < kWideMinT) {
    const int nlb = ((T + 3) / 4) * ((E + 7) / 8);
    return launch(router_logits_kernel<2, 4>, nlb + qblocks, 256, 0, s, x, wrP, T, h, E, logits, nlb, xq, xs, bp);
  }
  // large batches: the wide tiles, then (GEMV path only) the digit planes
  const unsigned nwb = (unsigned)(((T + kWideT - 1) / kWideT) * ((E + kWideE - 1) / kWideE));
  hipError_t err = launch(router_logits_wide_kernel, nwb, kWideWaves * 64, 0, s, x, wrP, T, h, E, logits);
  if (err != hipSuccess || qblocks == 0) return err;
  return launch(router_logits_kernel<2, 4>, qblocks, 256, 0, s, x, wrP, T, h, E, logits, 0, xq, xs, bp);
}

hipError_t launch_router_select(const float *logits, const float *bias, int T, int E, int k, float rsf,
                                RouteLimits lim, int32_t *idx, float *w, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  return launch(router_select_kernel, (T + 3) / 4, 256, 0, s, logits, bias, T, E, k, rsf, lim, idx, w);
}

hipError_t launch_select_dispatch(const float *logits, const float *bias, int T, int E, int k, float rsf,
                                  RouteLimits lim, int32_t *idx, float *w, int32_t *offsets, int32_t *sorted_ids,
                                  int32_t *inv, int32_t *active, int32_t *n_active, hipStream_t s) {
  return launch(select_dispatch_kernel, 1, kDispatchThreads, 0, s, logits, bias, T, E, k, rsf, lim, idx, w, offsets,
                sorted_ids, inv, active, n_active);
}

}  // namespace coli
