// Decode-sized expert FFN: int4 gs64 GEMV kernels, float32 accumulation.
//
// Source: "colibri engine teardown" page, "Three key engineering decisions",
// item 1 -- routed experts are int4 in the "gs64" container (64 weights share
// one scale); cf-1.com Colibri article, section 2.1 -- each expert is an FFN
// with three matrices (W1 gate, W3 up, W2 down), applied to the tokens
// grouped to it; section 3.3 step 4 skips experts with no tokens.
//
// Decode reads every selected expert's weights once per call, so these
// kernels are bound by HBM bandwidth: each wave streams RPW whole rows with
// 16-byte loads per lane (a wave covers 1 KB of a row per step, coalesced),
// unpacks the nibbles in registers and applies them to every token of the
// expert before the next load.  The activations come through the L1/L2
// caches (a token row is shared by all waves of the expert).
//
// Per 8 weights (one 32-bit word): the word is xored with 0x88888888, which
// turns each two's-complement code q into u = q + 8 in [0, 15]; the even and
// odd nibbles are split into bytes and converted with v_cvt_f32_ubyte*.  The
// sum over a 32-column lane chunk is then sum(u x) - 8 sum(x), scaled once by
// the chunk's group scale.  Everything accumulates in float32.
#include "internal.h"

namespace coli {
namespace {

__device__ __forceinline__ float ub(uint32_t v, int byte) { return (float)((v >> (8 * byte)) & 0xFFu); }

// acc += sum over the 8 columns of word w (codes) of u_c * x_c, u = q + 8.
__device__ __forceinline__ float dot8(uint32_t w, const float4 &xa, const float4 &xb, float acc) {
  const uint32_t u = w ^ 0x88888888u;
  const uint32_t lo = u & 0x0F0F0F0Fu;         // columns 0, 2, 4, 6
  const uint32_t hi = (u >> 4) & 0x0F0F0F0Fu;  // columns 1, 3, 5, 7
  acc = __builtin_fmaf(ub(lo, 0), xa.x, acc);
  acc = __builtin_fmaf(ub(hi, 0), xa.y, acc);
  acc = __builtin_fmaf(ub(lo, 1), xa.z, acc);
  acc = __builtin_fmaf(ub(hi, 1), xa.w, acc);
  acc = __builtin_fmaf(ub(lo, 2), xb.x, acc);
  acc = __builtin_fmaf(ub(hi, 2), xb.y, acc);
  acc = __builtin_fmaf(ub(lo, 3), xb.z, acc);
  acc = __builtin_fmaf(ub(hi, 3), xb.w, acc);
  return acc;
}

__device__ __forceinline__ uint32_t word(const uint4 &v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

struct Slot {
  const uint8_t *qa, *qb;
  const float *sa, *sb;
  int p_begin, cnt;
  bool routed;
};

// Rows [r0, r0 + RPW) of this slot's matrices applied to NT tokens starting
// at slot position tc.  GATE_UP: out = silu(A x) * (B x); else out = A x.
template <bool GATE_UP, int NT, int RPW>
__device__ __forceinline__ void rows_times_tokens(const GemvProblem &P, const Slot &S, int r0, int tc,
                                                  int lane) {
  const int rowq = P.cols >> 1, rows_s = P.cols >> 6, nchunks = P.cols >> 5;
  const float *xr[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int p = S.p_begin + tc + i;
    if (GATE_UP) {
      const int t = S.routed ? P.sorted_ids[p] / P.k : p - P.T * P.k;
      xr[i] = P.x + (size_t)t * P.cols;
    } else {
      xr[i] = P.x + (size_t)p * P.cols;
    }
  }
  float accA[RPW][NT], accB[RPW][NT];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int i = 0; i < NT; ++i) accA[r][i] = accB[r][i] = 0.0f;

  for (int lc = lane; lc < nchunks; lc += 64) {
    uint4 wa[RPW], wb[RPW];
    float sca[RPW], scb[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const size_t row = (size_t)(r0 + r);
      wa[r] = *reinterpret_cast<const uint4 *>(S.qa + row * rowq + (size_t)lc * 16);
      sca[r] = S.sa[row * rows_s + (lc >> 1)];
      if (GATE_UP) {
        wb[r] = *reinterpret_cast<const uint4 *>(S.qb + row * rowq + (size_t)lc * 16);
        scb[r] = S.sb[row * rows_s + (lc >> 1)];
      }
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const float4 *xv = reinterpret_cast<const float4 *>(xr[i] + (size_t)lc * 32);
      float pa[RPW], pb[RPW];
#pragma unroll
      for (int r = 0; r < RPW; ++r) pa[r] = pb[r] = 0.0f;
      float xs = 0.0f;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const float4 xa = xv[2 * wd], xb = xv[2 * wd + 1];
        xs += ((xa.x + xa.y) + (xa.z + xa.w)) + ((xb.x + xb.y) + (xb.z + xb.w));
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          pa[r] = dot8(word(wa[r], wd), xa, xb, pa[r]);
          if (GATE_UP) pb[r] = dot8(word(wb[r], wd), xa, xb, pb[r]);
        }
      }
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        accA[r][i] = __builtin_fmaf(sca[r], __builtin_fmaf(-8.0f, xs, pa[r]), accA[r][i]);
        if (GATE_UP) accB[r][i] = __builtin_fmaf(scb[r], __builtin_fmaf(-8.0f, xs, pb[r]), accB[r][i]);
      }
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1)
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        accA[r][i] += __shfl_xor(accA[r][i], d);
        if (GATE_UP) accB[r][i] += __shfl_xor(accB[r][i], d);
      }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const size_t p = (size_t)(S.p_begin + tc + i);
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        float v = accA[r][i];
        if (GATE_UP) v = v / (1.0f + expf(-v)) * accB[r][i];
        P.out[p * P.rows + r0 + r] = v;
      }
    }
  }
}

// grid = (rows / (4 RPW), n_routed_slots + has_shared); 4 waves per block,
// wave w owns rows [(4 bx + w) RPW, +RPW).  Slot s < n_routed_slots is the
// s-th active expert (blocks past n_active leave at once), the last slot is
// the shared expert over all T tokens.
template <bool GATE_UP, int NTMAX, int RPW>
__global__ __launch_bounds__(256) void gemv_kernel(GemvProblem P) {
  const int lane = threadIdx.x & 63;
  const int slot = blockIdx.y;
  Slot S;
  const size_t qstride = (size_t)P.rows * (P.cols >> 1), sstride = (size_t)P.rows * (P.cols >> 6);
  if (slot < P.n_routed_slots) {
    if (slot >= *P.n_active) return;
    const int e = P.active[slot];
    S.p_begin = P.offsets[e];
    S.cnt = P.offsets[e + 1] - S.p_begin;
    S.qa = P.a.q + e * qstride;
    S.sa = P.a.s + e * sstride;
    S.qb = GATE_UP ? P.b.q + e * qstride : nullptr;
    S.sb = GATE_UP ? P.b.s + e * sstride : nullptr;
    S.routed = true;
  } else {
    S.p_begin = P.T * P.k;
    S.cnt = P.T;
    S.qa = P.sh_a.q;
    S.sa = P.sh_a.s;
    S.qb = P.sh_b.q;
    S.sb = P.sh_b.s;
    S.routed = false;
  }
  const int r0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW;
  if (r0 >= P.rows) return;
  int tc = 0;
  if (NTMAX >= 4)
    for (; tc + 4 <= S.cnt; tc += 4) rows_times_tokens<GATE_UP, 4, RPW>(P, S, r0, tc, lane);
  if (NTMAX >= 2)
    for (; tc + 2 <= S.cnt; tc += 2) rows_times_tokens<GATE_UP, 2, RPW>(P, S, r0, tc, lane);
  for (; tc < S.cnt; ++tc) rows_times_tokens<GATE_UP, 1, RPW>(P, S, r0, tc, lane);
}

__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ y, const float *__restrict__ w,
                                                      const int32_t *__restrict__ inv, int T, int k, int h,
                                                      int has_shared, float *__restrict__ out) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= h) return;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int j = 0; j < k; ++j) {
    const int a = t * k + j;
    const float wj = w[a];
    const float4 v = *reinterpret_cast<const float4 *>(y + (size_t)inv[a] * h + c);
    acc.x = __builtin_fmaf(wj, v.x, acc.x);
    acc.y = __builtin_fmaf(wj, v.y, acc.y);
    acc.z = __builtin_fmaf(wj, v.z, acc.z);
    acc.w = __builtin_fmaf(wj, v.w, acc.w);
  }
  if (has_shared) {
    const float4 v = *reinterpret_cast<const float4 *>(y + ((size_t)T * k + t) * h + c);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  *reinterpret_cast<float4 *>(out + (size_t)t * h + c) = acc;
}

constexpr int kRowsPerWave = 4;

template <bool GATE_UP>
hipError_t launch_gemv(const GemvProblem &P, hipStream_t s) {
  const int slots = P.n_routed_slots + (P.has_shared ? 1 : 0);
  if (slots == 0 || P.T == 0) return hipSuccess;
  dim3 grid(P.rows / (4 * kRowsPerWave), slots);
  if (P.T == 1)
    gemv_kernel<GATE_UP, 1, kRowsPerWave><<<grid, 256, 0, s>>>(P);
  else if (P.T < 4)
    gemv_kernel<GATE_UP, 2, kRowsPerWave><<<grid, 256, 0, s>>>(P);
  else
    gemv_kernel<GATE_UP, 4, kRowsPerWave><<<grid, 256, 0, s>>>(P);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_gate_up(const GemvProblem &P, hipStream_t s) { return launch_gemv<true>(P, s); }
hipError_t launch_gemv_down(const GemvProblem &P, hipStream_t s) { return launch_gemv<false>(P, s); }

hipError_t launch_combine(const float *y, const float *w, const int32_t *inv, int T, int k, int h,
                          int has_shared, float *out, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  dim3 grid((h / 4 + 255) / 256, T);
  combine_kernel<<<grid, 256, 0, s>>>(y, w, inv, T, k, h, has_shared, out);
  return hipGetLastError();
}

}  // namespace coli
