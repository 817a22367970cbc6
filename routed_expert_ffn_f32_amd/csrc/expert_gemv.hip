// Decode-sized expert FFN: int4 gs64 GEMV kernels.
//
// Source: "colibri engine teardown" page, "Three key engineering decisions",
// item 1 -- routed experts are int4 in the "gs64" container (64 weights share
// one scale); cf-1.com Colibri article, section 2.1 -- each expert is an FFN
// with three matrices (W1 gate, W3 up, W2 down), applied to the tokens
// grouped to it; section 3.3 step 4 skips experts with no tokens.
//
// Decode reads every selected expert's weights once per call, so these
// kernels are bound by HBM bandwidth.  Each wave streams whole weight rows,
// 16 bytes per lane per step (a wave covers 1 KB of a row, coalesced).  The
// weights are never unpacked: the activations arrive as six signed 4-bit
// digit planes per 64-column group (wave.h), and v_dot8_i32_i4 multiplies a
// packed weight word by a plane word directly, 8 columns per instruction.
// Per 32-column half group, sum_c q_c x_c = s_x * sum_j 16^j dot8s_j is exact
// in int32; one float fma per half group applies the weight scale and the
// activation scale.  Results accumulate in float32.
//
// gate/up: a block owns 64 rows of I (one group of the down projection's
// input) for one expert, so it can finish SwiGLU and write the intermediate
// in digit-plane form itself.  down: a block owns 32 rows of h.
#include "internal.h"
#include "wave.h"

namespace coli {
namespace {

constexpr int kGuWaves = 8;        // gate/up block: 8 waves x 8 rows = 64 rows
constexpr int kGuRows = 8;
constexpr int kDnWaves = 4;        // down block: 4 waves x 8 rows = 32 rows
constexpr int kDnRows = 8;

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

struct Slot {
  const uint8_t *qa, *qb;
  const float *sa, *sb;
  int p_begin, cnt;
  bool routed;
};

// Slot s < n_routed_slots is the s-th active expert, the last slot the shared
// expert over all T tokens.  cnt < 0 marks a slot past n_active.
__device__ __forceinline__ Slot slot_of(const DecodeProblem &P, int slot, const ExpertTables &a,
                                       const ExpertTables &b, const ExpertTables &sha, const ExpertTables &shb,
                                       int rows, int cols) {
  Slot S;
  if (slot < P.n_routed_slots) {
    S.routed = true;
    if (slot >= *P.n_active) {
      S.cnt = -1;
      return S;
    }
    const int e = P.active[slot];
    const size_t qstride = (size_t)rows * (cols >> 1), sstride = (size_t)rows * (cols >> 6);
    S.p_begin = P.offsets[e];
    S.cnt = P.offsets[e + 1] - S.p_begin;
    S.qa = a.q + e * qstride;
    S.sa = a.s + e * sstride;
    S.qb = b.q ? b.q + e * qstride : nullptr;
    S.sb = b.s ? b.s + e * sstride : nullptr;
  } else {
    S.routed = false;
    S.p_begin = P.T * P.k;
    S.cnt = P.T;
    S.qa = sha.q;
    S.sa = sha.s;
    S.qb = shb.q;
    S.sb = shb.s;
  }
  return S;
}

// ---------------------------------------------------------------------------
// gate/up
// ---------------------------------------------------------------------------

// Rows [row0 + 8 wave, +8) of gate and up on NT tokens from slot position tc;
// lane 0 leaves silu(g) * u per row and token in mid_lds.
template <int NT>
__device__ __forceinline__ void gate_up_pass(const DecodeProblem &P, const Slot &S, int row0, int tc,
                                             float (*mid_lds)[4]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r0 = row0 + wave * kGuRows;
  const int h = P.h, rowq = h >> 1, groups = h >> 6, words = h >> 3, nch = h >> 5;
  int tok[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int p = S.p_begin + tc + i;
    tok[i] = S.routed ? P.sorted_ids[p] / P.k : p - P.T * P.k;
  }
  float ga[kGuRows][NT], ua[kGuRows][NT];
#pragma unroll
  for (int r = 0; r < kGuRows; ++r)
#pragma unroll
    for (int i = 0; i < NT; ++i) ga[r][i] = ua[r][i] = 0.0f;

  // per 32-column lane chunk: the gate rows, then the up rows (half the live
  // weight registers of doing both at once)
  for (int lc = lane; lc < nch; lc += 64) {
    uint4 xp[NT == 1 ? kPlanes : 1];
    float sx1 = 0.0f;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const uint8_t *q = half ? S.qb : S.qa;
      const float *sc = half ? S.sb : S.sa;
      uint4 wv[kGuRows];
      float ws[kGuRows];
#pragma unroll
      for (int r = 0; r < kGuRows; ++r) {
        const size_t row = (size_t)(r0 + r);
        wv[r] = ld16(q + row * rowq + (size_t)lc * 16);
        ws[r] = sc[row * groups + (lc >> 1)];
      }
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        uint4 xt[kPlanes];
        float sx;
        if (NT == 1 && half == 1) {
#pragma unroll
          for (int j = 0; j < kPlanes; ++j) xt[j] = xp[j < (NT == 1 ? kPlanes : 1) ? j : 0];
          sx = sx1;
        } else {
#pragma unroll
          for (int j = 0; j < kPlanes; ++j)
            xt[j] = ld16(P.xq + ((size_t)tok[i] * kPlanes + j) * words + (size_t)lc * 4);
          sx = P.xs[(size_t)tok[i] * groups + (lc >> 1)];
          if (NT == 1) {
#pragma unroll
            for (int j = 0; j < kPlanes; ++j) xp[j < (NT == 1 ? kPlanes : 1) ? j : 0] = xt[j];
            sx1 = sx;
          }
        }
#pragma unroll
        for (int r = 0; r < kGuRows; ++r) {
          const float v = (float)dot_planes(wv[r], xt);
          if (half == 0)
            ga[r][i] = __builtin_fmaf(v, ws[r] * sx, ga[r][i]);
          else
            ua[r][i] = __builtin_fmaf(v, ws[r] * sx, ua[r][i]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kGuRows; ++r)
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const float g = wave_sum(ga[r][i]);
      const float u = wave_sum(ua[r][i]);
      if (lane == 0) mid_lds[wave * kGuRows + r][i] = g / (1.0f + expf(-g)) * u;
    }
}

// grid = (I / 64, n_routed_slots + has_shared), 512 threads.
// Single-token calls: two blocks per CU (4 waves per SIMD) keep every block
// of the call resident at once.
template <int NTMAX>
__global__ __launch_bounds__(kGuWaves * 64, NTMAX == 1 ? 4 : 2) void gate_up_kernel(DecodeProblem P) {
  __shared__ float mid_lds[kGuWaves * kGuRows][4];
  const Slot S = slot_of(P, blockIdx.y, P.gate, P.up, P.sh_gate, P.sh_up, P.I, P.h);
  if (S.cnt <= 0) return;  // uniform over the block
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row0 = blockIdx.x * (kGuWaves * kGuRows);
  const int I = P.I, words = I >> 3;
  for (int tc = 0; tc < S.cnt;) {
    const int left = S.cnt - tc;
    const int nt = (NTMAX >= 4 && left >= 4) ? 4 : (NTMAX >= 2 && left >= 2) ? 2 : 1;
    if (nt == 4)
      gate_up_pass<(NTMAX >= 4 ? 4 : 1)>(P, S, row0, tc, mid_lds);
    else if (nt == 2)
      gate_up_pass<(NTMAX >= 2 ? 2 : 1)>(P, S, row0, tc, mid_lds);
    else
      gate_up_pass<1>(P, S, row0, tc, mid_lds);
    __syncthreads();
    // the 64 rows are one input group of the down projection: wave 0 writes
    // them as digit planes, eight lanes per token
    if (wave == 0) {
      const int i = lane >> 3, w = lane & 7;
      const bool store = i < nt;
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = store ? mid_lds[8 * w + q][i & 3] : 0.0f;
      const size_t p = (size_t)(S.p_begin + tc + (store ? i : 0));
      quantize_word(v, w == 0, store, P.mq + p * kPlanes * words + (row0 >> 3) + w, (size_t)words,
                    P.ms + p * (I >> 6) + (row0 >> 6));
    }
    __syncthreads();
    tc += nt;
  }
}

// ---------------------------------------------------------------------------
// down
// ---------------------------------------------------------------------------

template <int NT>
__device__ __forceinline__ void down_pass(const DecodeProblem &P, const Slot &S, int r0, int tc) {
  const int lane = threadIdx.x & 63;
  const int I = P.I, rowq = I >> 1, groups = I >> 6, words = I >> 3, nch = I >> 5;
  float acc[kDnRows][NT];
#pragma unroll
  for (int r = 0; r < kDnRows; ++r)
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[r][i] = 0.0f;
  for (int lc = lane; lc < nch; lc += 64) {
    uint4 dw[kDnRows];
    float ds[kDnRows];
#pragma unroll
    for (int r = 0; r < kDnRows; ++r) {
      const size_t row = (size_t)(r0 + r);
      dw[r] = ld16(S.qa + row * rowq + (size_t)lc * 16);
      ds[r] = S.sa[row * groups + (lc >> 1)];
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const size_t p = (size_t)(S.p_begin + tc + i);
      uint4 xp[kPlanes];
#pragma unroll
      for (int j = 0; j < kPlanes; ++j) xp[j] = ld16(P.mq + (p * kPlanes + j) * words + (size_t)lc * 4);
      const float sx = P.ms[p * groups + (lc >> 1)];
#pragma unroll
      for (int r = 0; r < kDnRows; ++r)
        acc[r][i] = __builtin_fmaf((float)dot_planes(dw[r], xp), ds[r] * sx, acc[r][i]);
    }
  }
#pragma unroll
  for (int r = 0; r < kDnRows; ++r)
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const float v = wave_sum(acc[r][i]);
      if (lane == 0) P.y[(size_t)(S.p_begin + tc + i) * P.h + r0 + r] = v;
    }
}

// grid = (h / 32, n_routed_slots + has_shared), 256 threads.
template <int NTMAX>
__global__ __launch_bounds__(kDnWaves * 64) void down_kernel(DecodeProblem P) {
  const ExpertTables none{nullptr, nullptr};
  const Slot S = slot_of(P, blockIdx.y, P.down, none, P.sh_down, none, P.h, P.I);
  if (S.cnt <= 0) return;
  const int r0 = (blockIdx.x * kDnWaves + (threadIdx.x >> 6)) * kDnRows;
  int tc = 0;
  if (NTMAX >= 4)
    for (; tc + 4 <= S.cnt; tc += 4) down_pass<4>(P, S, r0, tc);
  if (NTMAX >= 2)
    for (; tc + 2 <= S.cnt; tc += 2) down_pass<2>(P, S, r0, tc);
  for (; tc < S.cnt; ++tc) down_pass<1>(P, S, r0, tc);
}

// out[t][c..c+3]; the k slot weights and positions are loaded first (up to
// kMaxTopK, uniform per block), then all expert rows, then summed in slot
// order and the shared row added last.
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ y, const float *__restrict__ w,
                                                      const int32_t *__restrict__ inv, int T, int k, int h,
                                                      int has_shared, float *__restrict__ out) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= h) return;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int j0 = 0; j0 < k; j0 += 8) {
    float wj[8];
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int a = t * k + min(j0 + u, k - 1);
      wj[u] = w[a];
      v[u] = *reinterpret_cast<const float4 *>(y + (size_t)inv[a] * h + c);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (j0 + u < k) {
        acc.x = __builtin_fmaf(wj[u], v[u].x, acc.x);
        acc.y = __builtin_fmaf(wj[u], v[u].y, acc.y);
        acc.z = __builtin_fmaf(wj[u], v[u].z, acc.z);
        acc.w = __builtin_fmaf(wj[u], v[u].w, acc.w);
      }
    }
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

}  // namespace

hipError_t launch_gemv_gate_up(const DecodeProblem &P, hipStream_t s) {
  const int slots = P.n_routed_slots + (P.has_shared ? 1 : 0);
  if (slots == 0 || P.T == 0) return hipSuccess;
  dim3 grid(P.I / (kGuWaves * kGuRows), slots);
  // passes of at most two tokens: a four-token pass does not fit the
  // register file without spilling
  if (P.T == 1)
    gate_up_kernel<1><<<grid, kGuWaves * 64, 0, s>>>(P);
  else
    gate_up_kernel<2><<<grid, kGuWaves * 64, 0, s>>>(P);
  return hipGetLastError();
}

hipError_t launch_gemv_down(const DecodeProblem &P, hipStream_t s) {
  const int slots = P.n_routed_slots + (P.has_shared ? 1 : 0);
  if (slots == 0 || P.T == 0) return hipSuccess;
  dim3 grid(P.h / (kDnWaves * kDnRows), slots);
  if (P.T == 1)
    down_kernel<1><<<grid, kDnWaves * 64, 0, s>>>(P);
  else if (P.T < 4)
    down_kernel<2><<<grid, kDnWaves * 64, 0, s>>>(P);
  else
    down_kernel<4><<<grid, kDnWaves * 64, 0, s>>>(P);
  return hipGetLastError();
}

hipError_t launch_combine(const float *y, const float *w, const int32_t *inv, int T, int k, int h,
                          int has_shared, float *out, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  dim3 grid((h / 4 + 255) / 256, T);
  combine_kernel<<<grid, 256, 0, s>>>(y, w, inv, T, k, h, has_shared, out);
  return hipGetLastError();
}

}  // namespace coli
