// Decode-sized expert FFN: int4 gs64 GEMV kernels.
//
// Source: "colibri engine teardown" page, "Three key engineering decisions",
// item 1 -- routed experts are int4 in the "gs64" container (64 weights share
// one scale); cf-1.com Colibri article, section 2.1 -- each expert is an FFN
// with three matrices (W1 gate, W3 up, W2 down), applied to the tokens
// grouped to it, and the outputs are summed with the routing weights; section
// 3.3 step 4 skips experts with no tokens.
//
// Decode reads every selected expert's weights once per call, so these
// kernels are bound by HBM bandwidth.  Each wave streams whole weight rows,
// 16 bytes per lane per step (a wave covers 1 KB of a row, coalesced).  The
// weights are never unpacked: the activations arrive as six signed 4-bit
// digit planes per 32-column block (wave.h), and v_dot8_i32_i4 multiplies a
// packed weight word by a plane word directly, 8 columns per instruction.
// Per 32-column lane chunk, sum_c q_c x_c = s_x * sum_j 16^j dot8s_j is exact
// in int32; one float fma per chunk applies the weight scale and the
// activation scale.  Results accumulate in float32.
//
// Launch structure of one decode call (T tokens):
//   gate/up   grid (I/32, slots): slot 0 is the shared expert, which needs no
//             routing and starts streaming at once; the other slots are the
//             active routed experts.  For small batches every routed block
//             selects the experts of all T tokens and sorts the assignments
//             itself in LDS (a few microseconds, identical in every block)
//             instead of waiting for a separate launch; one block publishes
//             the routing.  A block owns 32 rows of I for one expert and
//             writes the SwiGLU result as digit planes.
//   down      small batches: grid (h/8): one wave per (token, slot) and per
//             shared-expert token computes 8 rows of its expert's output into
//             LDS; the block sums w_j * y_j in slot order plus the shared row
//             into the output (the weighted combine fused, no intermediate y
//             in HBM); larger batches: y per assignment, then a combine kernel.
#include "internal.h"
#include "select.h"
#include "wave.h"

namespace coli {
namespace {

#ifndef COLI_GU_ROWS
#define COLI_GU_ROWS 4
#endif
#ifndef COLI_GU_MIN_WAVES
#define COLI_GU_MIN_WAVES 1
#endif
constexpr int kGuRows = COLI_GU_ROWS;      // gate/up rows per wave
constexpr int kGuWaves = 32 / kGuRows;     // a block owns 32 rows of I
constexpr int kDnWaves = 4;  // down block (larger batches): 4 waves x 8 rows
constexpr int kDnRows = 8;
#ifndef COLI_DC_ROWS
#define COLI_DC_ROWS 8
#endif
constexpr int kDcRows = COLI_DC_ROWS;  // fused down + combine block: rows, one wave per slot

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// ---------------------------------------------------------------------------
// Routing of a small batch inside one block (T <= kSmallT tokens, T*k <= 64).
// ---------------------------------------------------------------------------
struct SmallRouting {
  SelectScratch sc[kSmallT];
  int32_t idx[kSmallAssign];
  float w[kSmallAssign];
  int32_t sorted_ids[kSmallAssign];
  int32_t inv[kSmallAssign];
  int32_t sorted_key[kSmallAssign];
  int32_t active[kSmallAssign];
  int32_t seg_begin[kSmallAssign + 1];
  int32_t n_active;
};

// Waves 0..T-1 select one token each; wave 0 then sorts the n = T*k
// assignments by expert, stably (position = smaller keys + equal keys of
// lower a), and lists the segments.  Ends with the block synchronised.
__device__ __forceinline__ void route_small(const float *__restrict__ logits, const float *__restrict__ bias, int T,
                                            int E, int k, float rsf, SmallRouting &R) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave < T) {
    int e;
    float w;
    select_token(logits + (size_t)wave * E, bias, E, k, rsf, e, w, R.sc[wave]);
    if (lane < k) {
      R.idx[wave * k + lane] = e;
      R.w[wave * k + lane] = w;
    }
  }
  __syncthreads();
  const int n = T * k;
  if (wave == 0) {
    const bool valid = lane < n;
    const int key = valid ? R.idx[lane] : 0;
    int before = 0;
    for (int b = 0; b < n; ++b) {
      const int kb = R.idx[b];
      before += (kb < key) || (kb == key && b < lane);
    }
    if (valid) {
      R.sorted_ids[before] = lane;
      R.inv[lane] = before;
      R.sorted_key[before] = key;
    }
  }
  __syncthreads();
  if (wave == 0) {
    const bool start = lane < n && (lane == 0 || R.sorted_key[lane] != R.sorted_key[lane > 0 ? lane - 1 : 0]);
    const uint64_t m = __ballot(start);
    const int slot = __popcll(m & ((1ull << lane) - 1));
    if (start) {
      R.active[slot] = R.sorted_key[lane];
      R.seg_begin[slot] = lane;
    }
    if (lane == 0) {
      R.n_active = __popcll(m);
      R.seg_begin[__popcll(m)] = n;
    }
  }
  __syncthreads();
}

// The routing of the call in the layout of the C ABI (idx, w, offsets[E+1],
// sorted_ids, inv, active, n_active), written by one block.
__device__ __forceinline__ void publish_routing(const SmallRouting &R, const DecodeProblem &P) {
  const int n = P.T * P.k;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    P.idx[i] = R.idx[i];
    P.wsel[i] = R.w[i];
    P.sorted_ids[i] = R.sorted_ids[i];
    P.inv[i] = R.inv[i];
  }
  for (int e = threadIdx.x; e <= P.E; e += blockDim.x) {
    int c = 0;
    for (int a = 0; a < n; ++a) c += R.idx[a] < e;
    P.offsets[e] = c;
  }
  for (int s = threadIdx.x; s < R.n_active; s += blockDim.x) P.active[s] = R.active[s];
  if (threadIdx.x == 0) *P.n_active = R.n_active;
}

struct Slot {
  const uint8_t *qa, *qb;
  const float *sa, *sb;
  int p_begin, cnt;
};

// ---------------------------------------------------------------------------
// gate/up
// ---------------------------------------------------------------------------

// Rows [row0 + 8 wave, +8) of gate and up on NT tokens from slot position tc;
// lane 0 leaves silu(g) * u per row and token in mid_lds.  tok_of(i) is the
// token of slot position i.
template <int NT, class TokOf>
__device__ __forceinline__ void gate_up_pass(const DecodeProblem &P, const Slot &S, int row0, int tc,
                                             const TokOf &tok_of, float (*mid_lds)[4]) {
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int r0 = row0 + wave * kGuRows;
  const int h = P.h, rowq = h >> 1, groups = h >> 6, blocks = h >> 5, words = h >> 3, nch = h >> 5;
  const uint32_t qbytes = (uint32_t)P.I * rowq, sbytes = (uint32_t)P.I * groups * 4;
  const Rsrc rqa = make_rsrc(S.qa, qbytes), rsa = make_rsrc(S.sa, sbytes);
  const Rsrc rqb = make_rsrc(S.qb, qbytes), rsb = make_rsrc(S.sb, sbytes);
  const Rsrc rx = make_rsrc(P.xq, (uint32_t)P.T * kPlanes * words * 4);
  const Rsrc rxs = make_rsrc(P.xs, (uint32_t)P.T * blocks * 4);
  int tok[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) tok[i] = uniform(tok_of(tc + i));
  float ga[kGuRows][NT], ua[kGuRows][NT];
#pragma unroll
  for (int r = 0; r < kGuRows; ++r)
#pragma unroll
    for (int i = 0; i < NT; ++i) ga[r][i] = ua[r][i] = 0.0f;

  // Stages alternate gate rows and up rows of one 32-column lane chunk; the
  // weights of the next stage are in flight while the current one is summed
  // (two stages of 8 rows x 16 bytes per lane).
  uint4 gw[kGuRows], uw[kGuRows];
  float gs[kGuRows], us[kGuRows];
  auto load_rows = [&](Rsrc rq, Rsrc rs, int lc, uint4(&wv)[kGuRows], float(&ws)[kGuRows]) {
#pragma unroll
    for (int r = 0; r < kGuRows; ++r) {
      wv[r] = bload16(rq, (uint32_t)lc * 16, (uint32_t)(r0 + r) * rowq);
      ws[r] = bloadf(rs, (uint32_t)(lc >> 1) * 4, (uint32_t)(r0 + r) * groups * 4);
    }
  };
  auto load_planes = [&](int t, int lc, uint4(&xt)[kPlanes]) -> float {
#pragma unroll
    for (int j = 0; j < kPlanes; ++j) xt[j] = bload16(rx, (uint32_t)lc * 16, (uint32_t)(t * kPlanes + j) * words * 4);
    return bloadf(rxs, (uint32_t)lc * 4, (uint32_t)t * blocks * 4);
  };
  int lc = lane;
  if (lc < nch) load_rows(rqa, rsa, lc, gw, gs);
  for (; lc < nch; lc += 64) {
    load_rows(rqb, rsb, lc, uw, us);  // up rows in flight during the gate sums
    uint4 xp[NT == 1 ? kPlanes : 1];
    float sx1 = 0.0f;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      uint4 xt[kPlanes];
      const float sx = load_planes(tok[i], lc, xt);
      if (NT == 1) {
#pragma unroll
        for (int j = 0; j < kPlanes; ++j) xp[NT == 1 ? j : 0] = xt[j];
        sx1 = sx;
      }
#pragma unroll
      for (int r = 0; r < kGuRows; ++r) ga[r][i] = __builtin_fmaf((float)dot_planes(gw[r], xt), gs[r] * sx, ga[r][i]);
    }
    if (lc + 64 < nch) load_rows(rqa, rsa, lc + 64, gw, gs);  // next gate rows in flight during the up sums
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      uint4 xt[kPlanes];
      float sx;
      if (NT == 1) {
#pragma unroll
        for (int j = 0; j < kPlanes; ++j) xt[j] = xp[NT == 1 ? j : 0];
        sx = sx1;
      } else {
        sx = load_planes(tok[i], lc, xt);
      }
#pragma unroll
      for (int r = 0; r < kGuRows; ++r) ua[r][i] = __builtin_fmaf((float)dot_planes(uw[r], xt), us[r] * sx, ua[r][i]);
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

// All token passes of one slot; after each pass the block's 32 rows (one
// 32-column block of the down projection's input) are written as digit
// planes by wave 0, four lanes per token.
template <int NTMAX, class TokOf>
__device__ __forceinline__ void gate_up_slot(const DecodeProblem &P, const Slot &S, int row0, const TokOf &tok_of,
                                             float (*mid_lds)[4]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int I = P.I, words = I >> 3;
  for (int tc = 0; tc < S.cnt;) {
    const int left = S.cnt - tc;
    const int nt = (NTMAX >= 2 && left >= 2) ? 2 : 1;
    if (nt == 2)
      gate_up_pass<(NTMAX >= 2 ? 2 : 1)>(P, S, row0, tc, tok_of, mid_lds);
    else
      gate_up_pass<1>(P, S, row0, tc, tok_of, mid_lds);
    __syncthreads();
    if (wave == 0) {
      const int i = lane >> 2, w = lane & 3;
      const bool store = i < nt;
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = store ? mid_lds[8 * w + q][i & 3] : 0.0f;
      const size_t p = (size_t)(S.p_begin + tc + (store ? i : 0));
      quantize_word(v, w == 0, store, P.mq + p * kPlanes * words + (row0 >> 3) + w, (size_t)words,
                    P.ms + p * (I >> 5) + (row0 >> 5));
    }
    __syncthreads();
    tc += nt;
  }
}

__device__ __forceinline__ Slot expert_slot(const DecodeProblem &P, int e, int p_begin, int cnt) {
  const size_t qstride = (size_t)P.I * (P.h >> 1), sstride = (size_t)P.I * (P.h >> 6);
  Slot S;
  S.p_begin = p_begin;
  S.cnt = cnt;
  S.qa = P.gate.q + e * qstride;
  S.sa = P.gate.s + e * sstride;
  S.qb = P.up.q + e * qstride;
  S.sb = P.up.s + e * sstride;
  return S;
}

// grid = (I / 32, has_shared + n_routed_slots), 256 threads.  ROUTE: the
// small-batch routing is computed in the block (and published by block
// (0, has_shared)); otherwise it is read from the dispatch arrays.
template <int NTMAX, bool ROUTE>
__global__ __launch_bounds__(kGuWaves * 64, COLI_GU_MIN_WAVES) void gate_up_kernel(DecodeProblem P) {
  __shared__ float mid_lds[kGuWaves * kGuRows][4];
  __shared__ SmallRouting R;
  const int row0 = blockIdx.x * (kGuWaves * kGuRows);
  const int slot = (int)blockIdx.y - P.has_shared;
  if (slot < 0) {  // shared expert: every token, weight 1
    Slot S;
    S.p_begin = P.T * P.k;
    S.cnt = P.T;
    S.qa = P.sh_gate.q;
    S.sa = P.sh_gate.s;
    S.qb = P.sh_up.q;
    S.sb = P.sh_up.s;
    gate_up_slot<NTMAX>(P, S, row0, [](int i) { return i; }, mid_lds);
    return;
  }
  const int k = P.k;
  if (ROUTE) {
    route_small(P.logits, P.bias, P.T, P.E, k, P.rsf, R);
    if (blockIdx.x == 0 && slot == 0) publish_routing(R, P);
    if (slot >= R.n_active) return;  // uniform over the block
    const int b = R.seg_begin[slot];
    const Slot S = expert_slot(P, R.active[slot], b, R.seg_begin[slot + 1] - b);
    gate_up_slot<NTMAX>(P, S, row0, [&](int i) { return R.sorted_ids[b + i] / k; }, mid_lds);
  } else {
    if (slot >= *P.n_active) return;
    const int e = P.active[slot];
    const int b = P.offsets[e];
    const Slot S = expert_slot(P, e, b, P.offsets[e + 1] - b);
    const int32_t *sid = P.sorted_ids;
    gate_up_slot<NTMAX>(P, S, row0, [&](int i) { return sid[b + i] / k; }, mid_lds);
  }
}

// ---------------------------------------------------------------------------
// down + combine, small batches: out[t][r] = sum_j w[t,j] y_(t,j)[r] + y_sh[t][r]
// ---------------------------------------------------------------------------

// grid = h / kDcRows, blockDim = 64 * min(16, S) with S = T*k + T*has_shared
// "slots": slot a < T*k is assignment a (expert idx[a], intermediate row
// inv[a]), slot T*k + t the shared expert on token t.  Wave w computes the
// kDcRows output rows of the block for slots w, w + waves, ... (one memory
// round trip per slot) into LDS; the block then sums, per token and row,
// w_j * y_j in slot order and the shared row last.
__global__ __launch_bounds__(1024) void down_combine_kernel(DecodeProblem P, float *__restrict__ out) {
  __shared__ float part[kSmallT * (kMaxTopK + 1)][kDcRows];
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6), waves = blockDim.x >> 6;
  const int r0 = blockIdx.x * kDcRows;
  const int h = P.h, I = P.I, k = P.k, T = P.T;
  const int rowq = I >> 1, groups = I >> 6, words = I >> 3, blocks = I >> 5, nch = I >> 5;
  const int n_slots = T * k + (P.has_shared ? T : 0);
  const size_t qstride = (size_t)h * (I >> 1), sstride = (size_t)h * (I >> 6);
  const uint32_t qbytes = (uint32_t)h * rowq, sbytes = (uint32_t)h * groups * 4;
  const int n_rows_mid = T * k + (P.has_shared ? T : 0);
  const Rsrc rm = make_rsrc(P.mq, (uint32_t)n_rows_mid * kPlanes * words * 4);
  const Rsrc rms = make_rsrc(P.ms, (uint32_t)n_rows_mid * blocks * 4);
  for (int sl = wave; sl < n_slots; sl += waves) {
    const uint8_t *q;
    const float *sc;
    int p;
    if (sl < T * k) {
      const int e = uniform(P.idx[sl]);
      q = P.down.q + e * qstride;
      sc = P.down.s + e * sstride;
      p = uniform(P.inv[sl]);
    } else {
      q = P.sh_down.q;
      sc = P.sh_down.s;
      p = sl;  // T*k + t
    }
    const Rsrc rq = make_rsrc(q, qbytes), rs = make_rsrc(sc, sbytes);
    float acc[kDcRows];
#pragma unroll
    for (int r = 0; r < kDcRows; ++r) acc[r] = 0.0f;
    for (int lc = lane; lc < nch; lc += 64) {
      uint4 dw[kDcRows];
      float ds[kDcRows];
#pragma unroll
      for (int r = 0; r < kDcRows; ++r) {
        dw[r] = bload16(rq, (uint32_t)lc * 16, (uint32_t)(r0 + r) * rowq);
        ds[r] = bloadf(rs, (uint32_t)(lc >> 1) * 4, (uint32_t)(r0 + r) * groups * 4);
      }
      uint4 xp[kPlanes];
#pragma unroll
      for (int j = 0; j < kPlanes; ++j) xp[j] = bload16(rm, (uint32_t)lc * 16, (uint32_t)(p * kPlanes + j) * words * 4);
      const float sx = bloadf(rms, (uint32_t)lc * 4, (uint32_t)p * blocks * 4);
#pragma unroll
      for (int r = 0; r < kDcRows; ++r) acc[r] = __builtin_fmaf((float)dot_planes(dw[r], xp), ds[r] * sx, acc[r]);
    }
#pragma unroll
    for (int r = 0; r < kDcRows; ++r) {
      const float v = wave_sum(acc[r]);
      if (lane == r) part[sl][r] = v;  // kDcRows <= 64
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < T * kDcRows; i += blockDim.x) {
    const int t = i / kDcRows, r = i % kDcRows;
    float o = 0.0f;
    for (int j = 0; j < k; ++j) o = __builtin_fmaf(P.wsel[t * k + j], part[t * k + j][r], o);
    if (P.has_shared) o += part[T * k + t][r];
    out[(size_t)t * h + r0 + r] = o;
  }
}

// ---------------------------------------------------------------------------
// down (larger batches): y[p] = Wd mid[p]
// ---------------------------------------------------------------------------

template <int NT>
__device__ __forceinline__ void down_pass(const DecodeProblem &P, const uint8_t *q, const float *s, int p_begin,
                                          int r0, int tc) {
  const int lane = threadIdx.x & 63;
  const int I = P.I, rowq = I >> 1, groups = I >> 6, words = I >> 3, blocks = I >> 5, nch = I >> 5;
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
      dw[r] = ld16(q + row * rowq + (size_t)lc * 16);
      ds[r] = s[row * groups + (lc >> 1)];
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const size_t p = (size_t)(p_begin + tc + i);
      uint4 xp[kPlanes];
#pragma unroll
      for (int j = 0; j < kPlanes; ++j) xp[j] = ld16(P.mq + (p * kPlanes + j) * words + (size_t)lc * 4);
      const float sx = P.ms[p * blocks + lc];
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
      if (lane == 0) P.y[(size_t)(p_begin + tc + i) * P.h + r0 + r] = v;
    }
}

// grid = (h / 32, has_shared + n_routed_slots), 256 threads; slot 0 is the
// shared expert when there is one.
template <int NTMAX>
__global__ __launch_bounds__(kDnWaves * 64) void down_kernel(DecodeProblem P) {
  const int slot = (int)blockIdx.y - P.has_shared;
  const uint8_t *q;
  const float *s;
  int p_begin, cnt;
  if (slot < 0) {
    q = P.sh_down.q;
    s = P.sh_down.s;
    p_begin = P.T * P.k;
    cnt = P.T;
  } else {
    if (slot >= *P.n_active) return;
    const int e = P.active[slot];
    const size_t qstride = (size_t)P.h * (P.I >> 1), sstride = (size_t)P.h * (P.I >> 6);
    q = P.down.q + e * qstride;
    s = P.down.s + e * sstride;
    p_begin = P.offsets[e];
    cnt = P.offsets[e + 1] - p_begin;
  }
  const int r0 = (blockIdx.x * kDnWaves + (threadIdx.x >> 6)) * kDnRows;
  int tc = 0;
  if (NTMAX >= 4)
    for (; tc + 4 <= cnt; tc += 4) down_pass<4>(P, q, s, p_begin, r0, tc);
  if (NTMAX >= 2)
    for (; tc + 2 <= cnt; tc += 2) down_pass<2>(P, q, s, p_begin, r0, tc);
  for (; tc < cnt; ++tc) down_pass<1>(P, q, s, p_begin, r0, tc);
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

bool small_batch(int T, int k) { return T <= kSmallT && T * k <= kSmallAssign; }

hipError_t launch_gemv_gate_up(const DecodeProblem &P, hipStream_t s) {
  const int slots = P.n_routed_slots + (P.has_shared ? 1 : 0);
  if (slots == 0 || P.T == 0) return hipSuccess;
  dim3 grid(P.I / (kGuWaves * kGuRows), slots);
  // passes of at most two tokens: wider passes do not fit the register file
  const bool route = small_batch(P.T, P.k);
  if (P.T == 1) {
    if (route)
      return launch(gate_up_kernel<1, true>, grid, kGuWaves * 64, 0, s, P);
    else
      return launch(gate_up_kernel<1, false>, grid, kGuWaves * 64, 0, s, P);
  } else {
    if (route)
      return launch(gate_up_kernel<2, true>, grid, kGuWaves * 64, 0, s, P);
    else
      return launch(gate_up_kernel<2, false>, grid, kGuWaves * 64, 0, s, P);
  }
}

hipError_t launch_down_combine(const DecodeProblem &P, float *out, hipStream_t s) {
  if (P.T == 0) return hipSuccess;
  const int n_slots = P.T * P.k + (P.has_shared ? P.T : 0);
  const int waves = n_slots < 16 ? n_slots : 16;
  return launch(down_combine_kernel, P.h / kDcRows, waves * 64, 0, s, P, out);
}

hipError_t launch_gemv_down(const DecodeProblem &P, hipStream_t s) {
  const int slots = P.n_routed_slots + (P.has_shared ? 1 : 0);
  if (slots == 0 || P.T == 0) return hipSuccess;
  dim3 grid(P.h / (kDnWaves * kDnRows), slots);
  if (P.T == 1)
    return launch(down_kernel<1>, grid, kDnWaves * 64, 0, s, P);
  else if (P.T < 4)
    return launch(down_kernel<2>, grid, kDnWaves * 64, 0, s, P);
  else
    return launch(down_kernel<4>, grid, kDnWaves * 64, 0, s, P);
}

hipError_t launch_combine(const float *y, const float *w, const int32_t *inv, int T, int k, int h,
                          int has_shared, float *out, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  dim3 grid((h / 4 + 255) / 256, T);
  return launch(combine_kernel, grid, 256, 0, s, y, w, inv, T, k, h, has_shared, out);
}

}  // namespace coli
