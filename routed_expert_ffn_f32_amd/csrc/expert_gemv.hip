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
//   small batches (T <= 4): gate/up with the routing computed inside every
//             block (a few microseconds, identical in every block; one block
//             publishes it) and the (slot, row) pairs split evenly over the
//             waves of the grid; then down fused with the weighted combine
//             (no intermediate y in HBM).  See the kernels' own comments.
//   larger batches: selection and dispatch in their own launch, gate/up over
//             grid (I/32, slots) -- slot 0 the shared expert, the others the
//             active routed experts, a block owning 32 rows of I and writing
//             the SwiGLU result as digit planes -- then y per assignment and
//             a combine kernel.
#include "internal.h"
#include "select.h"
#include "small_route.h"
#include "wave.h"

namespace coli {
namespace {

constexpr int kGuRows = 4;                 // gate/up rows per wave
constexpr int kGuWaves = 32 / kGuRows;     // a block owns 32 rows of I
constexpr int kDnWaves = 4;  // down block (larger batches): 4 waves x 8 rows
constexpr int kDnRows = 8;

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

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
  // one token's planes and scales (a descriptor per token: the whole batch
  // may pass 4 GiB)
  auto load_planes = [&](int t, int lc, uint4(&xt)[kPlanes]) -> float {
    const Rsrc rx = make_rsrc(P.xq + (size_t)t * kPlanes * words, (uint32_t)kPlanes * words * 4);
    const Rsrc rxs = make_rsrc(P.xs + (size_t)t * blocks, (uint32_t)blocks * 4);
#pragma unroll
    for (int j = 0; j < kPlanes; ++j) xt[j] = bload16(rx, (uint32_t)lc * 16, (uint32_t)j * words * 4);
    return bloadf(rxs, (uint32_t)lc * 4, 0);
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
  const size_t x = table_index(P.slot_of, e);
  S.qa = P.gate.q + x * qstride;
  S.sa = P.gate.s + x * sstride;
  S.qb = P.up.q + x * qstride;
  S.sb = P.up.s + x * sstride;
  return S;
}

// grid = (I / 32, has_shared + n_routed_slots), 256 threads; the routing
// and dispatch arrays come from the selection launch.
template <int NTMAX>
__global__ __launch_bounds__(kGuWaves * 64, 1) void gate_up_kernel(DecodeProblem P) {
  __shared__ float mid_lds[kGuWaves * kGuRows][4];
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
  if (slot >= *P.n_active) return;
  const int e = P.active[slot];
  const int b = P.offsets[e];
  const Slot S = expert_slot(P, e, b, P.offsets[e + 1] - b);
  const int32_t *sid = P.sorted_ids;
  gate_up_slot<NTMAX>(P, S, row0, [&](int i) { return sid[b + i] / k; }, mid_lds);
}

// Larger batches, rows held in registers: a block is one wave, which loads
// its kGuRows gate and up rows (all columns: chunks lc = lane + 64 cc,
// cc < NCH) once, then runs every token of the slot through them, one token
// at a time, the next chunk's digit planes in flight during the current
// chunk's sums, and writes silu(g) * u of its rows to midf (float32).  Each
// weight row is read from HBM once per call.  One-wave blocks share nothing,
// so the waves of a SIMD drift apart: one loads its rows while another
// computes.
template <int NCH, class TokOf>
__device__ __forceinline__ void gate_up_tokens(const DecodeProblem &P, const Slot &S, int r0, const TokOf &tok_of) {
  static_assert(kGuRows == 4, "the up sums sit 4 lanes from the gate sums");
  const int lane = threadIdx.x & 63;
  const int h = P.h, I = P.I, rowq = h >> 1, groups = h >> 6, words = h >> 3, nch = h >> 5;
  // the rows: one descriptor per row, so lanes past the row read zeros
  uint4 gw[NCH][kGuRows], uw[NCH][kGuRows];
  float gs[NCH][kGuRows], us[NCH][kGuRows];
#pragma unroll
  for (int r = 0; r < kGuRows; ++r) {
    const size_t row = (size_t)(r0 + r);
    const Rsrc qa = make_rsrc(S.qa + row * rowq, (uint32_t)rowq), qb = make_rsrc(S.qb + row * rowq, (uint32_t)rowq);
    const Rsrc sa = make_rsrc(S.sa + row * groups, (uint32_t)groups * 4);
    const Rsrc sb = make_rsrc(S.sb + row * groups, (uint32_t)groups * 4);
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
      const uint32_t lc = (uint32_t)(lane + 64 * cc);
      gw[cc][r] = bload16(qa, lc * 16, 0);
      uw[cc][r] = bload16(qb, lc * 16, 0);
      gs[cc][r] = bloadf(sa, (lc >> 1) * 4, 0);
      us[cc][r] = bloadf(sb, (lc >> 1) * 4, 0);
    }
  }
  // a token's planes: [6][h/8] words and scales [h/32], a descriptor per
  // token (the whole batch may pass 4 GiB); lanes past the row read zeros
  // (they meet zero weights anyway)
  auto load_planes = [&](int tok, int cc, uint4 (&xt)[kPlanes], float &sx) {
    const Rsrc rx = make_rsrc(P.xq + (size_t)tok * kPlanes * words, (uint32_t)kPlanes * words * 4);
    const Rsrc rxs = make_rsrc(P.xs + (size_t)tok * nch, (uint32_t)nch * 4);
    const uint32_t lc = (uint32_t)(lane + 64 * cc);
#pragma unroll
    for (int j = 0; j < kPlanes; ++j) xt[j] = bload16(rx, lc * 16, (uint32_t)j * words * 4);
    sx = bloadf(rxs, lc * 4, 0);
  };
  const int cnt = S.cnt;
  uint4 xn[kPlanes];
  float sxn;
  int tk = cnt > 0 ? uniform(tok_of(0)) : 0;  // the current token
  if (cnt > 0) load_planes(tk, 0, xn, sxn);
  for (int t = 0; t < cnt; ++t) {
    const int tn = t + 1 < cnt ? uniform(tok_of(t + 1)) : 0;  // the next one, read a token ahead
    float ga[kGuRows], ua[kGuRows];
#pragma unroll
    for (int r = 0; r < kGuRows; ++r) ga[r] = ua[r] = 0.0f;
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
      uint4 xt[kPlanes];
#pragma unroll
      for (int j = 0; j < kPlanes; ++j) xt[j] = xn[j];
      const float sx = sxn;
      // the next (token, chunk)'s planes in flight during these sums
      if (cc + 1 < NCH)
        load_planes(tk, cc + 1, xn, sxn);
      else if (t + 1 < cnt)
        load_planes(tn, 0, xn, sxn);
#pragma unroll
      for (int r = 0; r < kGuRows; ++r) {
        ga[r] = __builtin_fmaf((float)dot_planes(gw[cc][r], xt), gs[cc][r] * sx, ga[r]);
        ua[r] = __builtin_fmaf((float)dot_planes(uw[cc][r], xt), us[cc][r] * sx, ua[r]);
      }
    }
    // lane l: the sum of gate row l % 4 (l % 8 < 4) or up row l % 4; lane
    // r < kGuRows brings in its up sum from a lane 4 away, and the four
    // lanes write 16 bytes
    float v[2 * kGuRows];
#pragma unroll
    for (int r = 0; r < kGuRows; ++r) v[r] = ga[r], v[kGuRows + r] = ua[r];
    const float g = rows_sum<2 * kGuRows>(v);
    const float u = dpp_f<kDppRowRor4>(g);
    if (lane < kGuRows) P.midf[(size_t)(S.p_begin + t) * I + r0 + lane] = g / (1.0f + expf(-g)) * u;
    tk = tn;
  }
}

// grid = (I / kGuRows, has_shared + n_routed_slots), one wave per block; the
// routing and dispatch arrays come from the selection launch.
template <int NCH>
__global__ __launch_bounds__(64) void gate_up_tok_kernel(DecodeProblem P) {
  const int r0 = blockIdx.x * kGuRows;
  const int slot = (int)blockIdx.y - P.has_shared;
  if (slot < 0) {  // shared expert: every token, weight 1
    Slot S;
    S.p_begin = P.T * P.k;
    S.cnt = P.T;
    S.qa = P.sh_gate.q;
    S.sa = P.sh_gate.s;
    S.qb = P.sh_up.q;
    S.sb = P.sh_up.s;
    gate_up_tokens<NCH>(P, S, r0, [](int i) { return i; });
    return;
  }
  const int k = P.k;
  if (slot >= *P.n_active) return;
  const int e = P.active[slot];
  const int b = P.offsets[e];
  const Slot S = expert_slot(P, e, b, P.offsets[e + 1] - b);
  const int32_t *sid = P.sorted_ids;
  gate_up_tokens<NCH>(P, S, r0, [&](int i) { return sid[b + i] / k; });
}

// midf [n][I] (float32) as digit planes mq [n][6][I/8] words and scales
// ms [n][I/32], one thread per 8-column word; the four words of a 32-column
// block are a quad of lanes (I/8 is a multiple of 8, so a quad never
// straddles two rows).
__global__ __launch_bounds__(256) void quantize_mid_kernel(const float *__restrict__ midf, int n, int I,
                                                           uint32_t *__restrict__ mq, float *__restrict__ ms) {
  const int words = I >> 3;
  const size_t wg = (size_t)blockIdx.x * 256 + threadIdx.x;
  const bool valid = wg < (size_t)n * words;
  const size_t p = valid ? wg / words : 0;
  const int w = valid ? (int)(wg % words) : 0;
  float v[8];
  if (valid) {
    const float4 a = *reinterpret_cast<const float4 *>(midf + p * I + 8 * w);
    const float4 b = *reinterpret_cast<const float4 *>(midf + p * I + 8 * w + 4);
    v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
  quantize_word(v, (w & 3) == 0, valid, mq + p * kPlanes * words + w, (size_t)words, ms + p * (I >> 5) + (w >> 2));
}

// ---------------------------------------------------------------------------
// Small batches (T <= kSmallT): row-streaming kernels.
//
// gate/up: the (slot, row) pairs of the call -- slot 0 the shared expert,
// then the active routed experts in ascending order, I rows each -- are split
// into equal contiguous runs, one per wave of the grid, so every wave streams
// the same number of gate and up rows whatever the routing.  A row is h/32
// chunks of 32 columns (16 bytes of codes each); lane l takes chunks
// l, l + 64, ..., so one wave-load covers 1 KB of a row.  A wave's first
// shared-expert row is requested while the block computes the routing;
// kSbDepth rows are in flight after that.  The hidden rows' digit planes are
// held in registers (T = 1) or in LDS (T = 2..4).  Each row ends in two wave
// reductions per token and one float32 store of silu(g) * u.
//
// down + combine: every wave owns a few output rows and streams them from
// each slot's down matrix in turn, against the slot's intermediate row held
// in LDS as digit planes (see the kernel's comment).
// ---------------------------------------------------------------------------
constexpr int kSbDepth = 2;     // gate/up rows in flight per wave
constexpr int kGuQueues = 64;               // gate/up row queues (atomic counters)
constexpr int kGuQueueStride = 64;          // int32: one counter per 256 bytes
static_assert(kGuQueues * kGuQueueStride == kRowQueueWords, "row queue words");
constexpr int kSbBlocks = 512;   // gate/up grid, T = 1 (4 waves per block)
constexpr int kSbBlocksLds = kSbBlocks / 2; // gate/up grid, T = 2..4 (8 waves per block)
constexpr int kDcWaves = 8;     // down: waves per block
constexpr int kDcBlocks = 256;   // down: blocks (at most; fewer when h is small)
constexpr int kDcLds = 64 * 1024;           // down: LDS for the digit planes of a slot group
// down: LDS up to which every slot's planes are kept at once (one block per
// CU either way).  GLM-like T = 2 (18 slots, 115 KB): 27.5-28.1 us against
// 28.9-30.3 us in groups of 10; T = 3 and 4 do not fit, and larger groups
// measured slower for them than groups of 10.
constexpr int kDcLdsAll = 144 * 1024;
constexpr int kSbMaxXLds = 96 * 1024;       // bytes of hidden-row planes staged in LDS
constexpr int kDcMaxChunks = 4;             // down: I <= 64*32*4
constexpr int kDcMaxRing = 2;    // down: slots in flight per wave, at most

// Where the gate/up rows of a slot come from, and its assignment positions.
struct GuCursor {
  int slot, r;              // slot and row of I
  const uint8_t *qg, *qu;   // gate and up codes of the slot's expert
  const float *sg, *su;     // and scales
  int p_begin, cnt;         // positions p_begin .. p_begin + cnt - 1 of mid
};

template <class F>
__device__ __forceinline__ void gu_set_slot(const DecodeProblem &P, const SmallRouting &R, GuCursor &c) {
  const int hs = P.has_shared;
  if (c.slot < hs) {
    c.qg = P.sh_gate.q;
    c.sg = P.sh_gate.s;
    c.qu = P.sh_up.q;
    c.su = P.sh_up.s;
    c.p_begin = P.T * P.k;
    c.cnt = P.T;
    return;
  }
  const int s = min(c.slot - hs, kSmallAssign - 1);
  const int e = uniform(R.active[s]);
  const size_t qstride = (size_t)P.I * F::row_bytes(P.h), sstride = (size_t)P.I * F::row_scales(P.h);
  const size_t x = table_index(P.slot_of, e);
  c.qg = P.gate.q + x * qstride;
  c.sg = P.gate.s + x * sstride;
  c.qu = P.up.q + x * qstride;
  c.su = P.up.s + x * sstride;
  c.p_begin = uniform(R.seg_begin[s]);
  c.cnt = uniform(R.seg_begin[s + 1]) - c.p_begin;
}

// NS: scales per lane (one per chunk for int4 gs64, the row's one for int8)
template <int NCH, class F = FmtI4>
struct GuBuf {
  static constexpr int NS = F::kRowScale ? 1 : NCH;
  uint4 g[NCH], u[NCH];
  float gs[NS], us[NS];
};

// Codes and scales of row c.r of the slot's gate and up matrices for this
// lane's chunks; an invalid row (or chunks past the row) reads zeros.
template <int NCH, class F>
__device__ __forceinline__ void gu_load(GuBuf<NCH, F> &b, const GuCursor &c, bool valid, int h) {
  const int lane = threadIdx.x & 63;
  const uint32_t rowq = F::row_bytes(h), nsc = F::row_scales(h), rows = nsc * 4;
  const size_t r = (size_t)c.r;
  const Rsrc qg = make_rsrc(c.qg + r * rowq, valid ? rowq : 0u);
  const Rsrc qu = make_rsrc(c.qu + r * rowq, valid ? rowq : 0u);
  const Rsrc sg = make_rsrc(c.sg + r * nsc, valid ? rows : 0u);
  const Rsrc su = make_rsrc(c.su + r * nsc, valid ? rows : 0u);
#pragma unroll
  for (int cc = 0; cc < NCH; ++cc) {
    const uint32_t lc = (uint32_t)(lane + 64 * cc);
    b.g[cc] = bload16(qg, lc * 16, 0);
    b.u[cc] = bload16(qu, lc * 16, 0);
  }
  if constexpr (F::kRowScale) {
    b.gs[0] = bloadf(sg, 0, 0);
    b.us[0] = bloadf(su, 0, 0);
  } else {
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
      const uint32_t lc = (uint32_t)(lane + 64 * cc);
      b.gs[cc] = bloadf(sg, (lc >> 1) * 4, 0);
      b.us[cc] = bloadf(su, (lc >> 1) * 4, 0);
    }
  }
}

// silu(g) * u of one row for every token of the slot, stored as float32.
// XREG: the single token's planes are xr/xsr; otherwise they are read from
// LDS (planes [T][XP][nch] as uint4, then scales [T][h/32]), one token at a
// time.
template <int NCH, bool XREG, class F>
__device__ __forceinline__ void gu_consume(const GuBuf<NCH, F> &b, const GuCursor &c, bool valid,
                                           const uint4 (&xr)[XREG ? NCH : 1][F::kXPlanes],
                                           const float (&xsr)[XREG ? NCH : 1], const uint4 *xl, int nch,
                                           const SmallRouting &R, const DecodeProblem &P) {
  constexpr int XP = F::kXPlanes, CPB = 32 / F::kChunkCols;  // chunks per activation block
  const int lane = threadIdx.x & 63;
  const int cnt = XREG ? 1 : c.cnt, n_routed = P.T * P.k, nblk = P.h >> 5;
  for (int t = 0; t < cnt; ++t) {
    float g = 0.0f, u = 0.0f;
    const int pos = c.p_begin + t;
    const int tok = XREG ? 0 : pos < n_routed ? uniform(R.sorted_ids[pos]) / P.k : pos - n_routed;
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
      uint4 xt[XP];
      float sx;
      if (XREG) {
#pragma unroll
        for (int j = 0; j < XP; ++j) xt[j] = xr[XREG ? cc : 0][j];
        sx = xsr[XREG ? cc : 0];
      } else {
        const int lc = min(lane + 64 * cc, nch - 1);  // lanes past the row meet zero weights
#pragma unroll
        for (int j = 0; j < XP; ++j) xt[j] = xl[(tok * XP + j) * nch + lc];
        sx = reinterpret_cast<const float *>(xl + P.T * XP * nch)[tok * nblk + lc / CPB];
      }
      if constexpr (F::kRowScale) {
        g = __builtin_fmaf(F::dot(b.g[cc], xt), sx, g);
        u = __builtin_fmaf(F::dot(b.u[cc], xt), sx, u);
      } else {
        g = __builtin_fmaf(F::dot(b.g[cc], xt), b.gs[cc] * sx, g);
        u = __builtin_fmaf(F::dot(b.u[cc], xt), b.us[cc] * sx, u);
      }
    }
    if (valid) {
      float gg = wave_sum(g);
      float uu = wave_sum(u);
      if constexpr (F::kRowScale) {
        gg *= b.gs[0];
        uu *= b.us[0];
      }
      if (lane == 0) P.midf[(size_t)(c.p_begin + t) * P.I + c.r] = gg / (1.0f + expf(-gg)) * uu;
    }
  }
}

// grid = kSbBlocks (XREG: 4 waves) or kSbBlocksLds (8 waves) blocks.  Dynamic
// LDS: the hidden rows' digit planes [T][6][h/32] uint4, then scales
// [T][h/32].
//
// Every load is issued at a program point that all waves pass, with invalid
// rows reading zeros instead of being skipped, so the compiler's waits count
// exactly the loads issued after the ones awaited.  XREG (one token): wave
// 0 alone merges the selection and hands the routing to the other waves
// through an LDS flag, so that it never waits for waves stalled on issuing
// row loads; with several tokens the merging waves meet at a block barrier.
template <int NCH, bool XREG, class F>
__global__ __launch_bounds__(XREG ? 256 : 512) void gate_up_rows_kernel(DecodeProblem P) {
  extern __shared__ uint4 xl[];
  __shared__ SmallRouting R;
  __shared__ int routed;  // XREG: set by wave 0 once R holds the routing
  constexpr int kWaves = XREG ? 4 : 8;
  constexpr int XP = F::kXPlanes, CPB = 32 / F::kChunkCols;
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int h = P.h, I = P.I, T = P.T, nch = h / F::kChunkCols, nblk = h >> 5;
  uint4 xr[XREG ? NCH : 1][XP];
  float xsr[XREG ? NCH : 1];
  // 1. the selection inputs
  SelectInput sel;
  route_small_load(P.logits, P.bias, T, P.E, P.k, sel);
  // 2. the hidden rows' digit planes (written by the router launch), loaded
  // once per block (a share per thread, no branch) and kept in LDS; with
  // one token each wave then takes its lanes' chunks into registers
  const int nx = T * XP * nch, nxs = T * nblk;  // uint4 plane chunks, scales
  const Rsrc rx = make_rsrc(P.xq, (uint32_t)nx * 16), rxs = make_rsrc(P.xs, (uint32_t)nxs * 4);
  constexpr int kXPer = 5, kXsPer = 2;
  uint4 xv[kXPer];
  float xsv[kXsPer];
#pragma unroll
  for (int j = 0; j < kXPer; ++j) xv[j] = bload16(rx, (uint32_t)(threadIdx.x + j * blockDim.x) * 16, 0);
#pragma unroll
  for (int j = 0; j < kXsPer; ++j) xsv[j] = bloadf(rxs, (uint32_t)(threadIdx.x + j * blockDim.x) * 4, 0);
  // these small loads complete before any row is requested: behind the row
  // requests in the memory queues their latency grows several-fold, and the
  // routing, which needs them, is what the block waits for
  __builtin_amdgcn_s_waitcnt(0);
  // 3. the rows.  Flat row f < hs*I is row f of the shared expert (no
  // routing needed), f = hs*I + s*I + r row r of the s-th active routed
  // expert.  Wave gw takes row gw first if it is a shared row (requested
  // during the routing); the rows from P0 = min(W, hs*I) on are handed out
  // at run time: queue q = gw mod kGuQueues holds rows P0 + q + kGuQueues i,
  // i = 0, 1, ..., and a wave takes the next i of its queue with one atomic
  // increment, so waves that stream faster take more rows and all waves end
  // together.
  const int64_t W = (int64_t)gridDim.x * kWaves, gw = (int64_t)blockIdx.x * kWaves + wave;
  const int hs = P.has_shared, P0 = (int)min<int64_t>(W, (int64_t)hs * I);
  int32_t *const qctr = P.queues + (int)(gw % kGuQueues) * kGuQueueStride;
  const int qoff = P0 + (int)(gw % kGuQueues);
  constexpr int D = NCH > 4 ? 1 : kSbDepth;  // wide rows: one in flight (register file)
  GuBuf<NCH, F> bs;  // the wave's first shared row
  GuBuf<NCH, F> buf[D];
  GuCursor cs{};
  const bool has0 = gw < P0;
  if (has0) {
    cs.slot = 0;
    gu_set_slot<F>(P, R, cs);  // the shared expert: no routing needed
    cs.r = (int)gw;
  }
  // one atomic increment of this wave's queue: lane 0 receives the index of
  // its next row (read with uniform() only where it is used, so that the
  // wait for it comes as late as possible).  The first D + 1 indices are
  // requested now: they need no routing, and arrive while it is computed.
  auto grab = [&]() -> int {
    int v = 0;
    if (lane == 0) v = __hip_atomic_fetch_add(qctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return v;
  };
  int gi[D + 1];
#pragma unroll
  for (int d = 0; d <= D; ++d) gi[d] = grab();
  // the planes into LDS (more than one batch only for several long rows)
  float *xsl = reinterpret_cast<float *>(xl + nx);
#pragma unroll
  for (int j = 0; j < kXPer; ++j) {
    const int i = threadIdx.x + j * blockDim.x;
    if (i < nx) xl[i] = xv[j];
  }
#pragma unroll
  for (int j = 0; j < kXsPer; ++j) {
    const int i = threadIdx.x + j * blockDim.x;
    if (i < nxs) xsl[i] = xsv[j];
  }
  for (int i = threadIdx.x + kXPer * blockDim.x; i < nx; i += blockDim.x) xl[i] = bload16(rx, (uint32_t)i * 16, 0);
  for (int i = threadIdx.x + kXsPer * blockDim.x; i < nxs; i += blockDim.x) xsl[i] = bloadf(rxs, (uint32_t)i * 4, 0);
  if (XREG && threadIdx.x == 0) routed = 0;
  // 4. the routing of the batch: phase A (ends with a block barrier, which
  // also publishes the planes and the flag), then phase B
  route_small_a(sel, T, P.E, P.k, R);
  if (XREG) {  // token 0's planes for this lane's chunks (zeros past the row)
#pragma unroll
    for (int cc = 0; cc < (XREG ? NCH : 1); ++cc) {
      const int lc = lane + 64 * cc;
      const bool in = lc < nch;
#pragma unroll
      for (int j = 0; j < XP; ++j) xr[cc][j] = in ? xl[j * nch + lc] : make_uint4(0, 0, 0, 0);
      xsr[cc] = in ? xsl[lc / CPB] : 0.0f;
    }
  }
  bool have_routing = true;
  if (XREG) {
    if (wave == 0) {
      route_small_b1(P.E, P.k, P.rsf, P.lim, R);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // R written before the flag
      __hip_atomic_store(&routed, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    gu_load(bs, cs, has0, h);
    if (wave != 0) {
      // wave 0 sets the flag without waiting for any other wave; the bound
      // only guards against a hang: a wave that gives up streams no routed
      // row (the rows it took from its queue stay uncomputed) and stores 1
      // in the error word, so the call is reported as failed
      int spins = 0;
      while (__hip_atomic_load(&routed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0 &&
             ++spins < P.spin_limit)
        __builtin_amdgcn_s_sleep(1);
      asm volatile("" ::: "memory");  // R is read after the flag
      have_routing = __builtin_amdgcn_readfirstlane(spins < P.spin_limit ? 1 : 0) != 0;
      // every lane stores the same word: a store under a lane condition
      // here made the compiler keep the wave's uniform values in VGPRs
      if (!have_routing) __hip_atomic_store(P.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else {
    route_small_b(T, P.E, P.k, P.rsf, P.lim, R);
    gu_load(bs, cs, has0, h);
  }
  // rows of the call (a wave without the routing stops after the shared ones)
  const int N = hs * I + (have_routing ? R.n_active * I : 0);
  auto cursor_of = [&](int f, GuCursor &c) {
    const int fr = f - hs * I;
    c.slot = fr < 0 ? 0 : hs + fr / I;
    c.r = fr < 0 ? f : fr % I;
    gu_set_slot<F>(P, R, c);
  };
  auto row_of = [&](int i) { return qoff + kGuQueues * i < N ? qoff + kGuQueues * i : -1; };
  // 5. the handed-out rows through a ring of D buffers.  The index of the
  // next row is requested one step before it is used, and before that step's
  // row loads, so that waiting for it never waits for them.
  int fr[D];
  GuCursor cur[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    fr[d] = row_of(uniform(gi[d]));
    cur[d] = GuCursor{};
    if (fr[d] >= 0) cursor_of(fr[d], cur[d]);
    gu_load(buf[d], cur[d], fr[d] >= 0, h);
  }
  int pend = gi[D];
  if (blockIdx.x == 0 && have_routing) {
    const RoutingOut o{P.idx, P.wsel, P.sorted_ids, P.inv, P.offsets, P.active, P.n_active};
    publish_routing(R, T, P.k, P.E, o);
  }
  gu_consume<NCH, XREG, F>(bs, cs, has0, xr, xsr, xl, nch, R, P);
  // A queue hands out rows in increasing order, so once a ring entry is past
  // the end every later one is too.  The loop body is straight-line: absent
  // rows are summed from zeros and not stored, and every step issues its
  // atomic and its loads (absent rows read nothing), so the compiler's waits
  // count exactly the operations issued after the ones awaited.
  bool more = fr[0] >= 0;
#pragma unroll
  for (int d = 1; d < D; ++d) more = more || fr[d] >= 0;
  while (more) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      gu_consume<NCH, XREG, F>(buf[d], cur[d], fr[d] >= 0, xr, xsr, xl, nch, R, P);
      const int f = row_of(uniform(pend));
      pend = grab();
      fr[d] = f;
      if (f >= 0) cursor_of(f, cur[d]);
      gu_load(buf[d], cur[d], f >= 0, h);
    }
    more = fr[0] >= 0;
#pragma unroll
    for (int d = 1; d < D; ++d) more = more || fr[d] >= 0;
  }
}

template <int NCHD, class F>
struct DnBuf {
  static constexpr int NS = F::kRowScale ? 1 : NCHD;
  uint4 w[NCHD];
  float s[NS];
};

template <int NCHD, class F>
__device__ __forceinline__ void dn_load(DnBuf<NCHD, F> &b, const uint8_t *q, const float *sc, int row, bool valid,
                                        int I) {
  const int lane = threadIdx.x & 63;
  const uint32_t rowq = F::row_bytes(I), nsc = F::row_scales(I), rows = nsc * 4;
  const Rsrc rq = make_rsrc(q + (size_t)row * rowq, valid ? rowq : 0u);
  const Rsrc rs = make_rsrc(sc + (size_t)row * nsc, valid ? rows : 0u);
#pragma unroll
  for (int cc = 0; cc < NCHD; ++cc) b.w[cc] = bload16(rq, (uint32_t)(lane + 64 * cc) * 16, 0);
  if constexpr (F::kRowScale) {
    b.s[0] = bloadf(rs, 0, 0);
  } else {
#pragma unroll
    for (int cc = 0; cc < NCHD; ++cc) b.s[cc] = bloadf(rs, (uint32_t)((lane + 64 * cc) >> 1) * 4, 0);
  }
}

// Slot q of the down sequence: tokens in order; for each token its
// shared-expert slot first (those rows need no routing, so they can be
// requested before the routing has arrived), then its k routed assignments
// in slot order.  The block keeps the routing of every slot in LDS: expert
// (-1 for the shared expert, kDnDropped for a slot the routing limits
// dropped), position of the intermediate row, combine weight; one entry per
// thread of the block (entries past the last slot are written and never
// read).  A dropped slot reads no weights (its loads have an empty range
// and return zeros), has weight 0 and points at position 0, always a kept
// assignment's row, so that it adds exactly zero.
struct DnTable {
  int32_t e[kDcWaves * 64];
  int32_t p[kDcWaves * 64];
  float w[kDcWaves * 64];
};

constexpr int kDnDropped = -2;

struct DnSlot {
  const uint8_t *q;
  const float *s;
  int t;
  float w;
  bool live;  // false: a dropped slot, no rows read
};

// Thread q reads the routing of slot q (every slot has a thread: the block
// is larger than kSmallAssign + kSmallT); buffer loads without a branch,
// absent entries read zeros.
__device__ __forceinline__ void dn_table_load(const DecodeProblem &P, uint32_t (&v)[3]) {
  const int ks = P.k + P.has_shared, n_slots = P.T * ks, n_routed = P.T * P.k;
  const int qs = threadIdx.x, t = qs / ks, j = qs % ks - P.has_shared;
  const uint32_t off = qs < n_slots && j >= 0 ? (uint32_t)(t * P.k + j) * 4 : 0x7fff0000u;
  const uint32_t bytes = (uint32_t)n_routed * 4;
  v[0] = __float_as_uint(bloadf(make_rsrc(P.idx, bytes), off, 0));
  v[1] = __float_as_uint(bloadf(make_rsrc(P.inv, bytes), off, 0));
  v[2] = __float_as_uint(bloadf(make_rsrc(P.wsel, bytes), off, 0));
}

// Stores without a branch: a store under a branch would let the compiler
// sink the loads behind the rows requested after them.
__device__ __forceinline__ void dn_table_store(const DecodeProblem &P, const uint32_t (&v)[3], DnTable &D) {
  const int ks = P.k + P.has_shared;
  const int qs = threadIdx.x, t = qs / ks, j = qs % ks - P.has_shared;
  const bool routed = j >= 0, dropped = routed && (int)v[0] < 0;
  D.e[qs] = dropped ? kDnDropped : routed ? (int)v[0] : -1;
  D.p[qs] = dropped ? 0 : routed ? (int)v[1] : P.T * P.k + t;
  D.w[qs] = routed ? __uint_as_float(v[2]) : 1.0f;
}

__device__ __forceinline__ DnSlot dn_shared_slot(const DecodeProblem &P, int t) {
  return DnSlot{P.sh_down.q, P.sh_down.s, t, 1.0f, true};
}

template <class F>
__device__ __forceinline__ DnSlot dn_slot(const DecodeProblem &P, const DnTable &D, int qs) {
  DnSlot d;
  d.t = qs / (P.k + P.has_shared);
  const int e = uniform(D.e[qs]);
  d.live = e != kDnDropped;
  if (e >= 0) {
    const size_t x = table_index(P.slot_of, e);
    d.q = P.down.q + x * ((size_t)P.h * F::row_bytes(P.I));
    d.s = P.down.s + x * ((size_t)P.h * F::row_scales(P.I));
  } else if (e == -1) {
    d.q = P.sh_down.q;
    d.s = P.sh_down.s;
  } else {
    d.q = P.down.q;
    d.s = P.down.s;
  }
  d.w = __builtin_bit_cast(float, uniform(__builtin_bit_cast(int, D.w[qs])));
  return d;
}

__device__ __forceinline__ int dn_slot_token(const DecodeProblem &P, int qs) { return qs / (P.k + P.has_shared); }

// Slots in flight per wave in the down kernel: kDcMaxRing (two by default;
// deeper rings delay the reads of the intermediate rows, which every block
// waits for, more than they gain), fewer if the row buffers would pass about
// 96 VGPRs (5 per row and 32-column chunk), never below two.
template <int NCHD, int RM>
constexpr int dc_ring() {
  constexpr int n = 96 / (5 * NCHD * RM);
  return n < 2 ? 2 : n > kDcMaxRing ? kDcMaxRing : n;
}

// Down projection fused with the weighted combine, small batches.
// grid = Gd blocks of kDcWaves waves; wave w of the grid owns output rows
// [w h / W, (w + 1) h / W) (at most RM).  The intermediate rows are first
// written into LDS as digit planes (one thread per 8-column word, the four
// lanes of a quad sharing a 32-column block: [row][plane][chunk] uint4, then
// [row][chunk] scales); then every wave streams, slot by slot, its rows of
// the slot's down matrix, NS slots in flight (a ring of register buffers:
// buffer u holds slot base + u), and keeps per lane
// acc[r] += w_slot * (partial dot product of row r).  When the token
// changes the 64 lane partials of each row are summed (one wave reduction
// per row and token) into out: the weighted sum over the token's slots is
// formed before the reduction over lanes instead of after it.
//
// The ring's first slots are requested before the intermediate rows have
// arrived (their reads take microseconds: every block reads all of them),
// so HBM streams weights during the wait.  BYPOS: every intermediate row
// fits in LDS at once and is kept there by position (they are n_slots
// consecutive rows, so their loads need no routing and go out with it);
// otherwise the slots are taken in groups of gs, kept by slot, the next
// group quantised when the ring reaches it.  No load is issued under a
// branch that depends on the data, so the compiler's waits count exactly
// the loads issued after the ones awaited.
template <int NCHD, int RM, bool BYPOS, class F>
__global__ __launch_bounds__(kDcWaves * 64) void down_combine_rows_kernel(DecodeProblem P, float *__restrict__ out,
                                                                         int gs) {
  static_assert(kDcWaves * 64 >= kSmallAssign + kSmallT, "one thread per slot of the routing table");
  constexpr int NS = dc_ring<NCHD, RM>();
  constexpr int XP = F::kXPlanes, CPB = 32 / F::kChunkCols;
  extern __shared__ uint4 ml[];
  __shared__ DnTable tab;
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  // nchd 16-byte chunks of a down row; activation blocks of 32 and words of
  // 8 intermediate columns
  const int h = P.h, I = P.I, nchd = I / F::kChunkCols, nblk = I >> 5, words = I >> 3;
  const int n_slots = P.T * (P.k + P.has_shared);
  const int64_t W = (int64_t)gridDim.x * kDcWaves, gw = (int64_t)blockIdx.x * kDcWaves + wave;
  const int r0 = (int)((int64_t)h * gw / W), nr = (int)((int64_t)h * (gw + 1) / W) - r0;
  float *msc = reinterpret_cast<float *>(ml + (size_t)gs * XP * nchd);
  uint32_t *mw = reinterpret_cast<uint32_t *>(ml);
  const Rsrc rmid = make_rsrc(P.midf, (uint32_t)n_slots * I * 4);
  constexpr int kBatch = 5;  // 8-column words per thread and batch
  const int batch = kBatch * (int)blockDim.x;
  float acc[RM];
#pragma unroll
  for (int r = 0; r < RM; ++r) acc[r] = 0.0f;
  DnBuf<NCHD, F> buf[NS][RM];
  DnSlot ring[NS];

  // byte offsets of the batch's words in midf (past the group: an offset
  // that reads zeros); BYPOS: consecutive, else through the slots' positions
  auto mid_offsets = [&](int g0, int gn, int base, uint32_t (&off)[kBatch]) {
    const int total = gn * words;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = base + j * (int)blockDim.x + (int)threadIdx.x;
      if (BYPOS) {
        off[j] = i < total ? (uint32_t)i * 32 : 0x7fff0000u;
      } else {
        const int sl = min(i / words, gn - 1);
        off[j] = i < total ? (uint32_t)(((size_t)tab.p[g0 + sl] * I + 8 * (i % words)) * 4) : 0x7fff0000u;
      }
    }
  };
  auto mid_load = [&](const uint32_t (&off)[kBatch], uint4 (&va)[kBatch], uint4 (&vc)[kBatch]) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      va[j] = bload16(rmid, off[j], 0);
      vc[j] = bload16(rmid, off[j] + 16, 0);
    }
  };
  auto quantize = [&](int gn, int base, const uint4 (&va)[kBatch], const uint4 (&vc)[kBatch]) {
    const int total = gn * words;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = base + j * (int)blockDim.x + (int)threadIdx.x;
      const bool valid = i < total;
      const int sl = valid ? i / words : 0, w = valid ? i % words : 0;
      const float v[8] = {__uint_as_float(va[j].x), __uint_as_float(va[j].y), __uint_as_float(va[j].z),
                          __uint_as_float(va[j].w), __uint_as_float(vc[j].x), __uint_as_float(vc[j].y),
                          __uint_as_float(vc[j].z), __uint_as_float(vc[j].w)};
      F::quantize(v, (w & 3) == 0, valid, mw + (size_t)sl * XP * nchd * 4, I, w, msc + sl * nblk + (w >> 2));
    }
  };
  // the rest of a group's words, one batch at a time (several batches only
  // for long intermediate rows or several groups)
  auto quantize_rest = [&](int g0, int gn, int base0) {
    for (int base = base0; base < gn * words; base += batch) {
      uint32_t off[kBatch];
      uint4 va[kBatch], vc[kBatch];
      mid_offsets(g0, gn, base, off);
      mid_load(off, va, vc);
      quantize(gn, base, va, vc);
    }
  };
  // slot qs (past the last: no rows) into ring buffer u
  auto ring_load = [&](int u, int qs) {
    const bool v = qs < n_slots;
    ring[u] = v ? dn_slot<F>(P, tab, qs) : DnSlot{};
#pragma unroll
    for (int r = 0; r < RM; ++r) dn_load(buf[u][r], ring[u].q, ring[u].s, r0 + r, v && ring[u].live && r < nr, I);
  };

  // prologue: the routing table and the first batch of intermediate words,
  // then the ring's rows; the quantisation waits for the words only
  {
    const int gn = min(gs, n_slots);
    uint32_t tv[3];
    dn_table_load(P, tv);
    uint32_t off[kBatch];
    uint4 va[kBatch], vc[kBatch];
    if (BYPOS) {
      mid_offsets(0, gn, 0, off);
      mid_load(off, va, vc);
      // every wave's words requested before any row: a row request ahead
      // of them in the memory pipeline would hold them for an HBM latency
      block_barrier();
      // a shared expert's first slot needs no routing: its rows go out now
      ring[0] = dn_shared_slot(P, 0);
#pragma unroll
      for (int r = 0; r < RM; ++r) dn_load(buf[0][r], ring[0].q, ring[0].s, r0 + r, P.has_shared && r < nr, I);
    }
    dn_table_store(P, tv, tab);
    block_barrier();
    if (!BYPOS) {
      mid_offsets(0, gn, 0, off);
      mid_load(off, va, vc);
    }
    if (!BYPOS || !P.has_shared) ring_load(0, 0);
#pragma unroll
    for (int u = 1; u < NS; ++u) ring_load(u, u);
    quantize(gn, 0, va, vc);
    quantize_rest(0, gn, batch);
    block_barrier();
  }

  for (int base = 0; base < n_slots; base += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int qc = base + u;
      int sl = 0;
      if (BYPOS) {
        sl = qc < n_slots ? uniform(tab.p[qc]) : 0;
      } else {
        const int g0 = qc - qc % gs;
        if (qc < n_slots && qc == g0 && qc > 0) {  // uniform over the block: the next group's planes
          block_barrier();                          // the previous group's are no longer read
          quantize_rest(g0, min(gs, n_slots - g0), 0);
          block_barrier();
        }
        sl = qc - g0;
      }
      if (qc < n_slots) {
        const DnSlot &sc = ring[u];
        float part[RM];  // int8: the slot's sums before its row scales
#pragma unroll
        for (int r = 0; r < RM; ++r) part[r] = 0.0f;
#pragma unroll
        for (int cc = 0; cc < NCHD; ++cc) {
          const int lc = min(lane + 64 * cc, nchd - 1);  // lanes past the row meet zero weights
          uint4 xp[XP];
#pragma unroll
          for (int j2 = 0; j2 < XP; ++j2) xp[j2] = ml[(sl * XP + j2) * nchd + lc];
          const float sx = msc[sl * nblk + lc / CPB] * sc.w;
#pragma unroll
          for (int r = 0; r < RM; ++r) {
            if constexpr (F::kRowScale)
              part[r] = __builtin_fmaf(F::dot(buf[u][r].w[cc], xp), sx, part[r]);
            else
              acc[r] = __builtin_fmaf(F::dot(buf[u][r].w[cc], xp), buf[u][r].s[cc] * sx, acc[r]);
          }
        }
        if constexpr (F::kRowScale) {
#pragma unroll
          for (int r = 0; r < RM; ++r) acc[r] = __builtin_fmaf(part[r], buf[u][r].s[0], acc[r]);
        }
        // the token's last slot: reduce and store
        if (qc + 1 == n_slots || dn_slot_token(P, qc + 1) != sc.t) {
#pragma unroll
          for (int r = 0; r < RM; ++r) {
            if (r < nr) {
              const float v = wave_sum(acc[r]);
              if (lane == 0) out[(size_t)sc.t * h + r0 + r] = v;
            }
            acc[r] = 0.0f;
          }
        }
      }
      ring_load(u, qc + NS);
    }
  }
  // the gate/up launch of the next call finds its row queues at zero
  if (blockIdx.x == 0 && (int)threadIdx.x < kGuQueues)
    __hip_atomic_store(P.queues + threadIdx.x * kGuQueueStride, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
    q = P.down.q + table_index(P.slot_of, e) * qstride;
    s = P.down.s + table_index(P.slot_of, e) * sstride;
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

// Larger batches, rows held in registers: a block is one wave, which loads
// R down rows (all columns: chunks lc = lane + 64 cc, cc < NCHD) once and
// runs every intermediate row of the slot through them, the next chunk's
// digit planes in flight during the current chunk's sums.
template <int NCHD, int R>
__global__ __launch_bounds__(64) void down_tok_kernel(DecodeProblem P) {
  const int lane = threadIdx.x & 63;
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
    q = P.down.q + table_index(P.slot_of, e) * qstride;
    s = P.down.s + table_index(P.slot_of, e) * sstride;
    p_begin = P.offsets[e];
    cnt = P.offsets[e + 1] - p_begin;
  }
  const int h = P.h, I = P.I, rowq = I >> 1, groups = I >> 6, words = I >> 3, nch = I >> 5;
  const int r0 = blockIdx.x * R;
  uint4 dw[NCHD][R];
  float ds[NCHD][R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const size_t row = (size_t)(r0 + r);
    const Rsrc rq = make_rsrc(q + row * rowq, (uint32_t)rowq), rs = make_rsrc(s + row * groups, (uint32_t)groups * 4);
#pragma unroll
    for (int cc = 0; cc < NCHD; ++cc) {
      const uint32_t lc = (uint32_t)(lane + 64 * cc);
      dw[cc][r] = bload16(rq, lc * 16, 0);
      ds[cc][r] = bloadf(rs, (lc >> 1) * 4, 0);
    }
  }
  // an intermediate row's planes [6][I/8] words and scales [I/32], a
  // descriptor per row; lanes past the row read zeros
  auto load_planes = [&](int p, int cc, uint4 (&xt)[kPlanes], float &sx) {
    const Rsrc rx = make_rsrc(P.mq + (size_t)p * kPlanes * words, (uint32_t)kPlanes * words * 4);
    const Rsrc rxs = make_rsrc(P.ms + (size_t)p * nch, (uint32_t)nch * 4);
    const uint32_t lc = (uint32_t)(lane + 64 * cc);
#pragma unroll
    for (int j = 0; j < kPlanes; ++j) xt[j] = bload16(rx, lc * 16, (uint32_t)j * words * 4);
    sx = bloadf(rxs, lc * 4, 0);
  };
  uint4 xn[kPlanes];
  float sxn;
  if (cnt > 0) load_planes(p_begin, 0, xn, sxn);
  for (int t = 0; t < cnt; ++t) {
    const int p = p_begin + t;
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0f;
#pragma unroll
    for (int cc = 0; cc < NCHD; ++cc) {
      uint4 xt[kPlanes];
#pragma unroll
      for (int j = 0; j < kPlanes; ++j) xt[j] = xn[j];
      const float sx = sxn;
      if (cc + 1 < NCHD)
        load_planes(p, cc + 1, xn, sxn);
      else if (t + 1 < cnt)
        load_planes(p + 1, 0, xn, sxn);
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = __builtin_fmaf((float)dot_planes(dw[cc][r], xt), ds[cc][r] * sx, acc[r]);
    }
    // lane r < R holds row r's sum; R lanes write 4R contiguous bytes
    const float y = rows_sum<R>(acc);
    if (lane < R) P.y[(size_t)p * h + r0 + lane] = y;
  }
}

// out[t][c..c+3]; the k slot weights and positions are loaded first (up to
// kMaxTopK, uniform per block), then all expert rows, then summed in slot
// order and the shared row added last.
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ y, const float *__restrict__ w,
                                                      const int32_t *__restrict__ idx, const int32_t *__restrict__ inv,
                                                      int T, int k, int h, int has_shared, float *__restrict__ out) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= h) return;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int j0 = 0; j0 < k; j0 += 8) {
    float wj[8];
    float4 v[8];
    bool live[8];  // a slot of the token that the routing kept
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int a = t * k + min(j0 + u, k - 1);
      live[u] = j0 + u < k && idx[a] >= 0;
      wj[u] = w[a];
      v[u] = live[u] ? *reinterpret_cast<const float4 *>(y + (size_t)inv[a] * h + c) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (live[u]) {
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

namespace {
__global__ void fill_i32_kernel(int32_t *p, int n, int32_t v) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}
}  // namespace

hipError_t launch_fill_i32(int32_t *p, int n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  return launch(fill_i32_kernel, (n + 255) / 256, 256, 0, s, p, n, v);
}

bool small_batch(int T, int k, int h, int I, bool int8) {
  // down rows: at most kDcMaxChunks 16-byte chunks per lane
  const int max_i = 64 * (int8 ? 16 : 32) * kDcMaxChunks;
  if (T > kSmallT || T * k > kSmallAssign || I > max_i) return false;
  return T * (3 * h + 4 * (h >> 5)) <= kSbMaxXLds;  // the hidden rows' planes and scales in LDS
}

namespace {

template <int NCH, bool XREG, class F>
hipError_t launch_gu_rows_n(const DecodeProblem &P, hipStream_t s) {
  const uint32_t lds = (uint32_t)(P.T * (3 * P.h + 4 * (P.h >> 5)));
  {
    static bool attr_set = false;  // LDS above 64 KB must be allowed once per kernel
    if (!attr_set) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(gate_up_rows_kernel<NCH, XREG, F>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, kSbMaxXLds);
      if (e != hipSuccess) return e;
      attr_set = true;
    }
  }
  return launch(gate_up_rows_kernel<NCH, XREG, F>, XREG ? kSbBlocks : kSbBlocksLds, XREG ? 256 : 512, lds, s, P);
}

// Chunks per lane of a row: int4 h <= 64 * 32 * 8, int8 h <= 64 * 16 * 8.
// One token keeps its planes in registers up to 24 uint4 per lane.
template <class F>
hipError_t launch_gu_rows(const DecodeProblem &P, hipStream_t s) {
  const int per = 64 * F::kChunkCols, nchl = (P.h + per - 1) / per;
  const bool xreg = P.T == 1 && nchl * F::kXPlanes <= 24;
  if constexpr (F::kRowScale) {
    const int n = nchl <= 2 ? nchl : nchl <= 4 ? 4 : nchl <= 6 ? 6 : 8;
    if (xreg) {
      switch (n) {
        case 1: return launch_gu_rows_n<1, true, F>(P, s);
        case 2: return launch_gu_rows_n<2, true, F>(P, s);
        case 4: return launch_gu_rows_n<4, true, F>(P, s);
        case 6: return launch_gu_rows_n<6, true, F>(P, s);
        default: return launch_gu_rows_n<8, true, F>(P, s);
      }
    }
    switch (n) {
      case 1: return launch_gu_rows_n<1, false, F>(P, s);
      case 2: return launch_gu_rows_n<2, false, F>(P, s);
      case 4: return launch_gu_rows_n<4, false, F>(P, s);
      case 6: return launch_gu_rows_n<6, false, F>(P, s);
      default: return launch_gu_rows_n<8, false, F>(P, s);
    }
  } else {
    if (xreg) {
      switch (nchl) {
        case 1: return launch_gu_rows_n<1, true, F>(P, s);
        case 2: return launch_gu_rows_n<2, true, F>(P, s);
        case 3: return launch_gu_rows_n<3, true, F>(P, s);
        default: return launch_gu_rows_n<4, true, F>(P, s);
      }
    }
    switch (nchl) {
      case 1: return launch_gu_rows_n<1, false, F>(P, s);
      case 2: return launch_gu_rows_n<2, false, F>(P, s);
      case 3: return launch_gu_rows_n<3, false, F>(P, s);
      case 4: return launch_gu_rows_n<4, false, F>(P, s);
      case 5:
      case 6: return launch_gu_rows_n<6, false, F>(P, s);
      default: return launch_gu_rows_n<8, false, F>(P, s);
    }
  }
}

template <int NCHD, int RM, class F>
hipError_t launch_dc_rows_n(const DecodeProblem &P, float *out, int blocks, hipStream_t s) {
  const int per_slot = 3 * P.I + 4 * (P.I >> 5);  // planes and scales of one intermediate row
  const int n_slots = P.T * (P.k + P.has_shared);
  const int gs = kDcLds / per_slot;  // >= 2: small batches have I <= 8192
  if (gs >= n_slots || n_slots * per_slot <= kDcLdsAll)
    return launch(down_combine_rows_kernel<NCHD, RM, true, F>, blocks, kDcWaves * 64, (uint32_t)(n_slots * per_slot),
                  s, P, out, n_slots);
  return launch(down_combine_rows_kernel<NCHD, RM, false, F>, blocks, kDcWaves * 64, (uint32_t)(gs * per_slot), s, P,
                out, gs);
}

template <int NCHD, class F>
hipError_t launch_dc_rows_r(const DecodeProblem &P, float *out, hipStream_t s) {
  const int blocks = min(kDcBlocks, (P.h + kDcWaves - 1) / kDcWaves);
  const int rm = (P.h + blocks * kDcWaves - 1) / (blocks * kDcWaves);  // rows per wave, at most
  switch (rm) {
    case 1: return launch_dc_rows_n<NCHD, 1, F>(P, out, blocks, s);
    case 2: return launch_dc_rows_n<NCHD, 2, F>(P, out, blocks, s);
    case 3: return launch_dc_rows_n<NCHD, 3, F>(P, out, blocks, s);
    case 4: return launch_dc_rows_n<NCHD, 4, F>(P, out, blocks, s);
    default: return launch_dc_rows_n<NCHD, 8, F>(P, out, blocks, s);
  }
}

template <class F>
hipError_t launch_dc_rows(const DecodeProblem &P, float *out, hipStream_t s) {
  const int per = 64 * F::kChunkCols;
  switch ((P.I + per - 1) / per) {
    case 1: return launch_dc_rows_r<1, F>(P, out, s);
    case 2: return launch_dc_rows_r<2, F>(P, out, s);
    case 3: return launch_dc_rows_r<3, F>(P, out, s);
    default: return launch_dc_rows_r<4, F>(P, out, s);
  }
}

}  // namespace

namespace {

// Read probe: the gate and up codes and scales of n experts' rows (expert
// -1 = the shared expert; out-of-range ids read nothing), loaded with the
// small-batch gate/up launch's grid and a static split of the rows over its
// waves, two rows in flight per wave, and nothing computed but an XOR that
// keeps the loads.  Its time is the HBM read ceiling of the gate/up access
// pattern at the same size.
template <int NCH>
__global__ __launch_bounds__(256) void read_probe_kernel(DecodeProblem P, const int32_t *__restrict__ experts, int n,
                                                         uint32_t *__restrict__ sink) {
  const int wave = uniform(threadIdx.x >> 6);
  const int64_t W = (int64_t)gridDim.x * 4, gw = (int64_t)blockIdx.x * 4 + wave;
  const int I = P.I, h = P.h;
  const int64_t N = (int64_t)n * I;
  const int lo = (int)(N * gw / W), hi = (int)(N * (gw + 1) / W);
  const size_t qstride = (size_t)I * (h >> 1), sstride = (size_t)I * (h >> 6);
  uint32_t acc = 0;
  for (int f = lo; f < hi; f += 2) {
    GuBuf<NCH> b[2];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const int ff = min(f + d, hi - 1);
      const int e = uniform(experts[ff / I]);
      GuCursor c{};
      const bool shared = e == -1 && P.has_shared;
      const bool valid = shared || (e >= 0 && e < P.E);
      if (shared) {
        c.qg = P.sh_gate.q;
        c.sg = P.sh_gate.s;
        c.qu = P.sh_up.q;
        c.su = P.sh_up.s;
      } else if (valid) {
        c.qg = P.gate.q + e * qstride;
        c.sg = P.gate.s + e * sstride;
        c.qu = P.up.q + e * qstride;
        c.su = P.up.s + e * sstride;
      }
      c.r = ff % I;
      gu_load(b[d], c, valid, h);
    }
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc)
        acc ^= b[d].g[cc].x ^ b[d].g[cc].y ^ b[d].g[cc].z ^ b[d].g[cc].w ^ b[d].u[cc].x ^ b[d].u[cc].y ^
               b[d].u[cc].z ^ b[d].u[cc].w ^ __float_as_uint(b[d].gs[cc]) ^ __float_as_uint(b[d].us[cc]);
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;  // (almost) never taken; the loads must stay
}

// Read probe of the one-token down + combine launch: the down codes and
// scales of the n experts' rows, loaded with that launch's grid and row split
// (wave w of W owns rows [w h / W, (w + 1) h / W), at most RM), two experts
// in flight per wave, as its two-slot ring, and nothing computed but an XOR.
template <int NCHD, int RM>
__global__ __launch_bounds__(kDcWaves * 64) void read_probe_down_kernel(DecodeProblem P,
                                                                       const int32_t *__restrict__ experts, int n,
                                                                       uint32_t *__restrict__ sink) {
  const int wave = uniform(threadIdx.x >> 6);
  const int h = P.h, I = P.I;
  const int64_t W = (int64_t)gridDim.x * kDcWaves, gw = (int64_t)blockIdx.x * kDcWaves + wave;
  const int r0 = (int)((int64_t)h * gw / W), nr = (int)((int64_t)h * (gw + 1) / W) - r0;
  const size_t qstride = (size_t)h * (I >> 1), sstride = (size_t)h * (I >> 6);
  uint32_t acc = 0;
  for (int s0 = 0; s0 < n; s0 += 2) {
    DnBuf<NCHD, FmtI4> b[2][RM];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const int e = uniform(experts[min(s0 + d, n - 1)]);
      const bool shared = e == -1 && P.has_shared;
      const bool valid = shared || (e >= 0 && e < P.E);
      const uint8_t *q = shared ? P.sh_down.q : P.down.q + (valid ? (size_t)e * qstride : 0);
      const float *sc = shared ? P.sh_down.s : P.down.s + (valid ? (size_t)e * sstride : 0);
#pragma unroll
      for (int r = 0; r < RM; ++r) dn_load(b[d][r], q, sc, r0 + r, valid && r < nr, I);
    }
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int r = 0; r < RM; ++r)
#pragma unroll
        for (int cc = 0; cc < NCHD; ++cc)
          acc ^= b[d][r].w[cc].x ^ b[d][r].w[cc].y ^ b[d][r].w[cc].z ^ b[d][r].w[cc].w ^ __float_as_uint(b[d][r].s[cc]);
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;  // (almost) never taken; the loads must stay
}

template <int NCHD>
hipError_t launch_read_probe_down_r(const DecodeProblem &P, const int32_t *experts, int n, uint32_t *sink,
                                    hipStream_t s) {
  const int blocks = min(kDcBlocks, (P.h + kDcWaves - 1) / kDcWaves);
  const int rm = (P.h + blocks * kDcWaves - 1) / (blocks * kDcWaves);
  switch (rm) {
    case 1: return launch(read_probe_down_kernel<NCHD, 1>, blocks, kDcWaves * 64, 0, s, P, experts, n, sink);
    case 2: return launch(read_probe_down_kernel<NCHD, 2>, blocks, kDcWaves * 64, 0, s, P, experts, n, sink);
    case 3: return launch(read_probe_down_kernel<NCHD, 3>, blocks, kDcWaves * 64, 0, s, P, experts, n, sink);
    case 4: return launch(read_probe_down_kernel<NCHD, 4>, blocks, kDcWaves * 64, 0, s, P, experts, n, sink);
    default: return launch(read_probe_down_kernel<NCHD, 8>, blocks, kDcWaves * 64, 0, s, P, experts, n, sink);
  }
}

}  // namespace

hipError_t launch_read_probe_down(const DecodeProblem &P, const int32_t *experts, int n, uint32_t *sink,
                                  hipStream_t s) {
  switch ((P.I + 2047) / 2048) {
    case 1: return launch_read_probe_down_r<1>(P, experts, n, sink, s);
    case 2: return launch_read_probe_down_r<2>(P, experts, n, sink, s);
    case 3: return launch_read_probe_down_r<3>(P, experts, n, sink, s);
    default: return launch_read_probe_down_r<4>(P, experts, n, sink, s);
  }
}

hipError_t launch_read_probe(const DecodeProblem &P, const int32_t *experts, int n, uint32_t *sink,
                             hipStream_t s) {
  switch ((P.h + 2047) / 2048) {
    case 1: return launch(read_probe_kernel<1>, kSbBlocks, 256, 0, s, P, experts, n, sink);
    case 2: return launch(read_probe_kernel<2>, kSbBlocks, 256, 0, s, P, experts, n, sink);
    case 3: return launch(read_probe_kernel<3>, kSbBlocks, 256, 0, s, P, experts, n, sink);
    default: return launch(read_probe_kernel<4>, kSbBlocks, 256, 0, s, P, experts, n, sink);
  }
}

hipError_t launch_gemv_gate_up(const DecodeProblem &P, hipStream_t s) {
  if (P.T == 0) return hipSuccess;
  if (small_batch(P.T, P.k, P.h, P.I, P.int8)) return P.int8 ? launch_gu_rows<FmtI8>(P, s) : launch_gu_rows<FmtI4>(P, s);
  if (P.int8) return hipErrorInvalidValue;  // int8 tables take the small-batch launches only
  const int slots = P.n_routed_slots + (P.has_shared ? 1 : 0);
  if (slots == 0) return hipSuccess;
  // rows held in registers up to h = 6144 (wider rows do not fit the
  // register file), then the digit planes of midf for the down launch;
  // wider: passes of at most two tokens, planes written directly
  const int nchl = (P.h + 2047) / 2048;
  if (nchl <= 3) {
    const dim3 tg(P.I / kGuRows, slots);
    hipError_t err = nchl == 1   ? launch(gate_up_tok_kernel<1>, tg, 64, 0, s, P)
                     : nchl == 2 ? launch(gate_up_tok_kernel<2>, tg, 64, 0, s, P)
                                 : launch(gate_up_tok_kernel<3>, tg, 64, 0, s, P);
    if (err != hipSuccess) return err;
    const int n = P.T * (P.k + P.has_shared);
    const size_t nw = (size_t)n * (P.I >> 3);
    return launch(quantize_mid_kernel, dim3((unsigned)((nw + 255) / 256)), 256, 0, s, (const float *)P.midf, n,
                  P.I, P.mq, P.ms);
  }
  dim3 grid(P.I / (kGuWaves * kGuRows), slots);
  if (P.T == 1) return launch(gate_up_kernel<1>, grid, kGuWaves * 64, 0, s, P);
  return launch(gate_up_kernel<2>, grid, kGuWaves * 64, 0, s, P);
}

hipError_t launch_down_combine(const DecodeProblem &P, float *out, hipStream_t s) {
  if (P.T == 0) return hipSuccess;
  return P.int8 ? launch_dc_rows<FmtI8>(P, out, s) : launch_dc_rows<FmtI4>(P, out, s);
}

hipError_t launch_gemv_down(const DecodeProblem &P, hipStream_t s) {
  const int slots = P.n_routed_slots + (P.has_shared ? 1 : 0);
  if (slots == 0 || P.T == 0) return hipSuccess;
  // rows held in registers up to I = 8192 (16, 8 or 4 rows a wave; h is a
  // multiple of 64); wider: passes of up to four intermediate rows
  switch ((P.I + 2047) / 2048) {
    case 1: return launch(down_tok_kernel<1, 16>, dim3(P.h / 16, slots), 64, 0, s, P);
    case 2: return launch(down_tok_kernel<2, 8>, dim3(P.h / 8, slots), 64, 0, s, P);
    case 3: return launch(down_tok_kernel<3, 4>, dim3(P.h / 4, slots), 64, 0, s, P);
    case 4: return launch(down_tok_kernel<4, 4>, dim3(P.h / 4, slots), 64, 0, s, P);
    default: break;
  }
  dim3 grid(P.h / (kDnWaves * kDnRows), slots);
  if (P.T == 1)
    return launch(down_kernel<1>, grid, kDnWaves * 64, 0, s, P);
  else if (P.T < 4)
    return launch(down_kernel<2>, grid, kDnWaves * 64, 0, s, P);
  else
    return launch(down_kernel<4>, grid, kDnWaves * 64, 0, s, P);
}

hipError_t launch_combine(const float *y, const float *w, const int32_t *idx, const int32_t *inv, int T, int k,
                          int h, int has_shared, float *out, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  dim3 grid((h / 4 + 255) / 256, T);
  return launch(combine_kernel, grid, 256, 0, s, y, w, idx, inv, T, k, h, has_shared, out);
}


}  // namespace coli
