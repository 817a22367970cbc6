// Prefill-sized expert FFN: grouped GEMMs on the bf16 matrix cores (MFMA)
// with float32 accumulation.
//
// Source: "colibri engine teardown" page, "Three key engineering decisions",
// item 1 -- int4 "gs64" experts (64 weights share one scale); cf-1.com
// Colibri article, section 3.3 step 4 -- every expert with tokens runs one
// GEMM on its token group, fed by the expert offsets of step 3.  With
// thousands of tokens the expert FFN is a dense contraction per expert
// (M = tokens of the expert, N = rows, K = columns), so it runs on
// v_mfma_f32_32x32x16_bf16.
//
// Operands:
//  A  activations in bf16 ([T][h] for gate/up, the intermediate [P][I] for
//     down), stored with the 8 columns of every 8-column word in the order
//     0,2,4,6,1,3,5,7 (see below);
//  B  the int4 codes, made bf16 exactly without any arithmetic: the 4-bit
//     code q becomes u = q + 8 (xor 8) and the bf16 number 128 + u (bits
//     0x4300 | u, exact since bf16 spacing at 128 is 1), one v_perm_b32 per
//     pair; the even columns of a word fill the first four elements and the
//     odd columns the last four, which is why A is stored in that order (K is
//     a sum index, any order common to A and B gives the same products);
//  scale per 64-column group g: the MFMAs of one group accumulate
//     D = A (Q + 136) in float32, then acc += s[n][g] * (D - 136 * sum_k A[m][k]),
//     with the 64-column sums of A taken while staging A into LDS.
//
// Tiles: 128 rows of A (tokens of one expert) x 128 weight rows, 4 waves;
// wave w owns weight rows 32w..32w+31 and all 128 tokens (4 MFMA blocks of 32
// tokens).  gate/up: the tile holds the same 128 rows of gate and of up, so
// the epilogue applies SwiGLU and writes the intermediate in bf16 (in the A
// order of the down GEMM); down: y[p][r] in float32, followed by the
// deterministic combine.  The tile list (expert, first token) is built on the
// device from the dispatch offsets; the grid is launched for the largest
// possible list and surplus blocks leave at once.
#include "internal.h"
#include "wave.h"

namespace coli {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128;       // tokens per tile
constexpr int BN = 128;       // weight rows per tile (per matrix)
constexpr int BK = 64;        // columns per K step = one scale group
constexpr int kLdsRow = BK + 8;  // bf16 per LDS row (16-byte pad against bank conflicts)

// Column c of a word (c = 0..7) sits at position c/2 + 4 (c & 1) of the
// stored word: even columns first.
__device__ __forceinline__ int word_pos(int c) { return (c >> 1) + 4 * (c & 1); }

// 8 int4 codes (nibble i = column i) -> 8 bf16 values 136 + q in the stored
// column order (0,2,4,6,1,3,5,7).
__device__ __forceinline__ bf16x8 codes_to_bf16(uint32_t w) {
  const uint32_t v = w ^ 0x88888888u;
  const uint32_t lo = v & 0x0F0F0F0Fu;         // u of columns 0, 2, 4, 6 (bytes 0..3)
  const uint32_t hi = (v >> 4) & 0x0F0F0F0Fu;  // u of columns 1, 3, 5, 7
  const uint32_t k43 = 0x43434343u;
  // perm(a, b, sel): byte i of the result is byte sel_i of {b (0..3), a (4..7)}
  uint32_t p[4];
  p[0] = __builtin_amdgcn_perm(k43, lo, 0x04010400u);  // [u0, 43, u2, 43]
  p[1] = __builtin_amdgcn_perm(k43, lo, 0x04030402u);  // [u4, 43, u6, 43]
  p[2] = __builtin_amdgcn_perm(k43, hi, 0x04010400u);  // [u1, 43, u3, 43]
  p[3] = __builtin_amdgcn_perm(k43, hi, 0x04030402u);  // [u5, 43, u7, 43]
  return __builtin_bit_cast(bf16x8, p);
}

struct TileRows {
  int p_begin, cnt;   // sorted positions of the expert's tokens
  bool shared;
  int e;
};

__device__ __forceinline__ bool tile_rows(const PrefillProblem &P, int tile, int &m0, TileRows &R) {
  if (tile >= *P.n_tiles) return false;
  const int2 t = P.tiles[tile];
  m0 = t.y;
  if (t.x < 0) {
    R.shared = true;
    R.e = -1;
    R.p_begin = P.T * P.k;
    R.cnt = P.T;
  } else {
    R.shared = false;
    R.e = P.active[t.x];
    R.p_begin = P.offsets[R.e];
    R.cnt = P.offsets[R.e + 1] - R.p_begin;
  }
  return true;
}

// Stage one K step of A (BM rows x 64 columns) into LDS and the 64-column sums
// times 136: thread t copies 32 columns (64 bytes) of row t/2 and the pair of
// threads of a row adds its sums.
__device__ __forceinline__ void stage_a(const __bf16 *const *rowp, int g, __bf16 (*xs)[kLdsRow], float *xc) {
  const int t = threadIdx.x, m = t >> 1, part = t & 1;
  const uint4 *src = reinterpret_cast<const uint4 *>(rowp[m] + (size_t)g * BK + 32 * part);
  uint4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = src[i];
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x8 b = __builtin_bit_cast(bf16x8, v[i]);
#pragma unroll
    for (int j = 0; j < 8; ++j) sum += (float)b[j];
  }
  sum += __shfl_xor(sum, 1);
  uint4 *dst = reinterpret_cast<uint4 *>(&xs[m][32 * part]);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = v[i];
  if (part == 0) xc[m] = 136.0f * sum;
}

// ---------------------------------------------------------------------------
// gate/up
// ---------------------------------------------------------------------------

// grid = (I / BN, max tiles), 256 threads.
__global__ __launch_bounds__(256) void gate_up_mfma_kernel(PrefillProblem P) {
  __shared__ __bf16 xs[2][BM][kLdsRow];
  __shared__ float xc[2][BM];
  __shared__ const __bf16 *rowp[BM];
  int m0;
  TileRows R;
  if (!tile_rows(P, blockIdx.y, m0, R)) return;  // uniform over the block
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = P.h, I = P.I, G = h / BK;
  const int n0 = blockIdx.x * BN + wave * 32;  // this wave's 32 rows
  const int nl = lane & 31, half = lane >> 5;
  const int rows_here = min(BM, R.cnt - m0);
  if (threadIdx.x < BM) {
    const int m = min((int)threadIdx.x, rows_here - 1);  // padding rows repeat a valid token
    const int p = R.p_begin + m0 + m;
    const int tok = R.shared ? p - P.T * P.k : P.sorted_ids[p] / P.k;
    rowp[threadIdx.x] = P.xb + (size_t)tok * h;
  }
  // this lane's weight row n0 + nl: 16 bytes (32 columns) of each group
  const size_t qstride = (size_t)I * (h >> 1), sstride = (size_t)I * (h >> 6);
  const uint8_t *gq = (R.shared ? P.sh_gate.q : P.gate.q + (size_t)R.e * qstride) + (size_t)(n0 + nl) * (h >> 1);
  const uint8_t *uq = (R.shared ? P.sh_up.q : P.up.q + (size_t)R.e * qstride) + (size_t)(n0 + nl) * (h >> 1);
  const float *gs = (R.shared ? P.sh_gate.s : P.gate.s + (size_t)R.e * sstride) + (size_t)(n0 + nl) * (h >> 6);
  const float *us = (R.shared ? P.sh_up.s : P.up.s + (size_t)R.e * sstride) + (size_t)(n0 + nl) * (h >> 6);
  __syncthreads();

  f32x16 accg[4], accu[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) accg[mb] = accu[mb] = f32x16{};
  stage_a(rowp, 0, xs[0], xc[0]);
  uint4 wg = *reinterpret_cast<const uint4 *>(gq + 16 * half);
  uint4 wu = *reinterpret_cast<const uint4 *>(uq + 16 * half);
  float sg = gs[0], su = us[0];
  __syncthreads();
  for (int g = 0; g < G; ++g) {
    const int buf = g & 1;
    // next step's weights and scales in flight during this step
    uint4 wg_n = wg, wu_n = wu;
    float sg_n = sg, su_n = su;
    if (g + 1 < G) {
      wg_n = *reinterpret_cast<const uint4 *>(gq + (size_t)(g + 1) * 32 + 16 * half);
      wu_n = *reinterpret_cast<const uint4 *>(uq + (size_t)(g + 1) * 32 + 16 * half);
      sg_n = gs[g + 1];
      su_n = us[g + 1];
    }
    f32x16 dg[4], du[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) dg[mb] = du[mb] = f32x16{};
    const uint32_t wgs[4] = {wg.x, wg.y, wg.z, wg.w}, wus[4] = {wu.x, wu.y, wu.z, wu.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 bg = codes_to_bf16(wgs[j]), bu = codes_to_bf16(wus[j]);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&xs[buf][32 * mb + nl][32 * half + 8 * j]);
        dg[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bg, dg[mb], 0, 0, 0);
        du[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bu, du[mb], 0, 0, 0);
      }
    }
    if (g + 1 < G) stage_a(rowp, g + 1, xs[buf ^ 1], xc[buf ^ 1]);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float c = xc[buf][32 * mb + 4 * half + 8 * (i >> 2) + (i & 3)];
        accg[mb][i] = __builtin_fmaf(sg, dg[mb][i] - c, accg[mb][i]);
        accu[mb][i] = __builtin_fmaf(su, du[mb][i] - c, accu[mb][i]);
      }
    wg = wg_n;
    wu = wu_n;
    sg = sg_n;
    su = su_n;
    __syncthreads();
  }
  // SwiGLU; the intermediate row p, column n is stored at the A position of
  // the down GEMM (column order 0,2,4,6,1,3,5,7 within each word)
  const int n = n0 + nl;
  const int col = (n & ~7) | word_pos(n & 7);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = 32 * mb + 4 * half + 8 * (i >> 2) + (i & 3);
      if (m < rows_here) {
        const float gv = accg[mb][i], uv = accu[mb][i];
        const float v = gv / (1.0f + expf(-gv)) * uv;
        P.mid[(size_t)(R.p_begin + m0 + m) * I + col] = (__bf16)v;
      }
    }
}

// ---------------------------------------------------------------------------
// down: y[p][r] = sum_i mid[p][i] Wd[r][i]
// ---------------------------------------------------------------------------

// grid = (h / BN, max tiles), 256 threads.
__global__ __launch_bounds__(256) void down_mfma_kernel(PrefillProblem P) {
  __shared__ __bf16 xs[2][BM][kLdsRow];
  __shared__ float xc[2][BM];
  __shared__ const __bf16 *rowp[BM];
  int m0;
  TileRows R;
  if (!tile_rows(P, blockIdx.y, m0, R)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = P.h, I = P.I, G = I / BK;
  const int n0 = blockIdx.x * BN + wave * 32;
  const int nl = lane & 31, half = lane >> 5;
  const int rows_here = min(BM, R.cnt - m0);
  if (threadIdx.x < BM) {
    const int m = min((int)threadIdx.x, rows_here - 1);
    rowp[threadIdx.x] = P.mid + (size_t)(R.p_begin + m0 + m) * I;
  }
  const size_t qstride = (size_t)h * (I >> 1), sstride = (size_t)h * (I >> 6);
  const uint8_t *dq = (R.shared ? P.sh_down.q : P.down.q + (size_t)R.e * qstride) + (size_t)(n0 + nl) * (I >> 1);
  const float *ds = (R.shared ? P.sh_down.s : P.down.s + (size_t)R.e * sstride) + (size_t)(n0 + nl) * (I >> 6);
  __syncthreads();

  f32x16 acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x16{};
  stage_a(rowp, 0, xs[0], xc[0]);
  uint4 wd = *reinterpret_cast<const uint4 *>(dq + 16 * half);
  float sd = ds[0];
  __syncthreads();
  for (int g = 0; g < G; ++g) {
    const int buf = g & 1;
    uint4 wd_n = wd;
    float sd_n = sd;
    if (g + 1 < G) {
      wd_n = *reinterpret_cast<const uint4 *>(dq + (size_t)(g + 1) * 32 + 16 * half);
      sd_n = ds[g + 1];
    }
    f32x16 d[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) d[mb] = f32x16{};
    const uint32_t wds[4] = {wd.x, wd.y, wd.z, wd.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 b = codes_to_bf16(wds[j]);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&xs[buf][32 * mb + nl][32 * half + 8 * j]);
        d[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, d[mb], 0, 0, 0);
      }
    }
    if (g + 1 < G) stage_a(rowp, g + 1, xs[buf ^ 1], xc[buf ^ 1]);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float c = xc[buf][32 * mb + 4 * half + 8 * (i >> 2) + (i & 3)];
        acc[mb][i] = __builtin_fmaf(sd, d[mb][i] - c, acc[mb][i]);
      }
    wd = wd_n;
    sd = sd_n;
    __syncthreads();
  }
  const int n = n0 + nl;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = 32 * mb + 4 * half + 8 * (i >> 2) + (i & 3);
      if (m < rows_here) P.y[(size_t)(R.p_begin + m0 + m) * h + n] = acc[mb][i];
    }
}

// ---------------------------------------------------------------------------
// Tile list: (slot, first token) for every 128 tokens of every active expert,
// then of the shared expert.  One workgroup of 1024 threads, one slot per
// thread (n_active <= 512).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t *__restrict__ offsets,
                                                           const int32_t *__restrict__ active,
                                                           const int32_t *__restrict__ n_active, int T,
                                                           int has_shared, int2 *__restrict__ tiles,
                                                           int32_t *__restrict__ n_tiles) {
  __shared__ int32_t wave_sum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int na = *n_active;
  int cnt = 0;
  if (tid < na) {
    const int e = active[tid];
    cnt = offsets[e + 1] - offsets[e];
  } else if (tid == na && has_shared) {
    cnt = T;
  }
  const int mt = (cnt + BM - 1) / BM;
  int incl = mt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d);
    if (lane >= d) incl += v;
  }
  if (lane == 63) wave_sum[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wave_sum[w];
  const int start = before + incl - mt;
  const int slot = tid < na ? tid : -1;
  for (int i = 0; i < mt; ++i) tiles[start + i] = make_int2(slot, i * BM);
  if (tid == 1023) *n_tiles = before + incl;
}

// x [T][h] float -> bf16 in the stored column order of the A operand.
__global__ __launch_bounds__(256) void to_bf16_kernel(const float *__restrict__ x, size_t n_words,
                                                      __bf16 *__restrict__ xb) {
  const size_t w = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (w >= n_words) return;
  const float4 a = reinterpret_cast<const float4 *>(x)[2 * w];
  const float4 b = reinterpret_cast<const float4 *>(x)[2 * w + 1];
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  bf16x8 o;
#pragma unroll
  for (int c = 0; c < 8; ++c) o[word_pos(c)] = (__bf16)v[c];
  reinterpret_cast<bf16x8 *>(xb)[w] = o;
}

}  // namespace

int prefill_max_tiles(int T, int k, int E, int has_shared) {
  const int n = T * k, routed_slots = E < n ? E : n;
  return n / BM + routed_slots + (has_shared ? (T + BM - 1) / BM : 0);
}

hipError_t launch_prefill_prep(const float *x, int T, int h, __bf16 *xb, hipStream_t s) {
  const size_t n_words = (size_t)T * h / 8;
  to_bf16_kernel<<<(unsigned)((n_words + 255) / 256), 256, 0, s>>>(x, n_words, xb);
  return hipGetLastError();
}

hipError_t launch_build_tiles(const PrefillProblem &P, hipStream_t s) {
  build_tiles_kernel<<<1, 1024, 0, s>>>(P.offsets, P.active, P.n_active, P.T, P.has_shared, P.tiles, P.n_tiles);
  return hipGetLastError();
}

hipError_t launch_gate_up_mfma(const PrefillProblem &P, hipStream_t s) {
  dim3 grid(P.I / BN, prefill_max_tiles(P.T, P.k, P.E, P.has_shared));
  gate_up_mfma_kernel<<<grid, 256, 0, s>>>(P);
  return hipGetLastError();
}

hipError_t launch_down_mfma(const PrefillProblem &P, hipStream_t s) {
  dim3 grid(P.h / BN, prefill_max_tiles(P.T, P.k, P.E, P.has_shared));
  down_mfma_kernel<<<grid, 256, 0, s>>>(P);
  return hipGetLastError();
}

}  // namespace coli
