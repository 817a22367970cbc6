// Batched decode expert FFN on the int8 matrix cores (int4 gs64 tables,
// batches above the small-batch limits and below the prefill threshold).
//
// Sources: "colibri engine teardown" page, "Three key engineering decisions",
// item 1 -- routed experts are int4 in the "gs64" container (64 weights share
// one float32 scale); cf-1.com Colibri article, section 2.1 -- each expert is
// a SwiGLU FFN (gate, up, down) applied to the tokens routed to it; section
// 3.3 step 4 -- experts with no tokens are skipped.
//
// With several tokens per expert the v_dot8 GEMV (expert_gemv.hip) spends
// about 32 VALU instructions per weight row, token and 32 columns.  Here one
// v_mfma_i32_16x16x64_i8 multiplies a tile of 16 weight rows by 4 tokens
// over one weight group (64 columns), with exact integer products:
//   B (weights): lane l holds row l % 16 of the tile and 16 columns of the
//     group (its 8 code bytes), each code q as the byte 16 q (the nibble
//     moved to the top of the byte: exact, two's complement), even columns
//     of each 8 first;
//   A (activations): lane l holds vtoken l % 16 = 4 t + j, digit j of token
//     t's integers (j = 3 is zero) in the same 16 columns, same byte order.
// The int32 result C[4 t + j][r] = 16 sum_c q_c d_j,c is exact
// (|C| <= 64 * 128 * 128), and lane l of C holds the digits j = 0..2 of
// token l / 16 for row l % 16: the lane puts the group's sum together
// (65536 C2 + 256 C1 + C0, the low two in int32) and applies the weight
// scale times the token's group scale with one float32 fma per group, as
// the GEMV does per 32 columns.
//
// Activation format (byte planes over 64-column groups): for a row of `cols`
// floats and group g, s = 2^(E - 22) with 2^E > max |x| over the group, the
// integers N_c = rint(x_c / s) (|N_c| <= 2^22, a 23-bit signed mantissa per
// group), written as balanced base-256 digits N = d0 + 256 d1 + 65536 d2
// (d0, d1 in [-128, 127], d2 in [-64, 64]).  planes [row][cols/64][4][3][16]
// int8: per group, per 16-column chunk k (the columns of MFMA k-slot k), the
// three digits' 16 bytes in a row (48 bytes), each chunk in the byte order
// 0 2 4 6 1 3 5 7 8 10 12 14 9 11 13 15 (the order the code bytes unpack
// to); scales [row][cols/64] hold s / 16 (the factor of the code bytes
// folded in).
//
// Memory access: the MFMA layouts put 16 different weight rows in 16
// neighbouring lanes; loaded that way, every load touches a separate
// 32-byte piece of 16 rows, and the stream reached well under half the HBM
// rate.  The codes are instead read as the GEMV reads them, 512 contiguous
// bytes of a row per 32 lanes, staged in LDS and read back in the MFMA
// layout (see the block loop below); the activation layout above puts a
// token's 3 digits of a chunk, which 4 neighbouring A lanes take, in one
// 48-byte run.
#include "expert_batch.h"

#include "byte_planes.h"
#include "wave.h"

namespace coli {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kBtMinPass = 4;              // fewest tokens per pass over the rows (the grid's bound)
constexpr uint32_t kBtOut = 0x80000000u;   // a buffer offset past every table: the load returns zeros

// ---------------------------------------------------------------------------
// The block's product loop (gate/up and down).
//
// A block of 4 waves owns R weight rows (R / 16 MFMA tiles) of one slot and
// a pass of 4 NTT tokens (NTT token tiles of 4), and runs the columns in
// chunks of CG groups.  Each
// wave loads R / 4 of the rows, whole row pieces of 32 CG contiguous bytes
// (the access pattern of the GEMV: 512 or 1024 bytes per row and load), and
// their scales, into registers, then writes them to the block's LDS stage
// (two buffers, one barrier per chunk); every wave then takes CG / 4 of the
// chunk's groups for all tiles, reading the codes and scales from the stage
// in the MFMA layout, and its own activations from memory.  Piece p (16
// bytes) of stage row r sits at piece p ^ (r % 16), so that the 16 rows a
// read takes fall in 16 different bank groups; scale rows are padded to
// 4 CG + 16 bytes for the same reason.  The waves' partial sums meet in LDS
// in wave order at the end of the pass.
// Register rings: codes, scales and activations of 2 chunks; each chunk's
// activations are issued before the codes of the chunk after next, so the
// in-order completion of a wave's loads never holds an operand behind a
// later code load.
// ---------------------------------------------------------------------------
template <int R, int CG, int NTT>
struct BatchShape {
  static constexpr int kTiles = R / 16;
  static constexpr int kRowBytes = 32 * CG;       // codes per row and chunk
  static constexpr int kLpr = 2 * CG;             // load lanes per row (16 bytes each)
  static constexpr int kRpi = 64 / kLpr;          // rows per load
  static constexpr int kLoads = R / 4 / kRpi;     // code loads per wave and chunk
  static constexpr int kGw = CG / 4;              // groups per wave and chunk
  static constexpr int kSLanes = CG / 4;          // scale load lanes per row
  static constexpr int kSStride = 4 * CG;         // scale stage row stride
  static constexpr int kSWrap = 64 / CG;          // scale rows per turn of the 64 banks
  static constexpr int kStageCodes = R * kRowBytes;
  static constexpr int kStage = kStageCodes + R * kSStride;
  static constexpr int kTokens = 4 * NTT;           // tokens per pass
  static constexpr int kRed = 4 * NTT * kTiles * 64 * 4;  // partial sums of the 4 waves
  static constexpr int kOut = 4 * R * kTokens * 4;        // results of up to 4 row blocks
  static constexpr int kLds = 2 * kStage + kRed + kOut;
  static constexpr int kSActive = R / 4 * kSLanes;   // lanes of the scale load
  static_assert(kRpi * kLpr == 64 && kLoads >= 1 && kSActive <= 64, "shape");
};

__device__ __forceinline__ float4 bload16f(Rsrc r, uint32_t voff, uint32_t soff) {
  const uint4 v = bload16(r, voff, soff);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}

// This wave's sources: its rows' table (wave-uniform), their first row in
// it, and the activation rows of the pass.
struct BatchWaveSrc {
  Rsrc wq, ws;       // codes and scales of this wave's rows
  int row0;          // first row of the wave's R / 4 in those tables (row block 0)
  int xstep;         // rows of those tables from one row block to the next
  int rowq, G;       // code bytes per row, groups per row
  Rsrc a, as;        // activation byte planes and group scales
  uint32_t a_off[2];   // token tile t, A lane: its token's digit at chunk lane / 16 of group 0; kBtOut: zeros
  uint32_t as_off[2];  // token tile t, C lane: its token's scale row
};

// The partial sums of the 4 waves to LDS (then a barrier); batch_total adds
// them in wave order.
template <int R, int CG, int NTT>
__device__ __forceinline__ void batch_share(const float (&acc)[NTT][R / 16], char *lds) {
  using B = BatchShape<R, CG, NTT>;
  float *red = reinterpret_cast<float *>(lds + 2 * B::kStage);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int t = 0; t < NTT; ++t)
#pragma unroll
    for (int r = 0; r < R / 16; ++r) red[((wave * NTT + t) * (R / 16) + r) * 64 + lane] = acc[t][r];
  block_barrier();
}
template <int R, int CG, int NTT>
__device__ __forceinline__ float batch_total(const char *lds, int t, int r) {
  using B = BatchShape<R, CG, NTT>;
  const float *red = reinterpret_cast<const float *>(lds + 2 * B::kStage);
  const int lane = threadIdx.x & 63;
  float v = red[(t * (R / 16) + r) * 64 + lane];
#pragma unroll
  for (int w = 1; w < 4; ++w) v += red[((w * NTT + t) * (R / 16) + r) * 64 + lane];
  return v;
}

// The block's stream of nx row blocks x (each R rows of the slot) times
// the C chunks of the columns, one ring across all of them: acc[r] sums
// this wave's part (its groups) of the products of tile r's rows of the
// current row block and token tile t of the pass (lane: token 4 t + lane / 16,
// row lane % 16 of the tile; ntt of the NTT tiles hold tokens of this pass);
// after a row block's last chunk the waves' parts
// meet in LDS and epi(x) takes the totals.
template <int R, int CG, int NTT, class Epi>
__device__ __forceinline__ void batch_stream(const BatchWaveSrc &Q, int ntt, int nx, char *lds, const Epi &epi) {
  using B = BatchShape<R, CG, NTT>;
  const int lane = threadIdx.x & 63, j = lane & 15, kg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // scalar: buffer offsets come from it
  const int G = Q.G, C = (G + CG - 1) / CG, K = nx * C;
  uint4 wr[2][B::kLoads];
  float4 sr[2];
  v4i ar[2][B::kGw][NTT];
  float xr[2][B::kGw][NTT];
  const uint32_t w_voff = (uint32_t)((lane / B::kLpr) * Q.rowq + 16 * (lane % B::kLpr));
  const bool s_lane = lane < B::kSActive;
  const uint32_t s_voff = s_lane ? (uint32_t)((lane / B::kSLanes) * Q.G * 4 + 16 * (lane % B::kSLanes)) : kBtOut;
  auto load_w = [&](int k, uint4 (&w)[B::kLoads], float4 &sc) {
    k = min(k, K - 1);  // past the last job: the last again (no branch around loads)
    const int x = k / C, c = k - x * C, row = Q.row0 + x * Q.xstep;
#pragma unroll
    for (int i = 0; i < B::kLoads; ++i)
      w[i] = bload16(Q.wq, w_voff, (uint32_t)((row + i * B::kRpi) * Q.rowq + B::kRowBytes * c));
    sc = bload16f(Q.ws, s_voff, (uint32_t)(row * Q.G * 4 + 4 * CG * c));
  };
  auto load_a = [&](int k, v4i (&a)[B::kGw][NTT], float (&x)[B::kGw][NTT]) {
    k = min(k, K - 1);
    const int c = k % C;
#pragma unroll
    for (int i = 0; i < B::kGw; ++i) {
      const int g = min(CG * c + B::kGw * wave + i, G - 1);
#pragma unroll
      for (int t = 0; t < NTT; ++t) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(Q.a, (int)Q.a_off[t], 192 * g, 0);
        a[i][t] = v4i{(int)v[0], (int)v[1], (int)v[2], (int)v[3]};
        x[i][t] = bloadf(Q.as, Q.as_off[t], (uint32_t)(4 * g));
      }
    }
  };
  // stage addresses (relative to a buffer): this lane's code pieces and
  // scale piece as written; the MFMA reads
  const int my_row = wave * (R / 4) + lane / B::kLpr;  // + i * kRpi for load i
  int w_st[B::kLoads];
#pragma unroll
  for (int i = 0; i < B::kLoads; ++i) {
    const int row = my_row + i * B::kRpi;
    w_st[i] = row * B::kRowBytes + 16 * ((lane % B::kLpr) ^ (row & 15));
  }
  // scale piece p of row r at piece p ^ ((r / kSWrap) % kSLanes): the 16
  // rows a read takes fall in 16 different banks
  const int s_row = wave * (R / 4) + lane / B::kSLanes;
  const int s_st = B::kStageCodes + s_row * B::kSStride +
                   16 * ((lane % B::kSLanes) ^ ((s_row / B::kSWrap) % B::kSLanes));
  int rd_q[B::kGw];
#pragma unroll
  for (int i = 0; i < B::kGw; ++i)
    rd_q[i] = j * B::kRowBytes + 16 * ((2 * (B::kGw * wave + i) + (kg >> 1)) ^ j) + 8 * (kg & 1);
  int rd_s[B::kGw];
#pragma unroll
  for (int i = 0; i < B::kGw; ++i) {
    const int gi = B::kGw * wave + i;
    rd_s[i] = B::kStageCodes + j * B::kSStride + 16 * ((gi >> 2) ^ ((j / B::kSWrap) % B::kSLanes)) + 4 * (gi & 3);
  }
  // issue order: W0 A0 W1, then per job k: A(k + 1) W(k + 2)
  load_w(0, wr[0], sr[0]);
  __builtin_amdgcn_sched_barrier(0);
  load_a(0, ar[0], xr[0]);
  __builtin_amdgcn_sched_barrier(0);
  load_w(1, wr[1], sr[1]);
  __builtin_amdgcn_sched_barrier(0);
  const v4i zero = {0, 0, 0, 0};
  float acc[NTT][R / 16];
#pragma unroll
  for (int t = 0; t < NTT; ++t)
#pragma unroll
    for (int r = 0; r < R / 16; ++r) acc[t][r] = 0.0f;
  // jobs in pairs (ring slots 0, 1); an odd count ends with a job that only
  // loads and stages (no branch around loads, so every wait counts the same
  // loads in flight)
  for (int k0 = 0; k0 < K; k0 += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int k = k0 + u;
      const bool real = k < K;
      const int x = k / C, c = k - x * C;
      char *st = lds + u * B::kStage;  // buffer k % 2 (k0 is even)
      // job k to the stage: the buffer's last readers (job k - 2) are past
      // the previous job's barrier
#pragma unroll
      for (int i = 0; i < B::kLoads; ++i) *reinterpret_cast<uint4 *>(st + w_st[i]) = wr[u][i];
      if (s_lane) *reinterpret_cast<float4 *>(st + s_st) = sr[u];
      block_barrier();
      load_a(k + 1, ar[u ^ 1], xr[u ^ 1]);
      __builtin_amdgcn_sched_barrier(0);
      load_w(k + 2, wr[u], sr[u]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < B::kGw; ++i) {
        if (real && CG * c + B::kGw * wave + i < G) {
          v4i bq[R / 16];
          float sw[R / 16];
#pragma unroll
          for (int r = 0; r < R / 16; ++r) {
            const uint2 w = *reinterpret_cast<const uint2 *>(st + 16 * r * B::kRowBytes + rd_q[i]);
            // the codes as bytes 16 q: even columns of each word, then odd ones
            bq[r] = v4i{(int)((w.x << 4) & 0xF0F0F0F0u), (int)(w.x & 0xF0F0F0F0u), (int)((w.y << 4) & 0xF0F0F0F0u),
                        (int)(w.y & 0xF0F0F0F0u)};
            sw[r] = *reinterpret_cast<const float *>(st + 16 * r * B::kSStride + rd_s[i]);
          }
#pragma unroll
          for (int t = 0; t < NTT; ++t) {
            if (t < ntt) {
              v4i cc[R / 16];
#pragma unroll
              for (int r = 0; r < R / 16; ++r)
                cc[r] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ar[u][i][t], bq[r], zero, 0, 0, 0);
#pragma unroll
              for (int r = 0; r < R / 16; ++r) {
                const int lo = (int)((uint32_t)cc[r][1] << 8) + cc[r][0];  // |.| < 2^29
                const float y = __builtin_fmaf((float)cc[r][2], 65536.0f, (float)lo);
                acc[t][r] = __builtin_fmaf(sw[r] * xr[u][i][t], y, acc[t][r]);
              }
            }
          }
        }
      }
      if (real && c == C - 1) {
        // the row block's totals (the next job's barrier comes after every
        // wave has read them, before the sums are written again)
        batch_share<R, CG, NTT>(acc, lds);
        epi(x);
#pragma unroll
        for (int t = 0; t < NTT; ++t)
#pragma unroll
          for (int r = 0; r < R / 16; ++r) acc[t][r] = 0.0f;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// The slot of a block: the shared expert (routed = false) or routed expert
// e, its tables and its assignment positions [p_begin, p_begin + cnt).
struct BatchSlot {
  const uint8_t *q0, *q1;  // gate and up (down: q0)
  const float *s0, *s1;
  int p_begin, cnt, base;  // base: offsets[e] for a routed slot, -1 for the shared one
};

// Block y of the grid: y < n_sh is chunk y of the shared expert's tokens;
// then routed slot y - n_sh.  False when the block has no work.
__device__ __forceinline__ bool batch_slot(const DecodeProblem &P, int n_sh, bool down, int pass, BatchSlot &S,
                                           int &t_first,
                                           int &t_end) {
  const int y = (int)blockIdx.y;
  if (y < n_sh) {
    S.q0 = down ? P.sh_down.q : P.sh_gate.q;
    S.s0 = down ? P.sh_down.s : P.sh_gate.s;
    S.q1 = P.sh_up.q;
    S.s1 = P.sh_up.s;
    S.p_begin = P.T * P.k;
    S.cnt = P.T;
    S.base = -1;
    t_first = y * pass;
    t_end = min(P.T, t_first + pass);
    return t_first < t_end;
  }
  const int slot = y - n_sh;
  if (slot >= *P.n_active) return false;
  const int e = P.active[slot];
  S.base = P.offsets[e];
  S.cnt = P.offsets[e + 1] - S.base;
  S.p_begin = S.base;
  const size_t x = table_index(P.slot_of, e);
  if (down) {
    S.q0 = P.down.q + x * (size_t)P.h * (P.I >> 1);
    S.s0 = P.down.s + x * (size_t)P.h * (P.I >> 6);
  } else {
    const size_t qs = (size_t)P.I * (P.h >> 1), ss = (size_t)P.I * (P.h >> 6);
    S.q0 = P.gate.q + x * qs;
    S.s0 = P.gate.s + x * ss;
    S.q1 = P.up.q + x * qs;
    S.s1 = P.up.s + x * ss;
  }
  t_first = 0;
  t_end = S.cnt;
  return S.cnt > 0;
}

// gate/up: 16 gate + 16 up rows, 512 bytes of codes per row and chunk,
// one token tile (4 tokens a pass) or two (8 tokens a pass);
// down: 64 rows, 512 bytes per row and chunk, 4 tokens a pass.
constexpr int kGuR = 32, kGuCG = 16;
constexpr int kDnR = 64, kDnCG = 16, kDnTT = 1;

// Two gate/up token tiles halve the passes over the rows of an expert with
// more than 4 tokens and the chunks of the shared expert, which every pass
// reads again; in return each pass carries the second tile's registers and
// work.  Outputs are the same bits either way.  Measured (microseconds, one
// tile against two):
//  - GLM-like layer (E = 256, k = 8, a shared expert), gate/up kernel:
//    T = 16: 220 / 258, T = 32: 330 / 353, T = 40: 372 / 382,
//    T = 48: 413 / 410, T = 64: 510 / 480;
//  - OLMoE-like layer (E = 64, k = 8, no shared expert), whole calls with
//    the weights from HBM (8 copies in turn): T = 16: 82 / 85,
//    T = 24: 95 / 93, T = 32: 105 / 101, T = 64: 153 / 143.
// Two tiles therefore from 2.5 assignments per expert, or from 48 tokens
// with a shared expert (its passes are then the larger saving).  A variant
// held to 168 registers (three workgroups per CU) spilled and was slower.
bool gate_up_two_tiles(int T, int k, int E, bool shared) {
  return 2 * (int64_t)T * k >= 5 * (int64_t)E || (shared && T >= 48);
}

// gate/up: block x owns intermediate rows [16 nx x, 16 nx (x + 1)) (nx = 4:
// one 64-column group of mid, whose byte planes it writes), row block i of
// them rows 16 (nx x + i) + (0..15) (tile 0: gate rows, tile 1: up rows);
// waves 0, 1 load gate rows, waves 2, 3 up rows.
template <int TT>
__global__ __launch_bounds__(256) void gate_up_batch_kernel(DecodeProblem P, int n_sh, int nx) {
  using B = BatchShape<kGuR, kGuCG, TT>;
  __shared__ __attribute__((aligned(16))) char lds[B::kLds];
  BatchSlot S;
  int t_first, t_end;
  if (!batch_slot(P, n_sh, false, B::kTokens, S, t_first, t_end)) return;
  const int lane = threadIdx.x & 63, j = lane & 15, kg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // scalar: buffer offsets come from it
  const int h = P.h, I = P.I, G = h >> 6, rowq = h >> 1;
  const int r0 = blockIdx.x * 16 * nx;
  BatchWaveSrc Q;
  Q.rowq = rowq;
  Q.G = G;
  const bool up = wave >= 2;
  Q.wq = make_rsrc((up ? S.q1 : S.q0) + (size_t)r0 * rowq, (uint32_t)(16 * nx * rowq));
  Q.ws = make_rsrc((up ? S.s1 : S.s0) + (size_t)r0 * G, (uint32_t)(16 * nx * G * 4));
  Q.row0 = 8 * (wave & 1);
  Q.xstep = 16;
  Q.a = make_rsrc(P.xq, (uint32_t)((size_t)P.T * 3 * h));
  Q.as = make_rsrc(P.xs, (uint32_t)((size_t)P.T * G * 4));
  const int ti = (lane & 15) >> 2, d = lane & 3;
  auto token_of = [&](int i) { return S.base < 0 ? i : P.sorted_ids[S.base + i] / P.k; };
  for (int t0 = t_first; t0 < t_end; t0 += B::kTokens) {
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const int ia = t0 + 4 * t + ti;
      Q.a_off[t] = d < 3 && ia < t_end ? (uint32_t)(token_of(ia) * 3 * h + 48 * kg + 16 * d) : kBtOut;
      Q.as_off[t] = (uint32_t)(token_of(min(t0 + 4 * t + kg, t_end - 1)) * G * 4);
    }
    const int ntt = (min(B::kTokens, t_end - t0) + 3) >> 2;
    // wave 0 (token 4 t + kg, intermediate row 16 x + j of the block's)
    // leaves the results in LDS: global stores inside the stream would make
    // its waits count them
    float *outb = reinterpret_cast<float *>(lds + 2 * B::kStage + B::kRed);  // [x][token][16 rows]
    batch_stream<kGuR, kGuCG, TT>(Q, ntt, nx, lds, [&](int x) {
      if (wave == 0) {
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          const float g = batch_total<kGuR, kGuCG, TT>(lds, t, 0), u = batch_total<kGuR, kGuCG, TT>(lds, t, 1);
          outb[(x * B::kTokens + 4 * t + kg) * 16 + j] = g / (1.0f + expf(-g)) * u;
        }
      }
    });
    block_barrier();
    // the block holds one whole 64-column group of mid (4 row blocks of 16):
    // its byte planes for the down kernel straight from LDS, thread 8 t + i
    // taking word i of token t (an aligned octet per token)
    const int tt = threadIdx.x >> 3, wi = threadIdx.x & 7;
    if (tt < B::kTokens) {
      const bool valid = t0 + tt < t_end;
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = valid ? outb[((wi >> 1) * B::kTokens + tt) * 16 + 8 * (wi & 1) + i] : 0.0f;
      byte_planes_word(v, valid, valid ? (size_t)(S.p_begin + t0 + tt) : 0, (r0 >> 3) + wi, I,
                       reinterpret_cast<uint8_t *>(P.mq), P.ms);
    }
    block_barrier();  // the stage, the sums and the results are rewritten by the next pass
  }
}

// down: block x owns output rows [kDnR nx x, kDnR nx (x + 1)) (row block i:
// kDnR rows, tiles of 16), wave w loads rows kDnR / 4 * w .. of each; y per
// assignment position; wave r stores tile r.
__global__ __launch_bounds__(256) void down_batch_kernel(DecodeProblem P, int n_sh, int nx) {
  using B = BatchShape<kDnR, kDnCG, kDnTT>;
  __shared__ __attribute__((aligned(16))) char lds[B::kLds];
  BatchSlot S;
  int t_first, t_end;
  if (!batch_slot(P, n_sh, true, B::kTokens, S, t_first, t_end)) return;
  const int lane = threadIdx.x & 63, j = lane & 15, kg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // scalar: buffer offsets come from it
  const int h = P.h, I = P.I, G = I >> 6, rowq = I >> 1;
  const int r0 = blockIdx.x * kDnR * nx;
  BatchWaveSrc Q;
  Q.rowq = rowq;
  Q.G = G;
  Q.wq = make_rsrc(S.q0 + (size_t)r0 * rowq, (uint32_t)(kDnR * nx * rowq));
  Q.ws = make_rsrc(S.s0 + (size_t)r0 * G, (uint32_t)(kDnR * nx * G * 4));
  Q.row0 = kDnR / 4 * wave;
  Q.xstep = kDnR;
  const size_t n_rows = (size_t)P.T * (P.k + P.has_shared);
  Q.a = make_rsrc(P.mq, (uint32_t)(n_rows * 3 * I));
  Q.as = make_rsrc(P.ms, (uint32_t)(n_rows * G * 4));
  const int ti = (lane & 15) >> 2, d = lane & 3;
  for (int t0 = t_first; t0 < t_end; t0 += B::kTokens) {
    const int ia = t0 + ti;
    Q.a_off[0] = d < 3 && ia < t_end ? (uint32_t)((S.p_begin + ia) * 3 * I + 48 * kg + 16 * d) : kBtOut;
    Q.as_off[0] = (uint32_t)((S.p_begin + min(t0 + kg, t_end - 1)) * G * 4);
    // wave r (token kg, row kDnR x + 16 r + j of the block's) leaves the
    // results in LDS
    float *outb = reinterpret_cast<float *>(lds + 2 * B::kStage + B::kRed);  // [x][token][kDnR rows]
    batch_stream<kDnR, kDnCG, kDnTT>(Q, 1, nx, lds, [&](int x) {
      if (wave < kDnR / 16) outb[(x * 4 + kg) * kDnR + 16 * wave + j] = batch_total<kDnR, kDnCG, kDnTT>(lds, 0, wave);
    });
    block_barrier();
    for (int i = threadIdx.x; i < nx * 4 * kDnR; i += 256) {
      const int x = i / (4 * kDnR), t = (i / kDnR) & 3, row = i % kDnR;
      if (t0 + t < t_end) P.y[(size_t)(S.p_begin + t0 + t) * h + r0 + kDnR * x + row] = outb[i];
    }
    block_barrier();
  }
}

// Row blocks per workgroup: the most of 4, 2, 1 that divides the count.
int row_blocks_per_group(int n) { return n % 4 == 0 ? 4 : n % 2 == 0 ? 2 : 1; }


int shared_chunks(const DecodeProblem &P, int pass) { return P.has_shared ? (P.T + pass - 1) / pass : 0; }

}  // namespace

bool batch_mfma_fits(int T, int k, int has_shared, int h, int I) {
  // every table and activation buffer within a 32-bit buffer offset (below
  // the out-of-range offset kBtOut)
  const uint64_t rows = (uint64_t)T * (k + has_shared);
  return (uint64_t)T * 3 * h < kBtOut && rows * 3 * I < kBtOut && (uint64_t)I * (h >> 1) < kBtOut &&
         (uint64_t)T / kBtMinPass + 1 + kMaxExperts <= 65535;
}

hipError_t launch_batch_gate_up(const DecodeProblem &P, hipStream_t s) {
  const bool two = gate_up_two_tiles(P.T, P.k, P.E, P.has_shared != 0);
  const int n_sh = shared_chunks(P, two ? 8 : 4);
  if (P.I % 64) return hipErrorInvalidValue;  // a workgroup writes whole 64-column groups of mid
  if (P.T == 0 || n_sh + P.n_routed_slots == 0) return hipSuccess;
  const int nx = 4;
  const dim3 grid(P.I / 16 / nx, n_sh + P.n_routed_slots);
  if (two) return launch(gate_up_batch_kernel<2>, grid, 256, 0, s, P, n_sh, nx);
  return launch(gate_up_batch_kernel<1>, grid, 256, 0, s, P, n_sh, nx);
}

hipError_t launch_batch_down(const DecodeProblem &P, hipStream_t s) {
  const int n_sh = shared_chunks(P, 4 * kDnTT);
  if (P.T == 0 || n_sh + P.n_routed_slots == 0) return hipSuccess;
  const int nx = row_blocks_per_group(P.h / kDnR);
  return launch(down_batch_kernel, dim3(P.h / kDnR / nx, n_sh + P.n_routed_slots), 256, 0, s, P, n_sh, nx);
}

}  // namespace coli
