// Prefill-sized expert FFN: grouped GEMMs on the bf16 matrix cores (MFMA)
// with float32 accumulation.
//
// Source: "colibri engine teardown" page, "Three key engineering decisions",
// item 1 -- int4 "gs64" experts (64 weights share one scale); cf-1.com
// Colibri article, section 3.3 step 4 -- every expert with tokens runs one
// GEMM on its token group, fed by the expert offsets of step 3.  With
// thousands of tokens the expert FFN is a dense contraction per expert
// (M = tokens of the expert, N = weight rows, K = columns), so it runs on
// v_mfma_f32_32x32x16_bf16.
//
// Operands:
//  A  activations in bf16 ([T][h] hidden rows for gate/up, the intermediate
//     [P][I] for down), gathered per tile into LDS;
//  B  the weights dequantised in registers straight into bf16: code q of a
//     64-column group with scale s becomes bf16(q * s), computed as
//     fma(u, s, -8 s) with u = q + 8 taken as an unsigned byte (exact before
//     the one rounding to bf16).  Each weight is dequantised once per tile
//     and feeds the 8 MFMA blocks of the tile's 256 tokens.
//
// Tiles: 256 rows of A (tokens of one expert) x 256 weight rows (gate/up:
// 128 intermediate rows of gate and the same 128 of up; down: 256 output
// rows); 8 waves, two per SIMD so that one wave's dequantisation overlaps the
// other's MFMAs.  Wave w owns one 32-row MFMA block of B (gate/up: pair
// w / 2, gate for even w, up for odd w) and all 256 tokens (8 blocks of 32
// tokens, those wholly past the expert's last token skipped).  K runs in
// steps of 64 columns (one scale group); each lane owns 32 of the 64
// columns, so the 4 MFMAs of a step cover columns {8j..8j+7} and
// {32+8j..32+8j+7} -- K is a sum index, any order common to A and B gives
// the same products.  A rows and weights are copied into LDS rings ahead of
// use.  For SwiGLU the up waves hand their accumulators to the gate waves
// through LDS.
//
// The tile list (expert slot, first token) is built on the device from the
// dispatch offsets.  The grid is launched for the largest possible list; each
// block maps its hardware index to a (tile, column block) pair so that the
// column blocks of one tile run on one XCD (hardware block i runs on XCD
// i mod 8), where they share the tile's activation rows in that XCD's L2, and
// blocks past the real list leave at once.
#include "internal.h"
#include "wave.h"

namespace coli {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 256;          // tokens per tile
constexpr int BK = 64;           // columns per K step = one scale group
constexpr int kWaves = 8;        // waves per block
constexpr int kThreads = 64 * kWaves;
constexpr int kXcds = 8;

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ float ubyte(uint32_t v, int j) {
  float f;
  switch (j) {
    case 0: asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(f) : "v"(v)); break;
    case 1: asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(f) : "v"(v)); break;
    case 2: asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(f) : "v"(v)); break;
    default: asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(f) : "v"(v)); break;
  }
  return f;
}

// 8 int4 codes (nibble c = column c, two's complement) -> bf16(q * s) in
// column order.  m8s = -8 s.
__device__ __forceinline__ bf16x8 dequant_word(uint32_t w, float s, float m8s) {
  const uint32_t v = w ^ 0x88888888u;  // u = q + 8 in every nibble
  const uint32_t lo = v & 0x0F0F0F0Fu, hi = (v >> 4) & 0x0F0F0F0Fu;
  uint32_t p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    p[j] = pack_bf16(__builtin_fmaf(ubyte(lo, j), s, m8s), __builtin_fmaf(ubyte(hi, j), s, m8s));
  return __builtin_bit_cast(bf16x8, p);
}

struct Tile {
  int p_begin, rows;  // first sorted position of the tile, valid rows (1..BM)
  int e;              // expert, -1 = shared
};

// Maps the hardware block index to (tile, column block); false for surplus
// blocks.  Hardware block b runs on XCD b mod 8; XCD x takes tiles x, x + 8,
// x + 16, ... in that order (the list is sorted by size, largest first, so
// every XCD gets a similar share), all column blocks of a tile in a row, so
// that they share the tile's activation rows in the XCD's L2.
// nb = column blocks per tile.
__device__ __forceinline__ bool tile_of_block(const PrefillProblem &P, int nb, Tile &t, int &n_blk) {
  const int n_tiles = *P.n_tiles;
  const int b = blockIdx.x, xcd = b % kXcds, j = b / kXcds;
  const int tile = xcd + kXcds * (j / nb);
  if (tile >= n_tiles) return false;
  n_blk = j % nb;
  const int2 d = P.tiles[tile];
  int cnt;
  if (d.x < 0) {
    t.e = -1;
    t.p_begin = P.T * P.k + d.y;
    cnt = P.T;
  } else {
    t.e = P.active[d.x];
    const int o = P.offsets[t.e];
    t.p_begin = o + d.y;
    cnt = P.offsets[t.e + 1] - o;
  }
  t.rows = min(BM, cnt - d.y);
  return true;
}

// LDS rings, filled by LDS-DMA loads (global_load_lds, 16 or 4 bytes per
// lane, lane-linear in LDS):
//  A ring, 4 slots = two pairs of K steps (the pair being computed and the
//    next pair in flight): the tile's rows of 64 bf16 (128 bytes = 8 chunks
//    of 16 bytes); chunk c of row r sits in slot c ^ ((r >> 1) & 7), so that
//    the 16 rows read by 16 neighbouring lanes fall in 16 different bank
//    groups (64 banks).  One block barrier per pair of steps publishes a
//    pair and frees the previous one.
//  Q ring, 3 slots of one step of codes: 256 weight rows x 32 bytes (row
//    b = 32 w + l of wave w, lane row l; the two 16-byte halves of rows with
//    bit 3 set swapped, again for the banks).
//  S ring, 2 slots of four steps of scales: 256 rows x 16 bytes, so that a
//    row's 4 consecutive scales come in one 16-byte copy.
// The Q and S rows of a wave are copied and read by that wave only (no
// barrier).  Per pair of steps and wave: 2 (NMB + 1) / 2 copies of A rows
// (copy i of wave w holds tile rows 8 c .. 8 c + 7, c = 8 i + w, or c - 4
// where that passes the NMB * 32 rows: an identical second copy), 2 of codes,
// and every other pair 1 of scales.  Copies past the end re-fetch the last
// step (chunk) into a slot no later step reads, so the issue pattern never
// changes and the waits are constants.
constexpr int kASlots = 4, kQSlots = 3, kSSlots = 2, kSChunk = 4;
constexpr int kASlotBytes = BM * 128;              // 32 KB
constexpr int kQSlotBytes = 256 * 32;              // 8 KB
constexpr int kSSlotBytes = 256 * 4 * kSChunk;     // 4 KB
constexpr int kQRingOff = kASlots * kASlotBytes;
constexpr int kSRingOff = kQRingOff + kQSlots * kQSlotBytes;
constexpr int kLdsBytes = kSRingOff + kSSlots * kSSlotBytes;
static_assert(kLdsBytes <= 160 * 1024, "LDS rings exceed the 160 KB of a CU");

__device__ __forceinline__ uint32_t lds_addr(const char *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

// LDS-DMA loads: M0 holds the LDS address of lane 0's data (one wait state
// between the M0 write and the load).  Issued from inline assembly so that
// the compiler does not fold them into its own vmcnt bookkeeping; their
// completion is awaited explicitly (dma_wait).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(uint32_t lds, const void *base, uint32_t off) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(off), "s"(base)
               : "memory", "m0");
}
__device__ __forceinline__ void dma16v(uint32_t lds, const void *addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(addr)
               : "memory", "m0");
}
#pragma clang diagnostic pop
template <int N>
__device__ __forceinline__ void dma_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}



__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Where this lane's copies come from.
struct Sources {
  const char *a_base;    // A rows (byte base)
  uint32_t a_off[4];     // copy i: byte offset of its row for this lane plus this lane's chunk
  const uint8_t *q_base; // codes of this wave's 32 rows
  uint32_t q_off;        // row lane / 2 of the 32, this lane's 16 bytes
  const float *s_row;    // scales of row 32 w + lane (lanes 0..31)
};

template <int NMB>
struct ACopies {
  static constexpr int kPerWave = (NMB + 1) / 2;
  // A copy index (8 rows each) of copy i of wave w
  __device__ static __forceinline__ int index(int i, int w) {
    const int c = 8 * i + w;
    return c < 4 * NMB ? c : c - 4;
  }
};

// Byte offset of row r's chunk for copy lane `lane` (row r = 8 c + lane / 8).
__device__ __forceinline__ uint32_t a_chunk(int r, int lane) { return (uint32_t)(((lane & 7) ^ ((r >> 1) & 7)) * 16); }

template <int NMB>
__device__ __forceinline__ void copy_a(const Sources &S, int g, char *lds, int slot, int i) {
  const uint32_t base = lds_addr(lds) + slot * kASlotBytes;
  dma16(base + 8 * ACopies<NMB>::index(i, wave_id()) * 128, S.a_base + (size_t)g * (BK * 2), S.a_off[i]);
}

__device__ __forceinline__ void copy_q(const Sources &S, int g, char *lds, int slot) {
  dma16(lds_addr(lds) + kQRingOff + slot * kQSlotBytes + 32 * wave_id() * 32, S.q_base + (size_t)g * 32, S.q_off);
}

// scales of steps 4 c .. 4 c + 3 (lanes 0..31, one row each)
__device__ __forceinline__ void copy_s(const Sources &S, int c, char *lds, int slot) {
  if ((threadIdx.x & 63) < 32)
    dma16v(lds_addr(lds) + kSRingOff + slot * kSSlotBytes + 32 * wave_id() * 16, S.s_row + kSChunk * c);
}

// The copies of a pair of steps issued during its first step, one or two
// between MFMA groups so that no wave stalls on a burst of them: A(ga) copies,
// A(ga + 1) copies, the codes of step gq, then (when sc >= 0) the scales of
// chunk sc.
template <int NMB>
struct PairCopies {
  static constexpr int kA = ACopies<NMB>::kPerWave, kCount = 2 * kA + 1;
  const Sources &S;
  char *lds;
  int ga, sa, gq, sq, sc, ss;
  __device__ __forceinline__ void copy(int x) const {
    if (x < kA)
      copy_a<NMB>(S, ga, lds, sa, x);
    else if (x < 2 * kA)
      copy_a<NMB>(S, ga + 1, lds, (sa + 1) & 3, x - kA);
    else
      copy_q(S, gq, lds, sq);
  }
  // copies issued after MFMA group j (0..3) of the step
  __device__ __forceinline__ void after(int j) const {
#pragma unroll
    for (int x = j * kCount / 4; x < (j + 1) * kCount / 4; ++x) copy(x);
    if (j == 3 && sc >= 0) copy_s(S, sc, lds, ss);
  }
};

// The codes of step g into slot sq, issued after the first MFMA group.
struct QCopies {
  const Sources &S;
  char *lds;
  int g, sq;
  __device__ __forceinline__ void after(int j) const {
    if (j == 0) copy_q(S, g, lds, sq);
  }
};

// One wave's share of a tile: acc = A x B^T for its 32 weight rows over the
// K columns of the tile (G steps of 64), for the first NMB token blocks of
// the tile (NMB is uniform over the block, so the MFMA sequence is
// straight-line code).
template <int NMB>
struct WaveGemm {
  f32x16 acc[NMB];

  // One 64-column step.  Software-pipelined by MFMA group: while the NMB
  // MFMAs of group j run, the A fragments of group j + 1 are read from LDS
  // and its weights dequantised (the compiler interleaves them; a fixed
  // one MFMA : one LDS read : three VALU pattern measured 3% slower).
  // Step g from A slot g & 3, Q slot sq.
  template <class C>
  __device__ __forceinline__ void compute(const char *lds, int g, int sq, const C &copies) {
    const int lane = threadIdx.x & 63, wave = wave_id(), nl = lane & 31, half = lane >> 5;
    const char *A = lds + (g & 3) * kASlotBytes;
    const char *Q = lds + kQRingOff + sq * kQSlotBytes;
    const uint4 q = *reinterpret_cast<const uint4 *>(Q + 32 * wave * 32 + 16 * (2 * nl + (half ^ ((nl >> 3) & 1))));
    const float c = *reinterpret_cast<const float *>(lds + kSRingOff + ((g >> 2) & 1) * kSSlotBytes +
                                                     (32 * wave + nl) * 16 + (g & 3) * 4);
    const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
    const float m8c = -8.0f * c;
    // row r = 32 mb + nl of group j: chunk slot (4 half + j) ^ ((r >> 1) & 7), (r >> 1) & 7 = (nl >> 1) & 7
    const char *arow = A + nl * 128;
    const int sw_ = (nl >> 1) & 7;
    bf16x8 af[2][NMB], bf[2];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      af[0][mb] = *reinterpret_cast<const bf16x8 *>(arow + mb * 4096 + (((4 * half) ^ sw_) * 16));
    bf[0] = dequant_word(qw[0], c, m8c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cur = j & 1, nxt = cur ^ 1;
      if (j < 3) {
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
          af[nxt][mb] = *reinterpret_cast<const bf16x8 *>(arow + mb * 4096 + (((4 * half + j + 1) ^ sw_) * 16));
        bf[nxt] = dequant_word(qw[j + 1], c, m8c);
      }
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][mb], bf[cur], acc[mb], 0, 0, 0);
      copies.after(j);
    }
  }

  // Issue order (pair of steps g, g + 1, g even):
  //   [barrier] A(g+2) A(g+3) Q(g+2) (S(g/4 + 1) when g % 4 == 0) | step g |
  //   Q(g+3) | step g + 1
  // (indices past the end re-fetch the last one).  Before step g: A(g),
  // A(g+1), Q(g) and S(g/4) are done once at most Q(g+1) and, when g % 4 ==
  // 2, S(g/4) are pending; before step g + 1, Q(g+1) is done once at most the
  // pair's own copies are pending.
  static constexpr int kA = ACopies<NMB>::kPerWave;

  __device__ __forceinline__ void run(const Sources &S, int G, char *lds) {  // G >= 4, G % 4 == 0
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) acc[mb] = f32x16{};
    const int last_chunk = G / kSChunk - 1;
#pragma unroll
    for (int i = 0; i < kA; ++i) copy_a<NMB>(S, 0, lds, 0, i);
#pragma unroll
    for (int i = 0; i < kA; ++i) copy_a<NMB>(S, 1, lds, 1, i);
    copy_s(S, 0, lds, 0);
    copy_q(S, 0, lds, 0);
    copy_q(S, 1, lds, 1);
    int sq = 0;  // Q slot of step g (g % 3)
    for (int g = 0; g < G; g += 2) {
      if (g % 4 == 2)
        dma_wait<2>();
      else
        dma_wait<1>();
      block_barrier();  // pair visible to all waves; all waves done with the previous pair
      const int sq1 = sq == 2 ? 0 : sq + 1, sq2 = sq1 == 2 ? 0 : sq1 + 1;
      const bool chunk = g % 4 == 0;
      const PairCopies<NMB> pc{S,  lds, min(g + 2, G - 2), (g + 2) & 3, min(g + 2, G - 1), sq2,
                               chunk ? min(g / 4 + 1, last_chunk) : -1, (g / 4 + 1) & 1};
      compute(lds, g, sq, pc);
      if (chunk)
        dma_wait<2 * kA + 2>();
      else
        dma_wait<2 * kA + 1>();
      compute(lds, g + 1, sq1, QCopies{S, lds, min(g + 3, G - 1), sq});  // Q(g+3) into step g's slot
      sq = sq2;
    }
    dma_wait<0>();    // no copy may land in LDS after this point
    block_barrier();  // every wave done with the rings (free for the epilogue)
  }
};

// Row m of the tile held by register i of an MFMA block (token-block mb).
__device__ __forceinline__ int acc_row(int mb, int half, int i) { return 32 * mb + 4 * half + 8 * (i >> 2) + (i & 3); }

// ---------------------------------------------------------------------------
// gate/up: mid[p][n] = silu(x_t . Wg[n]) * (x_t . Wu[n]), bf16.
// Column blocks of 128 intermediate rows.
// ---------------------------------------------------------------------------
template <int NMB>
__device__ __forceinline__ void a_sources(Sources &S, const PrefillProblem &P, const Tile &t, bool gather, int row_bytes) {
  const int lane = threadIdx.x & 63, wave = wave_id();
#pragma unroll
  for (int i = 0; i < ACopies<NMB>::kPerWave; ++i) {
    // tile row of this lane in copy i (padding rows repeat the last valid row)
    const int r = 8 * ACopies<NMB>::index(i, wave) + (lane >> 3);
    const int p = t.p_begin + min(r, t.rows - 1);
    const int row = !gather ? p : (t.e < 0 ? p - P.T * P.k : P.sorted_ids[p] / P.k);
    S.a_off[i] = (uint32_t)row * (uint32_t)row_bytes + a_chunk(r, lane);
  }
}

template <int NMB>
__device__ __forceinline__ void gate_up_tile(const PrefillProblem &P, const Tile &t, int n_blk, char *lds) {
  const int h = P.h, I = P.I;
  const int lane = threadIdx.x & 63, wave = wave_id(), nl = lane & 31, half = lane >> 5;
  const int pair = wave >> 1, up = wave & 1;
  Sources S;
  S.a_base = reinterpret_cast<const char *>(P.xb);
  a_sources<NMB>(S, P, t, true, h * 2);
  const size_t qstride = (size_t)I * (h >> 1), sstride = (size_t)I * (h >> 6);
  const ExpertTables &M = t.e < 0 ? (up ? P.sh_up : P.sh_gate) : (up ? P.up : P.gate);
  const size_t eq = t.e < 0 ? 0 : (size_t)t.e * qstride, es = t.e < 0 ? 0 : (size_t)t.e * sstride;
  const int row0 = n_blk * 128 + pair * 32;  // this wave's gate or up rows row0 .. row0 + 31
  S.q_base = M.q + eq + (size_t)row0 * (h >> 1);
  S.q_off = (uint32_t)((lane >> 1) * (h >> 1) + ((lane & 1) ^ ((lane >> 4) & 1)) * 16);
  S.s_row = M.s + es + (size_t)(row0 + nl) * (h >> 6);

  WaveGemm<NMB> W;
  W.run(S, h / BK, lds);

  // up waves hand their accumulators to the gate wave of their pair, lane by
  // lane (the same lane holds the same (token, row) in both waves)
  float *xchg = reinterpret_cast<float *>(lds) + (size_t)pair * (NMB * 16 * 64);
  if (up) {
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) xchg[(mb * 16 + i) * 64 + lane] = W.acc[mb][i];
  }
  block_barrier();
  if (!up) {
    const int n = row0 + nl;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = acc_row(mb, half, i);
        if (m < t.rows) {
          const float gv = W.acc[mb][i], uv = xchg[(mb * 16 + i) * 64 + lane];
          // silu in float32 with the hardware exp and reciprocal (the result is
          // rounded to bf16)
          const float sg = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv));
          P.mid[(size_t)(t.p_begin + m) * I + n] = (__bf16)(sg * uv);
        }
      }
  }
}

// ---------------------------------------------------------------------------
// down: y[p][r] = mid[p] . Wd[r], float32.  Column blocks of 256 output rows.
// ---------------------------------------------------------------------------
template <int NMB>
__device__ __forceinline__ void down_tile(const PrefillProblem &P, const Tile &t, int n_blk, char *lds) {
  const int h = P.h, I = P.I;
  const int lane = threadIdx.x & 63, wave = wave_id(), nl = lane & 31, half = lane >> 5;
  Sources S;
  S.a_base = reinterpret_cast<const char *>(P.mid);
  a_sources<NMB>(S, P, t, false, I * 2);
  const size_t qstride = (size_t)h * (I >> 1), sstride = (size_t)h * (I >> 6);
  const ExpertTables &D = t.e < 0 ? P.sh_down : P.down;
  const int row0 = n_blk * 256 + wave * 32;  // this wave's rows row0 .. row0 + 31
  S.q_base = D.q + (t.e < 0 ? 0 : (size_t)t.e * qstride) + (size_t)row0 * (I >> 1);
  S.q_off = (uint32_t)((lane >> 1) * (I >> 1) + ((lane & 1) ^ ((lane >> 4) & 1)) * 16);
  S.s_row = D.s + (t.e < 0 ? 0 : (size_t)t.e * sstride) + (size_t)(row0 + nl) * (I >> 6);

  WaveGemm<NMB> W;
  W.run(S, I / BK, lds);

  const int r = row0 + nl;
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = acc_row(mb, half, i);
      if (m < t.rows) P.y[(size_t)(t.p_begin + m) * h + r] = W.acc[mb][i];
    }
}

#define COLI_NMB_SWITCH(FN)                \
  switch ((t.rows + 31) / 32) {            \
    case 1: FN<1>(P, t, n_blk, lds); break; \
    case 2: FN<2>(P, t, n_blk, lds); break; \
    case 3: FN<3>(P, t, n_blk, lds); break; \
    case 4: FN<4>(P, t, n_blk, lds); break; \
    case 5: FN<5>(P, t, n_blk, lds); break; \
    case 6: FN<6>(P, t, n_blk, lds); break; \
    case 7: FN<7>(P, t, n_blk, lds); break; \
    default: FN<8>(P, t, n_blk, lds); break; \
  }

// 1-D grids of kThreads threads (see tile_of_block).
__global__ __launch_bounds__(kThreads, 1) void gate_up_mfma_kernel(PrefillProblem P) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  Tile t;
  int n_blk;
  if (!tile_of_block(P, P.I / 128, t, n_blk)) return;  // uniform over the block
  COLI_NMB_SWITCH(gate_up_tile)
}

__global__ __launch_bounds__(kThreads, 1) void down_mfma_kernel(PrefillProblem P) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  Tile t;
  int n_blk;
  if (!tile_of_block(P, P.h / 256, t, n_blk)) return;
  COLI_NMB_SWITCH(down_tile)
}
#undef COLI_NMB_SWITCH

// ---------------------------------------------------------------------------
// Tile list: (slot, first token) for every BM tokens of every active expert,
// then of the shared expert (slot -1), ordered by the tile's count of 32-token
// blocks, largest first, and by slot within a count.  One workgroup of 1024 threads, one slot per thread
// (n_active <= 512).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t *__restrict__ offsets,
                                                           const int32_t *__restrict__ active,
                                                           const int32_t *__restrict__ n_active, int T,
                                                           int has_shared, int2 *__restrict__ tiles,
                                                           int32_t *__restrict__ n_tiles) {
  constexpr int kB = BM / 32;  // token-block counts 1..kB
  __shared__ int32_t wave_sum[16][kB + 1];
  __shared__ int32_t bucket_start[kB + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int na = *n_active;
  int cnt = 0;
  if (tid < na) {
    const int e = active[tid];
    cnt = offsets[e + 1] - offsets[e];
  } else if (tid == na && has_shared) {
    cnt = T;
  }
  const int full = cnt / BM, rest = cnt - full * BM;
  const int part_nb = (rest + 31) / 32;  // 0 = no partial tile
  // per bucket: full tiles go to bucket kB, the partial one to bucket part_nb;
  // exclusive scans over threads for each bucket (bucket kB counts full tiles)
  int mine[kB + 1], before[kB + 1];
#pragma unroll
  for (int k = 0; k <= kB; ++k) {
    mine[k] = (k == kB ? full : 0) + (k == part_nb && k > 0 ? 1 : 0);
    int incl = mine[k];
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d);
      if (lane >= d) incl += v;
    }
    before[k] = incl - mine[k];
    if (lane == 63) wave_sum[wave][k] = incl;
  }
  __syncthreads();
  if (tid == 0) {
    int o = 0;
    for (int k = kB; k >= 1; --k) {  // largest first
      bucket_start[k] = o;
      for (int w = 0; w < 16; ++w) o += wave_sum[w][k];
    }
    bucket_start[0] = o;
    *n_tiles = o;
  }
  __syncthreads();
  const int slot = tid < na ? tid : -1;
#pragma unroll
  for (int k = 1; k <= kB; ++k) {
    if (!mine[k]) continue;
    int o = bucket_start[k] + before[k];
    for (int w = 0; w < wave; ++w) o += wave_sum[w][k];
    if (k == kB) {
      for (int i = 0; i < full; ++i) tiles[o + i] = make_int2(slot, i * BM);
      if (part_nb == kB) tiles[o + full] = make_int2(slot, full * BM);
    } else {
      tiles[o] = make_int2(slot, full * BM);
    }
  }
}

// x [T][h] float -> bf16 (round to nearest even), 8 values per thread.
__global__ __launch_bounds__(256) void to_bf16_kernel(const float *__restrict__ x, size_t n_words,
                                                      __bf16 *__restrict__ xb) {
  const size_t w = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (w >= n_words) return;
  const float4 a = reinterpret_cast<const float4 *>(x)[2 * w];
  const float4 b = reinterpret_cast<const float4 *>(x)[2 * w + 1];
  const uint4 o = make_uint4(pack_bf16(a.x, a.y), pack_bf16(a.z, a.w), pack_bf16(b.x, b.y), pack_bf16(b.z, b.w));
  reinterpret_cast<uint4 *>(xb)[w] = o;
}

int grid_blocks(int nb, int max_tiles) { return kXcds * nb * ((max_tiles + kXcds - 1) / kXcds); }

}  // namespace

bool prefill_shape_ok(int h, int I) { return h % 256 == 0 && I % 256 == 0; }

int prefill_max_tiles(int T, int k, int E, int has_shared) {
  const int n = T * k, routed_slots = E < n ? E : n;
  return n / BM + routed_slots + (has_shared ? (T + BM - 1) / BM : 0);
}

hipError_t launch_prefill_prep(const float *x, int T, int h, __bf16 *xb, hipStream_t s) {
  const size_t n_words = (size_t)T * h / 8;
  return launch(to_bf16_kernel, (unsigned)((n_words + 255) / 256), 256, 0, s, x, n_words, xb);
}

hipError_t launch_build_tiles(const PrefillProblem &P, hipStream_t s) {
  return launch(build_tiles_kernel, 1, 1024, 0, s, P.offsets, P.active, P.n_active, P.T, P.has_shared, P.tiles, P.n_tiles);
}

hipError_t launch_gate_up_mfma(const PrefillProblem &P, hipStream_t s) {
  const int blocks = grid_blocks(P.I / 128, prefill_max_tiles(P.T, P.k, P.E, P.has_shared));
  return launch(gate_up_mfma_kernel, blocks, kThreads, 0, s, P);
}

hipError_t launch_down_mfma(const PrefillProblem &P, hipStream_t s) {
  const int blocks = grid_blocks(P.h / 256, prefill_max_tiles(P.T, P.k, P.E, P.has_shared));
  return launch(down_mfma_kernel, blocks, kThreads, 0, s, P);
}

}  // namespace coli
