// Prefill-sized expert FFN: grouped GEMMs on the fp16 matrix cores (MFMA)
// with float32 accumulation.
//
// Source: "colibri engine teardown" page, "Three key engineering decisions",
// item 1 -- int4 "gs64" experts (64 weights share one scale); cf-1.com
// Colibri article, section 3.3 step 4 -- every expert with tokens runs one
// GEMM on its token group, fed by the expert offsets of step 3.  With
// thousands of tokens the expert FFN is a dense contraction per expert
// (M = tokens of the expert, N = weight rows, K = columns), so it runs on
// v_mfma_f32_32x32x16_f16.
//
// Number format.  The 16-bit operands are IEEE half precision (11-bit
// significand): the matrix cores run it at the bf16 rate, the int4 codes
// become halves with two packed instructions per pair, and every operand
// rounding is 8 times smaller than bf16's.  Half precision has a narrow
// exponent range, which power-of-two factors recover exactly:
//  - hidden rows: x' = x * 2^-ex(t), ex(t) chosen per token so that
//    max |x'| lies in [2^14, 2^15) (prep kernel, which also records
//    ||x'||^2);
//  - weights: w' = half(q * half(s * 2^ew)), ew per expert matrix chosen so
//    that the largest scale times 2^ew lies in [2^11, 2^12), so |w'| < 2^15
//    (scale_stats_kernel, at init);
//  - intermediate: mid' = mid * 2^(14 - eb), with eb = floor(log2 B) for a
//    bound B >= |mid| of the (token, expert): |silu(g)| <= |g| and
//    |g_i| <= ||x|| ||G_i||, ||G_i|| <= 64 ||s_i|| (|q| <= 8, 64 codes per
//    scale), so B = 4096 ||x||^2 max_i ||sG_i|| max_i ||sU_i||, and
//    |mid'| < 2^15.
// The float32 epilogues undo each factor exactly (ldexp).
//
// Weight conversion: a 32-bit word holds 8 codes (nibble c = column c, two's
// complement).  Flipping a nibble's top bit turns it into u = q + 8; the
// halves 0x6400 | u and 0x6400 | (u << 4) are 1024 + u and 1024 + 16 u, so a
// packed add of -1032 (or -1152) leaves q (or 16 q) exactly, and a packed
// multiply by the group's half scale (or a sixteenth of it) rounds q * s
// once to half.  The 8 halves come out in the column order
// 0 4 1 5 2 6 3 7; K is a sum index, so the activations are stored in the
// same order within every 8 columns (prep kernel and the gate/up epilogue),
// and A and B agree.
//
// Tiles: 256 rows of A (tokens of one expert) x 256 weight rows (gate/up:
// 128 intermediate rows of gate and the same 128 of up; down: 256 output
// rows) in 8 groups of 32 rows; 8 waves, two per SIMD, wave w copying group
// w.  K runs in steps of 64 columns (one scale group); each lane owns 32 of
// the 64 columns, so the 4 MFMAs of a step cover columns {8j..8j+7} and
// {32+8j..32+8j+7}.  A rows and weights are copied into LDS rings ahead of
// use, the copies spread between MFMA groups.
//  - down: wave w computes group w for all 256 tokens (8 blocks of 32
//    tokens, those wholly past the expert's last token skipped), so each
//    converted weight feeds up to 8 MFMAs;
//  - gate/up: wave w computes the gate group and the up group of pair w % 4
//    for the 128 tokens of half w / 4, so each A fragment read from LDS
//    feeds two MFMAs (half the LDS reads per MFMA, twice the conversions:
//    4% faster than one group per wave) and SwiGLU needs no exchange.
// Tiles are long in M and short in N because a token row per step is one
// whole cache line while a weight row per step is a 32-byte piece of one: the
// copies cost least per MFMA that way.
//
// The tile list (expert slot, first token) is built on the device from the
// dispatch offsets, largest tiles first.  The grid is launched for the
// largest possible list; each block maps its hardware index to a (tile,
// column block) pair so that the column blocks of one tile run on one XCD
// (hardware block i runs on XCD i mod 8), where they share the tile's
// activation rows in that XCD's L2, and blocks past the real list leave at
// once.
#include "internal.h"
#include "wave.h"

namespace coli {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 256;          // tokens per tile
constexpr int BK = 64;           // columns per K step = one scale group
constexpr int kWaves = 8;        // waves per block
constexpr int kThreads = 64 * kWaves;
constexpr int kXcds = 8;

// Exponent range kept for the intermediate's bound.
constexpr int kMidExpMin = -100, kMidExpMax = 100;
// LDS after the K loop: the up waves' accumulators (up to 128 KB), then the
// tile rows' exponents.
constexpr int kRowExpOff = 128 * 1024;

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Storage position of column c within its group of 8 (column order
// 0 4 1 5 2 6 3 7 of the converted weights).
__device__ __forceinline__ int perm8(int c) { return (c & ~7) | ((c & 3) << 1) | ((c >> 2) & 1); }

// floor(log2 |v|) for v != 0 (denormals included).
__device__ __forceinline__ int ilog2f(float v) { return __builtin_amdgcn_frexp_expf(v) - 1; }

// Bits of k where m is clear, bits of a ^ k where m is set (one v_bitop3).
__device__ __forceinline__ uint32_t merge_xor(uint32_t a, uint32_t m, uint32_t k) { return ((a ^ k) & m) | (k & ~m); }

// 8 int4 codes -> half(q * s) in the order 0 4 1 5 2 6 3 7; s1 = (s, s),
// s16 = (s / 16, s / 16) as halves.  Each pair: the two nibbles with their
// sign bit flipped (u = q + 8) dropped into the low mantissa bits of 1024
// (bits 0-3) or, for the odd nibbles, bits 4-7 (1024 + 16 u).
__device__ __forceinline__ f16x8 convert8(uint32_t w, f16x2 s1, f16x2 s16) {
  const uint32_t w8 = w >> 8;
  constexpr uint32_t kLo = 0x000F000Fu, kHi = 0x00F000F0u;
  constexpr uint32_t kLoMagic = 0x64086408u, kHiMagic = 0x64806480u;  // 1024, 1024 with the sign bits to flip
  const f16x2 c0 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const f16x2 c1 = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  const f16x2 d0 = (__builtin_bit_cast(f16x2, merge_xor(w, kLo, kLoMagic)) + c0) * s1;
  const f16x2 d1 = (__builtin_bit_cast(f16x2, merge_xor(w, kHi, kHiMagic)) + c1) * s16;
  const f16x2 d2 = (__builtin_bit_cast(f16x2, merge_xor(w8, kLo, kLoMagic)) + c0) * s1;
  const f16x2 d3 = (__builtin_bit_cast(f16x2, merge_xor(w8, kHi, kHiMagic)) + c1) * s16;
  return f16x8{d0[0], d0[1], d1[0], d1[1], d2[0], d2[1], d3[0], d3[1]};
}

struct Tile {
  int p_begin, rows;  // first sorted position of the tile, valid rows (1..BM)
  int e;              // expert, -1 = shared
  int stat;           // index into the per-expert statistics (E for the shared expert)
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
    t.stat = P.E;
    t.p_begin = P.T * P.k + d.y;
    cnt = P.T;
  } else {
    t.e = P.active[d.x];
    t.stat = t.e;
    const int o = P.offsets[t.e];
    t.p_begin = o + d.y;
    cnt = P.offsets[t.e + 1] - o;
  }
  t.rows = min(BM, cnt - d.y);
  return true;
}

// LDS rings, filled by LDS-DMA loads (global_load_lds, 16 bytes per lane,
// lane-linear in LDS):
//  A ring, 4 slots = two pairs of K steps (the pair being computed and the
//    next pair in flight): the tile's rows of 64 halves (128 bytes = 8 chunks
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
template <int N>
__device__ __forceinline__ void dma_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
#pragma clang diagnostic pop

// Where this lane's copies come from.
struct Sources {
  const char *a_base;    // A rows (byte base)
  uint32_t a_off[4];     // copy i: byte offset of its row for this lane plus this lane's chunk
  const uint8_t *q_base; // codes of this wave's 32 rows
  uint32_t q_off;        // row lane / 2 of the 32, this lane's 16 bytes
  const float *s_row;    // scales of row 32 w + lane (lanes 0..31)
  float wm[2];           // 2^ew of the weight groups this wave computes
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

// One wave's share of a tile: acc = A x B^T for its weight rows over the K
// columns of the tile (G steps of 64).  Wave w copies weight group w (rows
// 32 w .. 32 w + 31 of the tile's 256) and
//  - PAIRS = false: computes group w for the first NMB token blocks;
//  - PAIRS = true: computes groups 2 (w % 4) and 2 (w % 4) + 1 (a gate/up
//    pair) for NMW token blocks of its token half (blocks 4 (w / 4) ..), so
//    that every A fragment read from LDS feeds two MFMAs; each weight is
//    converted by the two waves that read it.  Waves read groups that other
//    waves copy, so every step, not only every pair of steps, starts at a
//    block barrier.
// NMB / NMW are uniform over the wave, so the MFMA sequence is straight-line
// code.
template <int NMB, int NMW, bool PAIRS>
struct WaveGemm {
  static constexpr int NBW = PAIRS ? 2 : 1;         // weight groups computed
  static constexpr int NA = NMW > 0 ? NMW : 1;
  f32x16 acc[NBW][NA];

  // One 64-column step.  Software-pipelined by MFMA group: while the MFMAs
  // of group j run, the A fragments of group j + 1 are read from LDS and its
  // weights converted (the compiler interleaves them; a fixed one MFMA : one
  // LDS read : three VALU pattern measured 3% slower).  Step g from A slot
  // g & 3, Q slot sq.
  template <class C>
  __device__ __forceinline__ void compute(const char *lds, int g, int sq, const float (&wm)[2], const C &copies) {
    const int lane = threadIdx.x & 63, wave = wave_id(), nl = lane & 31, half = lane >> 5;
    if constexpr (NMW == 0) {  // a token half past the tile: copies only
#pragma unroll
      for (int j = 0; j < 4; ++j) copies.after(j);
      return;
    }
    const int grp = PAIRS ? 2 * (wave & 3) : wave, row0 = PAIRS ? 128 * (wave >> 2) : 0;
    const char *A = lds + (g & 3) * kASlotBytes + row0 * 128;
    const char *Q = lds + kQRingOff + sq * kQSlotBytes + grp * (32 * 32);
    const char *Sc = lds + kSRingOff + ((g >> 2) & 1) * kSSlotBytes + grp * (32 * 16);
    uint32_t qw[NBW][4];
    f16x2 s1[NBW], s16[NBW];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      const uint4 q = *reinterpret_cast<const uint4 *>(Q + nb * (32 * 32) + 16 * (2 * nl + (half ^ ((nl >> 3) & 1))));
      qw[nb][0] = q.x, qw[nb][1] = q.y, qw[nb][2] = q.z, qw[nb][3] = q.w;
      const float sc = *reinterpret_cast<const float *>(Sc + (32 * nb + nl) * 16 + (g & 3) * 4) * wm[nb];
      const _Float16 h1 = (_Float16)sc, h16 = (_Float16)(sc * 0.0625f);
      s1[nb] = f16x2{h1, h1};
      s16[nb] = f16x2{h16, h16};
    }
    // row r = row0 + 32 mb + nl of group j: chunk slot (4 half + j) ^ ((r >> 1) & 7),
    // (r >> 1) & 7 = (nl >> 1) & 7
    const char *arow = A + nl * 128;
    const int sw_ = (nl >> 1) & 7;
    f16x8 af[2][NA], bf[2][NBW];
#pragma unroll
    for (int mb = 0; mb < NMW; ++mb)
      af[0][mb] = *reinterpret_cast<const f16x8 *>(arow + mb * 4096 + (((4 * half) ^ sw_) * 16));
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) bf[0][nb] = convert8(qw[nb][0], s1[nb], s16[nb]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cur = j & 1, nxt = cur ^ 1;
      if (j < 3) {
#pragma unroll
        for (int mb = 0; mb < NMW; ++mb)
          af[nxt][mb] = *reinterpret_cast<const f16x8 *>(arow + mb * 4096 + (((4 * half + j + 1) ^ sw_) * 16));
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) bf[nxt][nb] = convert8(qw[nb][j + 1], s1[nb], s16[nb]);
      }
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int mb = 0; mb < NMW; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[cur][mb], bf[cur][nb], acc[nb][mb], 0, 0, 0);
      copies.after(j);
    }
  }

  // Issue order (pair of steps g, g + 1, g even):
  //   [barrier] A(g+2) A(g+3) Q(g+2) (S(g/4 + 1) when g % 4 == 0) | step g |
  //   ([barrier] when PAIRS) Q(g+3) | step g + 1
  // (indices past the end re-fetch the last one).  Before step g: A(g),
  // A(g+1), Q(g) and S(g/4) are done once at most Q(g+1) and, when g % 4 ==
  // 2, S(g/4) are pending; before step g + 1, Q(g+1) is done once at most the
  // pair's own copies are pending.
  static constexpr int kA = ACopies<NMB>::kPerWave;

  __device__ __forceinline__ void run(const Sources &S, int G, char *lds) {  // G >= 4, G % 4 == 0
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
      for (int mb = 0; mb < NA; ++mb) acc[nb][mb] = f32x16{};
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
      compute(lds, g, sq, S.wm, pc);
      if (chunk)
        dma_wait<2 * kA + 2>();
      else
        dma_wait<2 * kA + 1>();
      if constexpr (PAIRS) block_barrier();  // Q(g+1) of every wave visible; every wave done with step g's slot
      compute(lds, g + 1, sq1, S.wm, QCopies{S, lds, min(g + 3, G - 1), sq});  // Q(g+3) into step g's slot
      sq = sq2;
    }
    dma_wait<0>();    // no copy may land in LDS after this point
    block_barrier();  // every wave done with the rings (free for the epilogue)
  }
};

// Row m of the tile held by register i of an MFMA block (token-block mb).
__device__ __forceinline__ int acc_row(int mb, int half, int i) { return 32 * mb + 4 * half + 8 * (i >> 2) + (i & 3); }

// Token of sorted position p (routed: its assignment's token; shared: p - T k).
__device__ __forceinline__ int token_of(const PrefillProblem &P, const Tile &t, int p) {
  return t.e < 0 ? p - P.T * P.k : P.sorted_ids[p] / P.k;
}

// Exponent eb of the intermediate's bound for token tok and the tile's expert.
__device__ __forceinline__ int mid_exp(const PrefillProblem &P, const PrefillStats &st, float cmid, int tok) {
  const float f = P.xn2[tok] * cmid;
  if (!(f > 0.0f)) return kMidExpMin;
  const int eb = ilog2f(f) + 2 * P.xexp[tok] - st.ew[0] - st.ew[1];
  return min(max(eb, kMidExpMin), kMidExpMax);
}

// 4096 max ||sG_i|| max ||sU_i|| over the prescaled scales.
__device__ __forceinline__ float mid_coef(const PrefillStats &st) { return 4096.0f * sqrtf(st.n2[0] * st.n2[1]); }

__device__ __forceinline__ float pow2f(int e) { return __builtin_amdgcn_ldexpf(1.0f, e); }

template <int NMB>
__device__ __forceinline__ void a_sources(Sources &S, const PrefillProblem &P, const Tile &t, bool gather, int row_bytes) {
  const int lane = threadIdx.x & 63, wave = wave_id();
#pragma unroll
  for (int i = 0; i < ACopies<NMB>::kPerWave; ++i) {
    // tile row of this lane in copy i (padding rows repeat the last valid row)
    const int r = 8 * ACopies<NMB>::index(i, wave) + (lane >> 3);
    const int p = t.p_begin + min(r, t.rows - 1);
    const int row = !gather ? p : token_of(P, t, p);
    S.a_off[i] = (uint32_t)row * (uint32_t)row_bytes + a_chunk(r, lane);
  }
}

// Exponents of tile row m (0 for rows past the tile): the token's ex and the
// intermediate's eb.  Each thread of the block takes one row.
struct RowExp {
  int ex, eb;
};
__device__ __forceinline__ RowExp row_exp(const PrefillProblem &P, const Tile &t, const PrefillStats &st, int m) {
  RowExp r{0, 0};
  if (m < t.rows) {
    const int tok = token_of(P, t, t.p_begin + m);
    r.ex = P.xexp[tok];
    r.eb = mid_exp(P, st, mid_coef(st), tok);
  }
  return r;
}

// ---------------------------------------------------------------------------
// gate/up: mid'[p][c] = half(silu(g) * u * 2^(14 - eb)), g = x . Wg[c],
// u = x . Wu[c].  Column blocks of 128 intermediate rows: weight group 2 q
// holds the gate rows c0 .. c0 + 31, group 2 q + 1 the up rows of the same c
// (c0 = 128 n + 32 q); wave w computes the pair q = w % 4 for the tokens of
// its half w / 4 (WaveGemm with PAIRS), so SwiGLU needs nothing from another
// wave.
// ---------------------------------------------------------------------------
template <int NMB, int NMW>
__device__ __forceinline__ void gate_up_finish(const PrefillProblem &P, const Tile &t, int n_blk, char *lds,
                                               const Sources &S, const PrefillStats &st, const RowExp &rx) {
  const int lane = threadIdx.x & 63, wave = wave_id(), nl = lane & 31, half = lane >> 5;
  WaveGemm<NMB, NMW, true> W;
  W.run(S, P.h / BK, lds);
  int2 *rowx = reinterpret_cast<int2 *>(lds + kRowExpOff);
  if (threadIdx.x < BM) rowx[threadIdx.x] = make_int2(rx.ex, rx.eb);
  block_barrier();
  const int cs = perm8(n_blk * 128 + (wave & 3) * 32 + nl);
#pragma unroll
  for (int mb = 0; mb < NMW; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = 128 * (wave >> 2) + acc_row(mb, half, i);
      if (m < t.rows) {
        const int2 e = rowx[m];
        const float g = __builtin_amdgcn_ldexpf(W.acc[0][mb][i], e.x - st.ew[0]);
        const float u = __builtin_amdgcn_ldexpf(W.acc[1][mb][i], e.x - st.ew[1]);
        // silu in float32 with the hardware exp and reciprocal
        const float sg = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
        const float mid = __builtin_amdgcn_ldexpf(sg * u, 14 - e.y);
        P.mid[(size_t)(t.p_begin + m) * P.I + cs] = (_Float16)mid;
      }
    }
}

template <int NMB>
__device__ __forceinline__ void gate_up_tile(const PrefillProblem &P, const Tile &t, int n_blk, char *lds) {
  const int h = P.h, I = P.I;
  const int lane = threadIdx.x & 63, wave = wave_id(), nl = lane & 31;
  const int pair = wave >> 1, up = wave & 1;  // the group this wave copies
  const PrefillStats st = P.stats[t.stat];
  Sources S;
  S.a_base = reinterpret_cast<const char *>(P.xb);
  a_sources<NMB>(S, P, t, true, h * 2);
  const size_t qstride = (size_t)I * (h >> 1), sstride = (size_t)I * (h >> 6);
  const ExpertTables &M = t.e < 0 ? (up ? P.sh_up : P.sh_gate) : (up ? P.up : P.gate);
  const size_t eq = t.e < 0 ? 0 : (size_t)t.e * qstride, es = t.e < 0 ? 0 : (size_t)t.e * sstride;
  const int row0 = n_blk * 128 + pair * 32;  // gate or up rows row0 .. row0 + 31
  S.q_base = M.q + eq + (size_t)row0 * (h >> 1);
  S.q_off = (uint32_t)((lane >> 1) * (h >> 1) + ((lane & 1) ^ ((lane >> 4) & 1)) * 16);
  S.s_row = M.s + es + (size_t)(row0 + nl) * (h >> 6);
  S.wm[0] = pow2f(st.ew[0]);
  S.wm[1] = pow2f(st.ew[1]);
  // this thread's tile row: its token's exponent and the intermediate's
  // (loads issued now, used after the K loop)
  const RowExp rx = row_exp(P, t, st, threadIdx.x);
  constexpr int N0 = NMB < 4 ? NMB : 4, N1 = NMB > 4 ? NMB - 4 : 0;  // token blocks of the two halves
  if (wave < 4)
    gate_up_finish<NMB, N0>(P, t, n_blk, lds, S, st, rx);
  else
    gate_up_finish<NMB, N1>(P, t, n_blk, lds, S, st, rx);
}

// ---------------------------------------------------------------------------
// down: y[p][r] = mid[p] . Wd[r], float32.  Column blocks of 256 output rows;
// wave w computes its own group, rows 32 w .. 32 w + 31, for every token
// block (with pairs, the grid of the gate/up tiles, down measured 7% slower).
// ---------------------------------------------------------------------------
template <int NMB>
__device__ __forceinline__ void down_tile(const PrefillProblem &P, const Tile &t, int n_blk, char *lds) {
  const int h = P.h, I = P.I;
  const int lane = threadIdx.x & 63, wave = wave_id(), nl = lane & 31, half = lane >> 5;
  const PrefillStats st = P.stats[t.stat];
  Sources S;
  S.a_base = reinterpret_cast<const char *>(P.mid);
  a_sources<NMB>(S, P, t, false, I * 2);
  const size_t qstride = (size_t)h * (I >> 1), sstride = (size_t)h * (I >> 6);
  const ExpertTables &D = t.e < 0 ? P.sh_down : P.down;
  const int row0 = n_blk * 256 + wave * 32;  // this wave's rows row0 .. row0 + 31
  S.q_base = D.q + (t.e < 0 ? 0 : (size_t)t.e * qstride) + (size_t)row0 * (I >> 1);
  S.q_off = (uint32_t)((lane >> 1) * (I >> 1) + ((lane & 1) ^ ((lane >> 4) & 1)) * 16);
  S.s_row = D.s + (t.e < 0 ? 0 : (size_t)t.e * sstride) + (size_t)(row0 + nl) * (I >> 6);
  S.wm[0] = S.wm[1] = pow2f(st.ew[2]);
  const RowExp rx = row_exp(P, t, st, threadIdx.x);

  WaveGemm<NMB, NMB, false> W;
  W.run(S, I / BK, lds);
  int *rowe = reinterpret_cast<int *>(lds + kRowExpOff);
  if (threadIdx.x < BM) rowe[threadIdx.x] = rx.eb - st.ew[2] - 14;
  block_barrier();

  const int r = row0 + nl;
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = acc_row(mb, half, i);
      if (m < t.rows) P.y[(size_t)(t.p_begin + m) * h + r] = __builtin_amdgcn_ldexpf(W.acc[0][mb][i], rowe[m]);
    }
}

#define COLI_NMB_SWITCH(FN)                 \
  switch ((t.rows + 31) / 32) {             \
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
// then of the shared expert (slot -1), ordered by the tile's count of
// 32-token blocks, largest first, and by slot within a count.  One workgroup
// of 1024 threads, one slot per thread (n_active <= 512).
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
  // exclusive scans over threads for each bucket
  int mine[kB + 1], before[kB + 1];
#pragma unroll
  for (int b = 0; b <= kB; ++b) {
    mine[b] = (b == kB ? full : 0) + (b == part_nb && b > 0 ? 1 : 0);
    int incl = mine[b];
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d);
      if (lane >= d) incl += v;
    }
    before[b] = incl - mine[b];
    if (lane == 63) wave_sum[wave][b] = incl;
  }
  __syncthreads();
  if (tid == 0) {
    int o = 0;
    for (int b = kB; b >= 1; --b) {  // largest first
      bucket_start[b] = o;
      for (int w = 0; w < 16; ++w) o += wave_sum[w][b];
    }
    bucket_start[0] = o;
    *n_tiles = o;
  }
  __syncthreads();
  const int slot = tid < na ? tid : -1;
#pragma unroll
  for (int b = 1; b <= kB; ++b) {
    if (!mine[b]) continue;
    int o = bucket_start[b] + before[b];
    for (int w = 0; w < wave; ++w) o += wave_sum[w][b];
    if (b == kB) {
      for (int i = 0; i < full; ++i) tiles[o + i] = make_int2(slot, i * BM);
      if (part_nb == kB) tiles[o + full] = make_int2(slot, full * BM);
    } else {
      tiles[o] = make_int2(slot, full * BM);
    }
  }
}

// ---------------------------------------------------------------------------
// Hidden rows to half: one block per token.  x' = x * 2^-ex with ex =
// floor(log2 max |x|) - 14 (0 for an all-zero row), rounded once to half and
// stored in the column order of the converted weights; xexp[t] = ex,
// xn2[t] = sum of x'^2 (float32, fixed order).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float block_reduce(float v, float *red, bool is_max) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const float o = __shfl_xor(v, d);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  v = red[0];
  for (int i = 1; i < 4; ++i) v = is_max ? fmaxf(v, red[i]) : v + red[i];
  return v;
}

__global__ __launch_bounds__(256) void prep_x_kernel(const float *__restrict__ x, int h, _Float16 *__restrict__ xb,
                                                     int32_t *__restrict__ xexp, float *__restrict__ xn2) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const float4 *row = reinterpret_cast<const float4 *>(x + (size_t)t * h);
  const int n8 = h >> 3;
  float mx = 0.0f;
  for (int i = threadIdx.x; i < n8; i += 256) {
    const float4 a = row[2 * i], b = row[2 * i + 1];
    mx = fmaxf(mx, fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))));
    mx = fmaxf(mx, fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
  }
  mx = block_reduce(mx, red, true);
  const int ex = mx > 0.0f ? ilog2f(mx) - 14 : 0;
  float ss = 0.0f;
  uint4 *out = reinterpret_cast<uint4 *>(xb + (size_t)t * h);
  for (int i = threadIdx.x; i < n8; i += 256) {
    const float4 a = row[2 * i], b = row[2 * i + 1];
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    _Float16 o[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float s = __builtin_amdgcn_ldexpf(v[c], -ex);
      ss = __builtin_fmaf(s, s, ss);
      o[(c & 3) * 2 + (c >> 2)] = (_Float16)s;
    }
    out[i] = __builtin_bit_cast(uint4, o);
  }
  ss = block_reduce(ss, red, false);
  if (threadIdx.x == 0) {
    xexp[t] = ex;
    xn2[t] = ss;
  }
}

// ---------------------------------------------------------------------------
// Per-expert statistics of the prescaling, one block per (matrix, expert):
// ew = 11 - floor(log2 max s) (0 for an all-zero table), and for gate and up
// the largest squared row norm of the scales times 2^ew.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void scale_stats_kernel(PrefillProblem P, int n_stats) {
  __shared__ float red[4];
  const int mat = blockIdx.x, e = blockIdx.y;  // mat 0 gate, 1 up, 2 down
  const bool sh = e == P.E;
  const ExpertTables &tab = mat == 0 ? (sh ? P.sh_gate : P.gate) : mat == 1 ? (sh ? P.sh_up : P.up)
                                                                            : (sh ? P.sh_down : P.down);
  const int rows = mat < 2 ? P.I : P.h, groups = (mat < 2 ? P.h : P.I) >> 6;
  const float *s = tab.s + (sh ? 0 : (size_t)e * rows * groups);
  const size_t n = (size_t)rows * groups;
  float mx = 0.0f;
  for (size_t i = threadIdx.x; i < n; i += 256) mx = fmaxf(mx, fabsf(s[i]));
  mx = block_reduce(mx, red, true);
  const int ew = mx > 0.0f ? 11 - ilog2f(mx) : 0;
  if (threadIdx.x == 0) P.stats[e].ew[mat] = ew;
  if (mat == 2) return;
  float best = 0.0f;
  for (int r = threadIdx.x; r < rows; r += 256) {
    float acc = 0.0f;
    for (int g = 0; g < groups; ++g) {
      const float v = __builtin_amdgcn_ldexpf(s[(size_t)r * groups + g], ew);
      acc = __builtin_fmaf(v, v, acc);
    }
    best = fmaxf(best, acc);
  }
  best = block_reduce(best, red, true);
  if (threadIdx.x == 0) P.stats[e].n2[mat] = best;
  (void)n_stats;
}

int grid_blocks(int nb, int max_tiles) { return kXcds * nb * ((max_tiles + kXcds - 1) / kXcds); }

}  // namespace

bool prefill_shape_ok(int h, int I) { return h % 256 == 0 && I % 256 == 0; }

int prefill_max_tiles(int T, int k, int E, int has_shared) {
  const int n = T * k, routed_slots = E < n ? E : n;
  return n / BM + routed_slots + (has_shared ? (T + BM - 1) / BM : 0);
}

hipError_t launch_prefill_prep(const float *x, int T, int h, PrefillProblem &P, hipStream_t s) {
  return launch(prep_x_kernel, T, 256, 0, s, x, h, const_cast<_Float16 *>(P.xb), P.xexp, P.xn2);
}

hipError_t launch_prefill_stats(const PrefillProblem &P, hipStream_t s) {
  const int n = P.E + (P.has_shared ? 1 : 0);
  return launch(scale_stats_kernel, dim3(3, n), 256, 0, s, P, n);
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
