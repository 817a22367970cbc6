// Wavefront helpers for gfx950 (wave64): DPP reductions and the 23-bit
// digit-plane activation format used by the expert GEMV kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace coli {

// DPP controls (GFX9 encoding).
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;   // row_ror:4
constexpr int kDppRowRor8 = 0x128;   // row_ror:8
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK,
                                                                0xF, false));
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}

// Raw buffer loads: the descriptor covers [base, base + bytes); lanes pass a
// 32-bit byte offset (VGPR) and the wave a uniform one (SGPR).  Reads past
// `bytes` return zero instead of faulting.
using Rsrc = __amdgpu_buffer_rsrc_t;
constexpr int kRawBufferDword3 = 0x00020000;  // gfx9-family raw buffer, 32-bit elements

__device__ __forceinline__ Rsrc make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRawBufferDword3);
}

__device__ __forceinline__ uint4 bload16(Rsrc r, uint32_t voff, uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ float bloadf(Rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0));
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Block barrier for LDS data only: this wave's LDS accesses are complete
// (lgkmcnt 0) and kept on their side of it by the memory clobber, but global
// loads still in flight (prefetched rows) are not waited for, as
// __syncthreads() would.  Global memory written before it is not published.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void block_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
#pragma clang diagnostic pop

// Sum of v over the 64 lanes, returned uniformly (fixed combining order, so
// the result is the same on every run).
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kDppQuadXor1>(v);
  v += dpp_f<kDppQuadXor2>(v);
  v += dpp_f<kDppRowRor4>(v);
  v += dpp_f<kDppRowRor8>(v);       // every lane: its row's sum
  v += dpp_f<kDppRowBcast15, 0xA>(v);  // rows 1, 3 add rows 0, 2
  v += dpp_f<kDppRowBcast31, 0xC>(v);  // rows 2, 3 add lane 31
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// One halving step of rows_sum: the first N values become N/2, lane l
// keeping value 2i + hi of each pair and adding the other one from the lane
// CTRL brings in, which differs from l in the bit that hi is taken from.
template <int CTRL, int N, int R>
__device__ __forceinline__ void rows_halve(float (&v)[R], bool hi) {
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const float keep = hi ? v[2 * i + 1] : v[2 * i];
    const float send = hi ? v[2 * i] : v[2 * i + 1];
    v[i] = keep + dpp_f<CTRL>(send);
  }
}

// Sums over the 64 lanes of R values at once (R a power of two, <= 16):
// lane l receives the sum of v[l % R].  Bits 0 .. log2(R) - 1 of the lane
// number each halve the values (a quad swap for bits 0 and 1, a rotation by
// 4 or 8 within the 16-lane row for bits 2 and 3: the lane rotated in
// differs in that bit and agrees in the lower ones), so that each lane is
// left with one partial sum, of value l % R; the other lane bits are summed
// plainly, across rows with the 16- and 32-lane swaps.  Fixed order: the
// same result on every run.  Leaves v clobbered.
template <int R>
__device__ __forceinline__ float rows_sum(float (&v)[R]) {
  static_assert(R == 1 || R == 2 || R == 4 || R == 8 || R == 16, "R: a power of two up to 16");
  const int lane = threadIdx.x & 63;
  if constexpr (R >= 2) rows_halve<kDppQuadXor1, R>(v, lane & 1);
  if constexpr (R >= 4) rows_halve<kDppQuadXor2, R / 2>(v, lane & 2);
  if constexpr (R >= 8) rows_halve<kDppRowRor4, R / 4>(v, lane & 4);
  if constexpr (R >= 16) rows_halve<kDppRowRor8, R / 8>(v, lane & 8);
  float s = v[0];
  if constexpr (R < 2) s += dpp_f<kDppQuadXor1>(s);
  if constexpr (R < 4) s += dpp_f<kDppQuadXor2>(s);
  if constexpr (R < 8) s += dpp_f<kDppRowRor4>(s);
  if constexpr (R < 16) s += dpp_f<kDppRowRor8>(s);
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Max of v over the lanes 4a..4a+3 of a quad, in every lane of the quad.
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, dpp_f<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f<kDppQuadXor2>(v));
  return v;
}

// ---------------------------------------------------------------------------
// Digit-plane activations.
//
// A row of `cols` float activations is stored per block of 32 columns (half a
// weight group) as a power-of-two scale s_b = 2^(E_b - 22), 2^E_b > max |x|
// over the block, and integers N_c = rint(x_c / s_b) with |N_c| <= 2^22 (a
// 23-bit signed mantissa shared by the block: block floating point).  N_c is
// written as six balanced base-16 digits d_j in [-8, 7], N_c = sum_j 16^j d_j,
// and digit j of columns 8w..8w+7 forms word w of plane j, column 8w+i in
// nibble i -- the nibble order of the int4 weights, so v_dot8_i32_i4 on a
// weight word and a plane word multiplies matching columns.  sum_c q_c x_c
// over a block is then s_b * sum_j 16^j dot8s_j, exact in int32
// (|sum| <= 8 * 2^22 * 32 = 2^30).
// Layout: planes [row][kPlanes][cols/8] uint32, scales [row][cols/32] float.
// ---------------------------------------------------------------------------
constexpr int kPlanes = 6;
constexpr int kMantBits = 22;
constexpr int kMinExp = -100;  // blocks with max |x| < 2^-101 quantise to zero

// One thread holds 8 consecutive columns (word w); the four lanes of a quad
// hold the 32 columns of one block, and every lane of the wave takes part
// (padding lanes pass zeros and store = false).  Writes the plane words and,
// from the block's first lane, the scale.
//
// The digits come without a loop over planes: M = N + 0x888888 has the
// base-16 digits d_j + 8 (each in [0, 15], so no carries and 0 <= M < 2^24),
// and the code of digit j is ((M >> 4j) & 15) ^ 8.  N itself is read from
// the float y = x / s_b + 1.5 * 2^23: for |x / s_b| <= 2^22, y rounds
// x / s_b to the nearest integer (ties to even, as rint) and its bit pattern
// is 0x4B400000 + N.  The 8 x 6 nibbles are then transposed into the six
// plane words with bit-field inserts and byte permutes.
__device__ __forceinline__ void quantize_word(const float v[8], bool first_of_block, bool store,
                                              uint32_t *planes_w, size_t plane_stride, float *scale_b) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  m = quad_max(m);
  int e = 0;
  (void)__builtin_frexpf(m, &e);  // m < 2^e (m = 0 gives e = 0)
  e = m > 0.0f ? max(e, kMinExp) : kMinExp;
  const float to_int = __int_as_float((127 + kMantBits - e) << 23);   // 2^(22 - e)
  const float to_real = __int_as_float((127 - kMantBits + e) << 23);  // 2^(e - 22)
  constexpr uint32_t kRound = 0x4B400000u;  // 1.5 * 2^23
  uint32_t M[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    M[i] = __float_as_uint(__builtin_fmaf(v[i], to_int, __uint_as_float(kRound))) - (kRound - 0x888888u);
  // pairs (2p, 2p+1): byte k of lo[p] holds nibble 2k of both values (value
  // 2p in the low half), byte k of hi[p] nibble 2k + 1
  uint32_t lo[4], hi[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    lo[p] = (M[2 * p] & 0x0F0F0F0Fu) | ((M[2 * p + 1] << 4) & 0xF0F0F0F0u);
    hi[p] = ((M[2 * p] >> 4) & 0x0F0F0F0Fu) | (M[2 * p + 1] & 0xF0F0F0F0u);
  }
  // plane 2k (lo) or 2k + 1 (hi): byte p of the word is byte k of pair p
  uint32_t w[kPlanes];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const uint32_t *q = half == 0 ? lo : hi;
    // bytes 0, 1 of pairs (0, 1) and (2, 3) interleaved; then bytes 2
    const uint32_t a01 = __builtin_amdgcn_perm(q[1], q[0], 0x05010400u);
    const uint32_t a23 = __builtin_amdgcn_perm(q[3], q[2], 0x05010400u);
    const uint32_t b01 = __builtin_amdgcn_perm(q[1], q[0], 0x0C0C0602u);
    const uint32_t b23 = __builtin_amdgcn_perm(q[3], q[2], 0x0C0C0602u);
    w[half] = __builtin_amdgcn_perm(a23, a01, 0x05040100u);
    w[half + 2] = __builtin_amdgcn_perm(a23, a01, 0x07060302u);
    w[half + 4] = __builtin_amdgcn_perm(b23, b01, 0x05040100u);
  }
#pragma unroll
  for (int j = 0; j < kPlanes; ++j)
    if (store) planes_w[j * plane_stride] = w[j] ^ 0x88888888u;
  if (store && first_of_block) *scale_b = to_real;
}

// sum over 32 columns of weight codes (4 words) times the digit-plane
// integers of the activations: sum_j 16^j sum_k dot8(w_k, p_j,k), Horner over
// the planes, exact in int32.
__device__ __forceinline__ int dot_planes(const uint4 &w, const uint4 (&p)[kPlanes]) {
  int h = 0;
#pragma unroll
  for (int j = kPlanes - 1; j >= 0; --j) {
    h = (int)((uint32_t)h << 4);
    h = __builtin_amdgcn_sdot8((int)w.x, (int)p[j].x, h, false);
    h = __builtin_amdgcn_sdot8((int)w.y, (int)p[j].y, h, false);
    h = __builtin_amdgcn_sdot8((int)w.z, (int)p[j].z, h, false);
    h = __builtin_amdgcn_sdot8((int)w.w, (int)p[j].w, h, false);
  }
  return h;
}

// ---------------------------------------------------------------------------
// Byte-plane activations (int8 weights).
//
// The same block floating point as above (N_c = rint(x_c / s_b), |N_c| <=
// 2^22, one scale per 32 columns), written as three balanced base-256 digits
// b_j in [-128, 127] (b_2 in [-64, 64]), N_c = b_0 + 256 b_1 + 65536 b_2.
// Byte i of word w of plane j is digit j of column 4w + i: the byte order of
// an int8 weight row, so v_dot4_i32_i8 on a weight word and a plane word
// multiplies matching columns.
// Layout: planes [row][kBytePlanes][cols/4] uint32, scales [row][cols/32].
// ---------------------------------------------------------------------------
constexpr int kBytePlanes = 3;

// As quantize_word (same thread and quad layout, same scale), for byte
// planes: the thread's 8 columns are words 0 and 1 of each plane at
// planes_w[j * plane_stride + 0/1].  M = N + 0x808080 has the base-256
// digits b_j + 128 (no carries, 0 <= M < 2^24); byte j of M with its top bit
// flipped is b_j as a two's-complement byte.
__device__ __forceinline__ void quantize_word8(const float v[8], bool first_of_block, bool store,
                                               uint32_t *planes_w, size_t plane_stride, float *scale_b) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  m = quad_max(m);
  int e = 0;
  (void)__builtin_frexpf(m, &e);
  e = m > 0.0f ? max(e, kMinExp) : kMinExp;
  const float to_int = __int_as_float((127 + kMantBits - e) << 23);
  const float to_real = __int_as_float((127 - kMantBits + e) << 23);
  constexpr uint32_t kRound = 0x4B400000u;
  uint32_t M[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    M[i] = __float_as_uint(__builtin_fmaf(v[i], to_int, __uint_as_float(kRound))) - (kRound - 0x808080u);
#pragma unroll
  for (int j = 0; j < kBytePlanes; ++j) {
    // byte j of each value: pairs first, then the two pairs of a word
    const uint32_t sel = (uint32_t)j | ((uint32_t)(4 + j) << 8) | ((uint32_t)j << 16) | ((uint32_t)(4 + j) << 24);
    const uint32_t a = __builtin_amdgcn_perm(M[1], M[0], sel), b = __builtin_amdgcn_perm(M[3], M[2], sel);
    const uint32_t c = __builtin_amdgcn_perm(M[5], M[4], sel), d = __builtin_amdgcn_perm(M[7], M[6], sel);
    const uint32_t w0 = __builtin_amdgcn_perm(b, a, 0x05040100u), w1 = __builtin_amdgcn_perm(d, c, 0x05040100u);
    if (store) {
      planes_w[j * plane_stride] = w0 ^ 0x80808080u;
      planes_w[j * plane_stride + 1] = w1 ^ 0x80808080u;
    }
  }
  if (store && first_of_block) *scale_b = to_real;
}

// sum over 16 columns of int8 weights (4 words) times the byte-plane
// integers: d_j = sum_k dot4(w_k, p_j,k) is exact (|d_j| <= 16 * 128 * 128
// = 2^18), d_0 + 256 d_1 too (< 2^27); the top plane joins in float32.
__device__ __forceinline__ float dot_bytes(const uint4 &w, const uint4 (&p)[kBytePlanes]) {
  int d[kBytePlanes];
#pragma unroll
  for (int j = 0; j < kBytePlanes; ++j) {
    int a = __builtin_amdgcn_sdot4((int)w.x, (int)p[j].x, 0, false);
    a = __builtin_amdgcn_sdot4((int)w.y, (int)p[j].y, a, false);
    a = __builtin_amdgcn_sdot4((int)w.z, (int)p[j].z, a, false);
    d[j] = __builtin_amdgcn_sdot4((int)w.w, (int)p[j].w, a, false);
  }
  return __builtin_fmaf((float)d[2], 65536.0f, (float)(d[0] + (d[1] << 8)));
}

// ---------------------------------------------------------------------------
// Weight formats of the GEMV kernels.  A lane chunk is 16 bytes of a weight
// row (a wave-load covers 1 KB of the row).
//  - int4 gs64: 32 columns per chunk, a float32 scale per 64 columns;
//    activations as six 4-bit digit planes (dot_planes).
//  - int8 with one float32 scale per row: 16 columns per chunk; activations
//    as three byte planes (dot_bytes); the row scale is applied once per row
//    (and, in the down launch, per slot before the weighted sum).
// Both keep 3 bytes of planes per activation column and one activation scale
// per 32 columns, so plane buffers have the same size in either format.
// ---------------------------------------------------------------------------
struct FmtI4 {
  static constexpr int kChunkCols = 32;
  static constexpr int kXPlanes = kPlanes;
  static constexpr bool kRowScale = false;
  __device__ static uint32_t row_bytes(int cols) { return (uint32_t)cols >> 1; }
  __device__ static uint32_t row_scales(int cols) { return (uint32_t)cols >> 6; }
  __device__ static float dot(const uint4 &w, const uint4 (&p)[kXPlanes]) { return (float)dot_planes(w, p); }
  // the thread's 8-column word w of a row: its plane words
  __device__ static void quantize(const float v[8], bool first, bool store, uint32_t *row_planes, int cols, int w,
                                  float *scale_b) {
    quantize_word(v, first, store, row_planes + w, (size_t)(cols >> 3), scale_b);
  }
};

struct FmtI8 {
  static constexpr int kChunkCols = 16;
  static constexpr int kXPlanes = kBytePlanes;
  static constexpr bool kRowScale = true;
  __device__ static uint32_t row_bytes(int cols) { return (uint32_t)cols; }
  __device__ static uint32_t row_scales(int) { return 1u; }
  __device__ static float dot(const uint4 &w, const uint4 (&p)[kXPlanes]) { return dot_bytes(w, p); }
  __device__ static void quantize(const float v[8], bool first, bool store, uint32_t *row_planes, int cols, int w,
                                  float *scale_b) {
    quantize_word8(v, first, store, row_planes + 2 * w, (size_t)(cols >> 2), scale_b);
  }
};

}  // namespace coli
