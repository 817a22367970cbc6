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
  int n[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) n[i] = (int)__builtin_rintf(v[i] * to_int);
#pragma unroll
  for (int j = 0; j < kPlanes; ++j) {
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      word |= (uint32_t)(n[i] & 15) << (4 * i);
      n[i] = (n[i] + 8) >> 4;  // balanced digit: n = 16 n' + d, d = (n & 15) read as int4
    }
    if (store) planes_w[j * plane_stride] = word;
  }
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

}  // namespace coli
