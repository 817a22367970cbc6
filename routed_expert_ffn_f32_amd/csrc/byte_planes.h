// Byte planes of float32 activations for the int8 matrix-core kernels
// (expert_batch.hip describes the format): one thread per word of 8
// consecutive columns, the 8 threads of a 64-column group in consecutive
// lanes (an aligned octet).  Used by the standalone quantisation launch and
// by the router launch's plane blocks.
#pragma once

#include "internal.h"

namespace coli {

constexpr int kBtMant = 22;
constexpr int kBtMinExp = -100;  // groups with max |x| < 2^-101 quantise to zero

// Word w (columns 8w .. 8w + 7) of row p, values v (zeros for an invalid
// thread, which stores nothing but takes part in its octet's maximum).
__device__ __forceinline__ void byte_planes_word(const float (&v)[8], bool valid, size_t p, int w, int cols,
                                                 uint8_t *__restrict__ planes, float *__restrict__ scales) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  m = fmaxf(m, __shfl_xor(m, 1));
  m = fmaxf(m, __shfl_xor(m, 2));
  m = fmaxf(m, __shfl_xor(m, 4));
  int e = 0;
  (void)__builtin_frexpf(m, &e);  // m < 2^e
  e = m > 0.0f ? max(e, kBtMinExp) : kBtMinExp;
  const float to_int = __int_as_float((127 + kBtMant - e) << 23);  // 2^(22 - e)
  // y = x / s + 1.5 * 2^23 rounds x / s to the nearest integer N (ties to
  // even) and has the bit pattern 0x4B400000 + N; M = N + 0x808080 has the
  // bytes d_j + 128 (no carries, 0 <= M < 2^24)
  constexpr uint32_t kRound = 0x4B400000u;
  uint32_t M[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    M[i] = __float_as_uint(__builtin_fmaf(v[i], to_int, __uint_as_float(kRound))) - (kRound - 0x808080u);
  if (!valid) return;
  // group w / 8, chunk (w % 8) / 2, half w % 2 of the chunk
  uint8_t *dst = planes + p * 3 * (size_t)cols + 192 * (w >> 3) + 48 * ((w & 7) >> 1) + 8 * (w & 1);
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    // byte j of values (0, 2, 4, 6) and of (1, 3, 5, 7), top bits flipped
    const uint32_t sel = (uint32_t)j | ((uint32_t)(4 + j) << 8) | ((uint32_t)j << 16) | ((uint32_t)(4 + j) << 24);
    const uint32_t e01 = __builtin_amdgcn_perm(M[2], M[0], sel), e23 = __builtin_amdgcn_perm(M[6], M[4], sel);
    const uint32_t o01 = __builtin_amdgcn_perm(M[3], M[1], sel), o23 = __builtin_amdgcn_perm(M[7], M[5], sel);
    uint2 out;
    out.x = __builtin_amdgcn_perm(e23, e01, 0x05040100u) ^ 0x80808080u;
    out.y = __builtin_amdgcn_perm(o23, o01, 0x05040100u) ^ 0x80808080u;
    *reinterpret_cast<uint2 *>(dst + 16 * j) = out;
  }
  if ((w & 7) == 0) scales[p * (size_t)(cols >> 6) + (w >> 3)] = __int_as_float((127 - kBtMant - 4 + e) << 23);
}

}  // namespace coli
