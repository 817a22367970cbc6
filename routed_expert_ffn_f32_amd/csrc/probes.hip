// Measurement probes: the HBM read rate and the MFMA rates this GPU
// reaches, measured in the same run as the layer so that its figures can be
// set against them as well as against the published peaks.  Neither is part
// of the layer; both leave a checkable result, so that the work cannot have
// been skipped.
#include "internal.h"
#include "wave.h"

namespace coli {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kStreamUnroll = 4;  // 16-byte loads in flight per lane

// XOR of every 32-bit word of buf [n16 x 16 bytes], each word read exactly
// once: lane-strided 16-byte loads, kStreamUnroll in flight, one atomic XOR
// per wave into *sink (the order of XORs does not change the result).
__global__ __launch_bounds__(256) void stream_probe_kernel(const uint4 *__restrict__ buf, size_t n16,
                                                           uint32_t *__restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t x = 0;
  for (; i + (kStreamUnroll - 1) * stride < n16; i += kStreamUnroll * stride) {
    uint4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = buf[i + u * stride];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = buf[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // xor over the wave, then one atomic per wave
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x ^= (uint32_t)__shfl_xor((int)x, d);
  if ((threadIdx.x & 63) == 0) atomicXor(sink, x);
}

// Back-to-back v_mfma_f32_32x32x16_bf16: each wave runs `iters` rounds of
// 8 MFMAs on independent accumulators (enough to keep the pipe busy:
// eight chains of 32-cycle MFMAs), operands all ones: each MFMA adds
// 16 to every element, so every accumulator ends at exactly 16 * iters when
// iters < 2^20 (integers below 2^24 are exact in float32).  A wave whose
// accumulators all hold that value adds 1 to *sink.
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, uint32_t *__restrict__ sink) {
  bf16x8 a;
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = (__bf16)1.0f;
  f32x16 acc[kMfmaChains];
#pragma unroll
  for (int m = 0; m < kMfmaChains; ++m) acc[m] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < kMfmaChains; ++m) acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc[m], 0, 0, 0);
  }
  const float want = 16.0f * (float)iters;
  bool ok = true;
#pragma unroll
  for (int m = 0; m < kMfmaChains; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) ok = ok && acc[m][r] == want;
  const bool all = __ballot(!ok) == 0;
  if ((threadIdx.x & 63) == 0 && all) atomicAdd(sink, 1u);
}

// Back-to-back v_mfma_f32_32x32x16_f16 on varied operands: the matrix pipe
// draws more power when its inputs change from one instruction to the next,
// and the clock drops to hold the power limit, so the rate on ones above is
// an upper bound that real data does not reach.  Each wave holds four A and
// four B operand registers filled with pseudo-random halves (random sign and
// mantissa, exponent in [-4, 10]) and cycles four accumulators through all
// sixteen (A, B) pairs, so consecutive MFMAs never see the same operands.
// The result cannot be predicted exactly; a wave whose accumulators are all
// finite adds 1 to *sink, which keeps the work observable.
__device__ __forceinline__ uint32_t probe_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__global__ __launch_bounds__(256) void mfma_probe_f16_kernel(int iters, uint32_t seed, uint32_t *__restrict__ sink) {
  const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
  f16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t ra = probe_hash(seed ^ (gid * 64u + i * 8u + j));
      const uint32_t rb = probe_hash(~seed ^ (gid * 64u + i * 8u + j));
      // biased exponent 11..25 -> 2^-4 .. 2^10
      const uint16_t ha = (uint16_t)((ra & 0x8000u) | ((11u + (ra >> 16) % 15u) << 10) | (ra & 0x3ffu));
      const uint16_t hb = (uint16_t)((rb & 0x8000u) | ((11u + (rb >> 16) % 15u) << 10) | (rb & 0x3ffu));
      a[i][j] = __builtin_bit_cast(_Float16, ha);
      b[i][j] = __builtin_bit_cast(_Float16, hb);
    }
  f32x16 acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) acc[m] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[(i + m) & 3], acc[m], 0, 0, 0);
  }
  bool ok = true;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) ok = ok && __builtin_isfinite(acc[m][r]);
  const bool all = __ballot(!ok) == 0;
  if ((threadIdx.x & 63) == 0 && all) atomicAdd(sink, 1u);
}

}  // namespace

hipError_t launch_stream_probe(const void *buf, size_t bytes, uint32_t *sink, hipStream_t s) {
  return launch(stream_probe_kernel, dim3(kProbeStreamBlocks), dim3(256), 0, s, static_cast<const uint4 *>(buf),
                bytes / 16, sink);
}

hipError_t launch_mfma_probe(int iters, int blocks, uint32_t *sink, hipStream_t s) {
  return launch(mfma_probe_kernel, dim3(blocks), dim3(256), 0, s, iters, sink);
}

hipError_t launch_mfma_probe_f16(int iters, int blocks, uint32_t seed, uint32_t *sink, hipStream_t s) {
  return launch(mfma_probe_f16_kernel, dim3(blocks), dim3(256), 0, s, iters, seed, sink);
}

}  // namespace coli
