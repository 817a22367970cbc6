/*
 * Seeded synthetic inputs for the routed-MoE layer (test and benchmark
 * infrastructure shared by the oracle side and the GPU side).
 *
 * This file holds none of the layer's arithmetic: it only draws numbers and
 * writes them in the layer's storage format.
 *
 *  - Random bits: SplitMix64 (Steele, Lea & Flood, "Fast splittable
 *    pseudorandom number generators", OOPSLA 2014).  Stream (seed, tag) starts
 *    from state mix(seed * golden + mix(tag)); element j of the stream is the
 *    SplitMix64 output for counter j + 1, so any element can be regenerated on
 *    its own (counter-based).
 *  - Normals: Box-Muller (Box & Muller, 1958).  Pair p of a stream uses the
 *    outputs 2p and 2p+1 as two 24-bit uniforms u1 in (0,1] and u2 in [0,1);
 *    element 2p gets r*cos(2*pi*u2), element 2p+1 gets r*sin(2*pi*u2),
 *    r = sqrt(-2 ln u1).  log, sin and cos are the float32 polynomials below
 *    (so the loop vectorises and the values do not depend on the host libm).
 *  - Storage format of int4 "gs64" weights: for a row of `cols` weights,
 *    byte c/2 holds weight c in its low nibble when c is even and in its high
 *    nibble when c is odd, as a 4-bit two's-complement code in [-8, 7]; float
 *    scale [c/64] belongs to the 64 weights c in [64g, 64g+64).
 *  - Quantiser used to produce those codes from N(0, sigma) draws: per group
 *    of 64, s = absmax/7 (float division), q = clamp(rint(w/s), -8, 7); an
 *    all-zero group gets s = 0 and q = 0.
 *
 * Built with -ffp-contract=off so no multiply-add is fused behind our back.
 */
#include <math.h>
#include <stdlib.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ULL;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_stream_key(uint64_t seed, uint64_t tag) {
  return mix64(seed * GOLDEN + mix64(tag + GOLDEN));
}

/* j-th raw 64-bit output of stream `key` (j = 0, 1, ...) */
static inline uint64_t stream_bits(uint64_t key, uint64_t j) {
  return mix64(key + (j + 1) * GOLDEN);
}

uint64_t synth_bits(uint64_t seed, uint64_t tag, uint64_t j) {
  return stream_bits(synth_stream_key(seed, tag), j);
}

/* ln(u) for u in (0, 1], float32: u = m * 2^e with m in [sqrt(1/2), sqrt(2)),
 * ln m = 2 atanh(t), t = (m - 1)/(m + 1), |t| < 0.1716, odd series to t^11.
 * Branch-free so that the calling loop vectorises. */
static inline float poly_logf(float u) {
  uint32_t b;
  memcpy(&b, &u, 4);
  uint32_t mb = (b & 0x007FFFFFu) | 0x3F800000u; /* m in [1, 2) */
  int32_t big = mb > 0x3FB504F3u;                /* m > sqrt(2) */
  int32_t e = (int32_t)(b >> 23) - 127 + big;
  mb -= (uint32_t)big << 23; /* m / 2 when big */
  float m;
  memcpy(&m, &mb, 4);
  float t = (m - 1.0f) / (m + 1.0f);
  float t2 = t * t;
  float s = 1.0f / 11.0f;
  s = s * t2 + 1.0f / 9.0f;
  s = s * t2 + 1.0f / 7.0f;
  s = s * t2 + 1.0f / 5.0f;
  s = s * t2 + 1.0f / 3.0f;
  s = s * t2 + 1.0f;
  return (float)e * 0.693147182f + 2.0f * t * s;
}

/* sin and cos of 2*pi*v for v in [0, 1): nearest quarter turn q from 4v,
 * Taylor series on the remainder a in [-pi/4, pi/4], then rotation by q
 * quarter turns done with sign-bit and select arithmetic (branch-free). */
static inline void poly_sincos2pi(float v, float *sn, float *cs) {
  float w = v * 4.0f;
  int32_t qi = (int32_t)(w + 0.5f); /* w >= 0: truncation is floor */
  float a = (w - (float)qi) * 1.57079637f;
  float a2 = a * a;
  float ps = -1.0f / 39916800.0f;
  ps = ps * a2 + 1.0f / 362880.0f;
  ps = ps * a2 - 1.0f / 5040.0f;
  ps = ps * a2 + 1.0f / 120.0f;
  ps = ps * a2 - 1.0f / 6.0f;
  ps = ps * a2 + 1.0f;
  float s0 = a * ps;
  float pc = 1.0f / 479001600.0f;
  pc = pc * a2 - 1.0f / 3628800.0f;
  pc = pc * a2 + 1.0f / 40320.0f;
  pc = pc * a2 - 1.0f / 720.0f;
  pc = pc * a2 + 1.0f / 24.0f;
  pc = pc * a2 - 0.5f;
  pc = pc * a2 + 1.0f;
  /* q=0: ( s, c)  q=1: ( c,-s)  q=2: (-s,-c)  q=3: (-c, s)   as (sin, cos) */
  uint32_t swap = (uint32_t)(qi & 1) * 0xFFFFFFFFu;
  uint32_t bs, bc;
  memcpy(&bs, &s0, 4);
  memcpy(&bc, &pc, 4);
  uint32_t rs = (bs & ~swap) | (bc & swap);
  uint32_t rc = (bc & ~swap) | (bs & swap);
  rs ^= (uint32_t)(qi & 2) << 30;         /* q = 2, 3 negate sin */
  rc ^= (uint32_t)((qi + 1) & 2) << 30;   /* q = 1, 2 negate cos */
  memcpy(sn, &rs, 4);
  memcpy(cs, &rc, 4);
}

/* Normals for pairs [p0, p0 + np) of stream `key` (np <= PAIR_BLOCK):
 * z[2i] = r cos(2 pi u2), z[2i+1] = r sin(2 pi u2) for pair p0 + i.  The
 * integer part fills two arrays, the float part is a straight loop the
 * compiler can vectorise. */
#define PAIR_BLOCK 256
__attribute__((target_clones("avx2", "default")))
static void normal_pairs(uint64_t key, uint64_t p0, int np, float *z) {
  float u1[PAIR_BLOCK], u2[PAIR_BLOCK];
  for (int i = 0; i < np; i++) {
    uint64_t b1 = stream_bits(key, 2 * (p0 + i));
    uint64_t b2 = stream_bits(key, 2 * (p0 + i) + 1);
    u1[i] = (float)(int32_t)((b1 >> 40) + 1) * 0x1.0p-24f; /* (0, 1] */
    u2[i] = (float)(int32_t)(b2 >> 40) * 0x1.0p-24f;       /* [0, 1) */
  }
  for (int i = 0; i < np; i++) {
    float r = sqrtf(-2.0f * poly_logf(u1[i]));
    float sn, cs;
    poly_sincos2pi(u2[i], &sn, &cs);
    z[2 * i] = r * cs;
    z[2 * i + 1] = r * sn;
  }
}

/* Elements [first, last) of stream `key` scaled by sigma, written to out. */
static void normal_range(uint64_t key, uint64_t first, uint64_t last, float sigma, float *out) {
  float z[2 * PAIR_BLOCK];
  uint64_t pend = (last + 1) >> 1;
  for (uint64_t p = first >> 1; p < pend; p += PAIR_BLOCK) {
    int np = (int)(pend - p < PAIR_BLOCK ? pend - p : PAIR_BLOCK);
    normal_pairs(key, p, np, z);
    uint64_t e0 = 2 * p;
    for (int i = 0; i < 2 * np; i++) {
      uint64_t e = e0 + i;
      if (e >= first && e < last) out[e - first] = sigma * z[i];
    }
  }
}

/* out[i] = sigma * N_{start+i} of stream (seed, tag), i in [0, n). */
void synth_normal_f32(uint64_t seed, uint64_t tag, uint64_t start, size_t n, float sigma,
                      float *out) {
  uint64_t key = synth_stream_key(seed, tag);
  const uint64_t CH = 1u << 16; /* elements per parallel chunk (even) */
  int64_t nch = (int64_t)((n + CH - 1) / CH);
#pragma omp parallel for schedule(static) if (nch > 1)
  for (int64_t ci = 0; ci < nch; ci++) {
    uint64_t a = start + (uint64_t)ci * CH, b = a + CH;
    if (b > start + n) b = start + n;
    normal_range(key, a, b, sigma, out + (a - start));
  }
}

/* Uniform floats in [0, 1) with 24 random bits: out[i] = element start+i. */
void synth_uniform_f32(uint64_t seed, uint64_t tag, uint64_t start, size_t n, float *out) {
  uint64_t key = synth_stream_key(seed, tag);
  for (size_t i = 0; i < n; i++) out[i] = (float)(stream_bits(key, start + i) >> 40) * 0x1.0p-24f;
}

/* Quantise one row of `cols` float weights into codes (cols/2 bytes) and
 * scales (cols/64 floats) with the rule stated at the top of this file. */
__attribute__((target_clones("avx2", "default")))
static void quant_row(const float *w, int cols, uint8_t *codes, float *scales) {
  for (int g = 0; g < cols / 64; g++) {
    const float *wg = w + 64 * g;
    float amax = 0.0f;
    for (int c = 0; c < 64; c++) {
      float a = fabsf(wg[c]);
      amax = a > amax ? a : amax;
    }
    float s = amax / 7.0f;
    scales[g] = s;
    int32_t q[64];
    if (s > 0.0f) {
      for (int c = 0; c < 64; c++) {
        float r = rintf(wg[c] / s);
        r = r < -8.0f ? -8.0f : r;
        r = r > 7.0f ? 7.0f : r;
        q[c] = (int32_t)r;
      }
    } else {
      for (int c = 0; c < 64; c++) q[c] = 0;
    }
    uint8_t *cg = codes + 32 * g;
    for (int c = 0; c < 32; c++) cg[c] = (uint8_t)((q[2 * c] & 0xF) | ((q[2 * c + 1] & 0xF) << 4));
  }
}

/* Row-major [rows, cols] weight matrix w[r][c] = sigma * N_{r*cols + c} of
 * stream (seed, tag), quantised to codes [rows][cols/2] and scales
 * [rows][cols/64].  cols must be a multiple of 64.  Returns 0 or -1. */
int synth_quant_matrix(uint64_t seed, uint64_t tag, int rows, int cols, float sigma,
                       uint8_t *codes, float *scales) {
  if (rows < 0 || cols <= 0 || cols % 64) return -1;
  uint64_t key = synth_stream_key(seed, tag);
#pragma omp parallel
  {
    float wbuf[16384];
    int chunk = cols <= 16384 ? cols : 16384; /* a multiple of 64 */
#pragma omp for schedule(static)
    for (int r = 0; r < rows; r++) {
      for (int c0 = 0; c0 < cols; c0 += chunk) {
        int n = cols - c0 < chunk ? cols - c0 : chunk;
        uint64_t first = (uint64_t)r * cols + c0;
        normal_range(key, first, first + n, sigma, wbuf);
        quant_row(wbuf, n, codes + ((size_t)r * cols + c0) / 2, scales + ((size_t)r * cols + c0) / 64);
      }
    }
  }
  return 0;
}

/* int8 storage with one scale per row: s = absmax(row) / 127,
 * q = clamp(rne(w / s), -127, 127) as a two's-complement byte (an all-zero
 * row gives s = 0, q = 0; -128 never occurs here but is legal input). */
__attribute__((target_clones("avx2", "default")))
static void quant_row_i8(const float *w, int cols, uint8_t *codes, float *scale) {
  float amax = 0.0f;
  for (int c = 0; c < cols; c++) {
    float a = fabsf(w[c]);
    amax = a > amax ? a : amax;
  }
  float s = amax / 127.0f;
  *scale = s;
  for (int c = 0; c < cols; c++) {
    int32_t q = 0;
    if (s > 0.0f) {
      float r = rintf(w[c] / s);
      r = r < -127.0f ? -127.0f : r;
      r = r > 127.0f ? 127.0f : r;
      q = (int32_t)r;
    }
    codes[c] = (uint8_t)(q & 0xFF);
  }
}

/* As synth_quant_matrix, int8 with a scale per row: codes [rows][cols],
 * scales [rows].  cols must be a positive multiple of 64.  Returns 0 or -1. */
int synth_quant_matrix_i8(uint64_t seed, uint64_t tag, int rows, int cols, float sigma,
                          uint8_t *codes, float *scales) {
  if (rows < 0 || cols <= 0 || cols % 64 || cols > 65536) return -1;
  uint64_t key = synth_stream_key(seed, tag);
#pragma omp parallel
  {
    float *wbuf = (float *)malloc(sizeof(float) * (size_t)cols);
#pragma omp for schedule(static)
    for (int r = 0; r < rows; r++) {
      uint64_t first = (uint64_t)r * cols;
      normal_range(key, first, first + cols, sigma, wbuf);
      quant_row_i8(wbuf, cols, codes + (size_t)r * cols, scales + r);
    }
    free(wbuf);
  }
  return 0;
}

/* Caller-given float weights [rows, cols], int8 per row (crafted inputs). */
int synth_quantize_rows_i8(const float *w, int rows, int cols, uint8_t *codes, float *scales) {
  if (rows < 0 || cols <= 0) return -1;
  for (int r = 0; r < rows; r++) quant_row_i8(w + (size_t)r * cols, cols, codes + (size_t)r * cols, scales + r);
  return 0;
}

/* Fisher-Yates shuffle of 0..n-1 driven by stream (seed, tag): step i (from
 * n-1 down to 1) swaps perm[i] with perm[j], j = bits_i mod (i+1). */
void synth_permutation(uint64_t seed, uint64_t tag, int n, int32_t *perm) {
  uint64_t key = synth_stream_key(seed, tag);
  for (int i = 0; i < n; i++) perm[i] = i;
  for (int i = n - 1; i > 0; i--) {
    uint64_t j = stream_bits(key, (uint64_t)(n - 1 - i)) % (uint64_t)(i + 1);
    int32_t t = perm[i];
    perm[i] = perm[j];
    perm[j] = t;
  }
}

/* Quantise caller-given float weights [rows, cols] (cols a multiple of 64)
 * with the same rule as synth_quant_matrix (for crafted test inputs). */
int synth_quantize_rows(const float *w, int rows, int cols, uint8_t *codes, float *scales) {
  if (rows < 0 || cols <= 0 || cols % 64) return -1;
  for (int r = 0; r < rows; r++)
    quant_row(w + (size_t)r * cols, cols, codes + (size_t)r * cols / 2, scales + (size_t)r * cols / 64);
  return 0;
}
