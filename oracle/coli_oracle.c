/*
 * CPU ORACLE for the routed Mixture-of-Experts layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg load this file's library.  It shares no code,
 * header, table or constant with the GPU library; the only thing the two
 * sides have in common is the seeded input generator (synth/), which holds
 * none of the layer's arithmetic.
 *
 * Sources (web pages about the Colibri / colibri MoE inference engine):
 *  [T]  "colibri engine teardown: running a 744B MoE model on 25 GB of RAM in
 *       pure C" (text-matrix.pages.dev):
 *         "System map" section -- 256 routed experts per MoE layer, top-8 per
 *         token, a resident shared expert;
 *         "Three key engineering decisions", item 1 -- the engine header
 *         states a sigmoid router with noaux_tc top-k, n_group = 1, and a
 *         routed_scaling_factor; norm, router and bias stay float32 because
 *         they are small and sensitive; experts use the int4 "gs64"
 *         container in which 64 weights share one scale;
 *         "Task flow example" -- per token and layer: shared expert, float32
 *         router scores, top-8, then the routed-expert matmuls.
 *  [C]  cf-1.com article on Colibri, section 2.1 -- the MoE forward: router
 *       gives expert ids and weights per token, tokens are grouped by expert,
 *       each group runs its expert FFN (three matrices W1, W2, W3), outputs
 *       are summed with the routing weights; section 2.2 -- worked grouping
 *       example; section 3.3 -- colibri_forward step 3 (per-expert counts,
 *       prefix sum into expert offsets, scatter by expert id) and step 5
 *       (weighted assembly per token).
 *  [P]  trdm.cn article "Colibri: a pure-C lightweight inference engine built
 *       for MoE models", section 2.2 -- routing yields a [batch, top_k]
 *       integer index array; section 3.1 -- router stored as a
 *       [hidden_size, num_experts] float32 matrix.
 *  [N]  "Colibrì：蜂鸟驮巨兽——纯C语言打造的7440亿参数MoE本地推理引擎", the
 *       kernels paragraph (hand-written int8, packed int4 and packed int2
 *       kernels with per-row scaling) and the MTP paragraph (the MTP head
 *       must be int8).
 *  [K]  "Colibri 调优与运行时旋钮实战指南" (Colibri tuning and runtime knobs
 *       guide), the knob table (explicit
 *       smaller k and adaptive expert top-p, lossy overrides of the
 *       routing).
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes of the repository):
 *  - the input hidden state is already normed, the output is the MoE output
 *    only (no residual);
 *  - the selection bias only selects; weights use the unbiased sigmoid;
 *  - n_group = 1 makes the group-limited stage the identity;
 *  - top-k order: key c = s + b descending, ties by expert index ascending;
 *    slot j of a token is its j-th selected expert;
 *  - renormalisation: den = sum of the selected s in slot order (float32),
 *    w_j = (s_j / den) * routed_scaling_factor;
 *  - SwiGLU: y = down( silu(gate x) * (up x) ), silu(z) = z / (1 + e^-z),
 *    W1 = gate, W3 = up, W2 = down;
 *  - the shared expert is added with weight 1 (not scaled, not gated);
 *  - int4 storage: byte c/2 of a row holds weight c in its low nibble for
 *    even c and in its high nibble for odd c, a 4-bit two's-complement code;
 *    scale [c/64] is a float32 for the 64 consecutive weights of the group
 *    along the input (reduction) axis; weight = code * scale;
 *  - int8 storage (the multi-token prediction head's format, [T], [N]):
 *    byte c of a row is weight c as an 8-bit two's-complement code, one
 *    float32 scale per (output) row; weight = code * scale[row].
 *
 * Precision: routing is an exact float32 program (the pages keep the router
 * in float32), so that a GPU can reproduce it bit for bit; the expert FFN and
 * the combine are evaluated in float64 and rounded once to float32.
 *
 * Build: gcc -O2 -ffp-contract=off (no fused multiply-add except the explicit
 * fmaf calls, no fast-math), OpenMP for independent tokens/assignments only
 * (every output element is summed by one thread in a fixed order, so results
 * do not depend on the thread count).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL -4
#define ORACLE_EROUTE -2

/* ---------------------------------------------------------------------- */
/* exp and sigmoid in float32, as an exact program.                        */
/* ---------------------------------------------------------------------- */

/* 2^n as a float for n in [-126, 127] (exponent-field construction). */
static float pow2i(int n) {
  uint32_t b = (uint32_t)(n + 127) << 23;
  float f;
  memcpy(&f, &b, 4);
  return f;
}

/*
 * exp_spec(y): e^y in float32.
 * Cody & Waite (1980) reduction y = n ln2 + r with n = rint(y * log2 e)
 * (float product, round to nearest even), r = (y - n*LN2_HI) - n*LN2_LO with
 * two fmaf steps; LN2_HI is ln 2 rounded to 16 significant bits so n*LN2_HI
 * is exact, LN2_LO is the float nearest to ln 2 - LN2_HI.  e^r is the
 * degree-7 Taylor polynomial sum r^i / i! in Horner form with fmaf (|r| <=
 * ln2/2, truncation below 0.05 ulp).  The result p * 2^n is formed by
 * exponent construction, in two steps where 2^n leaves the normal range.
 */
float coli_oracle_exp_spec(float y) {
  const float LOG2E = 0x1.715476p+0f;
  const float LN2_HI = 0x1.62e4p-1f;
  const float LN2_LO = 0x1.7f7d1cp-20f;
  const float C2 = 0x1p-1f;          /* 1/2! */
  const float C3 = 0x1.555556p-3f;   /* 1/3! */
  const float C4 = 0x1.555556p-5f;   /* 1/4! */
  const float C5 = 0x1.111112p-7f;   /* 1/5! */
  const float C6 = 0x1.6c16c2p-10f;  /* 1/6! */
  const float C7 = 0x1.a01a02p-13f;  /* 1/7! */
  if (y != y) return y;
  if (y > 89.0f) return INFINITY;
  if (y < -104.0f) return 0.0f;
  float n = rintf(y * LOG2E);
  float r = fmaf(-n, LN2_HI, y);
  r = fmaf(-n, LN2_LO, r);
  float p = C7;
  p = fmaf(p, r, C6);
  p = fmaf(p, r, C5);
  p = fmaf(p, r, C4);
  p = fmaf(p, r, C3);
  p = fmaf(p, r, C2);
  p = fmaf(p, r, 1.0f);
  p = fmaf(p, r, 1.0f);
  int ni = (int)n;
  if (ni > 127) return (p * pow2i(127)) * pow2i(ni - 127);
  if (ni < -126) return (p * pow2i(ni + 64)) * pow2i(-64);
  return p * pow2i(ni);
}

/* sigmoid_spec(z) = 1 / (1 + exp_spec(-z)), float32, IEEE division. */
float coli_oracle_sigmoid_spec(float z) {
  float e = coli_oracle_exp_spec(-z);
  return 1.0f / (1.0f + e);
}

/* ---------------------------------------------------------------------- */
/* Router logits: l[t][e] = sum_i x[t][i] * Wr[i][e], float32, fixed order. */
/* ---------------------------------------------------------------------- */

/*
 * Summation order (the float32 router of [T], made exact): 64 partial sums
 * p[0..63]; for m = 0 .. h/64 - 1 in order, p[l] = fmaf(x[l+64m], Wr[l+64m][e],
 * p[l]); then the 64 partials are combined by the xor butterfly: for
 * d = 32, 16, 8, 4, 2, 1, every p[l] becomes p[l] + p[l ^ d] (all l at
 * once); the logit is p[0].  Requires h % 64 == 0.
 */
__attribute__((target_clones("fma", "default")))
static void logits_token(const float *x, const float *wr, int32_t h, int32_t E, float *out) {
  for (int32_t e = 0; e < E; e++) {
    float p[64], q[64];
    for (int l = 0; l < 64; l++) p[l] = 0.0f;
    for (int32_t m = 0; m < h / 64; m++)
      for (int l = 0; l < 64; l++) {
        int32_t i = l + 64 * m;
        p[l] = fmaf(x[i], wr[(size_t)i * E + e], p[l]);
      }
    for (int d = 32; d >= 1; d >>= 1) {
      for (int l = 0; l < 64; l++) q[l] = p[l] + p[l ^ d];
      memcpy(p, q, sizeof p);
    }
    out[e] = p[0];
  }
}

int coli_oracle_router_logits(const float *x, const float *wr, int32_t T, int32_t h, int32_t E,
                              float *logits) {
  if (T < 0 || h <= 0 || h % 64 || E <= 0 || !x || !wr || !logits) return ORACLE_EINVAL;
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t t = 0; t < T; t++) logits_token(x + (size_t)t * h, wr, h, E, logits + (size_t)t * E);
  return ORACLE_OK;
}

/* ---------------------------------------------------------------------- */
/* Selection: sigmoid scores, biased key, top-k, renormalised weights.      */
/* ---------------------------------------------------------------------- */

typedef struct {
  float c;
  int32_t e;
} sel_key_t;

/* c descending, then expert index ascending (a strict total order). */
static int key_cmp(const void *a, const void *b) {
  const sel_key_t *x = (const sel_key_t *)a, *y = (const sel_key_t *)b;
  if (x->c > y->c) return -1;
  if (x->c < y->c) return 1;
  return (x->e > y->e) - (x->e < y->e);
}

/*
 * For every token: s[e] = sigmoid_spec(l[e]); c[e] = s[e] + b[e] (float32);
 * n_group = 1 keeps the single group, so the group stage changes nothing;
 * the k experts first in the order (c desc, e asc) fill slots 0..k-1;
 * den = ((s_0 + s_1) + s_2) + ... in slot order; w_j = (s_j / den) * rsf.
 * Source: [T] "Three key engineering decisions" item 1 (sigmoid, noaux_tc,
 * n_group = 1, routed_scaling_factor); [P] section 2.2 ([batch, top_k]
 * index array).
 *
 * Run-time routing limits: two lossy overrides of the routing, an explicit
 * smaller k and adaptive expert top-p, named as engine knobs in the knob
 * table of [K] (top-p cuts the
 * expert bytes streamed; both are warned about as lossy).  The page names
 * the knobs and their effect only; the readings here:
 *  - k_use < k: the k_use experts first in the order above are the
 *    candidates, in slots 0..k_use-1; den sums their scores; slots
 *    k_use..k-1 are dropped;
 *  - top-p, 0 < p < 1: in slot order, cum_j = ((s_0 + s_1) + ...) + s_(j-1)
 *    is the score of the candidates before slot j (float32, cum_0 = 0);
 *    slot 0 is always kept and slot j >= 1 is kept while cum_j < p * den
 *    (one float32 product), so the kept slots are the shortest prefix whose
 *    score reaches the share p of the candidates' score.  p = 1: no top-p;
 *  - the m kept slots are renormalised over themselves:
 *    w_j = (s_j / cum_m) * rsf, cum_m summed in slot order as above;
 *  - a dropped slot has idx -1 and w 0.
 * With k_use = k and p = 1 this is the selection above.
 * Returns -2 for k or k_use out of [1, E] / [1, k], or p outside (0, 1].
 */
int coli_oracle_select_limited(const float *logits, const float *bias, int32_t T, int32_t E, int32_t k,
                               int32_t k_use, float top_p, float rsf, int32_t *idx, float *w) {
  if (T < 0 || E <= 0 || !logits || !idx || !w) return ORACLE_EINVAL;
  if (k < 1 || k > E || k_use < 1 || k_use > k || !(top_p > 0.0f && top_p <= 1.0f)) return ORACLE_EROUTE;
  sel_key_t *keys = (sel_key_t *)malloc(sizeof(sel_key_t) * (size_t)E);
  float *s = (float *)malloc(sizeof(float) * (size_t)E);
  if (!keys || !s) {
    free(keys);
    free(s);
    return -1;
  }
  for (int32_t t = 0; t < T; t++) {
    const float *l = logits + (size_t)t * E;
    for (int32_t e = 0; e < E; e++) {
      s[e] = coli_oracle_sigmoid_spec(l[e]);
      keys[e].c = s[e] + (bias ? bias[e] : 0.0f);
      keys[e].e = e;
    }
    qsort(keys, (size_t)E, sizeof(sel_key_t), key_cmp);
    float den = 0.0f;
    for (int32_t j = 0; j < k_use; j++) den = den + s[keys[j].e];
    int32_t m = k_use;
    float kept = den;
    if (top_p < 1.0f) {
      const float thr = top_p * den;
      m = 1;
      kept = s[keys[0].e];
      while (m < k_use && kept < thr) {
        kept = kept + s[keys[m].e];
        m++;
      }
    }
    for (int32_t j = 0; j < k; j++) {
      const size_t a = (size_t)t * k + j;
      if (j < m) {
        idx[a] = keys[j].e;
        w[a] = (s[keys[j].e] / kept) * rsf;
      } else {
        idx[a] = -1;
        w[a] = 0.0f;
      }
    }
  }
  free(keys);
  free(s);
  return ORACLE_OK;
}

int coli_oracle_select(const float *logits, const float *bias, int32_t T, int32_t E, int32_t k,
                       float rsf, int32_t *idx, float *w) {
  if (k < 1 || k > E) return (T < 0 || E <= 0 || !logits || !idx || !w) ? ORACLE_EINVAL : ORACLE_EROUTE;
  return coli_oracle_select_limited(logits, bias, T, E, k, k, 1.0f, rsf, idx, w);
}

/* ---------------------------------------------------------------------- */
/* Dispatch: stable counting sort of assignments by expert.                 */
/* ---------------------------------------------------------------------- */

/*
 * Assignment a = t*k + j (token t, slot j) goes to expert idx[a].
 * counts[e] = number of a with idx[a] == e; offsets = exclusive prefix sum
 * (E + 1 entries); sorted_ids lists the a grouped by expert ascending and,
 * inside a group, by a ascending; inv[a] is the position of a in
 * sorted_ids; active lists the experts with counts > 0 in ascending order,
 * n_active of them.
 * A negative idx[a] is a dropped slot (routing limits): it goes to no
 * expert, and the dropped assignments follow all the groups in sorted_ids
 * (a ascending), so offsets[E] is the number of kept assignments (T*k when
 * none is dropped).
 * Source: [C] section 3.3 step 3 (per-expert counts, prefix sum to offsets,
 * scatter by expert id) and section 2.2 (grouping example).
 */
int coli_oracle_dispatch(const int32_t *idx, int32_t T, int32_t k, int32_t E, int32_t *counts,
                         int32_t *offsets, int32_t *sorted_ids, int32_t *inv, int32_t *active,
                         int32_t *n_active) {
  if (T < 0 || k < 1 || E <= 0 || !idx || !counts || !offsets || !sorted_ids || !inv || !active ||
      !n_active)
    return ORACLE_EINVAL;
  int64_t n = (int64_t)T * k;
  for (int32_t e = 0; e < E; e++) counts[e] = 0;
  for (int64_t a = 0; a < n; a++) {
    if (idx[a] >= E) return ORACLE_EROUTE;
    if (idx[a] >= 0) counts[idx[a]]++;
  }
  offsets[0] = 0;
  for (int32_t e = 0; e < E; e++) offsets[e + 1] = offsets[e] + counts[e];
  int32_t *fill = (int32_t *)calloc((size_t)E, sizeof(int32_t));
  if (!fill) return -1;
  int32_t dropped = 0;
  for (int64_t a = 0; a < n; a++) {
    int32_t e = idx[a];
    int32_t pos = e >= 0 ? offsets[e] + fill[e]++ : offsets[E] + dropped++;
    sorted_ids[pos] = (int32_t)a;
    inv[a] = pos;
  }
  free(fill);
  int32_t na = 0;
  for (int32_t e = 0; e < E; e++)
    if (counts[e] > 0) active[na++] = e;
  *n_active = na;
  return ORACLE_OK;
}

/* ---------------------------------------------------------------------- */
/* int4 gs64 expert FFN in float64.                                         */
/* ---------------------------------------------------------------------- */

/* Code of weight c of a packed row: low nibble of byte c/2 for even c, high
 * nibble for odd c, read as 4-bit two's complement ([T] item 1, gs64). */
int32_t coli_oracle_unpack_code(const uint8_t *row, int32_t c) {
  int32_t nib = (row[c / 2] >> (4 * (c & 1))) & 0xF;
  return nib >= 8 ? nib - 16 : nib;
}

/* Dequantised weight c of a row: code * scale of its group of 64. */
static double dq(const uint8_t *codes, const float *scales, int32_t c) {
  return (double)coli_oracle_unpack_code(codes, c) * (double)scales[c / 64];
}

typedef struct {
  const uint8_t *gate_q; /* [inter][hidden/2] */
  const float *gate_s;   /* [inter][hidden/64] */
  const uint8_t *up_q;   /* [inter][hidden/2] */
  const float *up_s;
  const uint8_t *down_q; /* [hidden][inter/2] */
  const float *down_s;   /* [hidden][inter/64] */
} coli_oracle_expert_t;

/* ---------------------------------------------------------------------- */
/* int8 with one scale per row.                                             */
/* ---------------------------------------------------------------------- */

/* Code of weight c of an int8 row: byte c read as 8-bit two's complement.
 * Format: [T] "Three key engineering decisions" item 1 and the MTP
 * subsection (the multi-token prediction head must be int8), [N] (the
 * engine's quantised kernels: int8, packed int4, packed int2, per-row
 * scaling); reading: one float32 scale per output row, weight = code *
 * scale[row]. */
int32_t coli_oracle_int8_code(const uint8_t *row, int32_t c) {
  const int32_t b = row[c];
  return b >= 128 ? b - 256 : b;
}

/* Weight c of row r of a [rows][cols] matrix in format fmt (0: int4 gs64,
 * 1: int8 per row), dequantised in float64. */
static double weight_at(int32_t fmt, const uint8_t *codes, const float *scales, int32_t r, int32_t cols,
                        int32_t c) {
  if (fmt == 1) return (double)coli_oracle_int8_code(codes + (size_t)r * cols, c) * (double)scales[r];
  return dq(codes + (size_t)r * (cols / 2), scales + (size_t)r * (cols / 64), c);
}

/*
 * One SwiGLU expert on one token, float64 throughout:
 *   g_i = sum_c Wg[i][c] x[c],  u_i = sum_c Wu[i][c] x[c]   (i < inter)
 *   m_i = silu(g_i) * u_i,      silu(z) = z / (1 + e^-z)
 *   y_r = sum_i Wd[r][i] m_i    (r < hidden)
 * with the tables in storage format fmt (0: int4 gs64, 1: int8 per row).
 * Source: [C] section 2.1 (expert FFN with three matrices); the gated
 * (SwiGLU) form and the matrix roles are the reading stated at the top.
 */
void coli_oracle_expert_ffn_fmt(const coli_oracle_expert_t *ex, int32_t fmt, int32_t h, int32_t I,
                                const float *x, double *y) {
  double *m = (double *)malloc(sizeof(double) * (size_t)I);
  for (int32_t i = 0; i < I; i++) {
    double g = 0.0, u = 0.0;
    for (int32_t c = 0; c < h; c++) {
      g += weight_at(fmt, ex->gate_q, ex->gate_s, i, h, c) * (double)x[c];
      u += weight_at(fmt, ex->up_q, ex->up_s, i, h, c) * (double)x[c];
    }
    double silu = g / (1.0 + exp(-g));
    m[i] = silu * u;
  }
  for (int32_t r = 0; r < h; r++) {
    double acc = 0.0;
    for (int32_t i = 0; i < I; i++) acc += weight_at(fmt, ex->down_q, ex->down_s, r, I, i) * m[i];
    y[r] = acc;
  }
  free(m);
}

void coli_oracle_expert_ffn(const coli_oracle_expert_t *ex, int32_t h, int32_t I, const float *x,
                            double *y) {
  coli_oracle_expert_ffn_fmt(ex, 0, h, I, x, y);
}

/* ---------------------------------------------------------------------- */
/* The layer forward.                                                       */
/* ---------------------------------------------------------------------- */

typedef struct {
  int32_t hidden, n_experts, top_k, inter, n_shared; /* n_shared is 0 or 1 */
  float routed_scaling_factor;
  const float *router_w; /* [hidden][n_experts] */
  const float *sel_bias; /* [n_experts], NULL means zeros */
  /* n_experts + n_shared entries each, shared expert last; an entry may be
   * NULL for an expert that no token of the call selects. */
  const coli_oracle_expert_t *experts;
  int32_t weight_format; /* 0: int4 gs64, 1: int8 with a scale per row */
} coli_oracle_layer_t;

/*
 * out[t] = float32( sum_j w[t][j] * y_(t,j) + y_shared[t] ), the sum taken in
 * float64 in slot order, then the shared term.  Steps in the pages' order:
 * router logits and selection, grouping by expert (dispatch), the FFN of each
 * active expert over its group, then the weighted assembly per token
 * ([C] section 3.3 steps 2-5; [T] "Task flow example").
 * idx_out / w_out (optional) receive the routing, [T][k].
 * k_use / top_p: the run-time routing limits of coli_oracle_select_limited
 * (k_use = k, top_p = 1: none); dropped slots have no FFN and add nothing.
 * Returns 0, -1 (allocation), -2 (k, k_use or top_p out of range), -4 (bad
 * argument or an expert table missing for a selected expert).
 */
int coli_oracle_forward_limited(const coli_oracle_layer_t *L, const float *x, int32_t T, int32_t k_use,
                                float top_p, float *out, int32_t *idx_out, float *w_out) {
  if (!L || T < 0 || (T > 0 && (!x || !out))) return ORACLE_EINVAL;
  const int32_t h = L->hidden, E = L->n_experts, k = L->top_k, I = L->inter;
  if (h <= 0 || h % 64 || I <= 0 || I % 64 || E <= 0 || !L->router_w || !L->experts ||
      (L->n_shared != 0 && L->n_shared != 1) || (L->weight_format != 0 && L->weight_format != 1))
    return ORACLE_EINVAL;
  if (k < 1 || k > E || k_use < 1 || k_use > k || !(top_p > 0.0f && top_p <= 1.0f)) return ORACLE_EROUTE;
  if (T == 0) return ORACLE_OK;
  int rc = ORACLE_OK;
  size_t n = (size_t)T * k;
  float *logits = (float *)malloc(sizeof(float) * (size_t)T * E);
  int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * n);
  float *w = (float *)malloc(sizeof(float) * n);
  int32_t *counts = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
  int32_t *offsets = (int32_t *)malloc(sizeof(int32_t) * ((size_t)E + 1));
  int32_t *sorted_ids = (int32_t *)malloc(sizeof(int32_t) * n);
  int32_t *inv = (int32_t *)malloc(sizeof(int32_t) * n);
  int32_t *active = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
  double *y = (double *)malloc(sizeof(double) * n * (size_t)h);
  double *ysh = L->n_shared ? (double *)malloc(sizeof(double) * (size_t)T * h) : NULL;
  if (!logits || !idx || !w || !counts || !offsets || !sorted_ids || !inv || !active || !y ||
      (L->n_shared && !ysh)) {
    rc = -1;
    goto done;
  }
  int32_t n_active = 0;
  coli_oracle_router_logits(x, L->router_w, T, h, E, logits);
  rc = coli_oracle_select_limited(logits, L->sel_bias, T, E, k, k_use, top_p, L->routed_scaling_factor, idx, w);
  if (rc) goto done;
  rc = coli_oracle_dispatch(idx, T, k, E, counts, offsets, sorted_ids, inv, active, &n_active);
  if (rc) goto done;
  for (int32_t s = 0; s < n_active; s++) {
    const coli_oracle_expert_t *ex = &L->experts[active[s]];
    if (!ex->gate_q || !ex->gate_s || !ex->up_q || !ex->up_s || !ex->down_q || !ex->down_s) {
      rc = ORACLE_EINVAL;
      goto done;
    }
  }
  /* expert FFN over each group: position p < offsets[E] of the sorted order
   * holds assignment a = sorted_ids[p] of token a / k (the positions after
   * offsets[E] are dropped slots) */
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t p = 0; p < (int64_t)offsets[E]; p++) {
    int32_t a = sorted_ids[p];
    coli_oracle_expert_ffn_fmt(&L->experts[idx[a]], L->weight_format, h, I, x + (size_t)(a / k) * h,
                               y + (size_t)p * h);
  }
  if (L->n_shared) {
    const coli_oracle_expert_t *sh = &L->experts[E];
    if (!sh->gate_q || !sh->gate_s || !sh->up_q || !sh->up_s || !sh->down_q || !sh->down_s) {
      rc = ORACLE_EINVAL;
      goto done;
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t t = 0; t < T; t++)
      coli_oracle_expert_ffn_fmt(sh, L->weight_format, h, I, x + (size_t)t * h, ysh + (size_t)t * h);
  }
  /* weighted assembly per token */
  for (int32_t t = 0; t < T; t++) {
    for (int32_t r = 0; r < h; r++) {
      double acc = 0.0;
      for (int32_t j = 0; j < k; j++) {
        size_t a = (size_t)t * k + j;
        if (idx[a] >= 0) acc += (double)w[a] * y[(size_t)inv[a] * h + r];
      }
      if (L->n_shared) acc += ysh[(size_t)t * h + r];
      out[(size_t)t * h + r] = (float)acc;
    }
  }
  if (idx_out) memcpy(idx_out, idx, sizeof(int32_t) * n);
  if (w_out) memcpy(w_out, w, sizeof(float) * n);
done:
  free(logits);
  free(idx);
  free(w);
  free(counts);
  free(offsets);
  free(sorted_ids);
  free(inv);
  free(active);
  free(y);
  free(ysh);
  return rc;
}

int coli_oracle_forward(const coli_oracle_layer_t *L, const float *x, int32_t T, float *out, int32_t *idx_out,
                        float *w_out) {
  if (!L) return ORACLE_EINVAL;
  return coli_oracle_forward_limited(L, x, T, L->top_k, 1.0f, out, idx_out, w_out);
}

/* Threads the oracle's parallel loops use (for reporting). */
#ifdef _OPENMP
#include <omp.h>
#endif
int32_t coli_oracle_threads(void) {
#ifdef _OPENMP
  return (int32_t)omp_get_max_threads();
#else
  return 1;
#endif
}
