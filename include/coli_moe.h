/*
 * coli_moe.h -- C ABI of one routed Mixture-of-Experts layer forward on AMD
 * Instinct MI355X (gfx950), hand-written HIP kernels.
 *
 * The layer (sources: web pages about the Colibri / colibri MoE engine):
 *   1. float32 router: logits = hidden . Wr, sigmoid scores, a per-expert
 *      selection bias, noaux_tc top-k with n_group = 1, the selected scores
 *      renormalised and multiplied by routed_scaling_factor
 *      ("colibri engine teardown" page, "Three key engineering decisions",
 *      item 1: sigmoid router, noaux_tc, n_group = 1, routed_scaling_factor;
 *      norm, router and bias stay float32);
 *   2. grouping of (token, slot) assignments by expert with a counting sort
 *      and a prefix sum into per-expert offsets (cf-1.com Colibri article,
 *      section 3.3, colibri_forward step 3), done on the device with no host
 *      round trip;
 *   3. per-expert SwiGLU FFN over int4 weights with one float32 scale per 64
 *      weights ("gs64", same teardown page, item 1; three expert matrices,
 *      cf-1.com article section 2.1);
 *   4. weighted combine of the k expert outputs of each token (cf-1.com
 *      article section 3.3, step 5) plus a shared expert with weight 1
 *      (teardown page, "System map": the shared expert is resident).
 *
 * API shape: init / forward / free with negative integer error codes, a dry
 * run for zero tokens, and a handle that is not thread-safe (trdm.cn article
 * "Colibri: a pure-C lightweight inference engine built for MoE models",
 * sections 4.2, 5.1 and 5.2).
 *
 * Conventions for every function below:
 *  - "device" pointers point to HIP device memory of the current device;
 *    "host" pointers to ordinary host memory.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls only enqueue work on that stream; nothing synchronises with the
 *    host unless stated.  Device-side faults surface at the caller's next
 *    synchronisation.
 *  - The library never allocates device memory: weights, the workspace,
 *    inputs and outputs belong to the caller, who keeps them alive while a
 *    handle uses them.
 *  - A handle must not be used from two threads at once, nor on two streams
 *    whose work may overlap (calls share the handle's workspace).
 *  - Inputs must be finite.  NaN or Inf in the hidden state or weights gives
 *    unspecified routing and outputs.
 */
#ifndef COLI_MOE_H
#define COLI_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Error codes (0 = success). */
#define COLI_MOE_OK 0
#define COLI_MOE_ECAPACITY (-1) /* T > max_tokens, or the workspace is too small */
#define COLI_MOE_EROUTING (-2)  /* top_k < 1 or > n_experts or > 32, n_group != 1, group_size not the format's */
#define COLI_MOE_EDEVICE (-3)   /* a HIP launch or runtime call failed */
#define COLI_MOE_EARG (-4)      /* NULL or misaligned pointer, unsupported dimension */

/* Layer configuration, fixed at init. */
typedef struct {
  int32_t hidden;            /* h: multiple of 64, 64..16384 */
  int32_t n_experts;         /* E: routed experts, 1..512 */
  int32_t top_k;             /* k: experts per token, 1..min(E, 32) */
  int32_t inter;             /* I: expert intermediate size, multiple of 64, 64..16384 */
  int32_t n_shared;          /* shared experts: 0 or 1 */
  int32_t group_size;        /* weights per scale: 64 for int4 gs64, 0 (a whole row) for int8 */
  int32_t n_group;           /* expert groups of noaux_tc: must be 1 */
  int32_t max_tokens;        /* most tokens one forward may take, >= 1 */
  int32_t prefill_threshold; /* T >= this takes the MFMA (fp16) path; 0 = 256 */
  float routed_scaling_factor;
  int32_t weight_format;     /* COLI_MOE_WEIGHTS_*: storage of the expert tables */
} coli_moe_config_t;

/*
 * Expert table formats (weight_format).
 *
 * COLI_MOE_WEIGHTS_INT4_GS64 (0): the routed experts' format of the
 *   teardown page ("Three key engineering decisions", item 1): int4 codes,
 *   one float32 scale per 64 weights along the input axis (layout below).
 *
 * COLI_MOE_WEIGHTS_INT8_ROW (1): int8 codes with one float32 scale per
 *   output row, the precision the same page requires of the MTP head
 *   ("MTP head must be int8": int4 drafts are almost never accepted) and
 *   one of the engine's per-row-scaled kernel formats.  A matrix
 *   [rows][cols] is rows of cols int8 two's-complement codes (byte c =
 *   column c), scale s[row]; weight = q * s[row].  Tables: gate_q, up_q
 *   [E][inter][hidden] bytes, gate_s, up_s [E][inter] floats, down_q
 *   [E][hidden][inter] bytes, down_s [E][hidden] floats (shared expert
 *   alike).  group_size must be 0.  Every forward runs the GEMV kernels'
 *   small-batch launches (draft and verify shapes: 1 to 4 tokens);
 *   larger T runs them on consecutive groups of up to 4 tokens, each group
 *   reading its experts again, then publishes the routing of the whole
 *   batch.  Requires inter <= 4096 and a hidden row's planes to fit
 *   (hidden <= 16384); no prefill path and no expert cache.
 */
#define COLI_MOE_WEIGHTS_INT4_GS64 0
#define COLI_MOE_WEIGHTS_INT8_ROW 1

/*
 * Weight tables, all DEVICE pointers, borrowed (the caller owns them and
 * keeps them alive and unchanged while the handle exists).
 *
 * int4 gs64 storage of a weight matrix [rows][cols]: byte c/2 of a row holds
 * weight c in its low nibble when c is even and in its high nibble when c is
 * odd, as a 4-bit two's-complement code q in [-8, 7]; the float32 scale
 * s[row][c/64] belongs to the 64 weights of group c/64; weight = q * s.
 * Groups run along the input (reduction) axis.  Rows are contiguous.
 *
 * All code and scale arrays must be 16-byte aligned; router_w and sel_bias
 * 4-byte aligned.
 */
typedef struct {
  const float *router_w;   /* [hidden][n_experts] float32 */
  const float *sel_bias;   /* [n_experts] float32 selection bias; NULL = zeros */
  const uint8_t *gate_q;   /* [n_experts][inter][hidden/2]   (W1) */
  const float *gate_s;     /* [n_experts][inter][hidden/64] */
  const uint8_t *up_q;     /* [n_experts][inter][hidden/2]   (W3) */
  const float *up_s;       /* [n_experts][inter][hidden/64] */
  const uint8_t *down_q;   /* [n_experts][hidden][inter/2]   (W2) */
  const float *down_s;     /* [n_experts][hidden][inter/64] */
  /* the shared expert, same layout for one expert; NULL when n_shared == 0 */
  const uint8_t *sh_gate_q;
  const float *sh_gate_s;
  const uint8_t *sh_up_q;
  const float *sh_up_s;
  const uint8_t *sh_down_q;
  const float *sh_down_s;
} coli_moe_weights_t;

typedef struct coli_moe coli_moe_t; /* opaque handle */

/*
 * Bytes of DEVICE workspace a handle with this configuration needs (router
 * copy, routing and dispatch arrays, expert intermediates for max_tokens).
 * Returns 0 when the configuration is invalid.
 */
size_t coli_moe_workspace_bytes(const coli_moe_config_t *cfg);

/*
 * Create a handle.  `workspace` is caller-owned DEVICE memory of at least
 * coli_moe_workspace_bytes(cfg) bytes, 256-byte aligned, used only by this
 * handle until coli_moe_free.  Enqueues a copy of the router into the
 * workspace on `stream`.  On success *out receives the handle (host memory
 * the library owns).
 * Errors: -4 NULL/misaligned pointer or unsupported dimension, -2 routing
 * configuration, -1 workspace too small, -3 HIP error.
 */
int coli_moe_init(coli_moe_t **out, const coli_moe_config_t *cfg, const coli_moe_weights_t *w,
                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * out[t] = sum_j w[t][j] * FFN_{idx[t][j]}(hidden[t]) + FFN_shared(hidden[t])
 * for t < T.  `hidden` is DEVICE float32 [T][hidden] (16-byte aligned), `out`
 * DEVICE float32 [T][hidden] (16-byte aligned, may not alias `hidden`).
 * Asynchronous on `stream`; the host never reads device data.  T == 0 checks
 * the arguments and enqueues nothing (dry run).  T >= prefill_threshold runs
 * the MFMA grouped-GEMM path (fp16 operands, float32 accumulation) when
 * hidden and inter are multiples of 256 and the 16-bit copies of the
 * activations ([max_tokens][hidden] and [max_tokens*(top_k+n_shared)][inter])
 * stay under 4 GiB; every other call runs the float32-accumulate GEMV path.
 * Errors: -4 bad handle/pointer, -1 T > max_tokens (or T < 0 gives -4),
 * -3 HIP launch error.
 */
int coli_moe_forward(coli_moe_t *m, const float *hidden, float *out, int32_t T, void *stream);

/*
 * For callers that cannot allocate (code under HIP graph capture, serving
 * loops, harnesses that forbid hipMalloc): the same layer forward as
 * coli_moe_forward, with no handle and no workspace argument.  Its workspace
 * is a device array inside the library of COLI_MOE_STATIC_SCRATCH_BYTES
 * (64 MiB) per device, held from the first call on a device until the
 * process ends; the call allocates nothing, host or device.  Each call
 * re-stages the per-layer state in it (router copy, cleared counters,
 * prefill statistics) on `stream` and then runs the forward, so calls whose
 * work overlaps on one device race on that array: serialise them (one
 * stream, or events).  Arguments as for coli_moe_init (cfg, w: DEVICE weight
 * tables, borrowed for the call) and coli_moe_forward (hidden, out, T).
 * Errors: -1 T > max_tokens, or the configuration's workspace
 * (coli_moe_workspace_bytes) exceeds COLI_MOE_STATIC_SCRATCH_BYTES -- e.g.
 * a layer with h 6144, 256 experts, top-8, I 2048 and a shared expert fits
 * up to max_tokens 163; -2 routing configuration; -4 bad argument;
 * -3 HIP error.  T == 0 checks the arguments and enqueues nothing.
 */
#define COLI_MOE_STATIC_SCRATCH_BYTES (64u << 20)
int coli_moe_forward_noalloc(const coli_moe_config_t *cfg, const coli_moe_weights_t *w, const float *hidden,
                             float *out, int32_t T, void *stream);

/*
 * Run-time routing limits of the handle's later forwards: two lossy
 * overrides of the routing, an explicit smaller k and adaptive expert top-p
 * ("Colibri 调优与运行时旋钮实战指南" -- Colibri tuning and runtime knobs
 * guide -- knob table; the engine warns that both change the model's
 * output).  1 <= k_use <= top_k, 0 < top_p <= 1; (top_k, 1) restores the
 * plain routing (the default).  Per token:
 *  - the k_use experts first in the selection order are the candidates,
 *    in slots 0..k_use-1; den is the sum of their sigmoid scores, added in
 *    slot order in float32;
 *  - top_p < 1 keeps slot 0, then slot j while the candidates before it
 *    score less than top_p * den (float32 product; the running sum in slot
 *    order, float32): the shortest prefix of slots whose score reaches the
 *    share top_p;
 *  - the kept slots' weights are renormalised over them,
 *    w_j = (s_j / kept sum) * routed_scaling_factor;
 *  - the other slots of the k are dropped: idx -1, w 0, no expert work.
 * The routing arrays keep their [T][top_k] layout; dispatch puts the
 * dropped assignments after every expert's group in sorted_ids (ascending),
 * so offsets[n_experts] counts the kept ones.  Dropped experts' weights are
 * never read, which is the point: fewer expert bytes per token.  Not
 * thread-safe with the handle's forwards (set it between calls on the
 * handle's stream order).  Errors: -4 NULL handle, -2 out of range.
 */
int coli_moe_set_routing(coli_moe_t *m, int32_t k_use, float top_p);

/* Release the handle (host memory only).  NULL is a no-op.  The caller must
 * make sure no enqueued forward of the handle is still running. */
void coli_moe_free(coli_moe_t *m);

/*
 * Error word of the handle's launches.  The one-token gate/up launch hands
 * the routing from one wave of each workgroup to the others through a flag
 * in LDS; the others wait a bounded time (COLI_MOE_DEFAULT_SPIN_LIMIT polls
 * of about 64 cycles, about 0.1 s).  A wave that gives up computes none of
 * its routed rows and stores 1 in a device word of the workspace, so that
 * call's output is wrong.  This call waits for `stream`, reads the word and
 * clears it: COLI_MOE_OK when no launch since the last call (or since init)
 * gave up, COLI_MOE_EDEVICE when one did or the read failed, -4 for NULL.
 * Synchronous.  coli_moe_forward_noalloc has no handle and no such report.
 */
int coli_moe_status(coli_moe_t *m, void *stream);

/*
 * For tests of the error path: the bound of that wait, in polls (>= 0; 0:
 * every waiting wave gives up at once, so every one-token call fails and is
 * reported).  Takes effect from the next forward.  -4 for NULL or polls < 0.
 */
#define COLI_MOE_DEFAULT_SPIN_LIMIT (1 << 22)
int coli_moe_test_spin_limit(coli_moe_t *m, int32_t polls);

/*
 * For tests of both kernel families of the larger int4 batches (above the
 * small-batch limits, below the prefill threshold): mfma = 1 runs them on
 * the int8 matrix cores, mfma = 0 on the v_dot8 GEMV kernels (which also
 * serve batches too large for the former's 31-bit offsets), mfma = 2 (the
 * default) picks by size: the matrix cores from 16 tokens.  Takes effect
 * from the next forward.  -4 for NULL or mfma outside 0..2.
 */
int coli_moe_test_batch_kernels(coli_moe_t *m, int32_t mfma);

/*
 * Copy the routing and dispatch of the handle's last forward (T tokens) into
 * caller DEVICE buffers, enqueued on `stream` (for parity checks).  Any
 * pointer may be NULL to skip it.  Sizes: idx and w [T*k] (assignment
 * a = t*k + j, slot order = selection rank; -1 and 0 in slots the routing
 * limits dropped), offsets [E+1], sorted_ids and inv [T*k], active [E]
 * (experts with tokens, ascending; n_active of them are valid), n_active
 * [1].  Returns the T of the last forward (>= 0) or -4.
 */
int coli_moe_last_routing(const coli_moe_t *m, int32_t *idx, float *w, int32_t *offsets,
                          int32_t *sorted_ids, int32_t *inv, int32_t *active, int32_t *n_active,
                          void *stream);

/*
 * The dispatch kernel alone on caller data: a stable counting sort of the
 * assignments a = t*k + j of DEVICE idx [T*k] (values in [0, E), or
 * negative for a dropped slot) by expert, written to DEVICE offsets [E+1],
 * sorted_ids [T*k], inv [T*k], active [E], n_active [1] (same meaning as
 * above; dropped assignments follow every group).  1 <= E <= 512,
 * 1 <= k <= 32, 0 <= T*k <= 2^20.  (cf-1.com Colibri article, section 3.3,
 * step 3.)  Runs the same launches as coli_moe_forward for this T*k: one
 * workgroup up to 1024 assignments, else a count launch and a scatter launch
 * over ceil(T*k / 1024) workgroups, whose count array (that many times E+1
 * ints) this call allocates and frees in stream order.  Errors: -4.  Values
 * >= E give unspecified (but in-bounds) results.
 */
int coli_moe_test_dispatch(const int32_t *idx, int32_t T, int32_t k, int32_t E, int32_t *offsets,
                           int32_t *sorted_ids, int32_t *inv, int32_t *active, int32_t *n_active,
                           void *stream);

/*
 * Measurement only: the HBM read ceiling of the decode gate/up kernel's
 * access pattern.  Enqueues one launch with the small-batch gate/up launch's
 * grid that loads, and otherwise discards, the gate and up codes and scales
 * of every row of the n experts listed in DEVICE experts [n] (expert id, or
 * -1 for the shared expert; ids outside [-1, n_experts) read nothing),
 * split statically over its waves with two rows in flight per wave: the
 * bytes the gate/up step reads for those experts, with none of its
 * arithmetic.  Overwrites the handle's logits buffer.  1 <= n <= 64,
 * hidden <= 8192.  Errors: -4, -3.
 */
int coli_moe_probe_read(const coli_moe_t *m, const int32_t *experts, int32_t n, void *stream);

/*
 * Measurement only: the same for the one-token down + combine kernel.  One
 * launch with that kernel's grid and row split (each wave owns a contiguous
 * range of output rows) that loads, and otherwise discards, the down codes
 * and scales of those rows of the n experts listed in DEVICE experts [n]
 * (as above), two experts in flight per wave.  Overwrites the handle's
 * logits buffer.  1 <= n <= 64, inter <= 8192.  Errors: -4, -3.
 */
int coli_moe_probe_read_down(const coli_moe_t *m, const int32_t *experts, int32_t n, void *stream);

/*
 * Measurement only: the rates this GPU reaches, for setting the layer's
 * figures against them (no handle needed).
 *
 * coli_moe_probe_stream reads every byte of the DEVICE buffer buf [bytes]
 * once (16-byte loads, bytes a multiple of 16, buf 16-byte aligned) and
 * XORs all its 32-bit words into the DEVICE word *sink (the caller clears
 * it first; the result does not depend on the order of reads).
 *
 * coli_moe_probe_mfma runs `blocks` blocks of 4 waves, each wave `iters`
 * rounds of 8 back-to-back v_mfma_f32_32x32x16_bf16 (32768 flops each) on
 * all-ones operands; each wave whose results all equal 16 * iters adds 1 to
 * the DEVICE word *sink.  1 <= iters < 2^20, 1 <= blocks <= 2^20.
 *
 * coli_moe_probe_mfma_f16 is the same launch shape with
 * v_mfma_f32_32x32x16_f16 on operands that change from one MFMA to the next
 * (pseudo-random halves derived from `seed`, |v| in [2^-4, 2^11)): each
 * wave runs `iters` rounds of 16 MFMAs and adds 1 to *sink when all its
 * accumulators are finite.  Power draw depends on the data, so this is the
 * rate a GEMM on real operands can approach; the all-ones rate is higher.
 *
 * All three only enqueue on `stream`.  Errors: -4 NULL/misaligned pointer or
 * a size out of range, -3 HIP launch error.
 */
int coli_moe_probe_stream(const void *buf, size_t bytes, uint32_t *sink, void *stream);
int coli_moe_probe_mfma(int32_t iters, int32_t blocks, uint32_t *sink, void *stream);
int coli_moe_probe_mfma_f16(int32_t iters, int32_t blocks, uint32_t seed, uint32_t *sink, void *stream);

/*
 * Kernel timing.  coli_moe_profile_begin makes the next `max_calls` forwards
 * of the handle record a HIP event pair around each kernel they launch (host
 * allocations only; events are created here).  coli_moe_profile_end waits
 * for those events, writes the summed milliseconds and launch counts per
 * kernel (arrays of COLI_MOE_N_KERNELS entries, either may be NULL) and
 * stops recording.  Returns the number of forwards recorded, or -4/-3.
 */
#define COLI_MOE_N_KERNELS 10
int coli_moe_profile_begin(coli_moe_t *m, int32_t max_calls);
int coli_moe_profile_end(coli_moe_t *m, float *kernel_ms, int32_t *kernel_launches);
/* Name of kernel i (0 <= i < COLI_MOE_N_KERNELS), a static string. */
const char *coli_moe_kernel_name(int32_t i);

/*
 * ---------------------------------------------------------------------------
 * HBM expert cache with host-RAM backing (three tiers: HBM slots, pinned host
 * memory, and -- outside this library -- disk).  Source: "Colibri 调优与运行时
 * 旋钮实战指南" (tuning and runtime knobs guide), sections on the resource
 * plan (hot / warm / cold tiers, a per-layer expert LRU), online re-pinning
 * (LFRU score of decayed frequency and recency, at most four swaps, 25%
 * hysteresis) and the learning cache (.coli_usage routing counts, hottest
 * experts pinned); "colibrì 引擎拆解" (engine teardown), "System map".
 *
 * A cache handle is one layer whose routed experts live in host memory and
 * are copied on demand into n_slots HBM slots.  Each forward runs the router,
 * selection and dispatch on the device, reads the call's expert list back
 * (the host waits for `stream` once per call), copies the misses from the
 * host tables into slots on the cache's own copy stream, and then runs the
 * expert kernels on the slots: outputs are bit for bit those of
 * coli_moe_forward on fully resident tables.  Every call runs the
 * float32-accumulate GEMV path (prefill_threshold is ignored).  A cache's
 * calls must be issued on one stream (or serialised by the caller).
 * ---------------------------------------------------------------------------
 */
typedef struct coli_moe_cache coli_moe_cache_t; /* opaque */

/* The routed experts of one layer in HOST memory that stays valid for the
 * cache's lifetime, stacked as in coli_moe_weights_t ([n_experts][...]),
 * 16-byte aligned.  Pinned memory (hipHostMalloc) is needed for the copies to
 * run asynchronously. */
typedef struct {
  const uint8_t *gate_q;
  const float *gate_s;
  const uint8_t *up_q;
  const float *up_s;
  const uint8_t *down_q;
  const float *down_s;
} coli_moe_host_experts_t;

typedef struct {
  int32_t n_slots;     /* experts resident in HBM at once: min(E, top_k * max_tokens) .. n_experts */
  int32_t repin_every; /* a re-pinning round every this many forwards; 0 = never */
  float decay;         /* per-forward decay of the expert frequencies, (0, 1]; 0 = 0.9 */
} coli_moe_cache_config_t;

typedef struct {
  int64_t calls;         /* forwards */
  int64_t needed;        /* sum over forwards of the distinct experts routed to */
  int64_t hits;          /* of those, resident when the forward began (prefetched ones included) */
  int64_t misses;        /* copied in by the forward itself */
  int64_t prefetched;    /* copied in by coli_moe_cache_prefetch */
  int64_t prefetch_hits; /* prefetched experts that the next forward routed to */
  int64_t evictions;     /* slots overwritten */
  int64_t repin_swaps;   /* re-pinning swaps */
  int64_t bytes_copied;  /* host -> HBM expert bytes */
  int32_t pinned, resident;
} coli_moe_cache_stats_t;

/* DEVICE bytes for n_slots slots (the slot tables and the slot map); 0 when
 * the configuration or n_slots is invalid. */
size_t coli_moe_cache_slot_bytes(const coli_moe_config_t *cfg, int32_t n_slots);

/*
 * Create a cache handle.  `resident` holds the DEVICE router, selection bias
 * and shared expert (its routed tables are ignored); `host` the routed
 * experts; `slots` caller-owned DEVICE memory of coli_moe_cache_slot_bytes
 * bytes and `workspace` of coli_moe_workspace_bytes bytes (both 256-byte
 * aligned).  The library allocates its pinned staging buffers, events and
 * copy stream here (host and event resources, no device memory).
 * Errors: -4 bad argument, -2 routing configuration, -1 n_slots below
 * min(E, top_k * max_tokens) or memory too small, -3 HIP error.
 */
int coli_moe_cache_init(coli_moe_cache_t **out, const coli_moe_config_t *cfg, const coli_moe_cache_config_t *cc,
                        const coli_moe_weights_t *resident, const coli_moe_host_experts_t *host, void *slots,
                        size_t slot_bytes, void *workspace, size_t workspace_bytes, void *stream);

/* The layer forward through the cache (see above).  Errors as
 * coli_moe_forward. */
int coli_moe_cache_forward(coli_moe_cache_t *c, const float *hidden, float *out, int32_t T, void *stream);

/*
 * Router look-ahead prefetch (PILOT): runs this cache's router, selection and
 * dispatch on `hidden` [T][h] (DEVICE) -- the state the previous layer
 * consumes, a stand-in for this layer's own input -- and starts copying the
 * first n_predict selected experts of every token that are not resident,
 * without waiting for the copies.  They stay guarded from eviction until the
 * next forward of this cache, which counts them as hits.  Source: tuning
 * guide, "路由器前瞻预取" (router look-ahead prefetch: layer L+1's router on
 * layer L's state recalls 71.6% of the true top-8; PILOT_K experts per step;
 * PILOT_EVICT_GUARD).  1 <= n_predict <= top_k.  Errors as
 * coli_moe_forward.
 */
int coli_moe_cache_prefetch(coli_moe_cache_t *c, const float *hidden, int32_t T, int32_t n_predict, void *stream);

/* Pin HOST-listed experts (copying in those not resident), in order, until
 * the pin budget (n_slots - min(E, top_k * max_tokens)) is full.  Returns the
 * number pinned, or -4 / -3. */
int coli_moe_cache_pin(coli_moe_cache_t *c, const int32_t *experts, int32_t n, void *stream);

/* Counters; per-expert routing counts of the cache's lifetime (HOST int64
 * [n_experts], the learning cache's signal); the slot of each expert (HOST
 * int32 [n_experts], -1 = not resident).  Return 0 or -4. */
int coli_moe_cache_stats(const coli_moe_cache_t *c, coli_moe_cache_stats_t *stats);
int coli_moe_cache_usage(const coli_moe_cache_t *c, int64_t *counts);
int coli_moe_cache_slots(const coli_moe_cache_t *c, int32_t *slot_of);

/* The layer handle the cache runs (for coli_moe_last_routing and the
 * profiling calls); owned by the cache. */
coli_moe_t *coli_moe_cache_layer(coli_moe_cache_t *c);

/* Release the cache (waits for its copies).  NULL is a no-op. */
void coli_moe_cache_free(coli_moe_cache_t *c);

/*
 * Usage history file (text; the learning cache's record): header records
 * "-1 n_layers n_experts" and "-2 1 <engine id>" (coli_moe_usage_engine_id(),
 * FNV-1a 32 of the engine name), then one "layer expert count" record per
 * non-zero count; an empty history is an empty file.  Readers skip records
 * whose first field is negative and is not -1 / -2, and reject files of other
 * dimensions or engines (-2).  counts: HOST int64 [n_layers][n_experts].
 * Source: tuning guide, learning-cache section (.coli_usage format).
 * write returns 0 or -4; read the number of count records, or -4 / -2.
 */
uint32_t coli_moe_usage_engine_id(void);
int coli_moe_usage_write(const char *path, int32_t n_layers, int32_t n_experts, const int64_t *counts);
int coli_moe_usage_read(const char *path, int32_t n_layers, int32_t n_experts, int64_t *counts);

/*
 * Test only: the cache's residency policy alone, on the host.  Pins `pins`,
 * then plays n_calls calls, call i needing call_len[i] distinct experts taken
 * in order from `calls`; miss_out[i] receives call i's misses and slot_out
 * (HOST [n_experts], may be NULL) the final slot of each expert.  Returns the
 * re-pinning swaps, or -4 / -1.
 */
int coli_moe_test_cache_policy(int32_t n_experts, int32_t n_slots, int32_t reserve, float decay, int32_t repin_every,
                               const int32_t *pins, int32_t n_pins, const int32_t *calls, const int32_t *call_len,
                               int32_t n_calls, int32_t *miss_out, int32_t *slot_out);

/* Static description of an error code. */
const char *coli_moe_error_string(int32_t code);

#ifdef __cplusplus
}
#endif

#endif /* COLI_MOE_H */
