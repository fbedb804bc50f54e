/*
 * mk.h — C ABI of the MI355X (gfx950) decode megakernel.
 *
 * One decode step of a Llama-style decoder (RMSNorm, QKV projection, RoPE, GQA
 * attention over a bf16 KV cache, O projection, SwiGLU MLP, LM head + greedy
 * argmax) runs as ONE persistent HIP kernel with one workgroup per compute
 * unit.  A second kernel runs the parallel-block mixture-of-experts decoder of
 * Cohere's write-up (airebao.com, «快在哪里» item 1: attention and the MoE
 * both read one RMSNorm output, x_{l+1} = x_l + attn + MoE; a router picks the
 * top-k experts of every token, their softmax weights sum the experts' SwiGLU
 * outputs) for B <= 8 sequences per step, each streamed weight byte applied to
 * every sequence that uses it.  Each workgroup interprets a host-built queue of tile-sized
 * instructions; instructions wait on each other instead of on kernel
 * boundaries: every activation element carries the step that wrote it, so a
 * consumer polls its inputs until they are this step's (data without such a
 * tag sits behind counters in global memory).  This follows the design described in
 * Hazy Research's Llama-1B megakernel write-up ("Fusing Operations with an
 * On-GPU Interpreter", "Efficient Shared Memory Management" and "Custom
 * Synchronization Mechanism" in the rocketrecap.com summary) and the persistent
 * per-SM task-list kernel in Cohere's write-up (airebao.com, «Megakernel
 * 是什么»), re-designed for gfx950.
 *
 * Conventions
 *   - Every call returns an mk_status; nothing throws or aborts across the ABI.
 *     On error, mk_last_error() returns a message.
 *   - Weights, KV cache, tokens, next-token and logits buffers are device
 *     memory owned by the CALLER.  They must outlive the context and any step
 *     in flight.  The library never frees them.
 *   - The library owns its arena (activations, counters, RoPE tables, plan,
 *     argmax/attention scratch, status word) and frees it in mk_destroy.
 *   - bf16 tensors are row-major [out, in] (PyTorch nn.Linear layout), stacked
 *     over layers.  KV caches are bf16 [L][B][G][max_seq][Dh]; cached keys are
 *     stored after RoPE.
 *   - One context is used by one host thread at a time.
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mk_ctx mk_ctx; /* opaque, owned by the library */

typedef enum {
  MK_OK = 0,
  MK_ERR_INVALID_ARG = -1, /* bad pointer, shape, option or position       */
  MK_ERR_HIP = -2,         /* a HIP runtime call failed                     */
  MK_ERR_NO_PLAN = -3,     /* mk_decode_step before mk_build_plan           */
  MK_ERR_UNSUPPORTED = -4, /* shape the kernel has no code path for         */
  MK_ERR_OOM = -5,         /* device allocation failed                      */
  MK_ERR_TIMEOUT = -6,     /* a device wait exceeded the watchdog           */
  MK_ERR_DEVICE = -7       /* the kernel reported an error (e.g. NaN logits)*/
} mk_status;

/* Model shape.  Dense decoders (batch 1) set n_experts = top_k = expert_ffn = 0
 * and parallel_block = 0.  The mixture-of-experts decoder sets n_experts
 * (<= 64), top_k (<= min(8, n_experts)), expert_ffn (512, 1024 or 2048) and
 * parallel_block = 1, with batch <= 8, hidden and n_q_heads*head_dim
 * multiples of 512 and batch * max(hidden, n_q_heads*head_dim) <= 16384; ffn
 * and the dense MLP weights are unused.  Other shapes: MK_ERR_UNSUPPORTED. */
typedef struct {
  int32_t n_layers;       /* L                                   */
  int32_t hidden;         /* d                                   */
  int32_t n_q_heads;      /* H                                   */
  int32_t n_kv_heads;     /* G (H % G == 0)                      */
  int32_t head_dim;       /* Dh (64 or 128)                      */
  int32_t ffn;            /* F (dense SwiGLU width)              */
  int32_t vocab;          /* V                                   */
  int32_t max_seq;        /* KV-cache capacity in positions      */
  int32_t batch;          /* B (1 for the dense decoder)         */
  int32_t tied_embedding; /* 1: lm_head may equal embed          */
  int32_t n_experts;      /* MoE only                            */
  int32_t top_k;          /* MoE only                            */
  int32_t expert_ffn;     /* MoE only                            */
  int32_t parallel_block; /* MoE only                            */
  float rms_eps;          /* RMSNorm epsilon (inside the sqrt)   */
  float rope_theta;       /* RoPE base                           */
} mk_config;

/* Caller-owned DEVICE pointers.  bf16 unless noted.  Unused entries are NULL. */
typedef struct {
  const void *embed;      /* [V, d]                                */
  const void *lm_head;    /* [V, d]; may equal embed               */
  const void *final_norm; /* [d]                                   */
  const void *attn_norm;  /* [L, d]                                */
  const void *wq;         /* [L, H*Dh, d]                          */
  const void *wk;         /* [L, G*Dh, d]                          */
  const void *wv;         /* [L, G*Dh, d]                          */
  const void *wo;         /* [L, d, H*Dh]                          */
  const void *mlp_norm;   /* dense: [L, d]                         */
  const void *w_gate;     /* dense: [L, F, d]                      */
  const void *w_up;       /* dense: [L, F, d]                      */
  const void *w_down;     /* dense: [L, d, F]                      */
  const void *router;     /* MoE: [L, E, d] (attn_norm feeds it)   */
  const void *e_gate;     /* MoE: [L, E, Fe, d]                    */
  const void *e_up;       /* MoE: [L, E, Fe, d]                    */
  const void *e_down;     /* MoE: [L, E, d, Fe]                    */
  void *k_cache;          /* [L, B, G, max_seq, Dh], written at pos */
  void *v_cache;          /* [L, B, G, max_seq, Dh], written at pos */
} mk_weights;

/* Plan options.  Zero means "default" for every field. */
typedef struct {
  int32_t n_cus;      /* workgroups = CUs used (default: all CUs of the device) */
  int32_t mlp_chunks; /* MLP intermediate split into this many chunks, each with
                         staged on its own so down-projection tiles start early
                         (the Llama-1B megakernel write-up, "Custom
                         Synchronization Mechanism", uses 4).  Default: the
                         fewest chunks of at most 4096 values each, since
                         every chunk adds two instructions per CU */
  int32_t attn_block; /* KV positions per attention tile (a multiple of 8 for
                         the one-sequence decoder, of 64 for the MoE decoder;
                         default: chosen from max_seq and the CU count) */
  int32_t watchdog_ms;/* limit of any one wait on the device (a counter, a
                         step-tagged input, an LDS page or barrier) before
                         the step ends in MK_ERR_TIMEOUT (default 2000) */
  int32_t debug_corrupt_target; /* tests only: 1 makes one instruction wait for
                                   a counter target and an input tag that the
                                   step never reaches, so the step must end in
                                   MK_ERR_TIMEOUT */
  int32_t generic_kernel; /* 1: always launch the kernel built for every shape
                             (default 0: the kernel built for this shape when
                             the library has one; see kernel_variant) */
  int32_t attn_heads; /* query heads per attention tile, dividing the heads per
                         KV group (default: 1 while n_q_heads * position
                         blocks <= n_cus, else the whole group; the MoE
                         decoder: the whole group) */
  int32_t o_split;    /* the O projection: 1 = split-K per KV group, each
                         tile waiting only for its own group's attention and
                         the last tile of a row block adding the residual
                         and the group partials in group order (the Cohere
                         kernel's removal of the attention -> O false
                         dependency, airebao.com «快在哪里» item 2); -1 = whole
                         rows after the whole attention stage (default;
                         the MoE decoder always).  The split needs more than
                         one KV group and heads-per-group * head_dim of 256
                         or a multiple of 512 */
  int32_t mfma;       /* batched decoder: 1 = the LM head on matrix cores
                         (v_mfma_f32_16x16x32_bf16 tiles of 16 rows; the fp32
                         input split into bf16 high and low parts, fp32
                         accumulation), run by a kernel variant of its own
                         (default); -1 = on the vector ALUs.  Batch 1:
                         always -1 */
  int32_t edn_queue;  /* MoE decoder: q > 1 = a 1/q share of each layer's
                         expert down-projection units waits in a ready queue
                         (chunks handed out at run time, each to whichever CU
                         asks first: Cohere's «快在哪里» item 1), the rest split
                         evenly over the CUs; 1 = every unit in the queue;
                         -1 = every unit split evenly.  Default: 2 */
  int32_t egu_balance; /* MoE decoder with gate/up rows of at most 4 KiB:
                          1 = each CU takes a share of the layer's (expert,
                          row) gate/up items sized so that its attention
                          and router tiles plus its share take about the
                          same time on every CU; -1 = an even slice of
                          every selected expert's rows per CU (default) */
  int32_t gu_all;     /* one-sequence decoder with mlp_chunks > 1: 1 = each
                         CU's gate/up pairs of every MLP chunk in one
                         instruction, chunk by chunk (all chunks read the
                         same input, and the per-element step tags still let
                         a down-projection chunk start once its own chunk is
                         written: the early start of the write-up's chunk
                         counters, "Custom Synchronization Mechanism",
                         without one staging per chunk); -1 = one gate/up
                         instruction per chunk.  Default: 1 from four
                         chunks on, else -1.  The MoE decoder: unused */
} mk_plan_opts;

/* Plan summary (filled by mk_plan_info / mk_plan_check). */
typedef struct {
  int32_t n_cus;           /* workgroups in the launch                    */
  int32_t n_instr;         /* instructions over all queues                */
  int32_t max_queue;       /* longest per-CU queue                        */
  int32_t n_counters;      /* counters in use                             */
  int32_t lds_bytes;       /* LDS per workgroup                           */
  int32_t n_pages;         /* LDS weight pages per workgroup              */
  int32_t page_bytes;      /* bytes per page                              */
  int32_t attn_block;      /* KV positions per attention tile             */
  int32_t attn_tiles;      /* attention tiles per layer                   */
  int32_t mlp_chunks;
  int64_t weight_bytes;    /* weight bytes streamed per step (MoE: the
                              part that does not depend on the routing;
                              each selected expert adds 6 * d * Fe bytes
                              per layer)                                  */
  int64_t max_cu_bytes;    /* largest per-CU streamed bytes (KV at max_seq)*/
  int64_t min_cu_bytes;    /* smallest per-CU streamed bytes              */
  int32_t kernel_variant;  /* 0: the generic kernel; > 0: the kernel built
                              for this shape (the Llama-3.2-1B, Llama-3-8B
                              and small test decoder geometries; MoE: 1 for
                              4 query heads per group of head_dim 128)   */
  int32_t scratch_bytes;   /* device scratch one step of this plan uses in
                              mk_decode_step_noalloc (must not exceed
                              MK_NOALLOC_SCRATCH_BYTES)                   */
} mk_plan_summary;

/* Create a context on `device` for this model and these caller-owned buffers.
 * Source: the pages define no programming interface.  This call sets up the
 * resident decode of Cohere's write-up (airebao.com, «Megakernel 是什么»: one
 * persistent kernel per step over state the host prepared) for one model; the
 * model is the Llama-style decoder of the Llama-1B megakernel write-up
 * (rocketrecap.com summary, "Megakernel: The Core Solution").
 * Validates the shape, allocates the arena and builds the RoPE tables.
 * Errors: MK_ERR_INVALID_ARG (NULL/inconsistent arguments), MK_ERR_UNSUPPORTED
 * (shape outside the kernel's code paths), MK_ERR_HIP, MK_ERR_OOM. */
mk_status mk_create(const mk_config *cfg, const mk_weights *w, int device, mk_ctx **out);

/* Build, verify and upload the per-CU instruction queues (host-side static
 * scheduling: the Llama-1B write-up, javascript.cn article, section
 * "Megakernel：从零设计的融合思路").  opts may be NULL (all defaults).  A plan
 * that fails the verifier (counter targets, dependency order, page budgets,
 * read coverage) is rejected with MK_ERR_INVALID_ARG. */
mk_status mk_build_plan(mk_ctx *ctx, const mk_plan_opts *opts);

/* Enqueue one decode step on `stream` (a hipStream_t; NULL = default stream).
 * Source: the whole forward pass of one token as one kernel launch (the
 * javascript.cn article, "Megakernel：从零设计的融合思路"; airebao.com,
 * «Megakernel 是什么»); the pages define no signature.
 *   d_tokens: device int32 [B], the input token of each sequence;
 *   pos:      position of the new token (= cached positions), 0 <= pos < max_seq;
 *   d_next:   device int32 [B], receives the greedy next token;
 *   d_logits: device float [B, V] or NULL.
 * Every sequence of a batch is at the same position.
 * Appends the new key/value rows at `pos` to the caller's caches.  Asynchronous:
 * a watchdog timeout or device error surfaces from mk_sync (or the next call).
 * d_tokens may alias d_next of the previous step (device-side chaining).
 * The kernel is one workgroup per CU.  It is launched plainly: a workgroup
 * fills a CU's LDS and the grid is at most the device's CU count, so every
 * workgroup becomes resident once its CU is free of other work, and every
 * wait inside is bounded by the watchdog.  With MK_COOP=1 in the environment
 * at mk_create, the launch is cooperative instead (the runtime then checks
 * residency before the launch, at about 16 us more per step).
 * Errors: MK_ERR_NO_PLAN, MK_ERR_INVALID_ARG, MK_ERR_HIP. */
mk_status mk_decode_step(mk_ctx *ctx, const int32_t *d_tokens, int32_t pos,
                         int32_t *d_next, float *d_logits, void *stream);

/* Enqueue n_steps greedy decode steps in ONE launch (the resident decode of
 * the Llama-1B write-up's future work and of Cohere's kernel: the step
 * boundary is one more dependency inside the running kernel instead of a
 * kernel launch, whose gap the javascript.cn article, «传统推理方式效率低下的原因»,
 * and the rocketrecap.com summary, "Memory Pipeline Bubbles Explained", price
 * at 1.3-2.1 us even with CUDA Graphs).
 *   d_tokens: device int32 [B], the input tokens of the first step;
 *   pos:      position of the first step; steps run at pos .. pos+n_steps-1,
 *             which must lie in [0, max_seq);
 *   d_next:   device int32 [n_steps][B], receives every step's greedy token
 *             (step s > 0 takes step s-1's token as its input, on the device);
 *   d_logits: device float [n_steps][B][V] or NULL.
 * Results are those of n_steps mk_decode_step calls chained on the device.
 * The dense decoder runs the steps inside one kernel: its loader waves stream
 * the next step's weights while the current step finishes, the argmax's last
 * arriver publishes the token with its step's tag, and the next step's first
 * stage polls for it.  The mixture-of-experts decoder runs one launch per step
 * on `stream`.  Errors: as mk_decode_step, and MK_ERR_INVALID_ARG for
 * n_steps < 1 or pos + n_steps > max_seq. */
mk_status mk_decode_steps(mk_ctx *ctx, const int32_t *d_tokens, int32_t pos, int32_t n_steps,
                          int32_t *d_next, float *d_logits, void *stream);

/* Bytes of the fixed per-device scratch array of mk_decode_step_noalloc. */
#define MK_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)

/* mk_decode_step without any device allocation, for callers that cannot
 * allocate while they decode: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, kernels and results
 * as mk_decode_step.  The step's scratch (tagged activations, counters, argmax
 * slots, status word; mk_plan_summary.scratch_bytes of it) lives in a fixed
 * file-scope device array of MK_NOALLOC_SCRATCH_BYTES bytes, one per GPU,
 * held until the process ends, instead of the context's arena.  Each call
 * first clears the part it uses (a fill kernel on `stream`), then runs the
 * step, so a call does not depend on what an earlier call (of any context)
 * left there.  All contexts on one GPU share the array: calls that overlap
 * on one GPU (other streams, other threads) race and must not be issued.
 * Allocates nothing and calls no allocating routine; the plan (built by
 * mk_build_plan, which does allocate) is reused.  Errors and the device
 * status word surface from mk_sync as for mk_decode_step.
 * Errors: MK_ERR_NO_PLAN, MK_ERR_INVALID_ARG (as mk_decode_step),
 * MK_ERR_UNSUPPORTED (the plan needs more scratch than
 * MK_NOALLOC_SCRATCH_BYTES), MK_ERR_HIP. */
mk_status mk_decode_step_noalloc(mk_ctx *ctx, const int32_t *d_tokens, int32_t pos,
                                 int32_t *d_next, float *d_logits, void *stream);

/* Wait for the context's last step and read the device status word.
 * Source: none on the pages (they define no interface); the status word
 * reports the bounded waits of the counter system (rocketrecap.com summary,
 * "Custom Synchronization Mechanism") that ran out.
 * Returns MK_ERR_TIMEOUT / MK_ERR_DEVICE with a message if the kernel reported
 * one; the counters are then reset so the context can be used again. */
mk_status mk_sync(mk_ctx *ctx);

/* Destroy the context and free the arena.  NULL is accepted (MK_OK).
 * Source: none on the pages (they define no interface); the counterpart of
 * mk_create. */
mk_status mk_destroy(mk_ctx *ctx);

/* Message for the last error on ctx (or of the calling thread if ctx is NULL).
 * The string is owned by the library and valid until the next call.
 * Source: none on the pages (they define no interface); error reporting of
 * this C boundary. */
const char *mk_last_error(const mk_ctx *ctx);

/* Routing statistics of the mixture-of-experts decoder (Cohere's write-up,
 * airebao.com, «为什么值得做»: each step streams only the selected experts'
 * weights; this counts them so that a caller can price the step in bytes).
 * per_layer[l] receives
 * the number of distinct experts the router selected in layer l (union over
 * the batch), summed over the steps since the last reset; each selected
 * expert streams 6 * hidden * expert_ffn weight bytes.  n >= n_layers.
 * Waits for the context's last step; reset != 0 zeroes the sums.  Dense
 * decoders report zeros.  Errors: MK_ERR_NO_PLAN, MK_ERR_INVALID_ARG,
 * MK_ERR_HIP. */
mk_status mk_route_stats(mk_ctx *ctx, int64_t *per_layer, int32_t n, int reset);

/* Summary of the context's current plan (the host-side static schedule of
 * the javascript.cn article, "Megakernel：从零设计的融合思路").
 * Errors: MK_ERR_NO_PLAN. */
mk_status mk_plan_info(const mk_ctx *ctx, mk_plan_summary *out);

/* Host-only planning for tests and tools (the same static schedule as
 * mk_build_plan, javascript.cn article, "Megakernel：从零设计的融合思路"):
 * build and verify a plan for
 * `n_cus` workgroups without a device or buffers.  Writes a text report
 * (truncated to report_len, may be NULL) and the summary (may be NULL). */
mk_status mk_plan_check(const mk_config *cfg, const mk_plan_opts *opts, int32_t n_cus,
                        mk_plan_summary *summary, char *report, size_t report_len);

/* ---- diagnostics -------------------------------------------------------
 * Source: the per-stage runtime breakdown of the Llama-1B write-up
 * (rocketrecap.com summary, "Detailed Runtime Breakdown") is what these
 * stamps reproduce for this kernel.
 * Per-instruction timestamps of the next steps (s_memrealtime, 100 MHz, low
 * 32 bits): for every CU and queue slot 16 words
 *   {start, deps satisfied, inputs staged, leader's items done, signal,
 *    leader's page-wait ticks, header word 0, header word 1,
 *    leader's input vector ready, leader's first item done, leader's stores
 *    visible, previous inputs released, then for attention the ends of the
 *    score pass, the softmax statistics and the value pass, the leader's
 *    re-reads of inputs whose step tag was not yet current}.
 * For attention instructions words 8 and 9 are the end of the query
 * preparation and of the leader's own score work.
 * mk_trace_enable allocates (on != 0) or frees the trace buffer; it costs a
 * few stores per instruction.  mk_trace_read copies it to host memory
 * (n_words >= n_cus * stride * 16) after mk_sync; *stride receives the slots
 * per CU.  Errors: MK_ERR_NO_PLAN, MK_ERR_INVALID_ARG, MK_ERR_HIP. */
mk_status mk_trace_enable(mk_ctx *ctx, int on);

/* Calibration (the measurement plan of the Llama-1B write-up reports its step
 * against the memory system's rate; rocketrecap.com summary, "Performance
 * Metrics"): read `bytes` (a multiple of 16) of device memory at d_src
 * (16-byte aligned) once with 16-byte non-temporal loads over `blocks`
 * workgroups of 256 threads on `stream`, and store one fold word per block to
 * d_sink[blocks] (device memory, caller-owned).  Time it with events on the
 * stream to get the achievable streaming read rate.  Errors:
 * MK_ERR_INVALID_ARG, MK_ERR_HIP. */
mk_status mk_stream_read(const void *d_src, size_t bytes, uint32_t *d_sink, int32_t blocks, void *stream);
mk_status mk_trace_read(mk_ctx *ctx, uint32_t *host, size_t n_words, int32_t *stride);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
