// mk_runtime.cpp — the C ABI (include/mk.h) over the HIP host API: context,
// arena, RoPE tables, plan upload, launch, status readback.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "mk.h"
#include "mk_plan.h"

extern "C" hipError_t mk_launch_megakernel(const mk::KArgs* args, int n_cus, hipStream_t stream,
                                           int cooperative, int variant);
extern "C" int mk_pick_variant(int nd, int rd, int nq, int rq, int nf, int rf, int hpt, int dh, int os);
extern "C" hipError_t mk_launch_batched(const mk::KArgs* args, int n_cus, hipStream_t stream, int cooperative,
                                        int variant);
extern "C" int mk_pick_batched(int hpt, int dh, int mfma);
extern "C" hipError_t mk_launch_pack(const mk::PackCopy* copies, uint32_t n, void* base,
                                     hipStream_t stream);
extern "C" hipError_t mk_scratch_init(int device, void** out);
extern "C" hipError_t mk_launch_fill_zero(void* p, uint64_t bytes, hipStream_t stream);

struct mk_ctx {
  mk_config cfg;
  mk_weights w;
  int device = 0;
  int dev_cus = 0;
  std::string err;
  std::vector<float> rope_cos, rope_sin;
  // plan state
  bool planned = false;
  mk::PlanInput pin;
  mk::Plan plan;
  char* arena = nullptr;
  char* pack = nullptr;   // packed weight stream (library-owned copy)
  mk::Instr* d_instrs = nullptr;
  uint32_t* d_qoff = nullptr;
  uint32_t* d_counters = nullptr;
  uint32_t epoch = 0;
  hipStream_t last_stream = nullptr;
  bool has_step = false;
  int cooperative = 0;
  int variant = 0;        // kernel launched for the current plan
  uint32_t* d_trace = nullptr;
  uint32_t trace_stride = 0;
  // mk_decode_step_noalloc: this device's fixed scratch array, its layout for
  // the current plan and the plan's instructions rebased into it (null when
  // the plan needs more than MK_NOALLOC_SCRATCH_BYTES)
  void* scratch = nullptr;
  mk::ScratchLayout sc{};
  mk::Instr* d_instrs_static = nullptr;
  bool last_static = false;   // the last step ran on the scratch array
};

namespace {
thread_local std::string g_err;

mk_status fail(mk_ctx* c, mk_status st, const std::string& m) {
  if (c) c->err = m;
  g_err = m;
  return st;
}
mk_status hip_fail(mk_ctx* c, hipError_t e, const char* what) {
  return fail(c, e == hipErrorOutOfMemory ? MK_ERR_OOM : MK_ERR_HIP,
              std::string(what) + ": " + hipGetErrorString(e));
}

void free_trace(mk_ctx* c) {
  if (c->d_trace) (void)hipFree(c->d_trace);
  c->d_trace = nullptr;
  c->trace_stride = 0;
}

void free_plan(mk_ctx* c) {
  free_trace(c);
  if (c->arena) (void)hipFree(c->arena);
  if (c->pack) (void)hipFree(c->pack);
  c->pack = nullptr;
  if (c->d_instrs) (void)hipFree(c->d_instrs);
  if (c->d_qoff) (void)hipFree(c->d_qoff);
  if (c->d_counters) (void)hipFree(c->d_counters);
  if (c->d_instrs_static) (void)hipFree(c->d_instrs_static);
  c->d_instrs_static = nullptr;
  c->arena = nullptr;
  c->d_instrs = nullptr;
  c->d_qoff = nullptr;
  c->d_counters = nullptr;
  c->planned = false;
}

// RoPE tables: angle p * theta^(-2j/Dh) in double precision, stored as float.
void rope_tables(const mk_config& cfg, std::vector<float>* cs, std::vector<float>* sn) {
  const int half = cfg.head_dim / 2;
  cs->resize(size_t(cfg.max_seq) * half);
  sn->resize(size_t(cfg.max_seq) * half);
  for (int j = 0; j < half; j++) {
    const double inv = std::pow(double(cfg.rope_theta), -2.0 * j / cfg.head_dim);
    for (int p = 0; p < cfg.max_seq; p++) {
      const double ang = double(p) * inv;
      (*cs)[size_t(p) * half + j] = float(std::cos(ang));
      (*sn)[size_t(p) * half + j] = float(std::sin(ang));
    }
  }
}

// The shape-specific kernel for this plan, or 0 (the generic kernel).
int variant_for(const mk_config& cfg, const mk_plan_opts& o) {
  if (mk::is_batched(cfg)) return o.generic_kernel ? 0 : mk_pick_batched(o.attn_heads, cfg.head_dim, o.mfma > 0);
  if (o.generic_kernel) return 0;
  int nd, rd, nq, rq, nf, rf;
  // the O projection's input: the whole attention output, or one KV group's
  const int oq = o.o_split > 0 ? cfg.n_q_heads / cfg.n_kv_heads * cfg.head_dim : cfg.n_q_heads * cfg.head_dim;
  if (!mk::gemv_geometry(cfg.hidden, &nd, &rd) ||
      !mk::gemv_geometry(oq, &nq, &rq) ||
      !mk::gemv_geometry(cfg.ffn / o.mlp_chunks, &nf, &rf))
    return 0;
  return mk_pick_variant(nd, rd, nq, rq, nf, rf, o.attn_heads, cfg.head_dim, o.o_split > 0);
}

bool dense_pointers_ok(const mk_weights& w) {
  return w.embed && w.final_norm && w.attn_norm && w.wq && w.wk && w.wv && w.wo && w.mlp_norm &&
         w.w_gate && w.w_up && w.w_down && w.k_cache && w.v_cache;
}
bool moe_pointers_ok(const mk_weights& w) {
  return w.embed && w.final_norm && w.attn_norm && w.wq && w.wk && w.wv && w.wo && w.router && w.e_gate &&
         w.e_up && w.e_down && w.k_cache && w.v_cache;
}
}  // namespace

extern "C" {

mk_status mk_create(const mk_config* cfg, const mk_weights* w, int device, mk_ctx** out) {
  if (!out) return fail(nullptr, MK_ERR_INVALID_ARG, "mk_create: out is NULL");
  *out = nullptr;
  if (!cfg || !w) return fail(nullptr, MK_ERR_INVALID_ARG, "mk_create: cfg and w are required");
  std::string err;
  mk_status st = mk::check_config(*cfg, &err);
  if (st != MK_OK) return fail(nullptr, st, err);
  if (!(mk::is_batched(*cfg) ? moe_pointers_ok(*w) : dense_pointers_ok(*w)))
    return fail(nullptr, MK_ERR_INVALID_ARG, "mk_create: a weight or cache pointer is NULL");
  if (!w->lm_head && !cfg->tied_embedding)
    return fail(nullptr, MK_ERR_INVALID_ARG, "mk_create: lm_head is NULL and the embedding is not tied");
  int n_dev = 0;
  hipError_t e = hipGetDeviceCount(&n_dev);
  if (e != hipSuccess || n_dev <= 0) return fail(nullptr, MK_ERR_HIP, "mk_create: no HIP device");
  if (device < 0 || device >= n_dev) return fail(nullptr, MK_ERR_INVALID_ARG, "mk_create: bad device index");
  if ((e = hipSetDevice(device)) != hipSuccess) return hip_fail(nullptr, e, "hipSetDevice");
  hipDeviceProp_t prop;
  if ((e = hipGetDeviceProperties(&prop, device)) != hipSuccess) return hip_fail(nullptr, e, "hipGetDeviceProperties");
  if (size_t(prop.maxSharedMemoryPerMultiProcessor) < size_t(mk::is_batched(*cfg) ? mk::lb::kTotal : mk::kLdsTotal))
    return fail(nullptr, MK_ERR_UNSUPPORTED, "mk_create: device has too little LDS per CU");
  const void* aligned[] = {w->embed, w->lm_head, w->wq, w->wk, w->wv, w->wo, w->w_gate, w->w_up,
                           w->w_down, w->k_cache, w->v_cache, w->router, w->e_gate, w->e_up, w->e_down};
  for (const void* ptr : aligned)
    if (uintptr_t(ptr) % 16)
      return fail(nullptr, MK_ERR_INVALID_ARG, "mk_create: weight and cache pointers must be 16-byte aligned");
  // the no-allocation entry point's scratch array on this device (looked up
  // once per device, with the device current)
  void* scratch = nullptr;
  if ((e = mk_scratch_init(device, &scratch)) != hipSuccess) return hip_fail(nullptr, e, "mk_create: scratch array");
  mk_ctx* c = new mk_ctx();
  c->scratch = scratch;
  c->cfg = *cfg;
  c->w = *w;
  if (!c->w.lm_head) c->w.lm_head = c->w.embed;
  c->device = device;
  c->dev_cus = prop.multiProcessorCount;
  // plain launch unless MK_COOP=1 (see mk_decode_step in mk.h)
  const char* co = std::getenv("MK_COOP");
  c->cooperative = (co && co[0] == '1') ? 1 : 0;

  rope_tables(c->cfg, &c->rope_cos, &c->rope_sin);
  *out = c;
  return MK_OK;
}

mk_status mk_build_plan(mk_ctx* c, const mk_plan_opts* opts) {
  if (!c) return fail(nullptr, MK_ERR_INVALID_ARG, "mk_build_plan: ctx is NULL");
  hipError_t e = hipSetDevice(c->device);
  if (e != hipSuccess) return hip_fail(c, e, "hipSetDevice");
  if (c->has_step) (void)hipStreamSynchronize(c->last_stream);
  free_plan(c);
  int n_cus = (opts && opts->n_cus > 0) ? opts->n_cus : c->dev_cus;
  if (n_cus > c->dev_cus) return fail(c, MK_ERR_INVALID_ARG, "mk_build_plan: n_cus exceeds the device's CUs");
  mk::PlanInput& in = c->pin;
  in.cfg = c->cfg;
  in.opts = mk::resolve_opts(c->cfg, opts, n_cus);
  in.n_cus = n_cus;
  in.w = c->w;
  // (the one-sequence plan takes multiples of 8, the batched plan of 64)
  if (in.opts.attn_block <= 0 || in.opts.attn_block % 8)
    return fail(c, MK_ERR_INVALID_ARG, "mk_build_plan: attn_block must be a positive multiple of 8");
  if (mk::is_batched(c->cfg) && in.opts.generic_kernel)
    return fail(c, MK_ERR_UNSUPPORTED, "mk_build_plan: the batched decoder has no generic-kernel option");
  const int nblk = (c->cfg.max_seq + in.opts.attn_block - 1) / in.opts.attn_block;
  const mk::ArenaLayout lay = mk::arena_layout(c->cfg, n_cus, c->cfg.batch * c->cfg.n_kv_heads * nblk);
  if ((e = hipMalloc(&c->arena, lay.total)) != hipSuccess) return hip_fail(c, e, "hipMalloc(arena)");
  in.arena_base = uint64_t(c->arena);
  in.pack_base = 0;
  std::string err;
  c->plan = mk::Plan();
  mk_status st = mk::build_plan(in, &c->plan, &err);
  if (st == MK_OK) {
    if ((e = hipMalloc(&c->pack, std::max<uint64_t>(c->plan.pack_bytes, 16))) != hipSuccess) {
      free_plan(c);
      return hip_fail(c, e, "hipMalloc(packed weights)");
    }
    mk::rebase_pack(&c->plan, 0, uint64_t(c->pack));
    in.pack_base = uint64_t(c->pack);
    st = mk::verify_plan(in, c->plan, &err);
  }
  if (st != MK_OK) {
    free_plan(c);
    return fail(c, st, err);
  }
  if (in.opts.debug_corrupt_target) mk::corrupt_one_target(&c->plan);
  const mk::Plan& p = c->plan;
  (void)hipMemset(c->arena, 0, lay.total);
  e = hipMemcpy(c->arena + p.arena.rope_cos, c->rope_cos.data(), c->rope_cos.size() * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess)
    e = hipMemcpy(c->arena + p.arena.rope_sin, c->rope_sin.data(), c->rope_sin.size() * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMalloc(&c->d_instrs, std::max<size_t>(1, p.instrs.size()) * sizeof(mk::Instr));
  if (e == hipSuccess)
    e = hipMemcpy(c->d_instrs, p.instrs.data(), p.instrs.size() * sizeof(mk::Instr), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMalloc(&c->d_qoff, p.q_off.size() * 4);
  if (e == hipSuccess) e = hipMemcpy(c->d_qoff, p.q_off.data(), p.q_off.size() * 4, hipMemcpyHostToDevice);
  // fill the packed weight stream (zero padding, then the rows)
  mk::PackCopy* d_copies = nullptr;
  if (e == hipSuccess) e = hipMemset(c->pack, 0, p.pack_bytes);
  if (e == hipSuccess && !p.pack.empty()) {
    e = hipMalloc(&d_copies, p.pack.size() * sizeof(mk::PackCopy));
    if (e == hipSuccess)
      e = hipMemcpy(d_copies, p.pack.data(), p.pack.size() * sizeof(mk::PackCopy), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = mk_launch_pack(d_copies, uint32_t(p.pack.size()), c->pack, nullptr);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (d_copies) (void)hipFree(d_copies);
  }
  const size_t ctr_bytes = size_t(std::max(1, p.n_counters)) * mk::kCtrSpread * mk::kCtrStride * 4;
  if (e == hipSuccess) e = hipMalloc(&c->d_counters, ctr_bytes);
  if (e == hipSuccess) e = hipMemset(c->d_counters, 0, ctr_bytes);
  // the same instructions with the activations in the scratch array
  c->sc = mk::scratch_layout(p);
  if (e == hipSuccess && c->sc.total <= MK_NOALLOC_SCRATCH_BYTES) {
    const std::vector<mk::Instr> st = mk::rebase_to_scratch(p, uint64_t(c->arena), uint64_t(c->scratch));
    e = hipMalloc(&c->d_instrs_static, std::max<size_t>(1, st.size()) * sizeof(mk::Instr));
    if (e == hipSuccess)
      e = hipMemcpy(c->d_instrs_static, st.data(), st.size() * sizeof(mk::Instr), hipMemcpyHostToDevice);
  }
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    free_plan(c);
    return hip_fail(c, e, "mk_build_plan upload");
  }
  c->epoch = 0;
  c->variant = variant_for(c->cfg, in.opts);
  c->planned = true;
  return MK_OK;
}

}  // extern "C"

namespace {
// Shared by both decode entry points: validate, fill the launch arguments and
// launch.  `noalloc` puts every scratch buffer in the fixed array (cleared
// first) and runs the step as step 1 of that scratch.
mk_status decode_launch(mk_ctx* c, const int32_t* d_tokens, int32_t pos, int32_t* d_next, float* d_logits,
                        void* stream, bool noalloc, const char* who, int32_t n_steps = 1) {
  if (!c) return fail(nullptr, MK_ERR_INVALID_ARG, std::string(who) + ": ctx is NULL");
  if (!c->planned) return fail(c, MK_ERR_NO_PLAN, std::string(who) + ": call mk_build_plan first");
  if (!d_tokens || !d_next) return fail(c, MK_ERR_INVALID_ARG, std::string(who) + ": tokens and next are required");
  if (pos < 0 || pos >= c->cfg.max_seq)
    return fail(c, MK_ERR_INVALID_ARG, std::string(who) + ": pos outside [0, max_seq)");
  if (n_steps < 1 || int64_t(pos) + n_steps > c->cfg.max_seq)
    return fail(c, MK_ERR_INVALID_ARG, std::string(who) + ": n_steps < 1 or pos + n_steps > max_seq");
  if (noalloc && !c->d_instrs_static) {
    char msg[200];
    std::snprintf(msg, sizeof(msg), "%s: the plan needs %llu bytes of scratch, above the %u-byte limit", who,
                  (unsigned long long)c->sc.total, MK_NOALLOC_SCRATCH_BYTES);
    return fail(c, MK_ERR_UNSUPPORTED, msg);
  }
  const mk::Plan& p = c->plan;
  char* sc = static_cast<char*>(c->scratch);
  mk::KArgs a;
  std::memset(&a, 0, sizeof(a));
  a.instrs = noalloc ? c->d_instrs_static : c->d_instrs;
  a.q_off = c->d_qoff;
  a.counters = noalloc ? reinterpret_cast<uint32_t*>(sc + c->sc.ctr) : c->d_counters;
  a.status = reinterpret_cast<uint32_t*>(noalloc ? sc + c->sc.status : c->arena + p.arena.status);
  a.tokens = d_tokens;
  a.next = d_next;
  a.logits = d_logits;
  a.rope_cos = reinterpret_cast<const float*>(c->arena + p.arena.rope_cos);
  a.rope_sin = reinterpret_cast<const float*>(c->arena + p.arena.rope_sin);
  a.lm_slots = reinterpret_cast<float*>(noalloc ? sc + c->sc.slots : c->arena + p.arena.lm_slots);
  a.zero_page = c->arena + p.arena.zero_page;
  a.epoch = noalloc ? 1 : c->epoch + 1;
  a.pos = pos;
  a.vocab = c->cfg.vocab;
  a.hidden = c->cfg.hidden;
  a.head_dim = c->cfg.head_dim;
  a.hpg = c->cfg.n_q_heads / c->cfg.n_kv_heads;
  a.q_dim = c->cfg.n_q_heads * c->cfg.head_dim;
  a.kv_dim = c->cfg.n_kv_heads * c->cfg.head_dim;
  a.max_seq = c->cfg.max_seq;
  a.rms_eps = c->cfg.rms_eps;
  a.attn_scale = float(1.0 / std::sqrt(double(c->cfg.head_dim)));
  a.watchdog_ticks = uint64_t(c->pin.opts.watchdog_ms) * 100000ull;
  a.trace = noalloc ? nullptr : c->d_trace;
  a.trace_stride = noalloc ? 0 : c->trace_stride;
  a.batch = c->cfg.batch;
  a.n_experts = c->cfg.n_experts;
  a.top_k = c->cfg.top_k;
  a.expert_ffn = c->cfg.expert_ffn;
  a.route_stats = reinterpret_cast<uint32_t*>(noalloc ? sc + c->sc.route : c->arena + p.arena.route_stats);
  a.tok_tag = reinterpret_cast<uint64_t*>((noalloc ? sc + c->sc.act : c->arena) + p.arena.tok);
  a.n_steps = uint32_t(n_steps);

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  // the scratch array keeps the last call's contents: clear the span this
  // plan uses (tags, counters, status) so the step starts from step 1
  if (noalloc) e = mk_launch_fill_zero(sc, c->sc.total, s);
  if (e == hipSuccess)
    e = p.batched ? mk_launch_batched(&a, p.n_cus, s, c->cooperative, c->variant)
                  : mk_launch_megakernel(&a, p.n_cus, s, c->cooperative, c->variant);
  if (e != hipSuccess) return hip_fail(c, e, "launch");
  if (!noalloc) c->epoch += uint32_t(n_steps);
  c->last_static = noalloc;
  c->last_stream = s;
  c->has_step = true;
  return MK_OK;
}
}  // namespace

extern "C" {

mk_status mk_decode_step(mk_ctx* c, const int32_t* d_tokens, int32_t pos, int32_t* d_next,
                         float* d_logits, void* stream) {
  return decode_launch(c, d_tokens, pos, d_next, d_logits, stream, false, "mk_decode_step");
}

mk_status mk_decode_step_noalloc(mk_ctx* c, const int32_t* d_tokens, int32_t pos, int32_t* d_next,
                                 float* d_logits, void* stream) {
  return decode_launch(c, d_tokens, pos, d_next, d_logits, stream, true, "mk_decode_step_noalloc");
}

mk_status mk_decode_steps(mk_ctx* c, const int32_t* d_tokens, int32_t pos, int32_t n_steps, int32_t* d_next,
                          float* d_logits, void* stream) {
  if (c && c->planned && c->plan.batched) {
    // the batched kernel runs one step per launch: chain the launches on
    // the stream, each step's input being the previous step's output
    if (n_steps < 1) return fail(c, MK_ERR_INVALID_ARG, "mk_decode_steps: n_steps < 1");
    const int32_t B = c->cfg.batch;
    for (int32_t s = 0; s < n_steps; s++) {
      const mk_status st = decode_launch(c, s ? d_next + size_t(s - 1) * B : d_tokens, pos + s, d_next + size_t(s) * B,
                                         d_logits ? d_logits + size_t(s) * B * c->cfg.vocab : nullptr, stream,
                                         false, "mk_decode_steps");
      if (st != MK_OK) return st;
    }
    return MK_OK;
  }
  return decode_launch(c, d_tokens, pos, d_next, d_logits, stream, false, "mk_decode_steps", n_steps);
}

mk_status mk_sync(mk_ctx* c) {
  if (!c) return fail(nullptr, MK_ERR_INVALID_ARG, "mk_sync: ctx is NULL");
  if (!c->planned || !c->has_step) return MK_OK;
  hipError_t e = hipStreamSynchronize(c->last_stream);
  if (e != hipSuccess) return hip_fail(c, e, "hipStreamSynchronize");
  uint32_t stw[8];
  const char* st_src = c->last_static ? static_cast<const char*>(c->scratch) + c->sc.status
                                      : c->arena + c->plan.arena.status;
  e = hipMemcpy(stw, st_src, sizeof(stw), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(c, e, "status readback");
  if (stw[mk::ST_CODE] == 0 && stw[mk::ST_NAN] == 0 && stw[mk::ST_BADTOK] == 0) return MK_OK;
  char msg[256];
  mk_status st;
  if (stw[mk::ST_CODE] == mk::STC_TIMEOUT) {
    std::snprintf(msg, sizeof(msg),
                  "watchdog: CU %u instruction %u waited on counter %u (seen %u, target %u)",
                  stw[mk::ST_CU], stw[mk::ST_INSTR], stw[mk::ST_CTR], stw[mk::ST_SEEN], stw[mk::ST_TARGET]);
    st = MK_ERR_TIMEOUT;
  } else if (stw[mk::ST_CODE] == mk::STC_LOCAL_TIMEOUT) {
    std::snprintf(msg, sizeof(msg), "watchdog: workgroup %u stalled on its own LDS pages or barrier", stw[mk::ST_CU]);
    st = MK_ERR_TIMEOUT;
  } else if (stw[mk::ST_CODE] == mk::STC_TAG_TIMEOUT) {
    std::snprintf(msg, sizeof(msg), "watchdog: workgroup %u waited on inputs this step never wrote", stw[mk::ST_CU]);
    st = MK_ERR_TIMEOUT;
  } else if (stw[mk::ST_BADTOK]) {
    std::snprintf(msg, sizeof(msg), "device: input token outside [0, vocab)");
    st = MK_ERR_DEVICE;
  } else {
    std::snprintf(msg, sizeof(msg), "device: NaN logits in the LM head");
    st = MK_ERR_DEVICE;
  }
  // reset so the context can be used again: counters, status and the
  // activation tags (the step count restarts at 1)
  const size_t ctr_bytes = size_t(std::max(1, c->plan.n_counters)) * mk::kCtrSpread * mk::kCtrStride * 4;
  (void)hipMemset(c->d_counters, 0, ctr_bytes);
  (void)hipMemset(c->arena, 0, c->plan.arena.rope_cos);
  (void)hipMemset(c->arena + c->plan.arena.status, 0, 64);
  (void)hipDeviceSynchronize();
  c->epoch = 0;
  return fail(c, st, msg);
}

mk_status mk_destroy(mk_ctx* c) {
  if (!c) return MK_OK;
  (void)hipSetDevice(c->device);
  if (c->has_step) (void)hipStreamSynchronize(c->last_stream);
  free_plan(c);
  delete c;
  return MK_OK;
}

mk_status mk_trace_enable(mk_ctx* c, int on) {
  if (!c) return fail(nullptr, MK_ERR_INVALID_ARG, "mk_trace_enable: ctx is NULL");
  if (!c->planned) return fail(c, MK_ERR_NO_PLAN, "mk_trace_enable: no plan");
  if (c->has_step) (void)hipStreamSynchronize(c->last_stream);
  free_trace(c);
  if (!on) return MK_OK;
  uint32_t mq = 0;
  for (int cu = 0; cu < c->plan.n_cus; cu++) mq = std::max(mq, c->plan.q_off[cu + 1] - c->plan.q_off[cu]);
  const size_t bytes = size_t(c->plan.n_cus) * mq * mk::TR_WORDS * 4;
  hipError_t e = hipMalloc(&c->d_trace, std::max<size_t>(bytes, 4));
  if (e == hipSuccess) e = hipMemset(c->d_trace, 0, std::max<size_t>(bytes, 4));
  if (e != hipSuccess) {
    c->d_trace = nullptr;
    return hip_fail(c, e, "trace buffer");
  }
  c->trace_stride = mq;
  return MK_OK;
}

mk_status mk_trace_read(mk_ctx* c, uint32_t* host, size_t n_words, int32_t* stride) {
  if (!c || !host || !stride) return fail(c, MK_ERR_INVALID_ARG, "mk_trace_read: NULL argument");
  if (!c->d_trace) return fail(c, MK_ERR_NO_PLAN, "mk_trace_read: tracing is off");
  const size_t need = size_t(c->plan.n_cus) * c->trace_stride * mk::TR_WORDS;
  if (n_words < need) return fail(c, MK_ERR_INVALID_ARG, "mk_trace_read: buffer too small");
  hipError_t e = hipMemcpy(host, c->d_trace, need * 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(c, e, "trace readback");
  *stride = int32_t(c->trace_stride);
  return MK_OK;
}

const char* mk_last_error(const mk_ctx* c) { return c ? c->err.c_str() : g_err.c_str(); }

mk_status mk_route_stats(mk_ctx* c, int64_t* per_layer, int32_t n, int reset) {
  if (!c || !per_layer || n < 0) return fail(c, MK_ERR_INVALID_ARG, "mk_route_stats: NULL argument");
  if (!c->planned) return fail(c, MK_ERR_NO_PLAN, "mk_route_stats: no plan");
  if (n < c->cfg.n_layers) return fail(c, MK_ERR_INVALID_ARG, "mk_route_stats: buffer shorter than n_layers");
  if (c->has_step) {
    hipError_t e = hipStreamSynchronize(c->last_stream);
    if (e != hipSuccess) return hip_fail(c, e, "hipStreamSynchronize");
  }
  uint32_t v[128];
  const size_t L = size_t(c->cfg.n_layers);
  hipError_t e = hipMemcpy(v, c->arena + c->plan.arena.route_stats, 4 * L, hipMemcpyDeviceToHost);
  if (e == hipSuccess && reset) e = hipMemset(c->arena + c->plan.arena.route_stats, 0, 4 * L);
  if (e != hipSuccess) return hip_fail(c, e, "route statistics readback");
  for (size_t l = 0; l < L; l++) per_layer[l] = c->cfg.n_experts > 0 ? int64_t(v[l]) : 0;
  return MK_OK;
}

mk_status mk_plan_info(const mk_ctx* c, mk_plan_summary* out) {
  if (!c || !out) return fail(nullptr, MK_ERR_INVALID_ARG, "mk_plan_info: NULL argument");
  if (!c->planned) return fail(const_cast<mk_ctx*>(c), MK_ERR_NO_PLAN, "mk_plan_info: no plan");
  mk::summarize(c->pin, c->plan, out);
  out->kernel_variant = c->variant;
  return MK_OK;
}

mk_status mk_plan_check(const mk_config* cfg, const mk_plan_opts* opts, int32_t n_cus,
                        mk_plan_summary* summary, char* report, size_t report_len) {
  if (!cfg) return fail(nullptr, MK_ERR_INVALID_ARG, "mk_plan_check: cfg is NULL");
  if (n_cus <= 0) return fail(nullptr, MK_ERR_INVALID_ARG, "mk_plan_check: n_cus must be positive");
  std::string err;
  mk_status st = mk::check_config(*cfg, &err);
  if (st != MK_OK) return fail(nullptr, st, err);
  mk::PlanInput in;
  in.cfg = *cfg;
  in.opts = mk::resolve_opts(*cfg, opts, n_cus);
  in.n_cus = n_cus;
  // distinct fake device addresses: only the structure is checked
  uintptr_t base = uintptr_t(1) << 40;
  const void** fields[] = {&in.w.embed, &in.w.lm_head, &in.w.final_norm, &in.w.attn_norm, &in.w.wq,
                           &in.w.wk, &in.w.wv, &in.w.wo, &in.w.mlp_norm, &in.w.w_gate, &in.w.w_up,
                           &in.w.w_down, &in.w.router, &in.w.e_gate, &in.w.e_up, &in.w.e_down};
  for (size_t i = 0; i < sizeof(fields) / sizeof(fields[0]); i++)
    *fields[i] = reinterpret_cast<const void*>(base * (i + 1));
  in.w.k_cache = reinterpret_cast<void*>(base * 20);
  in.w.v_cache = reinterpret_cast<void*>(base * 21);
  in.arena_base = uint64_t(base) * 30;
  in.pack_base = uint64_t(base) * 31;
  mk::Plan p;
  st = mk::build_plan(in, &p, &err);
  if (st == MK_OK && in.opts.debug_corrupt_target) mk::corrupt_one_target(&p);
  if (st == MK_OK) st = mk::verify_plan(in, p, &err);
  if (st != MK_OK) return fail(nullptr, st, err);
  if (summary) {
    mk::summarize(in, p, summary);
    summary->kernel_variant = variant_for(*cfg, in.opts);
  }
  if (report && report_len) {
    std::string r = mk::plan_report(in, p);
    std::snprintf(report, report_len, "%s", r.c_str());
  }
  return MK_OK;
}

}  // extern "C"
