// mk_plan.cpp — host planner and plan verifier (pure C++).
//
// Stages per layer (each cut into tiles, one tile per CU where possible):
//   QKV   rows of [Wq; Wk; Wv] . RMSNorm(x_l)               -> qkv_l
//   ATTN  per KV group (and position block): RoPE, KV append, GQA attention
//   O     rows of Wo . o_l + x_l                            -> h_l
//   GU c  pairs of (gate, up) rows of MLP chunk c, SwiGLU    -> m_l[chunk c]
//   DOWN  rows of Wd, one instruction per chunk, accumulated -> x_{l+1}
// then the LM head with a tile argmax and a last-arriver reduction.
//
// The MLP intermediate is split into chunks with their own counters so that
// down-projection tiles can start early (Llama-1B megakernel write-up,
// rocketrecap.com summary, "Custom Synchronization Mechanism": four chunks).
// Attention and its consumers are synchronised through counters in global
// memory (same section; Cohere's write-up, «Megakernel 是什么»).
#include "mk_plan.h"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <random>
#include <sstream>

namespace mk {
namespace {

enum Buf { BUF_EMBED = 0, BUF_X, BUF_QKV, BUF_O, BUF_H, BUF_M, BUF_LOGITS, BUF_RL, BUF_Y, BUF_COUNT };
const char* kBufName[] = {"embed", "x", "qkv", "o", "h", "m", "logits", "router", "y"};
enum LStage { ST_QKV = 0, ST_ATTN = 1, ST_O = 2, ST_GU = 3, ST_DOWN = 4, ST_DRED = 5, ST_PER_LAYER = 8 };

uint64_t align256(uint64_t v) { return (v + 255) & ~uint64_t(255); }

struct Geo {
  int nit = 0, rpu = 0;
};

// Row geometry for a GEMV whose rows hold K bf16 values.
bool geo_for_k(int K, Geo* g) {
  int rb = 2 * K;
  if (rb >= kUnit && rb % kUnit == 0 && rb / kUnit <= 8) {
    g->nit = rb / kUnit;
    g->rpu = 1;
    return true;
  }
  if (rb == kUnit / 2) {
    g->nit = 1;
    g->rpu = 2;
    return true;
  }
  return false;
}

int ceil_div(int64_t a, int64_t b) { return int((a + b - 1) / b); }

struct Builder {
  const PlanInput& in;
  Plan* P;
  std::vector<std::vector<Instr>> q;
  std::vector<std::vector<InstrMeta>> qm;
  std::vector<uint32_t> page_cursor;
  std::vector<int64_t> cu_bytes;
  explicit Builder(const PlanInput& i, Plan* p) : in(i), P(p) {
    q.resize(i.n_cus);
    qm.resize(i.n_cus);
    page_cursor.assign(i.n_cus, 0);
    cu_bytes.assign(i.n_cus, 0);
  }
  uint32_t new_counter(int stage) {
    P->ctr_stage.push_back(stage);
    P->ctr_producers.push_back(0);
    return uint32_t(P->ctr_stage.size() - 1);
  }
  void push(int cu, Instr ins, InstrMeta m, int64_t stream_bytes) {
    ins.page0 = page_cursor[cu];
    page_cursor[cu] += ins.n_pages;
    cu_bytes[cu] += stream_bytes;
    m.cu = cu;
    q[cu].push_back(ins);
    qm[cu].push_back(std::move(m));
  }
};

Instr blank() {
  Instr i;
  std::memset(&i, 0, sizeof(i));
  i.sig_ctr = kNoCounter;
  i.wait_ctr[0] = i.wait_ctr[1] = kNoCounter;
  return i;
}

// Instructions that finish through a ticket: a split attention tile (its KV
// block's partials) and a split-K O tile (its KV group's partial rows).  Each
// tile of a set takes one of n tickets on counter ctr; the tile that takes
// the last one merges the set and signals the stage counter.
bool ticketed(const Instr& I, uint32_t* ctr, uint32_t* n) {
  if (I.op == OP_ATTN && I.aux[3] > 1) {
    *ctr = I.seg_rows[0];
    *n = I.aux[3];
    return true;
  }
  if (I.op == OP_GEMV && I.epi == EPI_OPART) {
    *ctr = I.aux[2];
    *n = I.aux[3];
    return true;
  }
  return false;
}

}  // namespace

bool gemv_geometry(int K, int* nit, int* rpu) {
  Geo g;
  if (!geo_for_k(K, &g)) return false;
  *nit = g.nit;
  *rpu = g.rpu;
  return true;
}

// ------------------------------------------------------------------ config
bool is_batched(const mk_config& c) { return c.n_experts > 0; }

// The batched kernel: parallel-block MoE decoder, B <= 8 sequences.  Every
// GEMV input length is a multiple of 512 and all B staged vectors fit the
// 16384-float x slot; an expert's intermediate fits it at least 8 times (one
// staging group holds every sequence routed to an expert).
static mk_status check_config_moe(const mk_config& c, std::string* err) {
  auto unsup = [&](const char* m) {
    *err = m;
    return MK_ERR_UNSUPPORTED;
  };
  if (c.n_experts < 0 || c.top_k <= 0 || c.expert_ffn <= 0) {
    *err = "config: n_experts, top_k and expert_ffn must be positive";
    return MK_ERR_INVALID_ARG;
  }
  if (!c.parallel_block) return unsup("config: the mixture-of-experts decoder is built as a parallel block only");
  if (c.batch > lb::kMaxB) return unsup("config: at most 8 sequences per step");
  if (c.n_experts > lb::kMaxExperts) return unsup("config: at most 64 experts");
  if (c.top_k > c.n_experts || c.top_k > lb::kMaxTopK) return unsup("config: top_k must be at most min(8, n_experts)");
  if (c.n_layers > 128) return unsup("config: at most 128 layers");
  if (c.head_dim != 64 && c.head_dim != 128) return unsup("config: head_dim must be 64 or 128");
  const int q = c.n_q_heads * c.head_dim;
  if (c.hidden % 512 || q % 512 || c.expert_ffn % 512)
    return unsup("config: hidden, n_q_heads*head_dim and expert_ffn must be multiples of 512");
  if (int64_t(c.batch) * std::max(c.hidden, q) > lb::kXFloats)
    return unsup("config: batch * max(hidden, n_q_heads*head_dim) must be at most 16384");
  if (c.expert_ffn != 512 && c.expert_ffn != 1024 && c.expert_ffn != 2048)
    return unsup("config: expert_ffn must be 512, 1024 or 2048");
  const int hpg = c.n_q_heads / c.n_kv_heads;
  if ((hpg & (hpg - 1)) || hpg > 8 || hpg * c.head_dim > 512)
    return unsup("config: query heads per KV group must be 1, 2, 4 or 8, with at most 512 query values per group");
  if (c.vocab % 2) {
    *err = "config: vocab must be even";
    return MK_ERR_INVALID_ARG;
  }
  return MK_OK;
}

mk_status check_config(const mk_config& c, std::string* err) {
  auto bad = [&](const char* m) {
    *err = m;
    return MK_ERR_INVALID_ARG;
  };
  if (c.n_layers <= 0 || c.hidden <= 0 || c.n_q_heads <= 0 || c.n_kv_heads <= 0 ||
      c.head_dim <= 0 || c.vocab <= 0 || c.max_seq <= 0 || c.batch <= 0)
    return bad("config: every dimension must be positive");
  if (c.n_q_heads % c.n_kv_heads) return bad("config: n_q_heads must be a multiple of n_kv_heads");
  if (!(c.rms_eps > 0.f) || !(c.rope_theta > 1.f)) return bad("config: rms_eps > 0 and rope_theta > 1 required");
  if (is_batched(c)) return check_config_moe(c, err);
  if (c.parallel_block || c.batch != 1) {
    *err = "config: batch > 1 and the parallel block run only with the mixture-of-experts decoder";
    return MK_ERR_UNSUPPORTED;
  }
  if (c.ffn <= 0) return bad("config: ffn must be positive");
  if (c.n_layers > 128) {
    *err = "config: at most 128 layers";
    return MK_ERR_UNSUPPORTED;
  }
  if (c.head_dim != 64 && c.head_dim != 128) {
    *err = "config: head_dim must be 64 or 128";
    return MK_ERR_UNSUPPORTED;
  }
  const int q = c.n_q_heads * c.head_dim;
  Geo g;
  if (!geo_for_k(c.hidden, &g) || !geo_for_k(q, &g) || c.hidden > kMaxK || q > kMaxK) {
    *err = "config: hidden and n_q_heads*head_dim must be 256 or a multiple of 512 up to 4096";
    return MK_ERR_UNSUPPORTED;
  }
  const int hpg = c.n_q_heads / c.n_kv_heads;
  if ((hpg & (hpg - 1)) || hpg > 8 || hpg * c.head_dim > 512) {
    *err = "config: query heads per KV group must be 1, 2, 4 or 8, with at most 512 query values per group";
    return MK_ERR_UNSUPPORTED;
  }
  // the x slot holds q, k, v, cos, sin of a group, then the value-pass
  // partials of every compute wave
  if ((hpg + 3) * c.head_dim * 4 > kLdsXBytes || hpg * c.head_dim * kNComp > kMaxK) {
    *err = "config: one KV group exceeds the staging buffer";
    return MK_ERR_UNSUPPORTED;
  }
  if (c.vocab % 2 || c.hidden % 2) return bad("config: vocab and hidden must be even");
  return MK_OK;
}

mk_plan_opts resolve_opts(const mk_config& c, const mk_plan_opts* o, int n_cus) {
  mk_plan_opts r;
  std::memset(&r, 0, sizeof(r));
  if (o) r = *o;
  r.n_cus = n_cus;
  if (is_batched(c)) {
    // experts are split over the CUs by rows; the MLP chunk option is unused
    if (r.mlp_chunks <= 0) r.mlp_chunks = 1;
    r.o_split = -1;
    // the LM head on matrix cores by default: with the current kernel its
    // variant measured 3845-3850 against 3872-3875 us per step on the MoE
    // shape (two interleaved rounds; on earlier builds the variant lost
    // elsewhere what its LM head gained)
    if (r.mfma == 0) r.mfma = 1;
    // half of the expert down-projection units in the ready queue (measured
    // on the MoE shape with the current kernel, two interleaved rounds: 1/2
    // 3878-3879, 1/3 3886, 1/4 3884-3890, 1/6 3942-3944, 1/8 3921-3930,
    // 1/16 3888-3891 and no queue 3939-3940 us per step; an earlier build
    // had measured 1/8 best by a few us)
    if (r.edn_queue == 0) r.edn_queue = 2;
    if (r.edn_queue < 0) r.edn_queue = 0;  // 1: every unit in the queue
    // even gate/up slices by default: the weighted shares measured slower
    // on the MoE shape (4137 against 4001 us per step)
    if (r.egu_balance == 0) r.egu_balance = -1;
    r.gu_all = -1;
    if (r.attn_block <= 0) {
      // K and V blocks of a tile in four of the five ring pages, scores in
      // the scratch, whole KV groups per tile
      const int hpg = c.n_q_heads / c.n_kv_heads;
      const int cap_pages = (lb::kPages / 2) * kPageBytes / (2 * c.head_dim);
      const int cap_scores = lb::kScoreFloats / hpg;
      int blk = std::min(cap_pages, cap_scores);
      blk = std::max(64, (blk / 64) * 64);
      const int want = ((c.max_seq + 63) / 64) * 64;
      r.attn_block = std::min(blk, want);
    }
    if (r.attn_heads <= 0) r.attn_heads = c.n_q_heads / c.n_kv_heads;
    if (r.watchdog_ms <= 0) r.watchdog_ms = 2000;
    return r;
  }
  if (r.mlp_chunks <= 0) {
    // the fewest chunks whose width has a GEMV code path: every chunk costs
    // each CU one more gate/up and one more down instruction (staging, item
    // latency, a signal), which outweighs the earlier start of the down
    // projection that more chunks allow
    r.mlp_chunks = 1;
    for (int ch = 1; ch <= 64; ch *= 2) {
      Geo g;
      if (c.ffn % ch == 0 && geo_for_k(c.ffn / ch, &g)) {
        r.mlp_chunks = ch;
        break;
      }
    }
  }
  // gate/up of every MLP chunk in one instruction per CU (see build_plan)
  // from four chunks on: measured on the 8B shape (4 chunks) 4034-4043
  // against 4061-4066 us per step; with two chunks the per-chunk
  // instructions keep the early loads of the first down-projection chunk's
  // input during the second gate/up chunk (1B shape, context 8192: 897-902
  // against 910 us; context 128: equal)
  if (r.gu_all == 0) r.gu_all = r.mlp_chunks >= 4 ? 1 : -1;
  if (r.attn_block <= 0) {
    const int rows_per_page = kPageBytes / (2 * c.head_dim);
    if (c.max_seq <= 512 && c.max_seq * 2 * c.head_dim <= (kPages / 2) * kPageBytes) {
      r.attn_block = ((c.max_seq + 63) / 64) * 64;
    } else {
      // blocks that give every CU about one tile: rounded up to 64
      // positions, or to 8 when a block holds at least 256, where the tile's
      // own work dominates and the CUs a coarser block leaves idle matter
      // (measured: 1B shape at context 8192, 264 against 320 positions,
      // 876-881 against 890 us; 8B shape at context 2048, 72, 96 and 128
      // positions, 4102, 4098 and 4076-4082 us)
      int64_t want = (int64_t(c.max_seq) * c.n_kv_heads + n_cus - 1) / n_cus;
      int64_t blk = ((want + 63) / 64) * 64;
      if (want >= 256) blk = ((want + 7) / 8) * 8;
      int64_t cap = int64_t(rows_per_page) * (kPages / 2);
      if (blk > cap) blk = cap;
      r.attn_block = int(blk);
    }
  }
  if (r.attn_heads <= 0) {
    // one query head per tile while the tiles still fit on the CUs (short
    // contexts: attention is a chain of latencies, so smaller tiles finish
    // sooner); otherwise the whole KV group per tile, so that every K/V row
    // is streamed once
    const int hpg = c.n_q_heads / c.n_kv_heads;
    const int nblk = (c.max_seq + r.attn_block - 1) / r.attn_block;
    r.attn_heads = (int64_t(c.n_q_heads) * nblk <= n_cus) ? 1 : hpg;
  }
  // whole O rows by default: on MI355X the split's ticket and cross-CU merge
  // cost more than the spread of the attention tiles it lets O overlap
  if (r.o_split == 0) r.o_split = -1;
  // batch 1: no matrix-core tiles (the GEMVs are a single column)
  r.mfma = -1;
  r.edn_queue = 0;
  r.egu_balance = 0;
  if (r.watchdog_ms <= 0) r.watchdog_ms = 2000;
  return r;
}

ArenaLayout arena_layout(const mk_config& c, int max_lm_tiles, int max_parts) {
  ArenaLayout a;
  std::memset(&a, 0, sizeof(a));
  const uint64_t B = c.batch;
  const uint64_t d = B * c.hidden, q = B * uint64_t(c.n_q_heads) * c.head_dim,
                 kv = B * uint64_t(c.n_kv_heads) * c.head_dim,
                 F = is_batched(c) ? B * uint64_t(c.top_k) * c.expert_ffn : uint64_t(c.ffn);
  const uint64_t hpg = c.n_q_heads / c.n_kv_heads;
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    uint64_t r = off;
    off = align256(off + bytes);
    return r;
  };
  // tagged activations first: the runtime clears [0, rope_cos) to reset tags
  const uint64_t E = kActBytes;
  for (int l = 1; l <= c.n_layers; l++) a.x[l] = take(E * d);
  for (int l = 0; l < c.n_layers; l++) {
    a.qkv[l] = take(E * (q + 2 * kv));
    a.o[l] = take(E * q);
    a.h[l] = take(E * d);
    a.m[l] = take(E * F);
    a.rl[l] = is_batched(c) ? take(E * B * c.n_experts) : 0;
    a.part[l] = take(4 * uint64_t(max_parts) * hpg * (c.head_dim + 2));
    a.opart[l] = is_batched(c) ? 0 : take(4 * uint64_t(c.n_kv_heads) * c.hidden);
  }
  // expert outputs [B][top_k][d] of the layer being computed (one buffer for
  // every layer: its tags carry the layer as well as the step)
  a.y = is_batched(c) ? take(E * B * uint64_t(c.top_k) * c.hidden) : 0;
  a.edn_ctr = is_batched(c) ? take(8ull * c.n_layers) : 0;
  a.tok = take(E * B);
  a.rope_cos = take(4 * uint64_t(c.max_seq) * (c.head_dim / 2));
  a.rope_sin = take(4 * uint64_t(c.max_seq) * (c.head_dim / 2));
  a.zero_page = take(kPageBytes);
  a.lm_slots = take(8 * uint64_t(max_lm_tiles) * (is_batched(c) ? lb::kMaxB : 1));
  a.status = take(64);
  a.route_stats = take(4 * 128);
  a.total = off;
  return a;
}

// ------------------------------------------------------- build (batched)
// Stages per layer of the parallel-block MoE decoder, for B sequences:
//   QKV    rows of [Wq; Wk; Wv] . RMSNorm(x_l), every sequence        -> qkv_l
//   ROUTER rows of Wr . RMSNorm(x_l) (same staged input)               -> rl_l
//   ATTN   per sequence, KV group and position block                   -> o_l
//   EGU    per CU: its slice of gate/up pairs of every selected expert -> m_l
//   O      rows of Wo . o_l + x_l                                      -> h_l
//   EDN    per CU: its rows of every selected expert's down projection,
//          weighted over the top-k, + h_l                              -> x_{l+1}
// (attention and the experts both read RMSNorm(x_l); their results meet in
// x_{l+1} = x_l + attn + MoE, Cohere's parallel block, airebao.com «快在哪里»
// item 1), then the LM head with a per-sequence argmax.
static mk_status build_plan_moe(const PlanInput& in, Plan* P, std::string* err) {
  const mk_config& c = in.cfg;
  const mk_plan_opts& o = in.opts;
  const int C = in.n_cus;
  if (C <= 0 || C > 4096) {
    *err = "plan: n_cus out of range";
    return MK_ERR_INVALID_ARG;
  }
  const int L = c.n_layers, d = c.hidden, H = c.n_q_heads, G = c.n_kv_heads, Dh = c.head_dim, V = c.vocab,
            S = c.max_seq, B = c.batch, E = c.n_experts, Fe = c.expert_ffn;
  const int qd = H * Dh, kvd = G * Dh, hpg = H / G, Rq = qd + 2 * kvd;
  const int Bat = o.attn_block, kv_rb = 2 * Dh;
  if (Bat <= 0 || Bat % 64) {
    *err = "plan: attn_block must be a positive multiple of 64";
    return MK_ERR_INVALID_ARG;
  }
  const int kp = ceil_div(int64_t(Bat) * kv_rb, kPageBytes);
  if (2 * kp > lb::kPages) {
    *err = "plan: attention tile (K and V blocks) exceeds the LDS page ring";
    return MK_ERR_INVALID_ARG;
  }
  const int hpt = o.attn_heads;
  if (hpt <= 0 || hpg % hpt) {
    *err = "plan: attn_heads must divide the query heads per KV group";
    return MK_ERR_INVALID_ARG;
  }
  if (hpt * Bat > lb::kScoreFloats) {
    *err = "plan: attention scores of one tile exceed the LDS scratch";
    return MK_ERR_INVALID_ARG;
  }
  const int nblk = ceil_div(S, Bat), tpg = hpg / hpt;
  *P = Plan();
  P->n_cus = C;
  P->attn_block = Bat;
  P->attn_nblk = nblk;
  P->attn_tiles = B * G * tpg * nblk;
  P->attn_heads = hpt;
  P->mlp_chunks = 1;
  P->batched = true;
  P->arena = arena_layout(c, C, B * G * nblk);
  const uint64_t A = in.arena_base;
  const ArenaLayout& ar = P->arena;
  Builder b(in, P);
  const uint64_t embed = uint64_t(in.w.embed), lm = uint64_t(in.w.lm_head);
  auto lptr = [](const void* base, int l, uint64_t per_layer_elems) {
    return uint64_t(base) + 2ull * per_layer_elems * uint64_t(l);
  };
  auto split = [&](int64_t N, int cu, int64_t* lo, int64_t* hi) {
    *lo = N * cu / C;
    *hi = N * (cu + 1) / C;
  };
  std::vector<uint32_t> c_qkv(L), c_rt(L), c_attn(L), c_gu(L), c_o(L), c_dny(L), c_dn(L);
  std::vector<std::vector<uint32_t>> c_ticket(L);
  for (int l = 0; l < L; l++) {
    c_qkv[l] = b.new_counter(l * ST_PER_LAYER + ST_QKV);
    c_rt[l] = b.new_counter(l * ST_PER_LAYER + ST_QKV);
    c_attn[l] = b.new_counter(l * ST_PER_LAYER + ST_ATTN);
    if (nblk > 1)
      for (int t = 0; t < B * G * tpg; t++) c_ticket[l].push_back(b.new_counter(l * ST_PER_LAYER + ST_ATTN));
    c_gu[l] = b.new_counter(l * ST_PER_LAYER + ST_ATTN);
    c_o[l] = b.new_counter(l * ST_PER_LAYER + ST_O);
    c_dny[l] = b.new_counter(l * ST_PER_LAYER + ST_DOWN);
    c_dn[l] = b.new_counter(l * ST_PER_LAYER + ST_DRED);
  }
  const uint32_t c_lm = b.new_counter(L * ST_PER_LAYER);
  // a batched GEMV tile: rows [r0, r1) of one matrix (or the Wq|Wk|Wv
  // segments), applied to the B staged vectors
  auto bgemv = [&](int l, int epi, int K, int r0, int r1) {
    Instr I = blank();
    I.op = OP_BGEMV;
    I.epi = uint8_t(epi);
    I.nit = uint8_t(K / 512);
    I.rpu = 1;
    I.layer = uint16_t(l);
    I.n_items = uint32_t((r1 - r0 + 1) / 2);
    I.row0 = uint32_t(r0);
    I.row_bytes = uint32_t(2 * K);
    I.n_rows = uint32_t(r1 - r0);
    I.k = uint32_t(K);
    I.n_pages = uint32_t(ceil_div(int64_t(2 * I.n_items) * I.row_bytes, kPageBytes));
    return I;
  };
  auto per_seq = [&](std::vector<Range>& v, int buf, int layer, uint64_t stride, uint64_t lo, uint64_t hi) {
    for (int s = 0; s < B; s++) v.push_back({buf, layer, s * stride + lo, s * stride + hi});
  };
  // matrix-core tiles for the LM head: items are blocks of 16 rows, streamed
  // in fragment order (its input is not shared with other instructions; the
  // O projection's 8 rows per CU would stream a half-empty block)
  const bool mfma = o.mfma > 0;
  auto to_mfma = [&](Instr& I) {
    I.flags |= F_MFMA;
    I.n_items = uint32_t(ceil_div(int64_t(I.n_rows), 16));
    I.n_pages = uint32_t(ceil_div(int64_t(I.n_items) * 16 * I.row_bytes, kPageBytes));
  };
  // attention tile -> CU.  The tiles of the last position block (the
  // positions past the pre-filled context: a few rows at most) cost a
  // fraction of a full block's; the full blocks are spread evenly and each
  // last-block tile goes to a CU with the fewest tiles, near an even spread,
  // so that the CUs that take one tile more take a light one.
  const int n_att = B * G * tpg * nblk;
  std::vector<int> att_cu_of(n_att);
  const int n_rt = (E + 1) / 2;  // router tiles of two rows
  auto rt_cu = [&](int t) { return int(int64_t(t) * C / n_rt); };
  {
    const bool split_last = nblk > 1;
    const int n_full = split_last ? B * G * tpg * (nblk - 1) : n_att, n_last = n_att - n_full;
    // a router tile counts as a tile here, so that the light tiles avoid
    // the CUs that compute the router
    std::vector<int> count(C, 0);
    for (int t = 0; t < n_rt; t++) count[rt_cu(t)]++;
    int j = 0, k = 0;
    for (int a = 0; a < n_att; a++) {
      if (split_last && a % nblk == nblk - 1) continue;
      const int cu = int((int64_t(j++) * C / n_full) % C);
      att_cu_of[a] = cu;
      count[cu]++;
    }
    for (int a = 0; split_last && a < n_att; a++) {
      if (a % nblk != nblk - 1) continue;
      const int want = int((int64_t(k++) * C / std::max(1, n_last)) % C);
      int best = want;
      for (int dc = 0; dc < C; dc++) {
        const int cu = (want + dc) % C;
        if (count[cu] < count[best]) best = cu;
        if (count[best] == 0) break;
      }
      // the first CU at or after the even position among those with the fewest tiles
      int mn = count[best];
      for (int dc = 0; dc < C; dc++)
        if (count[(want + dc) % C] == mn) {
          best = (want + dc) % C;
          break;
        }
      att_cu_of[a] = best;
      count[best]++;
    }
  }
  auto att_cu = [&](int a) { return att_cu_of[a]; };
  // Gate/up shares: cumulative 1/65536 fractions of a layer's (expert, row)
  // items per CU, so that the work each CU does before its gate/up items
  // (attention tiles, router tiles) plus its items ends at about the same
  // time everywhere.  The costs are MI355X measurements of this kernel: an
  // attention tile ~12 us, a router tile ~6 us, gate/up rows streamed at
  // ~27.5 GB/s per CU; the number of selected experts is its expectation
  // for uniform routing.
  std::vector<uint32_t> egu_cum;
  {
    constexpr double kAttnTileUs = 12.0, kRouterTileUs = 6.0, kCuBytesPerUs = 27500.0;
    std::vector<double> pre(C, 0.0);
    for (int a = 0; a < n_att; a++) pre[att_cu_of[a]] += kAttnTileUs;
    for (int t = 0; t < n_rt; t++) pre[rt_cu(t)] += kRouterTileUs;
    const double nsel = E * (1.0 - std::pow(1.0 - double(c.top_k) / E, B));
    const double total = C * (nsel * Fe * 4.0 * d / C / kCuBytesPerUs);
    // the level L with sum over CUs of max(0, L - pre) = total
    std::vector<double> srt(pre);
    std::sort(srt.begin(), srt.end());
    double level = srt[0], acc = 0.0;
    for (int i = 0; i < C; i++) {
      const double next = i + 1 < C ? srt[i + 1] : 1e300;
      // CUs 0..i are below the level: raising it to next adds (i + 1) (next - level)
      if (acc + (i + 1) * (next - level) >= total) {
        level += (total - acc) / (i + 1);
        break;
      }
      acc += (i + 1) * (next - level);
      level = next;
    }
    std::vector<double> w(C);
    double sw = 0.0;
    for (int cu = 0; cu < C; cu++) sw += (w[cu] = std::max(0.0, level - pre[cu]));
    egu_cum.assign(C + 1, 0u);
    double run = 0.0;
    for (int cu = 0; cu < C; cu++) {
      run += w[cu];
      egu_cum[cu + 1] = cu + 1 == C ? 65536u : uint32_t(std::llround(65536.0 * run / sw));
    }
  }
  auto egu_shares = [&](int) { return egu_cum; };
  const int max_res_rows = std::min(kMaxResRows / B, lb::kMaxDnRows);
  // pairs of an expert gate/up instruction (each pair is a gate row and an up
  // row side by side in the page stream): a slice of at most four pages
  const int max_pairs = std::max(1, 4 * kPageBytes / (4 * d));

  for (int l = 0; l < L; l++) {
    const int stg = l * ST_PER_LAYER;
    const uint64_t x_in = l == 0 ? embed : A + ar.x[l];
    const int x_buf = l == 0 ? BUF_EMBED : BUF_X;
    // ---------------------------------------------------------------- QKV
    for (int cu = 0; cu < C; cu++) {
      int64_t r0, r1;
      split(Rq, cu, &r0, &r1);
      if (r1 <= r0) continue;
      Instr I = bgemv(l, EPI_STORE, d, int(r0), int(r1));
      I.flags = F_NORM | F_SIGNAL | (l == 0 ? F_IN_EMBED : 0);
      const int bounds[4] = {0, qd, qd + kvd, qd + 2 * kvd};
      const void* mats[3] = {in.w.wq, in.w.wk, in.w.wv};
      const int mrows[3] = {qd, kvd, kvd};
      int ns = 0;
      for (int sg = 0; sg < 3; sg++) {
        int lo = std::max(int(r0), bounds[sg]), hi = std::min(int(r1), bounds[sg + 1]);
        if (hi <= lo) continue;
        I.seg_ptr[ns] = lptr(mats[sg], l, uint64_t(mrows[sg]) * d) + 2ull * d * (lo - bounds[sg]);
        I.seg_rows[ns] = uint32_t(hi - lo);
        I.seg_stride[ns] = uint32_t(2 * d);
        ns++;
      }
      I.aux[0] = uint32_t(Rq);
      I.aux[4] = uint32_t(ns);
      I.in_ptr = x_in;
      I.out_ptr = A + ar.qkv[l];
      I.gain_ptr = lptr(in.w.attn_norm, l, d);
      if (l > 0) I.wait_ctr[0] = c_dn[l - 1];
      I.sig_ctr = c_qkv[l];
      InstrMeta m;
      m.stage = stg + ST_QKV;
      m.merge_write = false;
      m.reads.push_back({x_buf, l, 0, uint64_t(B) * d});
      per_seq(m.writes, BUF_QKV, l, Rq, r0, r1);
      b.push(cu, I, std::move(m), (r1 - r0) * 2ll * d);
    }
    // ------------------------------------------------------------- ROUTER
    for (int t = 0; t < n_rt; t++) {
      const int r0 = 2 * t, r1 = std::min(E, r0 + 2);
      Instr I = bgemv(l, EPI_STORE, d, r0, r1);
      I.flags = F_NORM | F_SIGNAL | (l == 0 ? F_IN_EMBED : 0);
      I.seg_ptr[0] = lptr(in.w.router, l, uint64_t(E) * d) + 2ull * d * r0;
      I.seg_rows[0] = uint32_t(r1 - r0);
      I.seg_stride[0] = uint32_t(2 * d);
      I.aux[0] = uint32_t(E);
      I.aux[4] = 1;
      I.in_ptr = x_in;
      I.out_ptr = A + ar.rl[l];
      I.gain_ptr = lptr(in.w.attn_norm, l, d);
      if (l > 0) I.wait_ctr[0] = c_dn[l - 1];
      I.sig_ctr = c_rt[l];
      InstrMeta m;
      m.stage = stg + ST_QKV;
      m.merge_write = false;
      m.reads.push_back({x_buf, l, 0, uint64_t(B) * d});
      per_seq(m.writes, BUF_RL, l, E, r0, r1);
      b.push(rt_cu(t), I, std::move(m), (r1 - r0) * 2ll * d);
    }
    // --------------------------------------------------------------- ATTN
    for (int a = 0; a < n_att; a++) {
      // tile a: sequence sq, head tile tg of the layer, block blk
      const int per_seq_tiles = G * tpg * nblk;
      const int sq = a / per_seq_tiles, rem = a % per_seq_tiles;
      const int tg = rem / nblk, blk = rem % nblk;
      const int g = tg / tpg, h0 = (tg % tpg) * hpt;
      Instr I = blank();
      I.op = OP_ATTN;
      I.layer = uint16_t(l);
      I.flags = F_SIGNAL;
      I.n_items = uint32_t(hpt);
      I.row0 = uint32_t(h0);
      I.row_bytes = uint32_t(kv_rb);
      I.n_rows = uint32_t(2 * Bat);
      I.aux[0] = uint32_t(g);
      I.aux[1] = uint32_t(blk);
      I.aux[2] = uint32_t(Bat);
      I.aux[3] = uint32_t(nblk);
      I.aux[4] = uint32_t(kp);
      const uint64_t head_rows = uint64_t(S) * Dh;
      const uint64_t kvi = (uint64_t(l) * B + sq) * G + g;
      I.seg_ptr[0] = uint64_t(in.w.k_cache) + 2ull * head_rows * kvi;
      I.seg_ptr[1] = uint64_t(in.w.v_cache) + 2ull * head_rows * kvi;
      I.seg_rows[0] = nblk > 1 ? c_ticket[l][sq * G * tpg + tg] : kNoCounter;
      I.in_ptr = A + ar.qkv[l] + uint64_t(kActBytes) * sq * Rq;
      I.out_ptr = A + ar.o[l] + uint64_t(kActBytes) * sq * qd;
      I.res_ptr = A + ar.part[l] + 4ull * sq * H * nblk * (Dh + 2);
      I.wait_ctr[0] = c_qkv[l];
      I.sig_ctr = c_attn[l];
      I.n_pages = uint32_t(2 * kp);
      InstrMeta m;
      m.stage = stg + ST_ATTN;
      m.merge_write = nblk > 1;
      const uint64_t so = uint64_t(sq) * Rq;
      const uint64_t q0 = uint64_t(g * hpg + h0) * Dh, q1 = q0 + uint64_t(hpt) * Dh;
      m.reads.push_back({BUF_QKV, l, so + q0, so + q1});
      m.reads.push_back({BUF_QKV, l, so + qd + g * Dh, so + qd + (g + 1) * Dh});
      m.reads.push_back({BUF_QKV, l, so + qd + kvd + g * Dh, so + qd + kvd + (g + 1) * Dh});
      m.writes.push_back({BUF_O, l, uint64_t(sq) * qd + q0, uint64_t(sq) * qd + q1});
      const int64_t rows = std::min<int64_t>(Bat, std::max<int64_t>(0, int64_t(S) - int64_t(blk) * Bat));
      b.push(att_cu(a), I, std::move(m), 2 * rows * kv_rb);
    }
    // ---------------------------------------------------------------- EGU
    std::vector<char> routed(C, 0);  // CU already has an expert instruction of this layer
    // rows of at most 4 KiB are loaded by the compute waves directly
    const bool egu_direct = d / 512 == 1 || d / 512 == 2 || d / 512 == 4;
    if (egu_direct && o.egu_balance > 0) {
      // Weighted shares: CU c takes items [T f_c, T f_{c+1}) of the T =
      // (selected experts) x Fe (expert, row) items in expert order, its
      // share cut so that its earlier work of the layer plus its gate/up
      // items take about the same time on every CU.
      const std::vector<uint32_t> cum = egu_shares(l);
      for (int cu = 0; cu < C; cu++) {
        Instr I = blank();
        I.op = OP_EGU;
        I.epi = EPI_SWIGLU;
        I.nit = uint8_t(d / 512);
        I.rpu = 1;
        I.layer = uint16_t(l);
        I.flags = F_NORM | F_SIGNAL | F_DIRECT | F_SHARE | (l == 0 ? F_IN_EMBED : 0) | (routed[cu] ? 0 : F_ROUTE);
        routed[cu] = 1;
        I.n_items = uint32_t(Fe);
        I.row_bytes = uint32_t(2 * d);
        I.n_rows = uint32_t(2 * Fe);
        I.k = uint32_t(d);
        I.aux[0] = c_rt[l];
        I.aux[3] = uint32_t(Fe);
        I.aux[4] = uint32_t(E);
        I.seg_ptr[0] = A + ar.rl[l];
        I.seg_ptr[1] = lptr(in.w.e_gate, l, uint64_t(E) * Fe * d);
        I.seg_ptr[2] = lptr(in.w.e_up, l, uint64_t(E) * Fe * d);
        I.seg_stride[0] = uint32_t(2ull * Fe * d);
        I.seg_rows[0] = uint32_t(Fe * 2 * d);
        I.seg_rows[1] = cum[cu];
        I.seg_rows[2] = cum[cu + 1];
        I.in_ptr = x_in;
        I.out_ptr = A + ar.m[l];
        I.gain_ptr = lptr(in.w.attn_norm, l, d);
        I.wait_ctr[0] = c_rt[l];
        I.sig_ctr = c_gu[l];
        I.n_pages = 0;
        InstrMeta m;
        m.stage = stg + ST_ATTN;
        // the rows a CU writes are decided by the routing
        m.merge_write = true;
        m.reads.push_back({x_buf, l, 0, uint64_t(B) * d});
        m.reads.push_back({BUF_RL, l, 0, uint64_t(B) * E});
        m.writes.push_back({BUF_M, l, 0, uint64_t(B) * c.top_k * Fe});
        b.push(cu, I, std::move(m), int64_t((uint64_t(E) * Fe * 4 * d * (cum[cu + 1] - cum[cu])) >> 16));
      }
    }
    for (int cu = 0; cu < C && !(egu_direct && o.egu_balance > 0); cu++) {
      int64_t f0, f1;
      split(Fe, cu, &f0, &f1);
      for (int64_t p0 = f0; p0 < f1; p0 += max_pairs) {
        const int64_t p1 = std::min<int64_t>(f1, p0 + max_pairs), npu = p1 - p0;
        const int ppe = ceil_div(npu * 4 * d, kPageBytes);
        Instr I = blank();
        I.op = OP_EGU;
        I.epi = EPI_SWIGLU;
        I.nit = uint8_t(d / 512);
        I.rpu = 1;
        I.layer = uint16_t(l);
        const bool direct = egu_direct;
        I.flags = F_NORM | F_SIGNAL | (l == 0 ? F_IN_EMBED : 0) | (routed[cu] ? 0 : F_ROUTE) |
                  (direct ? F_DIRECT : 0);
        routed[cu] = 1;
        I.n_items = uint32_t(npu);
        I.row0 = uint32_t(p0);
        I.row_bytes = uint32_t(2 * d);
        I.n_rows = uint32_t(2 * npu);
        I.k = uint32_t(d);
        I.aux[0] = c_rt[l];
        I.aux[2] = uint32_t(ppe);
        I.aux[3] = uint32_t(npu);
        I.aux[4] = uint32_t(E);
        I.seg_ptr[0] = A + ar.rl[l];
        I.seg_ptr[1] = lptr(in.w.e_gate, l, uint64_t(E) * Fe * d) + 2ull * d * p0;
        I.seg_ptr[2] = lptr(in.w.e_up, l, uint64_t(E) * Fe * d) + 2ull * d * p0;
        I.seg_stride[0] = uint32_t(2ull * Fe * d);
        I.seg_rows[0] = uint32_t(npu * 2 * d);
        I.seg_stride[1] = 0;
        I.in_ptr = x_in;
        I.out_ptr = A + ar.m[l];
        I.gain_ptr = lptr(in.w.attn_norm, l, d);
        I.wait_ctr[0] = c_rt[l];
        I.sig_ctr = c_gu[l];
        I.n_pages = direct ? 0 : uint32_t(E * ppe);
        InstrMeta m;
        m.stage = stg + ST_ATTN;
        m.merge_write = false;
        m.reads.push_back({x_buf, l, 0, uint64_t(B) * d});
        m.reads.push_back({BUF_RL, l, 0, uint64_t(B) * E});
        for (int sq = 0; sq < B; sq++)
          for (int slot = 0; slot < c.top_k; slot++) {
            const uint64_t base = (uint64_t(sq) * c.top_k + slot) * Fe;
            m.writes.push_back({BUF_M, l, base + p0, base + p1});
          }
        b.push(cu, I, std::move(m), int64_t(E) * npu * 4 * d);
      }
    }
    // ------------------------------------------------------------------ O
    for (int cu = 0; cu < C; cu++) {
      int64_t c0, c1;
      split(d, cu, &c0, &c1);
      for (int64_t r0 = c0; r0 < c1; r0 += max_res_rows) {
        const int64_t r1 = std::min<int64_t>(c1, r0 + max_res_rows);
        Instr I = bgemv(l, EPI_RESID, qd, int(r0), int(r1));
        I.flags = F_SIGNAL | (l == 0 ? F_RES_EMBED : 0);
        I.seg_ptr[0] = lptr(in.w.wo, l, uint64_t(d) * qd) + 2ull * qd * r0;
        I.seg_rows[0] = uint32_t(r1 - r0);
        I.seg_stride[0] = uint32_t(2 * qd);
        I.aux[0] = uint32_t(d);
        I.aux[2] = uint32_t(d);
        I.aux[4] = 1;
        I.in_ptr = A + ar.o[l];
        I.res_ptr = x_in;
        I.out_ptr = A + ar.h[l];
        I.wait_ctr[0] = c_attn[l];
        I.sig_ctr = c_o[l];
        InstrMeta m;
        m.stage = stg + ST_O;
        m.merge_write = false;
        m.reads.push_back({BUF_O, l, 0, uint64_t(B) * qd});
        per_seq(m.reads, x_buf, l, d, r0, r1);
        per_seq(m.writes, BUF_H, l, d, r0, r1);
        b.push(cu, I, std::move(m), (r1 - r0) * 2ll * qd);
      }
    }
    // ---------------------------------------------------------------- EDN
    // The down projections of the selected experts, cut into units of Rb
    // rows (32 KiB of weights); the units of all selected experts, in expert
    // order, are split evenly over the CUs at run time.  A unit's outputs go
    // to y[b][slot][row] for the sequences routed to its expert.
    {
      const int Rb = std::max(4, 32768 / (2 * Fe));
      const int nb = ceil_div(d, Rb), ppu = ceil_div(int64_t(Rb) * 2 * Fe, kPageBytes);
      for (int cu = 0; cu < C; cu++) {
        Instr I = blank();
        I.op = OP_EDN;
        I.nit = uint8_t(Fe / 512);
        I.rpu = 1;
        I.layer = uint16_t(l);
        // rows of at most 2 KiB are loaded by the compute waves directly
        const bool direct = Fe / 512 <= 2;
        I.flags = F_SIGNAL | (routed[cu] ? 0 : F_ROUTE) | (direct ? F_DIRECT : 0);
        routed[cu] = 1;
        I.n_items = uint32_t(C);
        I.row_bytes = uint32_t(2 * Fe);
        I.n_rows = uint32_t(Rb);
        I.k = uint32_t(Fe);
        I.aux[0] = c_rt[l];
        I.aux[2] = uint32_t(ppu);
        I.aux[3] = uint32_t(Rb);
        I.aux[4] = uint32_t(nb);
        I.seg_ptr[0] = A + ar.rl[l];
        I.seg_ptr[1] = lptr(in.w.e_down, l, uint64_t(E) * d * Fe);
        I.seg_stride[0] = uint32_t(2ull * d * Fe);
        I.seg_rows[0] = uint32_t(Rb * 2 * Fe);
        I.in_ptr = A + ar.m[l];
        I.out_ptr = A + ar.y;
        I.res_ptr = A + ar.edn_ctr + 8ull * l;  // the layer's ready-queue counters
        I.row0 = uint32_t(std::max(0, o.edn_queue));
        I.wait_ctr[0] = c_gu[l];
        I.sig_ctr = c_dny[l];
        // at most every unit (the static share and the queue's chunks)
        I.n_pages = direct ? 0 : uint32_t(E * nb * ppu);
        InstrMeta m;
        m.stage = stg + ST_DOWN;
        // every unit's writes are decided by the routing: the tiles share
        // the layer's whole buffer
        m.merge_write = true;
        m.reads.push_back({BUF_M, l, 0, uint64_t(B) * c.top_k * Fe});
        m.reads.push_back({BUF_RL, l, 0, uint64_t(B) * E});
        m.writes.push_back({BUF_Y, l, 0, uint64_t(B) * c.top_k * d});
        b.push(cu, I, std::move(m), int64_t(E) * d * 2 * Fe / C);
      }
    }
    // ---------------------------------------------------------------- ERD
    // x_{l+1}[b][r] = h[b][r] + sum over the top-k slots s, in slot order, of
    // w[b][s] * y[b][s][r], for the CU's rows of every sequence
    for (int cu = 0; cu < C; cu++) {
      int64_t r0, r1;
      split(d, cu, &r0, &r1);
      if (r1 > r0) {
        const int64_t nr = r1 - r0;
        Instr I = blank();
        I.op = OP_ERD;
        I.layer = uint16_t(l);
        I.flags = F_SIGNAL;
        I.row0 = uint32_t(r0);
        I.n_rows = uint32_t(nr);
        I.in_ptr = A + ar.y;
        I.res_ptr = A + ar.h[l];
        I.out_ptr = A + ar.x[l + 1];
        if (r0 == 0) I.seg_ptr[0] = A + ar.edn_ctr + 8ull * l;  // clears the next step's counter
        I.wait_ctr[0] = c_dny[l];
        I.wait_ctr[1] = c_o[l];
        I.sig_ctr = c_dn[l];
        InstrMeta m;
        m.stage = stg + ST_DRED;
        m.merge_write = false;
        m.reads.push_back({BUF_Y, l, 0, uint64_t(B) * c.top_k * d});
        per_seq(m.reads, BUF_H, l, d, r0, r1);
        per_seq(m.writes, BUF_X, l + 1, d, r0, r1);
        b.push(cu, I, std::move(m), 0);
      }
    }
  }
  // ------------------------------------------------------------- LM head
  {
    std::vector<int> lm_cus;
    for (int cu = 0; cu < C; cu++) {
      int64_t i0, i1;
      split(V, cu, &i0, &i1);
      if (i1 > i0) lm_cus.push_back(cu);
    }
    const int n_lm = int(lm_cus.size());
    int tile = 0;
    for (int cu : lm_cus) {
      int64_t r0, r1;
      split(V, cu, &r0, &r1);
      Instr I = bgemv(L, EPI_ARGMAX, d, int(r0), int(r1));
      I.flags = F_NORM | F_SIGNAL;
      I.seg_ptr[0] = lm + 2ull * d * r0;
      I.seg_rows[0] = uint32_t(r1 - r0);
      I.seg_stride[0] = uint32_t(2 * d);
      I.aux[0] = uint32_t(V);
      I.aux[1] = uint32_t(tile);
      I.aux[3] = uint32_t(n_lm);
      I.aux[4] = 1;
      I.in_ptr = A + ar.x[L];
      I.gain_ptr = uint64_t(in.w.final_norm);
      I.wait_ctr[0] = c_dn[L - 1];
      I.sig_ctr = c_lm;
      if (mfma) to_mfma(I);
      InstrMeta m;
      m.stage = L * ST_PER_LAYER;
      m.merge_write = false;
      m.reads.push_back({BUF_X, L, 0, uint64_t(B) * d});
      per_seq(m.writes, BUF_LOGITS, 0, V, r0, r1);
      b.push(cu, I, std::move(m), (r1 - r0) * 2ll * d);
      tile++;
    }
    P->lm_tiles = n_lm;
  }
  // producers per counter (per step)
  for (int cu = 0; cu < C; cu++)
    for (const Instr& I : b.q[cu]) {
      if (I.op == OP_ATTN && I.aux[3] > 1) {
        P->ctr_producers[I.seg_rows[0]]++;
        continue;
      }
      if ((I.flags & F_SIGNAL) && I.sig_ctr != kNoCounter) P->ctr_producers[I.sig_ctr]++;
    }
  for (int l = 0; l < L; l++)
    if (nblk > 1) P->ctr_producers[c_attn[l]] = uint32_t(B * G * tpg);
  for (int cu = 0; cu < C; cu++)
    for (Instr& I : b.q[cu]) {
      for (int k = 0; k < 2; k++)
        if (I.wait_ctr[k] != kNoCounter) I.wait_cnt[k] = P->ctr_producers[I.wait_ctr[k]];
      if (I.op == OP_EGU || I.op == OP_EDN) I.aux[1] = P->ctr_producers[I.aux[0]];
    }
  P->q_off.assign(C + 1, 0);
  for (int cu = 0; cu < C; cu++) {
    P->q_off[cu + 1] = P->q_off[cu] + uint32_t(b.q[cu].size());
    P->instrs.insert(P->instrs.end(), b.q[cu].begin(), b.q[cu].end());
    P->meta.insert(P->meta.end(), b.qm[cu].begin(), b.qm[cu].end());
  }
  P->n_counters = int(P->ctr_stage.size());
  // packed weight stream of the batched GEMV tiles (experts are read in place)
  uint64_t pack = 0;
  for (Instr& I : P->instrs) {
    if (I.op != OP_BGEMV) continue;
    I.src_ptr = in.pack_base + pack;
    uint64_t row = 0;
    for (uint32_t sg = 0; sg < I.aux[4]; sg++) {
      if (!I.seg_rows[sg]) continue;
      PackCopy cp{};
      cp.src = I.seg_ptr[sg];
      cp.rows = I.seg_rows[sg];
      cp.row_bytes = I.row_bytes;
      cp.src_stride = I.seg_stride[sg];
      if (I.flags & F_MFMA) {
        // one segment, in fragment order from the start of the run
        cp.dst = pack;
        cp.frag = 1;
      } else {
        cp.dst = pack + row * I.row_bytes;
        cp.dst_stride = I.row_bytes;
      }
      row += cp.rows;
      P->pack.push_back(cp);
    }
    pack += uint64_t(I.n_pages) * kPageBytes;
  }
  P->pack_bytes = pack;
  // bytes that do not depend on the routing: attention and router
  // projections, norms, the LM head and B embedding rows (the experts add
  // 6 * d * Fe bytes per selected expert and layer)
  int64_t wbytes = int64_t(L) * 2 * (int64_t(Rq) * d + int64_t(d) * qd + int64_t(E) * d + d);
  wbytes += 2ll * V * d + 2ll * d + 2ll * d * B;
  P->weight_bytes = wbytes;
  P->max_cu_bytes = *std::max_element(b.cu_bytes.begin(), b.cu_bytes.end());
  P->min_cu_bytes = *std::min_element(b.cu_bytes.begin(), b.cu_bytes.end());
  return MK_OK;
}

// ------------------------------------------------------------------- build
mk_status build_plan(const PlanInput& in, Plan* P, std::string* err) {
  const mk_config& c = in.cfg;
  mk_status st = check_config(c, err);
  if (st != MK_OK) return st;
  if (is_batched(c)) return build_plan_moe(in, P, err);
  const mk_plan_opts& o = in.opts;
  const int C = in.n_cus;
  if (C <= 0 || C > 4096) {
    *err = "plan: n_cus out of range";
    return MK_ERR_INVALID_ARG;
  }
  const int L = c.n_layers, d = c.hidden, H = c.n_q_heads, G = c.n_kv_heads, Dh = c.head_dim,
            F = c.ffn, V = c.vocab, S = c.max_seq;
  const int qd = H * Dh, kvd = G * Dh, hpg = H / G;
  const int chunks = o.mlp_chunks;
  if (chunks <= 0 || F % chunks) {
    *err = "plan: mlp_chunks must divide ffn";
    return MK_ERR_INVALID_ARG;
  }
  const int Fc = F / chunks;
  const bool gu_all = chunks > 1 && o.gu_all > 0;
  Geo gd, gq, gf;
  if (!geo_for_k(d, &gd) || !geo_for_k(qd, &gq) || !geo_for_k(Fc, &gf) || Fc > kMaxK) {
    *err = "plan: ffn/mlp_chunks must be 256 or a multiple of 512 up to 4096";
    return MK_ERR_UNSUPPORTED;
  }
  const int Bat = o.attn_block;
  const int kv_rb = 2 * Dh;
  // whole 1 KiB units of K and V rows (8 rows at head size 64, 4 at 128)
  if (Bat <= 0 || Bat % 8) {
    *err = "plan: attn_block must be a positive multiple of 8";
    return MK_ERR_INVALID_ARG;
  }
  const int kp = ceil_div(int64_t(Bat) * kv_rb, kPageBytes);
  if (2 * kp > kPages) {
    *err = "plan: attention tile (K and V blocks) exceeds the LDS page ring";
    return MK_ERR_INVALID_ARG;
  }
  const int hpt = o.attn_heads;  // query heads per attention tile
  if (hpt <= 0 || hpg % hpt) {
    *err = "plan: attn_heads must divide the query heads per KV group";
    return MK_ERR_INVALID_ARG;
  }
  if (hpt * Bat > kAttnScoreFloats) {
    *err = "plan: attention scores of one tile exceed the LDS scratch";
    return MK_ERR_INVALID_ARG;
  }
  const int nblk = ceil_div(S, Bat);
  const int tpg = hpg / hpt;  // head tiles per KV group
  *P = Plan();
  P->n_cus = C;
  P->attn_block = Bat;
  P->attn_nblk = nblk;
  P->attn_tiles = G * tpg * nblk;
  P->attn_heads = hpt;
  P->mlp_chunks = chunks;
  P->arena = arena_layout(c, C, G * nblk);
  const uint64_t A = in.arena_base;
  const ArenaLayout& ar = P->arena;
  Builder b(in, P);

  const uint64_t embed = uint64_t(in.w.embed), lm = uint64_t(in.w.lm_head);
  auto lptr = [](const void* base, int l, uint64_t per_layer_elems) {
    return uint64_t(base) + 2ull * per_layer_elems * uint64_t(l);
  };

  std::vector<uint32_t> c_qkv(L), c_attn(L), c_o(L), c_down(L);
  std::vector<std::vector<uint32_t>> c_gu(L), c_ticket(L);
  for (int l = 0; l < L; l++) {
    c_qkv[l] = b.new_counter(l * ST_PER_LAYER + ST_QKV);
    c_attn[l] = b.new_counter(l * ST_PER_LAYER + ST_ATTN);
    if (nblk > 1)
      for (int t = 0; t < G * tpg; t++) c_ticket[l].push_back(b.new_counter(l * ST_PER_LAYER + ST_ATTN));
    c_o[l] = b.new_counter(l * ST_PER_LAYER + ST_O);
    for (int ch = 0; ch < (gu_all ? 1 : chunks); ch++) c_gu[l].push_back(b.new_counter(l * ST_PER_LAYER + ST_GU));
    c_down[l] = b.new_counter(l * ST_PER_LAYER + ST_DOWN);
  }
  const uint32_t c_lm = b.new_counter(L * ST_PER_LAYER);

  // evenly split N items over C CUs
  auto split = [&](int64_t N, int cu, int64_t* lo, int64_t* hi) {
    *lo = N * cu / C;
    *hi = N * (cu + 1) / C;
  };
  auto set_wait = [](Instr& I, int k, uint32_t ctr) { I.wait_ctr[k] = ctr; };

  // attention tile -> CU: spread over the CUs, and over XCDs when sparse
  const int n_att = G * tpg * nblk;
  auto att_cu = [&](int a) {
    int64_t spacing = C / std::max(1, n_att);
    int64_t cu = int64_t(a) * C / n_att;
    if (spacing >= 8) cu += a % 8;
    return int(cu % C);
  };

  // CUs that take O rows: all, or, with few attention tiles (at most one
  // CU in four), the CUs without one
  std::vector<int> o_rank(C, 0), o_cu_of_rank;
  const bool o_skip_att = int64_t(n_att) * 4 <= C;
  int o_cus = C;
  if (o_skip_att) {
    for (int a = 0; a < n_att; a++) o_rank[att_cu(a)] = -1;
    o_cus = 0;
    for (int cu = 0; cu < C; cu++)
      if (o_rank[cu] == 0) o_rank[cu] = o_cus++;
  }
  for (int cu = 0; cu < C; cu++)
    if (!o_skip_att || o_rank[cu] >= 0) o_cu_of_rank.push_back(cu);

  // Split-K O projection: tile (row block, KV group g) takes the rows of the
  // block over group g's Kg input columns, so it waits only for that group's
  // attention; G tiles per row block, one per O CU while they last.
  const int Kg = hpg * Dh;
  Geo gk;
  const bool osplit = o.o_split > 0;
  if (osplit && (G < 2 || !geo_for_k(Kg, &gk))) {
    *err = "plan: o_split needs more than one KV group and a GEMV width for heads-per-group * head_dim";
    return MK_ERR_UNSUPPORTED;
  }
  const int o_blocks = osplit ? int(std::max<int64_t>(1, std::min<int64_t>(o_cus / G, d / gk.rpu))) : 0;
  std::vector<std::vector<uint32_t>> c_oticket(L);
  if (osplit)
    for (int l = 0; l < L; l++)
      for (int rb = 0; rb < o_blocks; rb++) c_oticket[l].push_back(b.new_counter(l * ST_PER_LAYER + ST_O));

  for (int l = 0; l < L; l++) {
    const int stg = l * ST_PER_LAYER;
    // ------------------------------------------------------------ QKV
    {
      const int R = qd + 2 * kvd;
      const int64_t N = R / gd.rpu;
      for (int cu = 0; cu < C; cu++) {
        int64_t i0, i1;
        split(N, cu, &i0, &i1);
        if (i1 <= i0) continue;
        const int r0 = int(i0 * gd.rpu), r1 = int(i1 * gd.rpu);
        Instr I = blank();
        I.op = OP_GEMV;
        I.epi = EPI_STORE;
        I.nit = uint8_t(gd.nit);
        I.rpu = uint8_t(gd.rpu);
        I.layer = uint16_t(l);
        I.flags = F_NORM | F_SIGNAL | (l == 0 ? F_IN_EMBED : 0);
        I.n_items = uint32_t(i1 - i0);
        I.row0 = uint32_t(r0);
        I.row_bytes = uint32_t(2 * d);
        I.n_rows = uint32_t(r1 - r0);
        I.k = uint32_t(d);
        // split [r0, r1) over Wq | Wk | Wv
        const int bounds[4] = {0, qd, qd + kvd, qd + 2 * kvd};
        const void* mats[3] = {in.w.wq, in.w.wk, in.w.wv};
        const int mrows[3] = {qd, kvd, kvd};
        int ns = 0;
        for (int s = 0; s < 3; s++) {
          int lo = std::max(r0, bounds[s]), hi = std::min(r1, bounds[s + 1]);
          if (hi <= lo) continue;
          I.seg_ptr[ns] = lptr(mats[s], l, uint64_t(mrows[s]) * d) + 2ull * d * (lo - bounds[s]);
          I.seg_rows[ns] = uint32_t(hi - lo);
          I.seg_stride[ns] = uint32_t(2 * d);
          ns++;
        }
        I.aux[4] = uint32_t(ns);
        I.in_ptr = l == 0 ? embed : A + ar.x[l];
        I.out_ptr = A + ar.qkv[l];
        I.gain_ptr = lptr(in.w.attn_norm, l, d);
        if (l > 0) set_wait(I, 0, c_down[l - 1]);
        I.sig_ctr = c_qkv[l];
        I.n_pages = uint32_t(ceil_div(int64_t(I.n_rows) * I.row_bytes, kPageBytes));
        InstrMeta m;
        m.stage = stg + ST_QKV;
        m.merge_write = false;
        m.reads.push_back({l == 0 ? BUF_EMBED : BUF_X, l, 0, uint64_t(d)});
        m.writes.push_back({BUF_QKV, l, uint64_t(r0), uint64_t(r1)});
        b.push(cu, I, std::move(m), int64_t(I.n_rows) * I.row_bytes);
      }
    }
    // ----------------------------------------------------------- ATTN
    for (int a = 0; a < n_att; a++) {
      // tile a: head tile tg = a / nblk (heads tg*hpt .. of the layer), block a % nblk
      const int tg = a / nblk, blk = a % nblk;
      const int g = tg / tpg, h0 = (tg % tpg) * hpt;
      Instr I = blank();
      I.op = OP_ATTN;
      I.layer = uint16_t(l);
      I.flags = F_SIGNAL;
      I.n_items = uint32_t(hpt);  // query heads of the tile
      I.row0 = uint32_t(h0);      // first of them within the group
      I.row_bytes = uint32_t(kv_rb);
      I.n_rows = uint32_t(2 * Bat);
      I.aux[0] = uint32_t(g);
      I.aux[1] = uint32_t(blk);
      I.aux[2] = uint32_t(Bat);
      I.aux[3] = uint32_t(nblk);
      I.aux[4] = uint32_t(kp);
      const uint64_t head_rows = uint64_t(S) * Dh;  // elements per (layer, seq, group)
      I.seg_ptr[0] = uint64_t(in.w.k_cache) + 2ull * head_rows * (uint64_t(l) * G + g);
      I.seg_ptr[1] = uint64_t(in.w.v_cache) + 2ull * head_rows * (uint64_t(l) * G + g);
      I.seg_rows[0] = nblk > 1 ? c_ticket[l][tg] : kNoCounter;
      I.in_ptr = A + ar.qkv[l];
      I.out_ptr = A + ar.o[l];
      I.res_ptr = A + ar.part[l];
      set_wait(I, 0, c_qkv[l]);
      I.sig_ctr = c_attn[l];
      I.n_pages = uint32_t(2 * kp);
      InstrMeta m;
      m.stage = stg + ST_ATTN;
      m.merge_write = nblk > 1;
      const uint64_t q0 = uint64_t(g * hpg + h0) * Dh, q1 = q0 + uint64_t(hpt) * Dh;
      m.reads.push_back({BUF_QKV, l, q0, q1});
      m.reads.push_back({BUF_QKV, l, uint64_t(qd + g * Dh), uint64_t(qd + (g + 1) * Dh)});
      m.reads.push_back({BUF_QKV, l, uint64_t(qd + kvd + g * Dh), uint64_t(qd + kvd + (g + 1) * Dh)});
      m.writes.push_back({BUF_O, l, q0, q1});
      // bytes streamed at full context
      const int64_t rows = std::min<int64_t>(Bat, std::max<int64_t>(0, int64_t(S) - int64_t(blk) * Bat));
      b.push(att_cu(a), I, std::move(m), 2 * rows * kv_rb);
    }
    // -------------------------------------------------------------- O
    if (osplit) {
      const int64_t N = d / gk.rpu;
      for (int rb = 0; rb < o_blocks; rb++) {
        const int64_t i0 = N * rb / o_blocks, i1 = N * (rb + 1) / o_blocks;
        const int r0 = int(i0 * gk.rpu), r1 = int(i1 * gk.rpu);
        for (int g = 0; g < G; g++) {
          const int cu = o_cu_of_rank[(rb * G + g) % o_cus];
          Instr I = blank();
          I.op = OP_GEMV;
          I.epi = EPI_OPART;
          I.nit = uint8_t(gk.nit);
          I.rpu = uint8_t(gk.rpu);
          I.layer = uint16_t(l);
          I.flags = F_SIGNAL | (l == 0 ? F_RES_EMBED : 0);
          I.n_items = uint32_t(i1 - i0);
          I.row0 = uint32_t(r0);
          I.row_bytes = uint32_t(2 * Kg);
          I.n_rows = uint32_t(r1 - r0);
          I.k = uint32_t(Kg);
          I.seg_ptr[0] = lptr(in.w.wo, l, uint64_t(d) * qd) + 2ull * qd * r0 + 2ull * Kg * g;
          I.seg_rows[0] = uint32_t(r1 - r0);
          I.seg_stride[0] = uint32_t(2 * qd);
          I.aux[1] = uint32_t(g);
          I.aux[2] = c_oticket[l][rb];
          I.aux[3] = uint32_t(G);
          I.aux[4] = 1;
          I.in_ptr = A + ar.o[l] + uint64_t(kActBytes) * g * Kg;
          I.out_ptr = A + ar.opart[l] + 4ull * g * d;
          I.res_ptr = l == 0 ? embed : A + ar.x[l];
          I.seg_ptr[2] = A + ar.h[l];
          set_wait(I, 0, c_attn[l]);
          I.sig_ctr = c_o[l];
          I.n_pages = uint32_t(ceil_div(int64_t(I.n_rows) * I.row_bytes, kPageBytes));
          InstrMeta m;
          m.stage = stg + ST_O;
          // the block's G tiles share the merged rows of h (written by the
          // tile that takes the last ticket)
          m.merge_write = true;
          m.reads.push_back({BUF_O, l, uint64_t(g) * Kg, uint64_t(g + 1) * Kg});
          m.reads.push_back({l == 0 ? BUF_EMBED : BUF_X, l, uint64_t(r0), uint64_t(r1)});
          m.writes.push_back({BUF_H, l, uint64_t(r0), uint64_t(r1)});
          b.push(cu, I, std::move(m), int64_t(I.n_rows) * I.row_bytes);
        }
      }
    } else {
      const int64_t N = d / gq.rpu;
      for (int cu = 0; cu < C; cu++) {
        int64_t c0, c1;
        // With few attention tiles, their CUs take no O rows: they finish
        // attention when the O stage can start, and would otherwise be its
        // last to finish.  The other CUs share the rows evenly.
        if (o_skip_att) {
          if (o_rank[cu] < 0) continue;
          c0 = N * o_rank[cu] / o_cus;
          c1 = N * (o_rank[cu] + 1) / o_cus;
        } else {
          split(N, cu, &c0, &c1);
        }
        const int64_t step = kMaxResRows / gq.rpu;  // residual rows staged per tile
        for (int64_t i0 = c0; i0 < c1; i0 += step) {
        const int64_t i1 = std::min(c1, i0 + step);
        const int r0 = int(i0 * gq.rpu), r1 = int(i1 * gq.rpu);
        Instr I = blank();
        I.op = OP_GEMV;
        I.epi = EPI_RESID;
        I.nit = uint8_t(gq.nit);
        I.rpu = uint8_t(gq.rpu);
        I.layer = uint16_t(l);
        I.flags = F_SIGNAL | (l == 0 ? F_RES_EMBED : 0);
        I.n_items = uint32_t(i1 - i0);
        I.row0 = uint32_t(r0);
        I.row_bytes = uint32_t(2 * qd);
        I.n_rows = uint32_t(r1 - r0);
        I.k = uint32_t(qd);
        I.seg_ptr[0] = lptr(in.w.wo, l, uint64_t(d) * qd) + 2ull * qd * r0;
        I.seg_rows[0] = uint32_t(r1 - r0);
        I.seg_stride[0] = uint32_t(2 * qd);
        I.aux[4] = 1;
        I.in_ptr = A + ar.o[l];
        I.res_ptr = l == 0 ? embed : A + ar.x[l];
        I.out_ptr = A + ar.h[l];
        set_wait(I, 0, c_attn[l]);
        I.sig_ctr = c_o[l];
        I.n_pages = uint32_t(ceil_div(int64_t(I.n_rows) * I.row_bytes, kPageBytes));
        InstrMeta m;
        m.stage = stg + ST_O;
        m.merge_write = false;
        m.reads.push_back({BUF_O, l, 0, uint64_t(qd)});
        m.reads.push_back({l == 0 ? BUF_EMBED : BUF_X, l, uint64_t(r0), uint64_t(r1)});
        m.writes.push_back({BUF_H, l, uint64_t(r0), uint64_t(r1)});
        b.push(cu, I, std::move(m), int64_t(I.n_rows) * I.row_bytes);
        }
      }
    }
    // ------------------------------------------------------- GATE/UP
    // One instruction per chunk and CU, or (gu_all) one per CU holding its
    // pairs of every chunk, chunk by chunk: all chunks read the same input,
    // and the per-element tags let a down-projection chunk start on its
    // input while later chunks are still being computed.
    for (int ch = 0; ch < (gu_all ? 1 : chunks); ch++) {
      const int64_t N = Fc;  // pairs
      for (int cu = 0; cu < C; cu++) {
        int64_t i0, i1;
        split(N, cu, &i0, &i1);
        if (i1 <= i0) continue;
        const int p0 = ch * Fc + int(i0), p1 = ch * Fc + int(i1);
        const int nch = gu_all ? chunks : 1;  // chunks in the instruction
        Instr I = blank();
        I.op = OP_GEMV;
        I.epi = EPI_SWIGLU;
        I.nit = uint8_t(gd.nit);
        I.rpu = uint8_t(gd.rpu);
        I.layer = uint16_t(l);
        I.flags = F_NORM | F_SIGNAL | F_INTERLEAVE | (gu_all ? F_GU_ALL : 0);
        I.n_items = uint32_t(nch * (p1 - p0));
        I.row0 = uint32_t(p0);
        I.row_bytes = uint32_t(2 * d);
        I.n_rows = 2 * I.n_items;
        I.k = uint32_t(d);
        I.seg_ptr[0] = lptr(in.w.w_gate, l, uint64_t(F) * d) + 2ull * d * p0;
        I.seg_ptr[1] = lptr(in.w.w_up, l, uint64_t(F) * d) + 2ull * d * p0;
        I.seg_rows[0] = I.seg_rows[1] = I.n_items;
        I.seg_stride[0] = I.seg_stride[1] = uint32_t(2 * d);
        if (gu_all) {
          I.aux[1] = uint32_t(p1 - p0);
          I.aux[2] = uint32_t(Fc);
          I.aux[3] = uint32_t(chunks);
        }
        I.aux[4] = 2;
        I.in_ptr = A + ar.h[l];
        I.out_ptr = A + ar.m[l];
        I.gain_ptr = lptr(in.w.mlp_norm, l, d);
        set_wait(I, 0, c_o[l]);
        I.sig_ctr = c_gu[l][ch];
        I.n_pages = uint32_t(ceil_div(int64_t(I.n_rows) * I.row_bytes, kPageBytes));
        InstrMeta m;
        m.stage = stg + ST_GU;
        m.merge_write = false;
        m.reads.push_back({BUF_H, l, 0, uint64_t(d)});
        for (int k = 0; k < nch; k++)
          m.writes.push_back({BUF_M, l, uint64_t(k * Fc + p0), uint64_t(k * Fc + p1)});
        b.push(cu, I, std::move(m), int64_t(I.n_rows) * I.row_bytes);
      }
    }
    // ---------------------------------------------------------- DOWN
    {
      const int64_t N = d / gf.rpu;
      for (int cu = 0; cu < C; cu++) {
        int64_t c0, c1;
        split(N, cu, &c0, &c1);
        if ((c1 - c0) * gf.rpu > 256) {
          *err = "plan: more than 256 down-projection rows on one CU";
          return MK_ERR_UNSUPPORTED;
        }
        const int64_t step = kMaxResRows / gf.rpu;
        for (int64_t i0 = c0; i0 < c1; i0 += step) {
        const int64_t i1 = std::min(c1, i0 + step);
        const int r0 = int(i0 * gf.rpu), r1 = int(i1 * gf.rpu);
        const uint32_t acc_off = uint32_t((i0 - c0) * gf.rpu);
        for (int ch = 0; ch < chunks; ch++) {
          Instr I = blank();
          I.op = OP_GEMV;
          I.epi = chunks == 1 ? EPI_ACC_ONLY
                              : (ch == 0 ? EPI_ACC_FIRST : (ch == chunks - 1 ? EPI_ACC_LAST : EPI_ACC_MID));
          I.nit = uint8_t(gf.nit);
          I.rpu = uint8_t(gf.rpu);
          I.layer = uint16_t(l);
          const bool last = ch == chunks - 1;
          I.flags = last ? F_SIGNAL : 0;
          I.n_items = uint32_t(i1 - i0);
          I.row0 = uint32_t(r0);
          I.row_bytes = uint32_t(2 * Fc);
          I.n_rows = uint32_t(r1 - r0);
          I.k = uint32_t(Fc);
          I.seg_ptr[0] = lptr(in.w.w_down, l, uint64_t(d) * F) + 2ull * (uint64_t(F) * r0 + uint64_t(ch) * Fc);
          I.seg_rows[0] = uint32_t(r1 - r0);
          I.seg_stride[0] = uint32_t(2 * F);
          I.aux[0] = acc_off;  // LDS accumulator offset
          I.aux[4] = 1;
          I.in_ptr = A + ar.m[l] + uint64_t(kActBytes) * ch * Fc;
          I.res_ptr = A + ar.h[l];
          I.out_ptr = A + ar.x[l + 1];
          set_wait(I, 0, c_gu[l][gu_all ? 0 : ch]);
          I.sig_ctr = last ? c_down[l] : kNoCounter;
          I.n_pages = uint32_t(ceil_div(int64_t(I.n_rows) * I.row_bytes, kPageBytes));
          InstrMeta m;
          m.stage = stg + ST_DOWN;
          m.merge_write = false;
          m.reads.push_back({BUF_M, l, uint64_t(ch) * Fc, uint64_t(ch + 1) * Fc});
          if (ch == 0) m.reads.push_back({BUF_H, l, uint64_t(r0), uint64_t(r1)});
          if (last) m.writes.push_back({BUF_X, l + 1, uint64_t(r0), uint64_t(r1)});
          b.push(cu, I, std::move(m), int64_t(I.n_rows) * I.row_bytes);
        }
        }
      }
    }
  }
  // ------------------------------------------------------------ LM head
  {
    const int64_t N = V / gd.rpu;
    int tile = 0;
    std::vector<int> lm_cus;
    for (int cu = 0; cu < C; cu++) {
      int64_t i0, i1;
      split(N, cu, &i0, &i1);
      if (i1 > i0) lm_cus.push_back(cu);
    }
    const int n_lm = int(lm_cus.size());
    for (int cu : lm_cus) {
      int64_t i0, i1;
      split(N, cu, &i0, &i1);
      const int r0 = int(i0 * gd.rpu), r1 = int(i1 * gd.rpu);
      Instr I = blank();
      I.op = OP_GEMV;
      I.epi = EPI_ARGMAX;
      I.nit = uint8_t(gd.nit);
      I.rpu = uint8_t(gd.rpu);
      I.layer = uint16_t(L);
      I.flags = F_NORM | F_SIGNAL;
      I.n_items = uint32_t(i1 - i0);
      I.row0 = uint32_t(r0);
      I.row_bytes = uint32_t(2 * d);
      I.n_rows = uint32_t(r1 - r0);
      I.k = uint32_t(d);
      I.seg_ptr[0] = lm + 2ull * d * r0;
      I.seg_rows[0] = uint32_t(r1 - r0);
      I.seg_stride[0] = uint32_t(2 * d);
      I.aux[1] = uint32_t(tile);
      I.aux[3] = uint32_t(n_lm);
      I.aux[4] = 1;
      I.in_ptr = A + ar.x[L];
      I.gain_ptr = uint64_t(in.w.final_norm);
      set_wait(I, 0, c_down[L - 1]);
      I.sig_ctr = c_lm;
      I.n_pages = uint32_t(ceil_div(int64_t(I.n_rows) * I.row_bytes, kPageBytes));
      InstrMeta m;
      m.stage = L * ST_PER_LAYER;
      m.merge_write = false;
      m.reads.push_back({BUF_X, L, 0, uint64_t(d)});
      m.writes.push_back({BUF_LOGITS, 0, uint64_t(r0), uint64_t(r1)});
      b.push(cu, I, std::move(m), int64_t(I.n_rows) * I.row_bytes);
      tile++;
    }
    P->lm_tiles = n_lm;
  }

  // producers per counter (per step)
  for (int cu = 0; cu < C; cu++)
    for (const Instr& I : b.q[cu]) {
      uint32_t tc, tn;
      if (ticketed(I, &tc, &tn)) {
        // every tile of the set takes a ticket; the last one signals
        P->ctr_producers[tc]++;
        continue;
      }
      if ((I.flags & F_SIGNAL) && I.sig_ctr != kNoCounter) P->ctr_producers[I.sig_ctr]++;
    }
  for (int l = 0; l < L; l++) {
    if (nblk > 1) P->ctr_producers[c_attn[l]] = uint32_t(G * tpg);
    if (osplit) P->ctr_producers[c_o[l]] = uint32_t(o_blocks);
  }
  // fill wait counts
  for (int cu = 0; cu < C; cu++)
    for (Instr& I : b.q[cu])
      for (int k = 0; k < 2; k++)
        if (I.wait_ctr[k] != kNoCounter) I.wait_cnt[k] = P->ctr_producers[I.wait_ctr[k]];
  // flatten
  P->q_off.assign(C + 1, 0);
  for (int cu = 0; cu < C; cu++) {
    P->q_off[cu + 1] = P->q_off[cu] + uint32_t(b.q[cu].size());
    P->instrs.insert(P->instrs.end(), b.q[cu].begin(), b.q[cu].end());
    P->meta.insert(P->meta.end(), b.qm[cu].begin(), b.qm[cu].end());
  }
  P->n_counters = int(P->ctr_stage.size());
  // packed weight stream: each GEMV instruction's rows in consumption order
  uint64_t pack = 0;
  for (Instr& I : P->instrs) {
    if (I.op != OP_GEMV) continue;
    I.src_ptr = in.pack_base + pack;
    const bool inter = I.flags & F_INTERLEAVE;
    if (I.flags & F_GU_ALL) {
      // gate/up pairs of every chunk, chunk by chunk, each chunk's rows
      // interleaved
      const uint32_t n = I.aux[1];
      for (uint32_t ch = 0; ch < I.aux[3]; ch++)
        for (uint32_t sg = 0; sg < 2; sg++) {
          PackCopy cp{};
          cp.src = I.seg_ptr[sg] + uint64_t(ch) * I.aux[2] * I.seg_stride[sg];
          cp.rows = n;
          cp.row_bytes = I.row_bytes;
          cp.src_stride = I.seg_stride[sg];
          cp.dst = pack + (uint64_t(ch) * 2 * n + sg) * I.row_bytes;
          cp.dst_stride = 2 * I.row_bytes;
          P->pack.push_back(cp);
        }
      pack += uint64_t(I.n_pages) * kPageBytes;
      continue;
    }
    uint64_t row = 0;
    for (uint32_t sg = 0; sg < I.aux[4]; sg++) {
      if (!I.seg_rows[sg]) continue;
      PackCopy cp{};
      cp.src = I.seg_ptr[sg];
      cp.rows = I.seg_rows[sg];
      cp.row_bytes = I.row_bytes;
      cp.src_stride = I.seg_stride[sg];
      cp.dst = pack + (inter ? uint64_t(sg) * I.row_bytes : row * I.row_bytes);
      cp.dst_stride = inter ? 2 * I.row_bytes : I.row_bytes;
      row += cp.rows;
      P->pack.push_back(cp);
    }
    pack += uint64_t(I.n_pages) * kPageBytes;
  }
  P->pack_bytes = pack;
  // bytes
  int64_t wbytes = 0;
  wbytes += int64_t(L) * 2 * (int64_t(qd + 2 * kvd) * d + int64_t(d) * qd + 3ll * F * d + 2ll * d);
  wbytes += 2ll * V * d + 2ll * d + 2ll * d;
  P->weight_bytes = wbytes;
  P->max_cu_bytes = *std::max_element(b.cu_bytes.begin(), b.cu_bytes.end());
  P->min_cu_bytes = *std::min_element(b.cu_bytes.begin(), b.cu_bytes.end());
  return MK_OK;
}

// ------------------------------------------------------------------ verify
mk_status verify_plan(const PlanInput& in, const Plan& p, std::string* err, uint64_t seed) {
  auto fail = [&](const std::string& m) {
    *err = "verify: " + m;
    return MK_ERR_INVALID_ARG;
  };
  const int C = p.n_cus;
  const int NC = p.n_counters;
  const mk_config& c = in.cfg;
  // 1. counter producers match signalling instructions; waits use them
  std::vector<uint32_t> sig(NC, 0);
  for (const Instr& I : p.instrs) {
    uint32_t tc, tn;
    if (ticketed(I, &tc, &tn)) {
      if (tc >= uint32_t(NC)) return fail("ticket counter out of range");
      sig[tc]++;
    } else if ((I.flags & F_SIGNAL) && I.sig_ctr != kNoCounter) {
      if (I.sig_ctr >= uint32_t(NC)) return fail("signal counter out of range");
      sig[I.sig_ctr]++;
    }
  }
  for (size_t i = 0; i < p.instrs.size(); i++) {
    const Instr& I = p.instrs[i];
    for (int k = 0; k < 2; k++) {
      if (I.wait_ctr[k] == kNoCounter) continue;
      const uint32_t ct = I.wait_ctr[k];
      if (ct >= uint32_t(NC)) return fail("wait counter out of range");
      if (I.wait_cnt[k] != p.ctr_producers[ct]) {
        std::ostringstream s;
        s << "instruction " << i << " waits for " << I.wait_cnt[k] << " signals on counter " << ct
          << " which has " << p.ctr_producers[ct] << " producers";
        return fail(s.str());
      }
      // 2. stage order: every wait names a counter of a strictly earlier stage
      if (p.ctr_stage[ct] >= p.meta[i].stage) return fail("wait on a counter of the same or a later stage");
    }
    // expert instructions: the loader waits on the router counter
    if (I.op == OP_EGU || I.op == OP_EDN) {
      if (I.aux[0] >= uint32_t(NC) || I.aux[1] != p.ctr_producers[I.aux[0]])
        return fail("expert instruction router counter");
      if (p.ctr_stage[I.aux[0]] >= p.meta[i].stage) return fail("router counter of the same or a later stage");
    }
  }
  // a split attention signals once per head tile: by the tile that takes
  // the last ticket of that head tile's blocks
  std::vector<std::vector<uint32_t>> merged_by(NC);
  for (const Instr& I : p.instrs) {
    uint32_t tc, tn;
    if (ticketed(I, &tc, &tn) && I.sig_ctr < uint32_t(NC)) merged_by[I.sig_ctr].push_back(tc);
  }
  for (int ct = 0; ct < NC; ct++) {
    std::vector<uint32_t>& t = merged_by[ct];
    std::sort(t.begin(), t.end());
    t.erase(std::unique(t.begin(), t.end()), t.end());
    const uint32_t expect = t.empty() ? sig[ct] : uint32_t(t.size());
    if (expect != p.ctr_producers[ct]) {
      std::ostringstream s;
      s << "counter " << ct << " expects " << p.ctr_producers[ct] << " producers, plan has " << expect;
      return fail(s.str());
    }
  }
  // 3. queue order per CU is by stage; pages are contiguous and within budget
  std::vector<std::vector<std::pair<uint32_t, uint32_t>>> shares(c.n_layers);
  for (int cu = 0; cu < C; cu++) {
    uint32_t page = 0;
    int last_stage = -1;
    for (uint32_t i = p.q_off[cu]; i < p.q_off[cu + 1]; i++) {
      const Instr& I = p.instrs[i];
      const InstrMeta& m = p.meta[i];
      if (m.stage < last_stage) return fail("queue not ordered by stage");
      last_stage = m.stage;
      if (I.page0 != page) return fail("page stream not contiguous");
      page += I.n_pages;
      if (I.op == OP_BGEMV) {
        if (!p.batched) return fail("batched GEMV in a one-sequence plan");
        if (I.k % 512 || I.nit != I.k / 512 || I.row_bytes != 2 * I.k) return fail("batched row geometry");
        if (uint64_t(I.k) * c.batch > uint64_t(lb::kXFloats)) return fail("batched input exceeds the x slot");
        if (I.flags & F_MFMA) {
          // blocks of 16 rows in fragment order, consumed one 1 KiB column
          // step at a time by all compute waves
          if (I.aux[4] != 1 || I.n_items != uint32_t(ceil_div(I.n_rows, 16)) ||
              uint64_t(I.n_pages) * kPageBytes < uint64_t(16) * I.n_items * I.row_bytes)
            return fail("matrix-core tile geometry");
        } else {
          if (uint64_t(I.n_pages) * kPageBytes < uint64_t(2) * I.n_items * I.row_bytes)
            return fail("page budget smaller than the tile");
          if (I.n_items != (I.n_rows + 1) / 2) return fail("row pairs");
          if (uint32_t(ceil_div(2 * I.row_bytes, kPageBytes)) + 1 > uint32_t(lb::kPages))
            return fail("an item spans more pages than the ring holds");
        }
        uint32_t srows = 0;
        for (uint32_t sg = 0; sg < I.aux[4]; sg++) srows += I.seg_rows[sg];
        if (srows != I.n_rows) return fail("segments do not cover the stream rows");
        if (I.epi == EPI_RESID && uint64_t(I.n_rows) * c.batch > uint64_t(kMaxResRows))
          return fail("residual rows exceed the LDS staging slot");
        continue;
      }
      if (I.op == OP_EGU) {
        if (!p.batched) return fail("expert instruction in a one-sequence plan");
        const uint32_t ppe = I.aux[2];
        if (I.k % 512 || I.nit != I.k / 512 || I.row_bytes != 2 * I.k) return fail("expert row geometry");
        if (I.flags & F_SHARE) {
          // a weighted share of every selected expert's rows
          if (!(I.flags & F_DIRECT) || I.row0 || I.aux[3] != uint32_t(c.expert_ffn) ||
              I.seg_rows[1] > I.seg_rows[2] || I.seg_rows[2] > 65536u)
            return fail("expert gate/up share");
          shares[I.layer].push_back({I.seg_rows[1], I.seg_rows[2]});
        } else if (uint64_t(ppe) * kPageBytes < 2ull * I.seg_rows[0] || ppe > uint32_t(lb::kPages) - 1) {
          return fail("expert page regions");
        }
        if (I.n_pages != ((I.flags & F_DIRECT) ? 0 : ppe * I.aux[4]) || I.aux[4] != uint32_t(c.n_experts))
          return fail("expert page budget");
        if ((I.flags & F_DIRECT) && (I.nit != 1 && I.nit != 2 && I.nit != 4)) return fail("direct expert loads");
        if (I.seg_rows[0] != I.aux[3] * I.row_bytes) return fail("expert gate/up runs");
        continue;
      }
      if (I.op == OP_EDN) {
        if (!p.batched) return fail("expert instruction in a one-sequence plan");
        const uint32_t ppu = I.aux[2], Rb = I.aux[3], nb = I.aux[4];
        if (I.k % 512 || I.nit != I.k / 512 || I.row_bytes != 2 * I.k || I.k != uint32_t(c.expert_ffn))
          return fail("expert row geometry");
        if (!Rb || Rb != I.n_rows || nb != uint32_t(ceil_div(c.hidden, Rb)) || I.seg_rows[0] != Rb * I.row_bytes ||
            ppu != uint32_t(ceil_div(I.seg_rows[0], kPageBytes)))
          return fail("expert down-projection units");
        // a 4-row item lies in at most kPages - 1 pages; every sequence routed
        // to one expert fits the x slot at once
        if (uint32_t(ceil_div(4 * I.row_bytes, kPageBytes)) + 1 > uint32_t(lb::kPages) ||
            uint64_t(c.batch) * I.k > uint64_t(lb::kXFloats))
          return fail("expert down-projection items");
        if (I.n_items != uint32_t(C) ||
            I.n_pages != ((I.flags & F_DIRECT) ? 0u : uint32_t(c.n_experts) * nb * ppu) ||
            ((I.flags & F_DIRECT) && I.nit > 2))
          return fail("expert down-projection page budget");
        continue;
      }
      if (I.op == OP_ERD) {
        if (!p.batched) return fail("expert sum in a one-sequence plan");
        if (I.n_pages || !I.n_rows || I.row0 + I.n_rows > uint32_t(c.hidden)) return fail("expert sum rows");
        continue;
      }
      if (I.op == OP_GEMV) {
        if (p.batched) return fail("one-sequence GEMV in a batched plan");
        const uint64_t need = uint64_t(I.n_rows) * I.row_bytes;
        if (uint64_t(I.n_pages) * kPageBytes < need) return fail("page budget smaller than the tile");
        if (I.rpu == 1 && I.row_bytes != uint32_t(I.nit) * kUnit) return fail("row geometry");
        if (I.rpu == 2 && I.row_bytes != kUnit / 2) return fail("row geometry (512 B rows)");
        // bytes one compute wave needs resident at once (a row, or a gate/up pair)
        const uint32_t item_bytes = I.rpu == 2 ? uint32_t(kUnit)
                                               : (I.epi == EPI_SWIGLU ? 2 : 1) * I.row_bytes;
        if (uint32_t(ceil_div(item_bytes, kPageBytes)) + 1 > uint32_t(kPages))
          return fail("an item spans more pages than the ring holds");
        if (I.k > uint32_t(kMaxK)) return fail("input longer than the staging buffer");
        if (I.epi == EPI_SWIGLU && I.n_rows != 2 * I.n_items) return fail("gate/up pairs");
        if (I.epi != EPI_SWIGLU && I.n_rows != I.n_items * I.rpu) return fail("items vs rows");
        uint32_t srows = 0;
        for (uint32_t s = 0; s < I.aux[4]; s++) srows += I.seg_rows[s];
        if (srows != I.n_rows) return fail("segments do not cover the stream rows");
      } else {
        const int ring = p.batched ? lb::kPages : kPages;
        if (2 * I.aux[4] != I.n_pages || 2 * I.aux[4] > uint32_t(ring)) return fail("attention page regions");
        if (I.n_items * I.aux[2] > uint32_t(p.batched ? lb::kScoreFloats : kAttnScoreFloats))
          return fail("attention scores exceed the LDS scratch");
      }
    }
  }
  // weighted gate/up shares of a layer tile [0, 65536) exactly
  for (auto& sh : shares) {
    if (sh.empty()) continue;
    std::sort(sh.begin(), sh.end());
    uint32_t at = 0;
    for (const auto& s : sh) {
      if (s.first != at) return fail("gate/up shares do not tile the layer's items");
      at = s.second;
    }
    if (at != 65536u) return fail("gate/up shares do not tile the layer's items");
  }
  // 4. read coverage: every element read must be written by an instruction
  //    whose signal the reader transitively waits for; each element written once
  // happens-before closure over counters (bitsets)
  std::vector<std::vector<uint64_t>> hb(NC, std::vector<uint64_t>((NC + 63) / 64, 0));
  // counters each counter's producers wait on
  std::vector<std::vector<uint32_t>> waits_of(NC);
  for (const Instr& I : p.instrs) {
    uint32_t sc = kNoCounter;
    uint32_t tc, tn;
    const bool tk = ticketed(I, &tc, &tn);
    if (tk) sc = I.sig_ctr;  // the merger waits like every tile
    else if ((I.flags & F_SIGNAL) && I.sig_ctr != kNoCounter) sc = I.sig_ctr;
    if (tk) waits_of[tc].push_back(I.wait_ctr[0]);
    if (sc == kNoCounter) continue;
    for (int k = 0; k < 2; k++)
      if (I.wait_ctr[k] != kNoCounter) waits_of[sc].push_back(I.wait_ctr[k]);
  }
  // DOWN chunks other than the last do not signal, yet the last chunk's result
  // depends on them (same waves, program order): their waits belong to the
  // down counter's closure too.
  for (size_t i = 0; i < p.instrs.size(); i++) {
    const Instr& I = p.instrs[i];
    if (I.op == OP_GEMV && (I.epi == EPI_ACC_FIRST || I.epi == EPI_ACC_MID)) {
      // find the last chunk of the same tile later in the same queue
      for (size_t j = i + 1; j < p.instrs.size() && p.meta[j].cu == p.meta[i].cu; j++) {
        const Instr& J = p.instrs[j];
        if (J.op == OP_GEMV && J.epi == EPI_ACC_LAST && J.layer == I.layer && J.row0 == I.row0) {
          for (int k = 0; k < 2; k++)
            if (I.wait_ctr[k] != kNoCounter) waits_of[J.sig_ctr].push_back(I.wait_ctr[k]);
          break;
        }
      }
    }
  }
  // counters are numbered in stage order, so one pass in increasing order works
  std::vector<int> order(NC);
  for (int i = 0; i < NC; i++) order[i] = i;
  std::sort(order.begin(), order.end(), [&](int a, int b2) { return p.ctr_stage[a] < p.ctr_stage[b2]; });
  for (int ct : order) {
    hb[ct][ct / 64] |= 1ull << (ct % 64);
    for (uint32_t w : waits_of[ct]) {
      if (p.ctr_stage[w] >= p.ctr_stage[ct]) return fail("cyclic counter dependency");
      for (size_t k = 0; k < hb[ct].size(); k++) hb[ct][k] |= hb[w][k];
    }
  }
  auto in_closure = [&](const Instr& I, uint32_t ct) {
    for (int k = 0; k < 2; k++)
      if (I.wait_ctr[k] != kNoCounter && (hb[I.wait_ctr[k]][ct / 64] >> (ct % 64) & 1)) return true;
    return false;
  };
  // writers per buffer: (layer, lo, hi, signal counter, merge)
  struct W {
    uint64_t lo, hi;
    uint32_t ctr;
    bool merge;
  };
  std::map<std::pair<int, int>, std::vector<W>> writers;
  for (size_t i = 0; i < p.instrs.size(); i++) {
    const Instr& I = p.instrs[i];
    uint32_t ct = I.sig_ctr;
    if (I.op == OP_GEMV && I.epi == EPI_ACC_LAST) ct = I.sig_ctr;
    for (const Range& r : p.meta[i].writes) writers[{r.buf, r.layer}].push_back({r.lo, r.hi, ct, p.meta[i].merge_write});
  }
  for (auto& kv : writers) {
    auto& v = kv.second;
    std::sort(v.begin(), v.end(), [](const W& a, const W& b2) { return a.lo < b2.lo; });
    for (size_t k = 1; k < v.size(); k++)
      if (v[k].lo < v[k - 1].hi && !(v[k].merge && v[k - 1].merge && v[k].lo == v[k - 1].lo && v[k].hi == v[k - 1].hi))
        return fail(std::string("buffer ") + kBufName[kv.first.first] + " written twice");
  }
  for (size_t i = 0; i < p.instrs.size(); i++) {
    const Instr& I = p.instrs[i];
    for (const Range& r : p.meta[i].reads) {
      if (r.buf == BUF_EMBED) continue;  // input of the step
      auto it = writers.find({r.buf, r.layer});
      if (it == writers.end()) return fail(std::string("read of never-written buffer ") + kBufName[r.buf]);
      uint64_t covered = r.lo;
      for (const W& w : it->second) {
        if (w.hi <= r.lo || w.lo >= r.hi) continue;
        if (w.lo > covered) break;
        if (!in_closure(I, w.ctr)) {
          std::ostringstream s;
          s << "instruction " << i << " (stage " << p.meta[i].stage << ") reads " << kBufName[r.buf]
            << "[" << r.layer << "] without waiting for its writer's counter " << w.ctr;
          return fail(s.str());
        }
        covered = std::max(covered, w.hi);
      }
      if (covered < r.hi) {
        std::ostringstream s;
        s << "instruction " << i << " reads " << kBufName[r.buf] << "[" << r.layer << "][" << covered
          << "] which no instruction writes";
        return fail(s.str());
      }
    }
  }
  // 5. memory bounds: every DMA source range lies inside a weight tensor or
  //    the KV cache, every activation pointer inside the arena or embedding
  {
    struct Ext {
      uint64_t lo, hi;
      const char* name;
    };
    const uint64_t L = c.n_layers, d = c.hidden, qd = uint64_t(c.n_q_heads) * c.head_dim,
                   kvd = uint64_t(c.n_kv_heads) * c.head_dim, F = c.ffn, V = c.vocab;
    const uint64_t kv_bytes = 2ull * L * c.batch * c.n_kv_heads * c.max_seq * c.head_dim;
    const uint64_t NE = c.n_experts > 0 ? c.n_experts : 0, Fe = c.expert_ffn > 0 ? c.expert_ffn : 0,
                   NB = c.batch;
    const Ext ext[] = {
        {uint64_t(in.w.embed), uint64_t(in.w.embed) + 2 * V * d, "embed"},
        {uint64_t(in.w.lm_head), uint64_t(in.w.lm_head) + 2 * V * d, "lm_head"},
        {uint64_t(in.w.wq), uint64_t(in.w.wq) + 2 * L * qd * d, "wq"},
        {uint64_t(in.w.wk), uint64_t(in.w.wk) + 2 * L * kvd * d, "wk"},
        {uint64_t(in.w.wv), uint64_t(in.w.wv) + 2 * L * kvd * d, "wv"},
        {uint64_t(in.w.wo), uint64_t(in.w.wo) + 2 * L * d * qd, "wo"},
        {uint64_t(in.w.w_gate), uint64_t(in.w.w_gate) + 2 * L * F * d, "w_gate"},
        {uint64_t(in.w.w_up), uint64_t(in.w.w_up) + 2 * L * F * d, "w_up"},
        {uint64_t(in.w.w_down), uint64_t(in.w.w_down) + 2 * L * d * F, "w_down"},
        {uint64_t(in.w.k_cache), uint64_t(in.w.k_cache) + kv_bytes, "k_cache"},
        {uint64_t(in.w.v_cache), uint64_t(in.w.v_cache) + kv_bytes, "v_cache"},
        {uint64_t(in.w.router), uint64_t(in.w.router) + 2 * L * NE * d, "router"},
        {uint64_t(in.w.e_gate), uint64_t(in.w.e_gate) + 2 * L * NE * Fe * d, "e_gate"},
        {uint64_t(in.w.e_up), uint64_t(in.w.e_up) + 2 * L * NE * Fe * d, "e_up"},
        {uint64_t(in.w.e_down), uint64_t(in.w.e_down) + 2 * L * NE * d * Fe, "e_down"},
    };
    auto inside = [&](uint64_t lo, uint64_t hi) {
      for (const Ext& e : ext)
        if (lo >= e.lo && hi <= e.hi) return true;
      return false;
    };
    const uint64_t A = in.arena_base, Aend = in.arena_base + p.arena.total;
    auto in_arena = [&](uint64_t lo, uint64_t hi) { return lo >= A && hi <= Aend; };
    // packed stream: instruction runs back to back inside the buffer, and
    // every copy reads weight rows and writes inside the buffer
    uint64_t next_src = in.pack_base, stream_bytes = 0, copied = 0;
    for (const Instr& I : p.instrs) {
      if (I.op != OP_GEMV && I.op != OP_BGEMV) continue;
      if (I.src_ptr != next_src) return fail("packed weight runs are not back to back");
      next_src += uint64_t(I.n_pages) * kPageBytes;
      stream_bytes += uint64_t(I.n_rows) * I.row_bytes;
    }
    if (next_src != in.pack_base + p.pack_bytes) return fail("packed weight stream size");
    for (const PackCopy& cp : p.pack) {
      if (!cp.rows || cp.row_bytes % 16 || cp.src_stride % 16 || cp.dst_stride % 16 || cp.src % 16)
        return fail("packed copy not in 16-byte units");
      if (!inside(cp.src, cp.src + uint64_t(cp.rows - 1) * cp.src_stride + cp.row_bytes))
        return fail("packed copy reads outside every weight tensor");
      const uint64_t span = cp.frag ? uint64_t(ceil_div(cp.rows, 16)) * 16 * cp.row_bytes
                                    : uint64_t(cp.rows - 1) * cp.dst_stride + cp.row_bytes;
      if (cp.dst + span > p.pack_bytes) return fail("packed copy writes outside the packed stream");
      copied += uint64_t(cp.rows) * cp.row_bytes;
    }
    if (copied != stream_bytes) return fail("packed copies do not cover the weight streams");
    for (size_t i = 0; i < p.instrs.size(); i++) {
      const Instr& I = p.instrs[i];
      const uint64_t EB = kActBytes;
      if (I.op == OP_BGEMV) {
        for (uint32_t sg = 0; sg < I.aux[4]; sg++) {
          if (!I.seg_rows[sg]) continue;
          const uint64_t lo = I.seg_ptr[sg];
          if (!inside(lo, lo + uint64_t(I.seg_rows[sg] - 1) * I.seg_stride[sg] + I.row_bytes))
            return fail("batched GEMV streams bytes outside every weight tensor");
        }
        if (I.flags & F_IN_EMBED) {
          if (I.in_ptr != uint64_t(in.w.embed) || I.k != uint32_t(d)) return fail("embedding input pointer");
        } else if (!in_arena(I.in_ptr, I.in_ptr + EB * NB * I.k)) {
          return fail("batched GEMV input outside the arena");
        }
        const uint64_t last = (NB - 1) * I.aux[0] + I.row0 + I.n_rows;
        if (I.epi != EPI_ARGMAX && !in_arena(I.out_ptr, I.out_ptr + EB * last))
          return fail("batched GEMV output outside the arena");
        if (I.epi == EPI_ARGMAX && (I.aux[0] != V || I.row0 + I.n_rows > V || I.aux[1] >= I.aux[3] ||
                                    I.aux[3] > uint32_t(p.n_cus)))
          return fail("LM head tile");
        if (I.epi == EPI_RESID) {
          const uint64_t rl = (NB - 1) * I.aux[2] + I.row0 + I.n_rows;
          if ((I.flags & F_RES_EMBED) ? (I.res_ptr != uint64_t(in.w.embed) || I.aux[2] != d)
                                      : !in_arena(I.res_ptr, I.res_ptr + EB * rl))
            return fail("batched GEMV residual outside the arena");
        }
        continue;
      }
      if (I.op == OP_EGU || I.op == OP_EDN) {
        const uint64_t stride = I.seg_stride[0], run = I.seg_rows[0];
        const uint64_t mb = EB * NB * c.top_k * Fe;
        if (!in_arena(I.seg_ptr[0], I.seg_ptr[0] + EB * NB * NE)) return fail("router logits outside the arena");
        if (I.op == OP_EGU) {
          for (int r = 0; r < 2; r++) {
            const uint64_t lo = I.seg_ptr[1 + r];
            if (!inside(lo, lo + (NE - 1) * stride + run)) return fail("expert runs outside the expert tensors");
          }
          if (I.row0 + I.aux[3] > Fe) return fail("expert gate/up slice");
          if (!(I.flags & F_IN_EMBED) && !in_arena(I.in_ptr, I.in_ptr + EB * NB * d))
            return fail("expert input outside the arena");
          if (!in_arena(I.out_ptr, I.out_ptr + mb)) return fail("expert intermediate outside the arena");
        } else {
          // the loader clips a unit to the expert's d rows
          const uint64_t lo = I.seg_ptr[1];
          if (stride != 2ull * d * Fe || !inside(lo, lo + (NE - 1) * stride + d * I.row_bytes))
            return fail("expert units outside the expert tensors");
          if (!in_arena(I.in_ptr, I.in_ptr + mb)) return fail("expert intermediate outside the arena");
          if (!in_arena(I.out_ptr, I.out_ptr + EB * NB * c.top_k * d)) return fail("expert outputs outside the arena");
          if (!in_arena(I.res_ptr, I.res_ptr + 8)) return fail("ready-queue counters outside the arena");
        }
        continue;
      }
      if (I.op == OP_ERD) {
        const uint64_t rl = (NB - 1) * d + I.row0 + I.n_rows;
        if (!in_arena(I.in_ptr, I.in_ptr + EB * NB * c.top_k * d) || !in_arena(I.res_ptr, I.res_ptr + EB * rl) ||
            !in_arena(I.out_ptr, I.out_ptr + EB * rl) || (I.seg_ptr[0] && !in_arena(I.seg_ptr[0], I.seg_ptr[0] + 8)))
          return fail("expert sum rows outside the arena");
        continue;
      }
      if (I.op == OP_GEMV) {
        for (uint32_t sg = 0; sg < I.aux[4]; sg++) {
          if (!I.seg_rows[sg]) continue;
          const uint64_t lo = I.seg_ptr[sg];
          const uint64_t hi = lo + uint64_t(I.seg_rows[sg] - 1) * I.seg_stride[sg] + I.row_bytes;
          if (!inside(lo, hi)) {
            std::ostringstream m;
            m << "instruction " << i << " streams bytes outside every weight tensor";
            return fail(m.str());
          }
        }
        const uint64_t kb = uint64_t(kActBytes) * I.k;
        if (I.flags & F_IN_EMBED) {
          if (I.in_ptr != uint64_t(in.w.embed)) return fail("embedding input pointer");
        } else if (!in_arena(I.in_ptr, I.in_ptr + kb)) {
          return fail("GEMV input outside the arena");
        }
        uint64_t out_rows = I.rpu == 2 && I.epi != EPI_SWIGLU ? uint64_t(I.n_items) * 2 : I.n_items;
        if (I.epi == EPI_OPART) {
          // the layer's partials [G][d] (fp32), the merged rows of h and the
          // residual rows the merging tile reads
          const uint64_t pb = I.out_ptr - 4ull * I.aux[1] * d;
          if (I.aux[3] != uint32_t(c.n_kv_heads) || I.aux[1] >= I.aux[3] || I.row0 + out_rows > d ||
              !in_arena(pb, pb + 4ull * I.aux[3] * d))
            return fail("split-K O partials outside the arena");
          if (!in_arena(I.seg_ptr[2] + 8 * I.row0, I.seg_ptr[2] + 8 * (I.row0 + out_rows)))
            return fail("split-K O output outside the arena");
          if ((I.flags & F_RES_EMBED) ? I.res_ptr != uint64_t(in.w.embed)
                                      : !in_arena(I.res_ptr + 8 * I.row0, I.res_ptr + 8 * (I.row0 + out_rows)))
            return fail("split-K O residual outside the arena");
        }
        uint64_t out_hi = I.row0 + out_rows;  // one past the last output row
        if (I.flags & F_GU_ALL) {
          if (I.epi != EPI_SWIGLU || !I.aux[1] || I.aux[3] < 2 || I.n_items != I.aux[1] * I.aux[3] ||
              uint64_t(I.aux[2]) * I.aux[3] != uint64_t(c.ffn) || I.row0 + I.aux[1] > I.aux[2])
            return fail("gate/up over every chunk: chunk geometry");
          out_hi = I.row0 + uint64_t(I.aux[3] - 1) * I.aux[2] + I.aux[1];
        }
        if (I.epi != EPI_ARGMAX && I.epi != EPI_ACC_FIRST && I.epi != EPI_ACC_MID && I.epi != EPI_OPART &&
            !in_arena(I.out_ptr + uint64_t(kActBytes) * I.row0, I.out_ptr + uint64_t(kActBytes) * out_hi))
          return fail("GEMV output outside the arena");
        if ((I.epi == EPI_RESID || I.epi == EPI_ACC_ONLY || I.epi == EPI_ACC_FIRST) &&
            !(I.flags & F_RES_EMBED) &&
            !in_arena(I.res_ptr + uint64_t(kActBytes) * I.row0, I.res_ptr + uint64_t(kActBytes) * (I.row0 + out_rows)))
          return fail("GEMV residual outside the arena");
        if ((I.epi == EPI_ACC_FIRST || I.epi == EPI_ACC_MID || I.epi == EPI_ACC_LAST) &&
            I.aux[0] + out_rows > 256)
          return fail("down-projection accumulators exceed the LDS area");
        if ((I.epi == EPI_RESID || I.epi == EPI_ACC_ONLY || I.epi == EPI_ACC_FIRST) &&
            out_rows > uint64_t(kMaxResRows))
          return fail("residual rows exceed the LDS staging slot");
      } else {
        const uint64_t span = uint64_t(c.max_seq) * I.row_bytes;
        if (!inside(I.seg_ptr[0], I.seg_ptr[0] + span) || !inside(I.seg_ptr[1], I.seg_ptr[1] + span))
          return fail("attention cache rows outside the KV cache");
        const uint64_t hpg = c.n_q_heads / c.n_kv_heads, hpt = I.n_items;
        if (!hpt || hpg % hpt || I.row0 % hpt || I.row0 + hpt > hpg) return fail("attention head tile");
        // partial records of the tile's head group: [tg][nblk][hpt][Dh + 2]
        const uint64_t tg = (uint64_t(I.aux[0]) * hpg + I.row0) / hpt;
        const uint64_t rec = hpt * (c.head_dim + 2) * 4;
        if (I.aux[3] > 1 && !in_arena(I.res_ptr, I.res_ptr + rec * (tg + 1) * I.aux[3]))
          return fail("attention partials outside the arena");
        if (!in_arena(I.in_ptr, I.in_ptr + uint64_t(kActBytes) * (qd + 2 * kvd)) ||
            !in_arena(I.out_ptr, I.out_ptr + uint64_t(kActBytes) * qd))
          return fail("attention activations outside the arena");
      }
    }
  }
  // 6. randomized execution of the queues: every instruction must run
  std::mt19937_64 rng(seed);
  for (int trial = 0; trial < 3; trial++) {
    std::vector<uint32_t> val(NC, 0), head(C, 0), ticket(NC, 0);
    size_t done = 0, total = p.instrs.size();
    std::vector<int> cus(C);
    for (int i = 0; i < C; i++) cus[i] = i;
    while (done < total) {
      std::shuffle(cus.begin(), cus.end(), rng);
      bool progress = false;
      for (int cu : cus) {
        uint32_t idx = p.q_off[cu] + head[cu];
        if (idx >= p.q_off[cu + 1]) continue;
        const Instr& I = p.instrs[idx];
        bool ready = true;
        for (int k = 0; k < 2; k++)
          if (I.wait_ctr[k] != kNoCounter && val[I.wait_ctr[k]] < I.wait_cnt[k]) ready = false;
        if (!ready) continue;
        uint32_t tc, tn;
        if (ticketed(I, &tc, &tn)) {
          if (++ticket[tc] == tn) val[I.sig_ctr]++;
        } else if ((I.flags & F_SIGNAL) && I.sig_ctr != kNoCounter) {
          val[I.sig_ctr]++;
        }
        head[cu]++;
        done++;
        progress = true;
      }
      if (!progress) {
        std::ostringstream s;
        s << "deadlock in queue simulation after " << done << " of " << total << " instructions";
        return fail(s.str());
      }
    }
  }
  return MK_OK;
}

void corrupt_one_target(Plan* p) {
  // the first waiting instruction of the last CU queue: raise its counter
  // target and make its staging expect a tag that this step never writes
  for (int cu = p->n_cus - 1; cu >= 0; cu--)
    for (uint32_t i = p->q_off[cu]; i < p->q_off[cu + 1]; i++)
      if (p->instrs[i].wait_ctr[0] != kNoCounter) {
        p->instrs[i].wait_cnt[0] += 1;
        p->instrs[i].flags |= F_DEBUG_STALL;
        return;
      }
}

void rebase_pack(Plan* p, uint64_t old_base, uint64_t base) {
  for (Instr& I : p->instrs)
    if (I.op == OP_GEMV || I.op == OP_BGEMV) I.src_ptr = I.src_ptr - old_base + base;
}

void summarize(const PlanInput& in, const Plan& p, mk_plan_summary* s) {
  std::memset(s, 0, sizeof(*s));
  s->n_cus = p.n_cus;
  s->n_instr = int32_t(p.instrs.size());
  uint32_t mq = 0;
  for (int cu = 0; cu < p.n_cus; cu++) mq = std::max(mq, p.q_off[cu + 1] - p.q_off[cu]);
  s->max_queue = int32_t(mq);
  s->n_counters = p.n_counters;
  s->lds_bytes = p.batched ? lb::kTotal : kLdsTotal;
  s->n_pages = p.batched ? lb::kPages : kPages;
  s->page_bytes = kPageBytes;
  s->attn_block = p.attn_block;
  s->attn_tiles = p.attn_tiles;
  s->mlp_chunks = p.mlp_chunks;
  s->weight_bytes = p.weight_bytes;
  s->max_cu_bytes = p.max_cu_bytes;
  s->min_cu_bytes = p.min_cu_bytes;
  const uint64_t sc = scratch_layout(p).total;
  s->scratch_bytes = int32_t(std::min<uint64_t>(sc, uint64_t(INT32_MAX)));
  (void)in;
}

ScratchLayout scratch_layout(const Plan& p) {
  ScratchLayout s;
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t r = off;
    off = align256(off + bytes);
    return r;
  };
  s.act = take(p.arena.rope_cos);
  s.slots = take(p.arena.status - p.arena.lm_slots);
  s.status = take(64);
  s.route = take(4 * 128);
  s.ctr_bytes = uint64_t(std::max(1, p.n_counters)) * kCtrSpread * kCtrStride * 4;
  s.ctr = take(s.ctr_bytes);
  s.total = off;
  return s;
}

std::vector<Instr> rebase_to_scratch(const Plan& p, uint64_t arena_base, uint64_t scratch_base) {
  const uint64_t lo = arena_base, hi = arena_base + p.arena.rope_cos;
  auto mv = [&](uint64_t& v) {
    if (v >= lo && v < hi) v = scratch_base + (v - lo);
  };
  std::vector<Instr> out = p.instrs;
  for (Instr& I : out) {
    mv(I.in_ptr);
    mv(I.res_ptr);
    mv(I.out_ptr);
    mv(I.gain_ptr);
    mv(I.src_ptr);
    for (int k = 0; k < 3; k++) mv(I.seg_ptr[k]);
  }
  return out;
}

std::string plan_report(const PlanInput& in, const Plan& p) {
  std::ostringstream s;
  mk_plan_summary sm;
  summarize(in, p, &sm);
  s << "{\"n_cus\": " << sm.n_cus << ", \"n_instr\": " << sm.n_instr << ", \"max_queue\": " << sm.max_queue
    << ", \"n_counters\": " << sm.n_counters << ", \"lds_bytes\": " << sm.lds_bytes
    << ", \"n_pages\": " << sm.n_pages << ", \"attn_block\": " << sm.attn_block
    << ", \"attn_tiles\": " << sm.attn_tiles << ", \"mlp_chunks\": " << sm.mlp_chunks
    << ", \"lm_tiles\": " << p.lm_tiles << ", \"weight_bytes\": " << sm.weight_bytes
    << ", \"max_cu_bytes\": " << sm.max_cu_bytes << ", \"min_cu_bytes\": " << sm.min_cu_bytes
    << ", \"arena_bytes\": " << p.arena.total << ", \"queue_lengths\": [";
  for (int cu = 0; cu < p.n_cus; cu++) s << (cu ? ", " : "") << (p.q_off[cu + 1] - p.q_off[cu]);
  s << "]}";
  return s.str();
}

}  // namespace mk
