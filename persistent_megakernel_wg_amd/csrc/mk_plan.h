// mk_plan.h — host planner for the decode megakernel (pure C++, no HIP).
//
// Static scheduling as in the Llama-1B megakernel write-up (javascript.cn
// article, "Megakernel：从零设计的融合思路": every SM gets an execution plan,
// dependencies are settled before the run): the planner cuts each stage of the
// decoder into tiles, places them on per-CU queues ordered by (layer, stage),
// gives every counter its producer count, sizes each tile's LDS page budget,
// and verifies the result.
#pragma once
#include <stdint.h>

#include <string>
#include <vector>

#include "mk.h"
#include "mk_isa.h"

namespace mk {

// Activation buffers of one step, as offsets from the arena base (bytes).
struct ArenaLayout {
  uint64_t x[129];        // residual stream entering layer l (x[0] unused: embedding)
  uint64_t qkv[128], o[128], h[128], m[128], part[128];
  uint64_t opart[128];    // [G][d] fp32 split-K O partials (one-sequence decoder)
  uint64_t rl[128];       // router logits (mixture-of-experts decoder)
  uint64_t y;             // [B][top_k][d] tagged expert outputs (mixture-of-experts decoder)
  uint64_t edn_ctr;       // [L][2] u32 ready-queue counters of the expert down projection
  uint64_t tok;           // [B] tagged greedy token of the last step
  uint64_t rope_cos, rope_sin, zero_page, lm_slots, status;
  uint64_t route_stats;   // [128] u32: selected experts per layer, summed over steps
  uint64_t total;
};

// Everything the planner needs: shape, options and the device addresses it
// bakes into the instructions (fake but consistent addresses in a dry run).
struct PlanInput {
  mk_config cfg;
  mk_plan_opts opts;
  int n_cus;
  mk_weights w;          // device pointers (may be fake)
  uint64_t arena_base;   // device address of the arena
  uint64_t pack_base;    // device address of the packed weight stream
};

// Verification view of one instruction.
struct Range {
  int buf;               // buffer id (see kBuf*)
  int layer;
  uint64_t lo, hi;       // element range [lo, hi)
};
struct InstrMeta {
  int cu;
  int stage;             // global stage order
  std::vector<Range> reads, writes;
  bool merge_write;      // writes shared by the tiles of one attention group
};

struct Plan {
  ArenaLayout arena;
  std::vector<uint32_t> q_off;      // [n_cus + 1]
  std::vector<Instr> instrs;        // queues back to back
  std::vector<InstrMeta> meta;      // parallel to instrs
  std::vector<uint32_t> ctr_producers;  // per counter: signals per step
  std::vector<int> ctr_stage;       // stage of the counter's producers
  std::vector<PackCopy> pack;       // copies that fill the packed weight stream
  uint64_t pack_bytes = 0;          // size of the packed weight stream
  int n_cus = 0, n_counters = 0;
  int attn_block = 0, attn_nblk = 0, attn_tiles = 0, attn_heads = 0, mlp_chunks = 0, lm_tiles = 0;
  bool batched = false;             // built for the batched (mixture-of-experts) kernel
  int64_t weight_bytes = 0, max_cu_bytes = 0, min_cu_bytes = 0;
};

// Arena layout for a shape (does not depend on the plan options).
ArenaLayout arena_layout(const mk_config& cfg, int max_lm_tiles, int max_parts);

// true for shapes run by the batched kernel (the mixture-of-experts decoder).
bool is_batched(const mk_config& cfg);

// Validate a shape for the kernel's code paths.  Returns MK_OK or an error
// with a message.
mk_status check_config(const mk_config& cfg, std::string* err);

// Build the plan.  Returns MK_OK, or MK_ERR_* with a message in *err.
mk_status build_plan(const PlanInput& in, Plan* out, std::string* err);

// Verify a plan: counter targets, stage order (no cycles), page budgets, read
// coverage through counter waits, single writers, and a randomized
// queue-order simulation that must run every instruction.  Returns MK_OK or
// MK_ERR_INVALID_ARG with the first violation in *err.
mk_status verify_plan(const PlanInput& in, const Plan& p, std::string* err, uint64_t seed = 1);

// Move the packed weight stream to `base` (the plan is built against
// in.pack_base; the runtime allocates the stream once its size is known).
void rebase_pack(Plan* p, uint64_t old_base, uint64_t base);

// Test hook: make one wait target unreachable (applied after verification by
// the runtime so that a step must end in the watchdog; mk_plan_check applies
// it before verification to show that the verifier rejects it).
void corrupt_one_target(Plan* p);

// Human-readable report (used by mk_plan_check).
std::string plan_report(const PlanInput& in, const Plan& p);

void summarize(const PlanInput& in, const Plan& p, mk_plan_summary* s);

// Scratch of one step in the fixed device array of mk_decode_step_noalloc
// (byte offsets): the tagged activations (the arena's [0, rope_cos)), the
// argmax slots, the status word, the routing statistics and the counters.
// The whole span is cleared before every such step.
struct ScratchLayout {
  uint64_t act, slots, status, route, ctr, ctr_bytes, total;
};
ScratchLayout scratch_layout(const Plan& p);

// The plan's instructions with every arena activation address moved into the
// scratch at `scratch_base` (weights, packed stream and caches unchanged).
std::vector<Instr> rebase_to_scratch(const Plan& p, uint64_t arena_base, uint64_t scratch_base);

// GEMV row geometry for input length K: 1 KiB units per row (nit) and rows
// per unit (rpu).  false if the kernel has no code path for K.
bool gemv_geometry(int K, int* nit, int* rpu);

// Resolved defaults for the options.
mk_plan_opts resolve_opts(const mk_config& cfg, const mk_plan_opts* opts, int n_cus);

}  // namespace mk
