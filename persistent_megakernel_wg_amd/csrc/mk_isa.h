// mk_isa.h — instruction records and launch arguments shared by the host
// planner and the persistent megakernel.
//
// Every instruction follows one template, as in the Llama-1B megakernel
// write-up (javascript.cn article, "Megakernel：从零设计的融合思路": each
// instruction standardises load, compute and store): its weight (or KV) stream
// is copied into LDS pages by the loader waves, its input dependencies are
// counters in global memory, its compute waves read the pages, and its last
// wave increments one counter when the outputs are visible.
#pragma once
#include <stdint.h>

namespace mk {

// ---------------------------------------------------------------- constants
constexpr int kNLoad = 2;            // loader waves per workgroup
constexpr int kNComp = 6;            // compute waves per workgroup (2 waves per SIMD with the loaders)
constexpr int kThreads = 64 * (kNLoad + kNComp);
constexpr int kUnit = 1024;          // bytes per wave-wide 16 B/lane DMA
constexpr int kPageBytes = 16384;    // LDS page (16 KiB, as on the pages' design)
constexpr int kUnitsPerPage = kPageBytes / kUnit;
constexpr int kPages = 8;            // pages in the LDS ring
constexpr int kCtrStride = 32;       // u32 per counter line (128 B apart)
// A counter is kCtrSpread lines: a producer on CU c adds to line
// c % kCtrSpread and a waiter sums the lines.  Many producers adding to one
// line serialise on it (256 atomics on one address take several
// microseconds); spread, each line takes a sixteenth of them.  Tickets
// (counters whose returned value picks the last arriver) use line 0 only.
constexpr int kCtrSpread = 16;
constexpr int kMaxK = 4096;          // largest GEMV input length
constexpr int kDoneRing = 4;         // per-instruction completion counters
// Activation element in global memory: fp32 value | u32 tag (the step that
// wrote it).  A consumer accepts an element only when its tag is the current
// step, so producers signal their counters without waiting for their stores.
constexpr int kActBytes = 8;

// LDS layout (bytes)
constexpr int kLdsCtrl = 0;          // control words
constexpr int kLdsSS = 512;          // per-wave shares of an input's sum of squares
constexpr int kLdsPf = 768;          // 256 B sink of the loaders' L2 prefetch loads (never read)
constexpr int kLdsAcc = 1024;        // down-projection accumulators (256 floats)
constexpr int kLdsX = 2048;          // staged input vector / q,k,v (16 KiB)
constexpr int kLdsXBytes = 4 * kMaxK;
constexpr int kLdsAttn = kLdsX + kLdsXBytes;   // attention scratch
constexpr int kLdsAttnBytes = 12800;   // scores 8 KiB, new V row 512 B, partials 4 KiB
constexpr int kLdsPages = kLdsAttn + kLdsAttnBytes;
// staged residual rows: two slots (by instruction parity) of 128 floats
constexpr int kLdsRes = kLdsPages + kPages * kPageBytes;
constexpr int kMaxResRows = 128;
constexpr int kLdsTotal = kLdsRes + 2 * 4 * kMaxResRows;      // 163328
constexpr int kAttnScoreFloats = 2048;                       // 8 KiB of scores

// LDS layout of the batched kernel (several sequences per step).  The staged
// GEMV input holds all B sequences' vectors ([B][K] fp32, 64 KiB), so the page
// ring is shorter.  Control words keep the offsets of the layout above.
namespace lb {
constexpr int kMaxB = 8;             // sequences per step
constexpr int kPages = 5;
constexpr int kSS = 512;             // sum of squares per 128-value chunk [128]
constexpr int kArg = 1024;           // argmax per compute wave and sequence [kNComp][kMaxB][2]
constexpr int kMfma = 1536;          // 4 KiB: the matrix-core GEMV's per-wave partial block sums
                                     // (LM head), and the expert down projection's ready queue
                                     // (two layer parities of 512 entries)
constexpr int kMfmaWaveBytes = 512;  // [16 rows][8 sequences] fp32 per wave
constexpr int kMaxDnRows = 16;
constexpr int kMaxTopK = 8;
constexpr int kRoute = kMfma + 4 * kMaxB * kMaxTopK * kMaxDnRows;   // 5632: routing tables
constexpr int kRouteBytes = 1280;    // one table per layer parity
constexpr int kRes = kRoute + 2 * kRouteBytes;                      // 8192: residual rows
constexpr int kX = kRes + 2 * 4 * kMaxResRows;                      // 9216
constexpr int kXFloats = 16384;      // [B][K] staged input, K <= 16384 / B
constexpr int kAttn = kX + 4 * kXFloats;                            // 74752
constexpr int kScoreFloats = 512;    // attention scores of one tile
constexpr int kAttnBytes = 4 * kScoreFloats + 512 + 64;
constexpr int kPg = ((kAttn + kAttnBytes + 1023) / 1024) * 1024;   // 77824
constexpr int kTotal = kPg + kPages * kPageBytes;                   // 159744
static_assert(kTotal <= 163840, "batched LDS layout exceeds 160 KiB");
static_assert(kRoute % 16 == 0 && kX % 16 == 0 && kAttn % 16 == 0, "alignment");
constexpr int kMaxExperts = 64;
}  // namespace lb

// ------------------------------------------------------------------- opcodes
enum Op : uint8_t {
  OP_GEMV = 1,        // one-sequence GEMV tile
  OP_ATTN = 2,        // decode attention tile (one sequence)
  OP_BGEMV = 3,       // batched GEMV tile: every row applied to all B sequences
  OP_EGU = 4,         // expert gate/up slice of every selected expert (SwiGLU)
  OP_EDN = 5,         // expert down-projection units of the selected experts
  OP_ERD = 6,         // weighted sum of the top-k expert outputs + residual
};

// GEMV epilogues
enum Epi : uint8_t {
  EPI_STORE = 0,      // out[r] = dot                        (q/k/v projection)
  EPI_RESID = 1,      // out[r] = res[r] + dot               (O projection)
  EPI_SWIGLU = 2,     // out[r] = silu(dot_gate) * dot_up    (gate/up pairs)
  EPI_ACC_FIRST = 3,  // acc[r] = res[r] + dot               (down-proj chunk 0)
  EPI_ACC_MID = 4,    // acc[r] += dot
  EPI_ACC_LAST = 5,   // out[r] = acc[r] + dot               (last chunk)
  EPI_ACC_ONLY = 6,   // out[r] = res[r] + dot  (single-chunk down projection)
  EPI_ARGMAX = 7,     // logits + greedy argmax              (LM head)
  EPI_OPART = 8,      // part[g][r] = dot, split-K O projection of KV group g
};

// instruction flags
enum Flag : uint16_t {
  F_NORM = 1,         // RMSNorm the input vector with gain_ptr before the GEMV
  F_IN_EMBED = 2,     // input vector is the bf16 embedding row of the token
  F_RES_EMBED = 4,    // residual is the bf16 embedding row of the token
  F_INTERLEAVE = 8,   // stream rows alternate between segments 0 and 1
  F_SIGNAL = 16,      // increment sig_ctr when done
  F_OWN_POS = 32,     // (attention) placeholder, decided at run time
  F_ROUTE = 64,       // (experts) first expert instruction of its layer on the CU:
                      // take the top-k routing decision from the router logits
  F_DIRECT = 128,     // (expert gate/up and down) the compute waves load the
                      // weight rows themselves; the instruction takes no LDS pages
  F_DEBUG_STALL = 256,  // tests only: staging expects the next step's tag, so the
                        // inputs never turn fresh and the watchdog ends the step
  F_MFMA = 512,         // (batched GEMV) matrix-core tiles of 16 rows: the input
                        // is staged as bf16 hi + lo parts in MFMA operand order
                        // and the packed rows are in MFMA fragment order
  F_SHARE = 1024,       // (expert gate/up) a weighted share of the layer's (expert,
                        // row) items instead of a slice of rows of every expert
  F_GU_ALL = 2048,      // (gate/up) the CU's pairs of every MLP chunk in one
                        // instruction, chunk by chunk (GEMV aux fields below)
};

constexpr uint32_t kNoCounter = 0xFFFFFFFFu;

// One instruction.  Pointers are device addresses fixed at plan time.
struct alignas(16) Instr {
  uint8_t op;
  uint8_t epi;
  uint8_t nit;         // 1 KiB units per stream row (rows >= 1 KiB), else 1
  uint8_t rpu;         // stream rows per 1 KiB unit (1, or 2 for 512 B rows)
  uint16_t flags;
  uint16_t layer;
  uint32_t n_items;    // GEMV: output items; ATTN: unused
  uint32_t row0;       // first output row
  uint32_t page0;      // first page of this instruction in the CU's page stream
  uint32_t n_pages;    // pages reserved for this instruction
  uint32_t row_bytes;  // bytes per stream row
  uint32_t n_rows;     // stream rows (all segments)
  uint32_t k;          // GEMV input length (floats)
  uint32_t wait_ctr[2];
  uint32_t wait_cnt[2];  // producers per step (0 = no wait); target = epoch * cnt
  uint32_t sig_ctr;
  uint32_t aux[5];     // op-specific
  uint64_t seg_ptr[3]; // stream segment base addresses
  uint32_t seg_rows[3];
  uint32_t seg_stride[3];
  uint64_t in_ptr;     // input vector (fp32) or embedding table (bf16)
  uint64_t res_ptr;    // residual (fp32) or embedding table (bf16)
  uint64_t out_ptr;    // output
  uint64_t gain_ptr;   // RMSNorm gain (bf16)
  uint64_t src_ptr;    // GEMV: this instruction's packed weight stream
};
static_assert(sizeof(Instr) % 16 == 0, "Instr must stay 16 B aligned");

// Packed weight stream.  At plan time every GEMV instruction's rows are copied,
// in the order the compute waves consume them (interleaved gate/up pairs,
// down-projection column chunks, the Wq|Wk|Wv concatenation), into one
// contiguous zero-padded run of n_pages * kPageBytes bytes at src_ptr, so
// that the loader waves stream plain consecutive 1 KiB units.
struct PackCopy {
  uint64_t src;        // first source row (device address)
  uint64_t dst;        // byte offset of the first row in the packed buffer
  uint32_t rows;
  uint32_t row_bytes;  // multiple of 16
  uint32_t src_stride; // bytes between source rows
  uint32_t dst_stride; // bytes between packed rows (0 with frag)
  uint32_t frag;       // 1: MFMA fragment order for blocks of 16 rows (below)
  uint32_t pad;
};
// MFMA fragment order (F_MFMA tiles, v_mfma_f32_16x16x32_bf16): rows go in
// blocks of 16, each block's K columns in steps of 32; step s of block b is
// one 1 KiB unit at (b * K / 32 + s) KiB, in which lane l's 16 bytes are the
// 8 values of row 16 b + (l % 16) at columns 32 s + 8 (l / 16) .. + 7, the A
// operand of that lane.  A block's rows past the copy are zero.

// Attention instruction aux fields
//   aux[0] = kv group g         aux[1] = block index b
//   aux[2] = positions/block    aux[3] = blocks per group (1 = no merge)
//   aux[4] = pages per K (and V) region
//   seg_ptr[0] = K cache rows of (layer, seq, g) from position 0
//   seg_ptr[1] = V cache rows of (layer, seq, g) from position 0
//   in_ptr = q|k|v activations of the layer; out_ptr = attention output
//   res_ptr = split partials of the layer; wait/sig as usual
//   seg_rows[0] = merge-ticket counter (blocks > 1)
// GEMV aux fields
//   aux[0] = LDS accumulator offset (down projection)
//   aux[1] = argmax slot index (LM head)
//   aux[2] = LM-head ticket counter, aux[3] = LM-head tiles
// Gate/up over every MLP chunk (EPI_SWIGLU with F_GU_ALL): aux[1] = pairs of
//   one chunk on this CU (n), aux[2] = pairs per chunk (Fc), aux[3] = chunks;
//   item t is pair row0 + (t / n) * Fc + t % n, and segment s (gate, up)
//   holds the n rows from seg_ptr[s] + ch * Fc * row_bytes for each chunk ch
// Split-K O projection (OP_GEMV, EPI_OPART): rows row0 .. row0 + n_rows of
// Wo[:, g*Kg .. (g+1)*Kg) . o_g, with Kg = (query heads per KV group) * Dh:
//   aux[1] = g, aux[2] = ticket counter of the row block, aux[3] = G (tiles
//   per row block); in_ptr = o + g*Kg (tagged); out_ptr = part + g*d (fp32,
//   untagged, behind the ticket); res_ptr = x_l (tagged) or the embedding
//   (F_RES_EMBED); seg_ptr[2] = h_l.  The tile taking the block's last ticket
//   writes h_l[r] = x_l[r] + part[0][r] + ... + part[G-1][r] (in g order).
// Batched GEMV (OP_BGEMV): rows are taken in pairs (n_items pairs); the input
// is [B][k], the output [B][aux[0]] and the residual [B][aux[2]] (elements);
//   aux[1] = argmax slot index, aux[3] = LM-head tiles (EPI_ARGMAX)
// Expert gate/up (OP_EGU): the weight runs are read in place.
//   aux[0] = router counter, aux[1] = its producers per step
//   aux[2] = pages per expert region, aux[3] = gate/up pairs, aux[4] = experts
//   seg_ptr[0] = router logits [B][E] (tagged)
//   seg_ptr[1] = first gate row, seg_ptr[2] = first up row of expert 0
//   seg_stride[0] = bytes between experts' runs; seg_rows[0] = bytes of a run
//   seg_stride[1] = pages of the gate run within an expert region
//   row0 = first FFN row of the slice; in_ptr = x; out_ptr = m [B][top_k][Fe]
//   F_SHARE (direct only): row0 = 0, seg_ptr[1], seg_ptr[2] = expert 0's
//   first rows; the CU takes items [T s0, T s1) / 65536 of the T =
//   (selected experts) x Fe (expert rank, row) items in that order, with
//   s0 = seg_rows[1] and s1 = seg_rows[2]
// Expert down projection (OP_EDN): units of n_rows (= aux[3]) consecutive
// down rows of one selected expert; the U = (selected experts) x aux[4] units
// of a layer, in expert order, go to the n_items CUs in even contiguous
// ranges, decided at run time from the routing.
//   aux[0], aux[1] as for OP_EGU; aux[2] = pages per unit; aux[4] = units per expert
//   seg_ptr[0] = router logits; seg_ptr[1] = expert 0's first down row
//   seg_stride[0] = bytes between experts; seg_rows[0] = bytes of a full unit
//   in_ptr = m [B][top_k][Fe]; out_ptr = y [B][top_k][d], tagged with
//   (step << 7) | layer
//   n_pages = the most pages a CU can take (the loader streams the CU's units),
//   or 0 with F_DIRECT (rows of at most 2 KiB: the compute waves load them)
//   row0 = q > 0: a 1/q share of the units waits in the ready queue, handed
//   out in chunks by the counter at res_ptr + 4 (step parity)
// Expert sum (OP_ERD): rows row0 .. row0 + n_rows of x_{l+1} for every sequence:
//   in_ptr = y, res_ptr = h, out_ptr = x_{l+1}

// Kernel launch arguments.
struct KArgs {
  const Instr* instrs;      // all queues back to back
  const uint32_t* q_off;    // [n_cus + 1] queue offsets
  uint32_t* counters;       // [n_ctr][kCtrSpread][kCtrStride]
  uint32_t* status;         // [16] error record
  const int32_t* tokens;    // [B], the input tokens of the launch's first step
  int32_t* next;            // [n_steps][B], the greedy token of every step
  float* logits;            // [n_steps][B, V] or null
  const float* rope_cos;    // [max_seq][Dh/2]
  const float* rope_sin;
  float* lm_slots;          // [n_lm_tiles][2] (value, index)
  const void* zero_page;    // 16 KiB of zeros (padding DMA source)
  uint32_t epoch;           // 1-based step count since the counters were zeroed
  int32_t pos;
  int32_t vocab;
  int32_t hidden;
  int32_t head_dim;
  int32_t hpg;              // query heads per KV group
  int32_t q_dim;            // H * Dh (offset of k in the qkv buffer)
  int32_t kv_dim;           // G * Dh
  int32_t max_seq;
  float rms_eps;
  float attn_scale;         // 1/sqrt(Dh)
  uint64_t watchdog_ticks;  // s_memrealtime ticks (100 MHz)
  uint32_t* trace;          // [n_cus][trace_stride][8] timestamps, or null
  uint32_t trace_stride;    // instructions per CU in the trace buffer
  int32_t batch;            // sequences per step
  int32_t n_experts;        // experts per layer (0 = dense MLP)
  int32_t top_k;            // experts per token
  int32_t expert_ffn;       // intermediate size of one expert
  uint32_t* route_stats;    // [L] distinct experts selected per layer, summed over steps
  uint32_t n_steps;         // decode steps run back to back by this launch (>= 1;
                            // only the one-sequence kernel runs more than one)
  uint64_t* tok_tag;        // [B] tagged copy of the last greedy token: value |
                            // epoch of the step that chose it (steps after the
                            // first read their input token here)
};

// trace record words (s_memrealtime, 100 MHz, low 32 bits)
enum TraceWord { TR_START = 0, TR_DEPS = 1, TR_STAGED = 2, TR_ITEMS = 3, TR_SIGNAL = 4,
                 TR_PAGEWAIT = 5, TR_HW0 = 6, TR_HW1 = 7, TR_XREADY = 8, TR_ITEM0 = 9,
                 TR_VISIBLE = 10, TR_XFREE = 11, TR_A_PASS1 = 12, TR_A_STATS = 13,
                 TR_A_PASS3 = 14, TR_RETRY = 15, TR_WORDS = 16 };

// status words
enum StatusWord { ST_CODE = 0, ST_CU = 1, ST_INSTR = 2, ST_CTR = 3, ST_SEEN = 4, ST_TARGET = 5,
                  ST_NAN = 6, ST_BADTOK = 7 };
enum StatusCode { STC_OK = 0, STC_TIMEOUT = 1, STC_LOCAL_TIMEOUT = 2, STC_TAG_TIMEOUT = 3 };

}  // namespace mk
