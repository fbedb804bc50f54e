// mk_dev.h — device code shared by the one-sequence and the batched
// megakernels: instruction field access, LDS control words, counters in global
// memory, bounded waits, the LDS page DMA of the loader waves, and the decode
// attention tile.
//
// The counter system follows the Llama-1B megakernel write-up (rocketrecap.com
// summary, "Custom Synchronization Mechanism"); the paged LDS follows its
// "Efficient Shared Memory Management" section; weights are fetched before the
// activation dependency is met (Cohere's write-up, airebao.com, «三点关键差异»
// item 3).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "mk_isa.h"

#define DEV __device__ __forceinline__
// Global memory is addressed through address-space-1 pointers so that every
// access is a global_* instruction: a flat access would also count on the
// LDS counter, and every LDS wait after it would wait for global memory.
#define GLB __attribute__((address_space(1)))

namespace mk {

template <class T>
DEV GLB T* gp(T* p) { return (GLB T*)p; }
template <class T>
DEV GLB T* gp(const T* p) { return (GLB T*)const_cast<T*>(p); }

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(4))) const Instr* InstrCP;

extern __shared__ __attribute__((aligned(1024))) char lds[];

// Sub-dword header fields are read as whole dwords (scalar loads only move
// dwords; a byte field would otherwise become a vector load, whose vmcnt would
// disturb the loader's DMA accounting).
typedef __attribute__((address_space(4))) const uint32_t* WordCP;
DEV uint32_t hw0(InstrCP I) { return reinterpret_cast<WordCP>(I)[0]; }
DEV uint32_t hw1(InstrCP I) { return reinterpret_cast<WordCP>(I)[1]; }
DEV uint32_t i_op(InstrCP I) { return hw0(I) & 0xFFu; }
DEV uint32_t i_epi(InstrCP I) { return (hw0(I) >> 8) & 0xFFu; }
DEV uint32_t i_nit(InstrCP I) { return (hw0(I) >> 16) & 0xFFu; }
DEV uint32_t i_rpu(InstrCP I) { return hw0(I) >> 24; }
DEV uint32_t i_flags(InstrCP I) { return hw1(I) & 0xFFFFu; }

// --------------------------------------------------------------- LDS control
enum : int {
  C_FILLED = 0,        // [kNLoad] pages published by each loader
  C_RELEASED = 16,     // [kNComp] pages below this index are done, per wave
  C_XOK = 64,          // instructions whose inputs are staged (leader staging)
  C_DEPOK = 68,        // instructions whose counter waits are satisfied
  C_MARR = 72,         // matrix-core GEMV: wave arrivals at block ends (all blocks)
  C_MRED = 76,         // matrix-core GEMV: blocks reduced so far
  C_RTOK = 80,         // batched kernel: layer + 1 of the last routing table written
  C_XCONS = 96,        // [kNComp] instructions whose staged inputs each wave read
  C_DONE = 128,        // [kDoneRing] waves finished, per instruction slot
  C_ABORT = 160,
  C_BAR = 176,
  C_ARGV = 192,        // [kNComp] best value per wave
  C_ARGI = 224,        // [kNComp] best index per wave
  C_STATUS_LO = 256,   // status pointer (written once at kernel entry)
  C_STATUS_HI = 260,
  C_LIMIT_LO = 264,    // time limit of local waits, s_memrealtime ticks
  C_LIMIT_HI = 268,
  C_TR_LOOP = 272,     // traced runs: earliest, latest end of the attention waves' loops
  C_CTRL_END = 280,
};
static_assert(C_FILLED + 4 * kNLoad <= C_RELEASED, "ctrl layout");
static_assert(C_RELEASED + 4 * kNComp <= C_XOK, "ctrl layout");
static_assert(C_XCONS + 4 * kNComp <= C_DONE, "ctrl layout");
static_assert(C_DONE + 4 * kDoneRing <= C_ABORT, "ctrl layout");
static_assert(C_CTRL_END <= kLdsSS && kLdsSS + 4 * kNComp <= kLdsPf && kLdsPf + 256 <= kLdsAcc, "ctrl layout");

DEV uint32_t* lw(int off) { return reinterpret_cast<uint32_t*>(lds + off); }
DEV uint32_t lds_ld(int off) {
  return __hip_atomic_load(lw(off), __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// relaxed LDS read: several of them are issued together; the caller adds a
// workgroup acquire fence once it has seen what it waited for
DEV uint32_t lds_ld_rlx(int off) {
  return __hip_atomic_load(lw(off), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
DEV void lds_st(int off, uint32_t v) {
  __hip_atomic_store(lw(off), v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
DEV uint32_t lds_add(int off, uint32_t v) {
  return __hip_atomic_fetch_add(lw(off), v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
}
DEV bool aborted() { return lds_ld(C_ABORT) != 0; }

// The status pointer and the local time limit live in LDS so that wait loops
// deep in the call tree can reach them.
DEV uint32_t* status_ptr() {
  return reinterpret_cast<uint32_t*>((uint64_t(*lw(C_STATUS_HI)) << 32) | *lw(C_STATUS_LO));
}
DEV uint64_t local_limit() { return (uint64_t(*lw(C_LIMIT_HI)) << 32) | *lw(C_LIMIT_LO); }
DEV uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
DEV uint64_t uni64(uint64_t v) {
  return (uint64_t(uni(uint32_t(v >> 32))) << 32) | uni(uint32_t(v));
}
// LDS layouts: the one-sequence kernel's and the batched kernel's (page ring,
// staged input slot, attention scratch).
struct LayA {
  static constexpr int pages = kPages, pg = kLdsPages, x = kLdsX, x_floats = kMaxK, attn = kLdsAttn,
                       score_floats = kAttnScoreFloats;
};
struct LayB {
  static constexpr int pages = lb::kPages, pg = lb::kPg, x = lb::kX, x_floats = lb::kXFloats,
                       attn = lb::kAttn, score_floats = lb::kScoreFloats;
};
template <class Lay>
DEV uint32_t page_off(uint32_t g) { return Lay::pg + (g % uint32_t(Lay::pages)) * kPageBytes; }

// ------------------------------------------------------ global memory access
DEV void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Counters and activations use device-scope (sc1) loads and stores; no L2
// writeback or invalidate is issued.
DEV uint32_t ctr_load(const uint32_t* p) {
  return __hip_atomic_load(gp(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Signal: the counter is bumped without waiting for this wave's stores.
// Consumers take activations only with the current step's tag, so the
// counter only says when it is worth looking.
DEV uint32_t ctr_signal(uint32_t* p) {
  return __hip_atomic_fetch_add(gp(p), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Ticket of the untagged data behind it (attention partials, argmax slots,
// split-K O partials).  Default: this wave's stores are waited for
// (s_waitcnt vmcnt(0): they are device-scope stores, acknowledged once
// visible at device scope) and the count moves with a relaxed add; the
// taker of the last ticket issues its loads of the others' data only after
// the add has returned (a control dependency), with device-scope loads.
// MK_ACQREL=1 builds the formal device-scope release / acquire pair instead
// (an L2 write-back before every ticket and an L2 invalidate by the last
// taker), which measured 2-21 % slower.
#ifndef MK_ACQREL
#define MK_ACQREL 0
#endif
DEV uint32_t ctr_release(uint32_t* p) {
#if MK_ACQREL
  return __hip_atomic_fetch_add(gp(p), 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
#else
  wait_vm0();
  return __hip_atomic_fetch_add(gp(p), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#endif
}
DEV void ctr_acquire() {
#if MK_ACQREL
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#endif
}
// untagged device-coherent scalar store / load
DEV void st_act(float* p, float v) {
  __hip_atomic_store(gp(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV float ld_act(const float* p) {
  return __hip_atomic_load(gp(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Tagged activation element (8 bytes): the fp32 value in the low word, the
// step (epoch) that wrote it in the high word, stored as one 8-byte access.
DEV void st_tag(uint64_t* p, float v, uint32_t tag) {
  const uint64_t w = uint64_t(__float_as_uint(v)) | (uint64_t(tag) << 32);
  __hip_atomic_store(gp(p), w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Loads through buffer resources: reads past the resource's size return
// zero without touching memory.  sc1 = device scope.
DEV __amdgpu_buffer_rsrc_t act_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
// The same for a base and size the compiler cannot prove wave-uniform (they
// are): readfirstlane keeps the descriptor in scalar registers, where the
// compiler would otherwise loop over the lanes for every load.
DEV __amdgpu_buffer_rsrc_t act_rsrc_u(const void* base, uint32_t bytes) {
  return act_rsrc(reinterpret_cast<const void*>(uni64(reinterpret_cast<uint64_t>(base))), uni(bytes));
}
DEV f4 ld_act4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16 /* sc1 */));
}
// two tagged elements {v0, tag0, v1, tag1}
DEV u4 ld_tag2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16));
}

DEV float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
DEV float bf_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
DEV uint16_t f2bf(float f) {  // round to nearest even (no NaN inputs expected)
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}
// input token of a step, checked against the vocabulary (an out-of-range id
// is reported and replaced by 0 so that no access leaves the embedding
// table).  The first step of a launch reads the caller's token; a later step
// reads the tagged copy the previous step's argmax wrote, polling until it
// carries that step's epoch (bounded by the watchdog: a stale tag past the
// limit aborts the workgroup and reads token 0).
DEV bool local_timeout_tok(uint64_t& t0, uint32_t& n, uint64_t limit);
DEV uint32_t token_of(const KArgs& a, uint32_t step, uint32_t ep) {
  int32_t t;
  if (step == 0) {
    t = *gp(a.tokens);
  } else {
    uint64_t t0 = 0;
    uint32_t n = 0;
    for (;;) {
      const uint64_t w = __hip_atomic_load(gp(a.tok_tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (uint32_t(w >> 32) == ep - 1) {
        t = int32_t(uint32_t(w));
        break;
      }
      if (local_timeout_tok(t0, n, a.watchdog_ticks)) {
        t = 0;
        break;
      }
    }
  }
  if (t >= 0 && t < a.vocab) return uint32_t(t);
  __hip_atomic_store(gp(a.status) + ST_BADTOK, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return 0;
}
DEV float silu(float z) { return z / (1.0f + __expf(-z)); }

DEV float dot8(u4 w, const float* x) {
  float a = bf_lo(w.x) * x[0];
  a = fmaf(bf_hi(w.x), x[1], a);
  float b = bf_lo(w.y) * x[2];
  b = fmaf(bf_hi(w.y), x[3], b);
  a = fmaf(bf_lo(w.z), x[4], a);
  a = fmaf(bf_hi(w.z), x[5], a);
  b = fmaf(bf_lo(w.w), x[6], b);
  b = fmaf(bf_hi(w.w), x[7], b);
  return a + b;
}

// Cross-lane reductions with DPP (quad permutes and row rotates/shifts inside
// 16-lane rows) and readlane across rows.  Fixed order: deterministic.
template <int CTRL>
DEV float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
DEV float rl(float v, int lane) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane)); }
// The value of lane l ^ OFF, exchanged in registers rather than through the
// LDS crossbar (what a generic shuffle compiles to): a DPP rotation by 8
// inside each 16-lane row for OFF = 8, and for 16 and 32 gfx950's lane-swap
// instructions, whose two results hold the lower and the upper row (half) of
// each pair; a lane takes the one it is not in.
template <int OFF>
DEV float lane_xor(float v) {
  const uint32_t l = threadIdx.x & 63;
  if constexpr (OFF == 8) {
    return dpp<0x128>(v);  // row_ror:8
  } else if constexpr (OFF == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((l & 16) ? r[0] : r[1]);
  } else if constexpr (OFF == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((l & 32) ? r[0] : r[1]);
  } else {
    return __shfl_xor(v, OFF, 64);
  }
}
// every lane receives the sum of its 16-lane row
DEV float row_sum16(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x124>(v);  // row_ror:4
  v += dpp<0x128>(v);  // row_ror:8
  return v;
}
// wave-uniform sum of all 64 lanes
DEV float sum64(float v) {
  v = row_sum16(v);
  return (rl(v, 0) + rl(v, 16)) + (rl(v, 32) + rl(v, 48));
}
// wave-uniform sums of two values at once: the first exchange leaves a's
// pair sums in even lanes and b's in odd lanes, which the remaining
// (parity-preserving) steps reduce side by side; each sum is added in the
// same order as sum64 adds it
DEV void sum64x2(float a, float b, float& sa, float& sb) {
  const bool odd = threadIdx.x & 1;
  const float pa = dpp<0xB1>(a), pb = dpp<0xB1>(b);  // quad_perm [1,0,3,2]
  float v = odd ? b + pb : a + pa;
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x124>(v);  // row_ror:4
  v += dpp<0x128>(v);  // row_ror:8
  sa = (rl(v, 0) + rl(v, 16)) + (rl(v, 32) + rl(v, 48));
  sb = (rl(v, 1) + rl(v, 17)) + (rl(v, 33) + rl(v, 49));
}
// sums of lanes [0,32) and [32,64)
DEV void sum32x2(float v, float& lo, float& hi) {
  v = row_sum16(v);
  lo = rl(v, 0) + rl(v, 16);
  hi = rl(v, 32) + rl(v, 48);
}
// sum over aligned groups of G (8 or 16) lanes, valid in the group's first lane
template <int G>
DEV float group_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x104>(v);              // row_shl:4
  if (G == 16) v += dpp<0x108>(v); // row_shl:8
  return v;
}
// sum over aligned groups of G (8 or 16) lanes, in every lane of the group
template <int G>
DEV float group_allsum(float v) {
  v += dpp<0xB1>(v);                // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);                // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);               // row_half_mirror: the other quad of the 8
  if (G == 16) v += dpp<0x140>(v);  // row_mirror: the other 8 of the row
  return v;
}
template <int CTRL>
DEV float dpp_max(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF, false));
}
DEV float max64(float v) {
  v = fmaxf(v, dpp_max<0xB1>(v));
  v = fmaxf(v, dpp_max<0x4E>(v));
  v = fmaxf(v, dpp_max<0x124>(v));
  v = fmaxf(v, dpp_max<0x128>(v));
  return fmaxf(fmaxf(rl(v, 0), rl(v, 16)), fmaxf(rl(v, 32), rl(v, 48)));
}

// ----------------------------------------------------------------- watchdog
DEV void record_timeout(const KArgs& a, int cu, uint32_t instr, uint32_t ctr, uint32_t seen,
                        uint32_t target) {
  uint32_t expected = 0;
  if (__hip_atomic_compare_exchange_strong(gp(a.status) + ST_CODE, &expected, uint32_t(STC_TIMEOUT),
                                           __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT)) {
    __hip_atomic_store(gp(a.status) + ST_CU, uint32_t(cu), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(gp(a.status) + ST_INSTR, instr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(gp(a.status) + ST_CTR, ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(gp(a.status) + ST_SEEN, seen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(gp(a.status) + ST_TARGET, target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Wait until counter >= target (wrap-safe).  false = watchdog or abort.
DEV uint32_t* ctr_line(const KArgs& a, uint32_t ctr, uint32_t line) {
  return a.counters + (size_t(ctr) * kCtrSpread + line) * kCtrStride;
}
// sum of the counter's lines (lanes 0 .. kCtrSpread-1 load one line each)
DEV uint32_t ctr_sum(const KArgs& a, uint32_t ctr) {
  static_assert(kCtrSpread == 16, "one DPP row per counter");
  const uint32_t lane = threadIdx.x & 63;
  int v = lane < uint32_t(kCtrSpread) ? int(ctr_load(ctr_line(a, ctr, lane))) : 0;
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, true);   // quad_perm [1,0,3,2]
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, true);   // quad_perm [2,3,0,1]
  v += __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, true);  // row_ror:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, true);  // row_ror:8
  return uint32_t(__builtin_amdgcn_readlane(v, 0));
}
DEV bool wait_counter(const KArgs& a, uint32_t ctr, uint32_t target, int cu, uint32_t instr) {
  uint64_t t0 = 0;
  for (uint32_t it = 0;; it++) {
    const uint32_t v = ctr_sum(a, ctr);
    if (int32_t(v - target) >= 0) return true;
    // The clock is a scalar memory read: read it every 64 polls only, so that
    // a poll is not held up by its latency.
    if ((it & 63) != 63) continue;
    const uint64_t now = __builtin_amdgcn_s_memrealtime();
    if (t0 == 0) t0 = now;
    if (now - t0 > a.watchdog_ticks) {
      record_timeout(a, cu, instr, ctr, v, target);
      return false;
    }
    if (__hip_atomic_load(gp(a.status) + ST_CODE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
      return false;
  }
}

// Time limit of waits inside the workgroup (pages, staged inputs, barriers).
// They can only stall if the workgroup itself is stuck; the limit turns that
// into an error instead of a hang.  The clock (a scalar memory read, waited
// for together with LDS reads) is read every 256 polls, so the limit counts
// from the 256th poll.
struct Watch {
  uint32_t n = 0;
  uint64_t t0 = 0;
};
DEV bool local_timeout(Watch& w, uint64_t limit) {
  if ((++w.n & 255) != 0) return false;
  const uint64_t now = __builtin_amdgcn_s_memrealtime();
  if (w.t0 == 0) w.t0 = now;
  return now - w.t0 > limit;
}
// the token poll's limit: on expiry the step is recorded as a tag timeout
DEV bool local_timeout_tok(uint64_t& t0, uint32_t& n, uint64_t limit) {
  if ((++n & 255) != 0) return false;
  const uint64_t now = __builtin_amdgcn_s_memrealtime();
  if (t0 == 0) t0 = now;
  if (now - t0 <= limit) return false;
  uint32_t expected = 0;
  __hip_atomic_compare_exchange_strong(gp(status_ptr()) + ST_CODE, &expected, uint32_t(STC_TAG_TIMEOUT),
                                       __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  lds_st(C_ABORT, 1);
  return true;
}

DEV void local_abort(uint32_t code) {
  uint32_t expected = 0;
  if (__hip_atomic_compare_exchange_strong(gp(status_ptr()) + ST_CODE, &expected, code, __ATOMIC_RELAXED,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
    __hip_atomic_store(gp(status_ptr()) + ST_CU, uint32_t(blockIdx.x), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  lds_st(C_ABORT, 1);
}

// Wait for an LDS word to reach `want` (or abort).
DEV bool wait_lds_ge(int off, uint32_t want) {
  Watch t0;
  while (int32_t(lds_ld(off) - want) < 0) {
    if (aborted()) return false;
    if (local_timeout(t0, local_limit())) {
      local_abort(STC_LOCAL_TIMEOUT);
      return false;
    }
    __builtin_amdgcn_s_sleep(0);
  }
  return true;
}
// Wait until every compute wave's word at off + 4*w has reached `want` (the
// kNComp words are read together each poll).
DEV bool wait_all_ge(int off, uint32_t want) {
  Watch t0;
  for (;;) {
    uint32_t m = lds_ld_rlx(off);
#pragma unroll
    for (int w = 1; w < kNComp; w++) m = min(m, lds_ld_rlx(off + 4 * w));
    if (int32_t(m - want) >= 0) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      return true;
    }
    if (aborted()) return false;
    if (local_timeout(t0, local_limit())) {
      local_abort(STC_LOCAL_TIMEOUT);
      return false;
    }
    __builtin_amdgcn_s_sleep(0);
  }
}
// The per-instruction completion counters (C_DONE) are a ring of kDoneRing
// slots, each cleared by the last wave to add to it; a wave adds to
// instruction i's slot after its work on i.  An instruction that stages its
// inputs synchronises the waves: each has read the inputs of the previous
// instruction (its C_XCONS word has reached i), so each has added to the
// slots up to i - 2.  Between two such instructions a fast wave can run ahead
// through instructions without a wait (one that reuses the staged input, an
// expert sum); at kDoneRing - 1 or more instructions past the last
// synchronisation it first waits until every wave's word has reached
// i - kDoneRing + 2, i.e. every wave has added to (and the last one has
// cleared) the slot of instruction i - kDoneRing.
DEV bool done_slot_free(uint32_t i, uint32_t last_sync) {
  return i - last_sync < uint32_t(kDoneRing - 1) || wait_all_ge(C_XCONS, i - kDoneRing + 2);
}
DEV uint32_t min_filled() {
  uint32_t m = lds_ld_rlx(C_FILLED);
#pragma unroll
  for (int v = 1; v < kNLoad; v++) m = min(m, lds_ld_rlx(C_FILLED + 4 * v));
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  return m;
}
// Wait until page g is published by every loader.
DEV bool wait_page(uint32_t g, uint32_t& cache) {
  Watch t0;
  while (cache <= g) {
    cache = min_filled();
    if (cache > g) break;
    if (aborted()) return false;
    if (local_timeout(t0, local_limit())) {
      local_abort(STC_LOCAL_TIMEOUT);
      return false;
    }
    __builtin_amdgcn_s_sleep(0);
  }
  return true;
}

// Software barrier of the compute waves (monotonic count).
DEV bool comp_barrier() {
  uint32_t c = 0;
  if ((threadIdx.x & 63) == 0) c = lds_add(C_BAR, 1) + 1;
  c = uni(c);
  const uint32_t target = ((c + kNComp - 1) / kNComp) * kNComp;
  return wait_lds_ge(C_BAR, target);
}

// ------------------------------------------------------------------- trace
DEV uint32_t now32() { return uint32_t(__builtin_amdgcn_s_memrealtime()); }
DEV void trace_put(const KArgs& a, int cu, uint32_t i, int word, uint32_t v) {
  if (a.trace && i < a.trace_stride)
    gp(a.trace)[(size_t(cu) * a.trace_stride + i) * TR_WORDS + word] = v;
}
// ================================================================== loader
// One wave-wide 16 B/lane DMA from global memory into LDS at M0.  M0 is set
// per DMA and not restored: the loader waves use M0 for nothing else, and
// writing M0 back right after an LDS DMA stalls issue until that DMA has been
// accepted, which cut the streaming rate by more than half.
#ifndef MK_DMA_NOP
#define MK_DMA_NOP "s_nop 0"
#endif
DEV void dma_uniform(uint32_t lds_addr, uint64_t src, uint32_t voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t" MK_DMA_NOP "\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(lds_addr), "v"(voff), "s"(src)
      : "memory", "m0");
}
DEV void dma_lane(uint32_t lds_addr, uint64_t src) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t" MK_DMA_NOP "\n\t"
      "global_load_lds_dwordx4 %1, off"
      :
      : "s"(lds_addr), "v"(src)
      : "memory", "m0");
}

constexpr uint32_t kDmaPerPage = kUnitsPerPage / kNLoad;  // 8

// Pages of weights a loader wave brings into L2 ahead of its DMA while the
// page ring is full (the compute waves are staging or waiting on a producer,
// so HBM would otherwise idle for this CU).  With 32 CUs per XCD, 4 pages
// ahead hold 2 MiB of the XCD's 4 MiB L2.
#ifndef MK_PF_PAGES
#define MK_PF_PAGES 4
#endif
constexpr uint32_t kPfPages = MK_PF_PAGES;

// One wave-wide 4 B/lane load with its lanes 128 B (one L2 line) apart: it
// brings the 8 KiB that a loader wave later copies into a page half into the
// XCD's L2, so that copy does not wait on HBM.  The words land in a 256 B LDS
// sink nobody reads; no register holds them.
DEV void l2_touch(uint32_t sink, uint64_t src, uint32_t voff128) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t" MK_DMA_NOP "\n\t"
      "global_load_lds_dword %1, %2"
      :
      : "s"(sink), "v"(voff128), "s"(src)
      : "memory", "m0");
}

// wait until at most `pages_after` pages of this loader's DMA are in flight
DEV void wait_vm_pages(uint32_t pages_after) {
  static_assert(kDmaPerPage == 8, "vmcnt table assumes 8 DMA per page");
  switch (pages_after) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(32)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(40)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(48)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

DEV uint32_t min_released() {
  uint32_t m = lds_ld_rlx(C_RELEASED);
#pragma unroll
  for (int w = 1; w < kNComp; w++) m = min(m, lds_ld_rlx(C_RELEASED + 4 * w));
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  return m;
}

// Per-instruction loader view: every field the DMA address arithmetic needs,
// loaded once into registers (the DMA asm clobbers memory, so fields read
// through the instruction pointer would be reloaded for every DMA).
struct LoadView {
  uint64_t src;            // GEMV: packed stream of the instruction
  uint64_t kv_base[2];     // ATTN: first K / V row of the position block
  uint32_t op, stream_units, kp, valid_bytes;
  bool deep;               // deep DMA queue (the LM head)
};

DEV void load_view(const KArgs& a, InstrCP I, LoadView& L, int32_t pos) {
  L.op = i_op(I);
  L.deep = (L.op == OP_GEMV || L.op == OP_BGEMV) && i_epi(I) == EPI_ARGMAX;
  // packed rows (matrix-core tiles: whole blocks of 16 rows, zero-padded)
  const uint32_t rows = (i_flags(I) & F_MFMA) ? 16 * I->n_items : I->n_rows;
  L.stream_units = (rows * I->row_bytes + kUnit - 1) / kUnit;
  L.src = I->src_ptr;
  L.kp = I->aux[4];
  L.valid_bytes = 0;
  L.kv_base[0] = L.kv_base[1] = 0;
  if (L.op == OP_ATTN) {
    const int32_t p0 = int32_t(I->aux[1] * I->aux[2]);
    int32_t nc = pos - p0;
    nc = nc < 0 ? 0 : (nc > int32_t(I->aux[2]) ? int32_t(I->aux[2]) : nc);
    L.valid_bytes = uint32_t(nc) * I->row_bytes;
    L.kv_base[0] = I->seg_ptr[0] + uint64_t(p0) * I->row_bytes;
    L.kv_base[1] = I->seg_ptr[1] + uint64_t(p0) * I->row_bytes;
  }
}

// DMAs each loader wave keeps in flight.  A DMA is issued, then the wave
// waits until at most kVmT of its DMAs are outstanding: vmcnt decrements in
// issue order, so every DMA older than the last kVmT has landed in LDS.
// Issuing one DMA per wait (rather than a page-sized burst per wait) keeps
// the request stream smooth; bursts streamed at well under half the rate.
#ifndef MK_VMT
#define MK_VMT 8
#endif
#ifndef MK_VMT_DEEP
#define MK_VMT_DEEP 24
#endif
#define MK_STR2(x) #x
#define MK_STR(x) MK_STR2(x)
// DMAs in flight per loader wave: shallow while the layers run (their weights
// are prefetched during the waits between stages, and a deep queue only
// lengthens the latency of the activation loads behind it), deep for the LM
// head, which is the one long pure stream of the step.
constexpr uint32_t kVmT = MK_VMT, kVmTDeep = MK_VMT_DEEP;
static_assert(kVmT % kDmaPerPage == 0 && kVmT >= kDmaPerPage && kVmTDeep % kDmaPerPage == 0 &&
                  kVmTDeep >= kVmT && kVmTDeep <= 48,
              "throttles are whole numbers of pages within the vmcnt range");

// Eight DMAs of 8 consecutive 1 KiB units starting at `src` into LDS at
// `lds_addr`, marked non-temporal (weights are read once per step).  The
// instruction offset moves the global source and the LDS destination
// together, so four DMAs share one M0 value; the second four use a VGPR
// offset 4 KiB higher and M0 + 4 KiB.  Each DMA is followed by the in-flight
// throttle (a no-op while fewer than T DMAs are outstanding).
#define MK_DMA8(T)                                                                                  \
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\t"                                                   \
               "global_load_lds_dwordx4 %1, %3 nt\n\ts_waitcnt vmcnt(" MK_STR(T) ")\n\t"              \
               "global_load_lds_dwordx4 %1, %3 offset:1024 nt\n\ts_waitcnt vmcnt(" MK_STR(T) ")\n\t"  \
               "global_load_lds_dwordx4 %1, %3 offset:2048 nt\n\ts_waitcnt vmcnt(" MK_STR(T) ")\n\t"  \
               "global_load_lds_dwordx4 %1, %3 offset:3072 nt\n\ts_waitcnt vmcnt(" MK_STR(T) ")\n\t"  \
               "s_add_u32 m0, %0, 0x1000\n\ts_nop 0\n\t"                                              \
               "global_load_lds_dwordx4 %2, %3 nt\n\ts_waitcnt vmcnt(" MK_STR(T) ")\n\t"              \
               "global_load_lds_dwordx4 %2, %3 offset:1024 nt\n\ts_waitcnt vmcnt(" MK_STR(T) ")\n\t"  \
               "global_load_lds_dwordx4 %2, %3 offset:2048 nt\n\ts_waitcnt vmcnt(" MK_STR(T) ")\n\t"  \
               "global_load_lds_dwordx4 %2, %3 offset:3072 nt\n\ts_waitcnt vmcnt(" MK_STR(T) ")"        \
               :                                                                                    \
               : "s"(lds_addr), "v"(voff), "v"(voff4k), "s"(src)                                    \
               : "memory", "m0")
DEV void dma_run8(uint32_t lds_addr, uint64_t src, uint32_t voff, uint32_t voff4k, bool deep) {
  lds_addr = uni(lds_addr);  // wave-uniform; the DMA takes scalar operands
  src = uni64(src);
  if (deep)
    MK_DMA8(MK_VMT_DEEP);
  else
    MK_DMA8(MK_VMT);
}

DEV void vm_throttle(uint32_t& nd) {
  if (++nd > kVmT) asm volatile("s_waitcnt vmcnt(" MK_STR(MK_VMT) ")" ::: "memory");
}

// Issue this loader wave's half (units v*8 .. v*8+7) of one page of a run of
// `valid` bytes at `base`, from byte off0 of the run: whole units past the run
// read the zero page, a unit that straddles its end is read per lane.
DEV void issue_run(const KArgs& a, uint32_t dst, uint64_t base, uint32_t off0, uint32_t valid,
                   uint32_t voff, uint32_t voff4k, uint32_t& nd, bool deep = false) {
  // every operand is wave-uniform (the DMA takes scalar addresses)
  dst = uni(dst);
  base = uni64(base);
  off0 = uni(off0);
  valid = uni(valid);
  const uint64_t zero = uint64_t(a.zero_page);
  if (off0 + kDmaPerPage * kUnit <= valid) {
    dma_run8(dst, base + off0, voff, voff4k, deep);
    nd += kDmaPerPage;
  } else if (off0 >= valid) {
    dma_run8(dst, zero, voff, voff4k, deep);
    nd += kDmaPerPage;
  } else {
    for (uint32_t j = 0; j < kDmaPerPage; j++) {
      const uint32_t off = off0 + j * kUnit;
      const uint32_t d = dst + j * kUnit;
      if (off + kUnit <= valid) {
        dma_uniform(d, base + off, voff);
      } else if (off >= valid) {
        dma_uniform(d, zero, voff);
      } else {
        const uint32_t lo = off + voff;
        dma_lane(d, lo < valid ? base + lo : zero + voff);
      }
      vm_throttle(nd);
    }
  }
}

// Issue this loader wave's half of page p (units v*8 .. v*8+7): one
// contiguous 8 KiB run, so consecutive DMAs of a wave read consecutive bytes.
template <class Lay>
DEV void issue_page(const KArgs& a, const LoadView& L, uint32_t p, uint32_t g, int v,
                    uint32_t voff, uint32_t voff4k, uint32_t& nd) {
  const uint32_t half = uint32_t(v) * kDmaPerPage;
  const uint32_t dst = uint32_t(size_t(lds)) + page_off<Lay>(g) + half * kUnit;
  if (L.op == OP_GEMV || L.op == OP_BGEMV) {
    // Packed stream: the run is inside the instruction's zero-padded pages;
    // a half page wholly past the rows reads the zero page instead of HBM.
    const uint32_t u0 = p * kUnitsPerPage + half;
    dma_run8(dst, u0 < L.stream_units ? L.src + uint64_t(u0) * kUnit : uint64_t(a.zero_page), voff, voff4k,
             L.deep);
    nd += kDmaPerPage;
    return;
  }
  // OP_ATTN: K block region then V block region; rows < n_cached are valid
  const uint32_t region = p < L.kp ? 0 : 1;
  const uint64_t base = region ? L.kv_base[1] : L.kv_base[0];
  issue_run(a, dst, base, ((p - region * L.kp) * kUnitsPerPage + half) * kUnit, L.valid_bytes, voff, voff4k, nd);
}

DEV void publish(uint32_t& g_pub, uint32_t upto, int v) {
  if (upto > g_pub) {
    g_pub = upto;
    if ((threadIdx.x & 63) == 0) lds_st(C_FILLED + 4 * v, g_pub);
  }
}

// ================================================================ compute
struct Comp {
  const KArgs* a;
  int cu;
  int w;          // compute wave index
  uint32_t lane;
  uint32_t fcache;  // cached min published page
  uint32_t pagewait;  // ticks spent waiting for pages (leader, traced runs)
  uint32_t retries;   // re-reads of stale tagged inputs (leader, traced runs)
  uint32_t ep;        // epoch (1-based step count) of the step being run
  int32_t pos;        // its position
  uint32_t step;      // its index within the launch
  uint32_t pbase;     // the step's first page in the CU's page stream
};


// ---- GEMV epilogue for one output row
struct ArgBest {
  float v;
  uint32_t i;
};
DEV void arg_update(ArgBest& b, float v, uint32_t i) {
  if (v > b.v || (v == b.v && i < b.i)) {
    b.v = v;
    b.i = i;
  }
}

// ---- attention: one KV group, one position block
// The x slot holds, staged by the leader: q [HPT*Dh] of the tile's heads | k [Dh] | v [Dh] of the
// group | cos [Dh/2] | sin [Dh/2] of the position.  The waves' softmax
// records go to the x slot after those inputs, so the instruction releases
// the slot (C_XCONS) only at its end.
template <int HPT, int DH, class Lay>
DEV bool attn(Comp& c, InstrCP I, uint32_t i, uint32_t page0) {
  const KArgs& a = *c.a;
  const uint32_t lane = c.lane;
  constexpr int LPRA = DH / 8;            // lanes per cached row (8 dims per lane)
  constexpr int UPOS = kUnit / (2 * DH);  // rows per 1 KiB unit
  constexpr int HALF = DH / 2;
  constexpr int OUT = HPT * DH;           // outputs of the group
  static_assert(64 % LPRA == 0 && LPRA >= 4 && LPRA <= 32 && HPT >= 1 && HPT <= 8, "attention shape");
  const uint32_t g = I->aux[0], blk = I->aux[1], Bat = I->aux[2], nblk = I->aux[3], kp = I->aux[4];
  const uint32_t h0 = I->row0;                  // first query head of the tile in its group
  const uint32_t head0 = g * uint32_t(a.hpg) + h0;  // ... in the layer
  const int32_t P = c.pos;
  const int32_t p0 = int32_t(blk * Bat);
  int32_t nc = P - p0;
  nc = nc < 0 ? 0 : (nc > int32_t(Bat) ? int32_t(Bat) : nc);
  const bool own = P >= p0 && P < p0 + int32_t(Bat);
  float* xs = reinterpret_cast<float*>(lds + Lay::x);
  const float* cs = xs + HPT * DH + 2 * DH;
  const float* sn = cs + HALF;
  const uint32_t s = lane % LPRA;        // dims [8s, 8s+8)
  const uint32_t jrow = lane / LPRA;     // row within a unit
  const bool trl = a.trace && c.w == 0 && lane == 0;

  // rotated (RoPE, rotate-half pairing), scaled query slices of every head.
  // A lane's 8 dims [8s, 8s+8) lie in one half, so every operand is two
  // 16-byte LDS reads: the dims themselves, their partners in the other
  // half, and cos / sin at the dims' frequencies.
  const uint32_t d0 = 8 * s;
  const bool first_half = d0 < uint32_t(HALF);
  const uint32_t pd = first_half ? d0 + HALF : d0 - HALF;  // partner dims
  const uint32_t fd = first_half ? d0 : d0 - HALF;         // frequency index
  const float sgn = first_half ? -1.f : 1.f;
  auto ld8 = [&](const float* p, float (&o)[8]) {
    const f4 lo = *reinterpret_cast<const f4*>(p);
    const f4 hi = *reinterpret_cast<const f4*>(p + 4);
    o[0] = lo.x; o[1] = lo.y; o[2] = lo.z; o[3] = lo.w;
    o[4] = hi.x; o[5] = hi.y; o[6] = hi.z; o[7] = hi.w;
  };
  float cv[8], sv[8];
  ld8(cs + fd, cv);
  ld8(sn + fd, sv);
  auto rot8 = [&](const float* vec, float (&o)[8], float scale) {
    float self[8], part[8];
    ld8(vec + d0, self);
    ld8(vec + pd, part);
#pragma unroll
    for (int e = 0; e < 8; e++) o[e] = (self[e] * cv[e] + sgn * part[e] * sv[e]) * scale;
  };
  float qr[HPT][8];
#pragma unroll
  for (int h = 0; h < HPT; h++) rot8(xs + h * DH, qr[h], a.attn_scale);
  // the new key/value row, rounded to bf16
  float kr[8], vr[8], kn[8];
  uint16_t kb[8], vb[8];
  rot8(xs + HPT * DH, kr, 1.f);
  ld8(xs + HPT * DH + DH + d0, vr);
#pragma unroll
  for (int e = 0; e < 8; e++) {
    kb[e] = f2bf(kr[e]);
    kn[e] = __uint_as_float(uint32_t(kb[e]) << 16);
    vb[e] = f2bf(vr[e]);
  }
  if (trl) trace_put(a, c.cu, i, TR_XREADY, now32());

  // One pass per wave, softmax online: wave w takes the position units
  // u = w (mod waves); in a unit, lane group jrow holds row u*UPOS + jrow,
  // its lanes 8 dims each of k and v.  Every lane group keeps, per head, a
  // reference m (at most kLazy below the maximum of its scores), the sum l
  // of exp(score - m) and o~ = sum exp(score - m) v over its rows; the
  // groups of a wave, then the waves, are merged by the log-sum-exp rule.
  // The wave after the last unit's takes the new row.
  const uint32_t n_units = (uint32_t(nc) + UPOS - 1) / UPOS;
  float m[HPT], l[HPT], acc[HPT][8];
#pragma unroll
  for (int h = 0; h < HPT; h++) {
    m[h] = -__builtin_inff();
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; e++) acc[h][e] = 0.f;
  }
  // m is the reference of a group's sums (l and o~ are taken relative to
  // exp(m)): it moves to a row's score only when the score exceeds it by
  // more than kLazy, which rescales the old sums, so every weight
  // exp(score - m) stays below e^kLazy and most rows cost one exponential
  // and one fused multiply-add per dimension.  The first row moves it from
  // -inf (the old sums, all zero, scale by 0).
  constexpr float kLazy = 8.f;
  auto update = [&](int h, float sc, const float (&v)[8]) {
    if (sc > m[h] + kLazy) {
      const float sa = __expf(m[h] - sc);  // m = -inf: exp(-inf) = 0
      l[h] *= sa;
#pragma unroll
      for (int e = 0; e < 8; e++) acc[h][e] *= sa;
      m[h] = sc;
    }
    const float w = __expf(sc - m[h]);
    l[h] += w;
#pragma unroll
    for (int e = 0; e < 8; e++) acc[h][e] = fmaf(w, v[e], acc[h][e]);
  };
  for (uint32_t u = c.w; u < n_units; u += kNComp) {
    // the v unit streams after every k unit of the tile
    if (!wait_page(page0 + kp + u / kUnitsPerPage, c.fcache)) return false;
    const uint32_t lo = (u % kUnitsPerPage) * kUnit + lane * 16;
    const u4 kw = *reinterpret_cast<const u4*>(lds + page_off<Lay>(page0 + u / kUnitsPerPage) + lo);
    const u4 vw = *reinterpret_cast<const u4*>(lds + page_off<Lay>(page0 + kp + u / kUnitsPerPage) + lo);
    const bool valid = u * UPOS + jrow < uint32_t(nc);
    const float v[8] = {bf_lo(vw.x), bf_hi(vw.x), bf_lo(vw.y), bf_hi(vw.y),
                        bf_lo(vw.z), bf_hi(vw.z), bf_lo(vw.w), bf_hi(vw.w)};
#pragma unroll
    for (int h = 0; h < HPT; h++) {
      const float sc = group_allsum<LPRA>(dot8(kw, qr[h]));
      if (valid) update(h, sc, v);
    }
  }
  if (own && uint32_t(c.w) == n_units % kNComp) {
    // (every tile of the group scores the new row; the one holding the
    // group's first head appends it to the cache)
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; e++) v[e] = __uint_as_float(uint32_t(vb[e]) << 16);
#pragma unroll
    for (int h = 0; h < HPT; h++) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; e++) d = fmaf(qr[h][e], kn[e], d);
      d = group_allsum<LPRA>(d);
      if (jrow == 0) update(h, d, v);
    }
    if (lane < uint32_t(LPRA) && h0 == 0) {
      // device-scope stores: a later step of the same launch streams this
      // row from another CU (ordered behind every CU's LM-head release)
      const size_t row = size_t(P) * DH + 8 * s;
      uint64_t* kc = reinterpret_cast<uint64_t*>(reinterpret_cast<uint16_t*>(I->seg_ptr[0]) + row);
      uint64_t* vc = reinterpret_cast<uint64_t*>(reinterpret_cast<uint16_t*>(I->seg_ptr[1]) + row);
      const uint64_t k0 = uint64_t(kb[0] | uint32_t(kb[1]) << 16) | uint64_t(kb[2] | uint32_t(kb[3]) << 16) << 32;
      const uint64_t k1 = uint64_t(kb[4] | uint32_t(kb[5]) << 16) | uint64_t(kb[6] | uint32_t(kb[7]) << 16) << 32;
      const uint64_t v0 = uint64_t(vb[0] | uint32_t(vb[1]) << 16) | uint64_t(vb[2] | uint32_t(vb[3]) << 16) << 32;
      const uint64_t v1 = uint64_t(vb[4] | uint32_t(vb[5]) << 16) | uint64_t(vb[6] | uint32_t(vb[7]) << 16) << 32;
      __hip_atomic_store(gp(kc), k0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(gp(kc + 1), k1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(gp(vc), v0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(gp(vc + 1), v1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (lane == 0) lds_st(C_RELEASED + 4 * c.w, page0 + I->n_pages);
  if (trl) trace_put(a, c.cu, i, TR_ITEM0, now32());
  if constexpr (std::is_same<Lay, LayA>::value) {
    // traced runs: earliest and latest end of the waves' position loops
    if (a.trace && lane == 0) {
      const uint32_t t = now32();
      __hip_atomic_fetch_min(lw(C_TR_LOOP), t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      __hip_atomic_fetch_max(lw(C_TR_LOOP + 4), t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  // Merge the lane groups of the wave.  A butterfly gives every lane the
  // wave's maximum of each head; each group rescales its sums to it once;
  // a butterfly sums the weights, and a reduce-scatter the value sums: each
  // exchange keeps half of a lane's values and adds the partner's copy of
  // that half, so the NG groups' 8 values per lane end as 8 / NG sums per
  // lane, each added in one fixed tree.
  constexpr int NG = 64 / LPRA, NV = 8 / NG;  // lane groups, sums per lane
  static_assert(NG * NV == 8 && (LPRA == 8 || LPRA == 16), "lane groups");
  // register exchanges in the one-sequence kernel; the batched kernel keeps
  // the generic shuffle, which measured faster there
  auto xch = [](auto off_c, float v) {
    constexpr int OFF = decltype(off_c)::value;
    if constexpr (std::is_same<Lay, LayA>::value) return lane_xor<OFF>(v);
    else return __shfl_xor(v, OFF, 64);
  };
  // the exchange offsets between lane groups: LPRA, 2 LPRA, ..., 32
  auto over_groups = [&](auto f) {
    if constexpr (LPRA <= 8) f(std::integral_constant<int, 8>{});
    f(std::integral_constant<int, 16>{});
    f(std::integral_constant<int, 32>{});
  };
  float M[HPT];
#pragma unroll
  for (int h = 0; h < HPT; h++) M[h] = m[h];
  over_groups([&](auto oc) {
#pragma unroll
    for (int h = 0; h < HPT; h++) M[h] = fmaxf(M[h], xch(oc, M[h]));
  });
#pragma unroll
  for (int h = 0; h < HPT; h++) {
    // a group without rows (m = -inf) adds nothing
    const float sc = m[h] == -__builtin_inff() ? 0.f : __expf(m[h] - M[h]);
    l[h] *= sc;
#pragma unroll
    for (int e = 0; e < 8; e++) acc[h][e] *= sc;
  }
  over_groups([&](auto oc) {
#pragma unroll
    for (int h = 0; h < HPT; h++) l[h] += xch(oc, l[h]);
  });
  over_groups([&](auto oc) {
    constexpr int OFF = decltype(oc)::value, HN = 4 * LPRA / OFF;  // values kept: 4, 2, 1
    const bool up = lane & OFF;
#pragma unroll
    for (int h = 0; h < HPT; h++)
#pragma unroll
      for (int e = 0; e < HN; e++) {
        const float send = up ? acc[h][e] : acc[h][HN + e];
        const float keep = up ? acc[h][HN + e] : acc[h][e];
        acc[h][e] = keep + xch(oc, send);
      }
  });
  // lane (group j, slice s) holds the sums of dims 8 s + dof .. + NV - 1,
  // dof from the bits of j that chose the kept halves
  const uint32_t dof = ((lane & uint32_t(LPRA)) ? 4u : 0u) + ((lane & uint32_t(2 * LPRA)) ? 2u : 0u) +
                       ((NG == 8 && (lane & uint32_t(4 * LPRA))) ? 1u : 0u);
  // the wave's record per head after the staged inputs: o~ [DH] | m | l
  constexpr int REC = DH + 2;
  constexpr int PBASE = (HPT * DH + 3 * DH + 3) & ~3;
  static_assert(PBASE + kNComp * HPT * REC <= Lay::x_floats, "attention partials");
  float* wrec = xs + PBASE;
#pragma unroll
  for (int h = 0; h < HPT; h++) {
    float* r = wrec + (c.w * HPT + h) * REC;
#pragma unroll
    for (int e = 0; e < NV; e++) r[8 * s + dof + e] = acc[h][e];
    if (lane == 0) {
      r[DH] = M[h];
      r[DH + 1] = l[h];
    }
  }
  if (!comp_barrier()) return false;
  if (trl) {
    trace_put(a, c.cu, i, TR_A_PASS3, now32());
    if constexpr (std::is_same<Lay, LayA>::value) {
      trace_put(a, c.cu, i, TR_A_PASS1, *lw(C_TR_LOOP));
      trace_put(a, c.cu, i, TR_A_STATS, *lw(C_TR_LOOP + 4));
    }
  }

  // final: merge the waves' records in order, normalise, store
  for (uint32_t o = c.w * 64 + lane; o < uint32_t(OUT); o += 64 * kNComp) {
    const uint32_t h = o / DH, d = o % DH;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kNComp; w++) M = fmaxf(M, wrec[(w * HPT + h) * REC + DH]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kNComp; w++) {
      const float* r = wrec + (w * HPT + h) * REC;
      const float sw = r[DH] == -__builtin_inff() ? 0.f : __expf(r[DH] - M);
      num = fmaf(sw, r[d], num);
      den = fmaf(sw, r[DH + 1], den);
    }
    const uint32_t head = head0 + h;
    if (nblk == 1) {
      st_tag(reinterpret_cast<uint64_t*>(I->out_ptr) + head * DH + d, num / den, c.ep);
    } else {
      // partial record of (head tile, block, head): o~ [DH] | m | l
      const size_t tg = head0 / HPT;
      float* part = reinterpret_cast<float*>(I->res_ptr) + ((tg * nblk + blk) * HPT + h) * (DH + 2);
      st_act(part + d, num);
      if (d == 0) {
        st_act(part + DH, M);
        st_act(part + DH + 1, den);
      }
    }
  }
  // every wave has read the x slot: the next inputs may be staged
  if (!comp_barrier()) return false;
  if (lane == 0) lds_st(C_XCONS + 4 * c.w, i + 1);
  return true;
}

// Last-arriving tile of a head tile's blocks merges their partials
// (log-sum-exp of the block maxima, taken as a running maximum over batches
// of blocks).  Lane l merges the PER consecutive outputs from l*PER (one
// head); every load of a batch of blocks is issued before the first is used,
// so a merge of n blocks costs about n/NB memory round trips.
template <int HPT, int DH, int NB = 8>
DEV void attn_merge(Comp& c, InstrCP I) {
  constexpr int OUT = HPT * DH, PER = OUT / 64, REC = DH + 2;
  static_assert(PER == 1 || PER == 2 || PER == 4 || PER == 8, "merge lane shape");
  const uint32_t g = I->aux[0], nblk = I->aux[3];
  const uint32_t head0 = g * uint32_t(c.a->hpg) + I->row0;
  const float* part = reinterpret_cast<const float*>(I->res_ptr) + size_t(head0 / HPT) * nblk * (HPT * REC);
  const __amdgpu_buffer_rsrc_t r = act_rsrc_u(part, nblk * HPT * REC * 4);
  const uint32_t o0 = c.lane * PER, h = o0 / DH, d0 = o0 % DH;
  float M = -__builtin_inff(), den = 0.f, num[PER];
#pragma unroll
  for (int e = 0; e < PER; e++) num[e] = 0.f;
  for (uint32_t b0 = 0; b0 < nblk; b0 += NB) {
    float mb[NB], lb_[NB], v[NB][PER];
#pragma unroll
    for (int k = 0; k < NB; k++) {
      // blocks past the end read past the resource: zero, and are skipped
      const uint32_t rec = ((b0 + k) * HPT + h) * REC * 4;
      mb[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, rec + DH * 4, 0, 16 /* sc1 */));
      lb_[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, rec + (DH + 1) * 4, 0, 16));
      if constexpr (PER >= 4) {
#pragma unroll
        for (int q4 = 0; q4 < PER / 4; q4++) {
          const f4 t = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, rec + (d0 + 4 * q4) * 4, 0, 16));
          v[k][4 * q4] = t.x; v[k][4 * q4 + 1] = t.y; v[k][4 * q4 + 2] = t.z; v[k][4 * q4 + 3] = t.w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < PER; e++)
          v[k][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, rec + (d0 + e) * 4, 0, 16));
      }
    }
    float Mn = M;
#pragma unroll
    for (int k = 0; k < NB; k++)
      if (b0 + k < nblk) Mn = fmaxf(Mn, mb[k]);
    const float scale = M == -__builtin_inff() ? 0.f : __expf(M - Mn);
    den *= scale;
#pragma unroll
    for (int e = 0; e < PER; e++) num[e] *= scale;
#pragma unroll
    for (int k = 0; k < NB; k++) {
      const float w = (b0 + k >= nblk || mb[k] == -__builtin_inff()) ? 0.f : __expf(mb[k] - Mn);
      den = fmaf(w, lb_[k], den);
#pragma unroll
      for (int e = 0; e < PER; e++) num[e] = fmaf(w, v[k][e], num[e]);
    }
    M = Mn;
  }
  uint64_t* out = reinterpret_cast<uint64_t*>(I->out_ptr) + (head0 + h) * DH + d0;
#pragma unroll
  for (int e = 0; e < PER; e++) st_tag(out + e, num[e] / den, c.ep);
}

// ---- staging of the instruction's inputs into the LDS x slot (leader wave)
// Re-read tagged entries of `t` (the first `live` of this lane) until every
// one holds the current step's tag: a stale entry is a row its producer has
// not stored yet, or a store still in flight.  The wait is bounded by the
// watchdog limit.  T is u4 (two elements) or uint2 (one).
DEV bool is_fresh(const u4& t, uint32_t tag) { return t.y == tag && t.w == tag; }
DEV bool is_fresh(const uint2& t, uint32_t tag) { return t.y == tag; }
DEV void reload(u4& t, __amdgpu_buffer_rsrc_t r, uint32_t off) { t = ld_tag2(r, off); }
DEV void reload(uint2& t, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  t = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 16));
}
template <typename T, int N, typename Off>
DEV bool wait_fresh(T (&t)[N], uint32_t live, __amdgpu_buffer_rsrc_t r, Off off, int h, uint32_t tag,
                    uint32_t& retries) {
  Watch wt;
  for (;;) {
    bool ok = true;
#pragma unroll
    for (int j = 0; j < N; j++)
      if (j < int(live) && !is_fresh(t[j], tag)) ok = false;
    if (__builtin_amdgcn_ballot_w64(!ok) == 0) return true;
    retries++;
#pragma unroll
    for (int j = 0; j < N; j++)
      if (j < int(live) && !is_fresh(t[j], tag)) reload(t[j], r, off(h, j));
    if (aborted()) return false;
    if (local_timeout(wt, local_limit())) {
      local_abort(STC_TAG_TIMEOUT);
      return false;
    }
  }
}

// The tag that an instruction's inputs carry once this step has written them.
DEV uint32_t in_tag(uint32_t ep, InstrCP I) { return ep + ((i_flags(I) & F_DEBUG_STALL) ? 1u : 0u); }

// Leader staging of an attention tile: the tile's q, the group's k and v
// (tagged) and cos | sin of the position into the x slot.  Every load is
// issued before the first is waited for: one memory round trip.
template <class Lay>
DEV bool stage_attn(Comp& c, InstrCP I) {
  const KArgs& a = *c.a;
  const uint32_t lane = c.lane;
  const uint32_t tag = in_tag(c.ep, I);
  float* xs = reinterpret_cast<float*>(lds + Lay::x);
  {
      // attention: q, k, v of the group (tagged) and cos | sin (tables)
      const int dh = a.head_dim;
      const uint32_t g = I->aux[0], hpt = I->n_items, head0 = g * uint32_t(a.hpg) + I->row0;
      const char* qkv = reinterpret_cast<const char*>(I->in_ptr);
      const uint32_t nq = hpt * dh, half = dh / 2;
      const __amdgpu_buffer_rsrc_t rq = act_rsrc(qkv + size_t(head0) * dh * kActBytes, nq * kActBytes);
      const __amdgpu_buffer_rsrc_t rk = act_rsrc(qkv + size_t(a.q_dim + g * dh) * kActBytes, dh * kActBytes);
      const __amdgpu_buffer_rsrc_t rv =
          act_rsrc(qkv + size_t(a.q_dim + a.kv_dim + g * dh) * kActBytes, dh * kActBytes);
      const __amdgpu_buffer_rsrc_t rc = act_rsrc(a.rope_cos + size_t(c.pos) * half, half * 4);
      const __amdgpu_buffer_rsrc_t rs = act_rsrc(a.rope_sin + size_t(c.pos) * half, half * 4);
      static_assert(kMaxK >= 512, "q staging");
      constexpr int NQ = 4;  // up to 512 q values
      u4 tq[NQ], tk[1], tv[1];
      uint32_t oq[NQ], ok1[1] = {lane * 16};
#pragma unroll
      for (int j = 0; j < NQ; j++) {
        oq[j] = (2 * lane + 128 * j) * kActBytes;
        tq[j] = ld_tag2(rq, oq[j]);
      }
      tk[0] = ld_tag2(rk, ok1[0]);
      tv[0] = ld_tag2(rv, ok1[0]);
      const f4 cv = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rc, lane * 16, 0, 0));
      const f4 sv = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rs, (lane - half / 4) * 16, 0, 0));
      const bool kv_lane = 2 * lane < uint32_t(dh);
      const uint32_t q_live = nq > 2 * lane ? (nq - 2 * lane + 127) / 128 : 0;
      if (!wait_fresh(tq, q_live, rq, [&](int, int j) { return oq[j]; }, 0, tag, c.retries)) return false;
      if (!wait_fresh(tk, kv_lane ? 1 : 0, rk, [&](int, int) { return ok1[0]; }, 0, tag, c.retries)) return false;
      if (!wait_fresh(tv, kv_lane ? 1 : 0, rv, [&](int, int) { return ok1[0]; }, 0, tag, c.retries)) return false;
#pragma unroll
      for (int j = 0; j < NQ; j++)
        if (2 * lane + 128 * j < nq)
          *reinterpret_cast<float2*>(xs + 2 * lane + 128 * j) =
              float2{__uint_as_float(tq[j].x), __uint_as_float(tq[j].z)};
      if (kv_lane) {
        *reinterpret_cast<float2*>(xs + nq + 2 * lane) = float2{__uint_as_float(tk[0].x), __uint_as_float(tk[0].z)};
        *reinterpret_cast<float2*>(xs + nq + dh + 2 * lane) =
            float2{__uint_as_float(tv[0].x), __uint_as_float(tv[0].z)};
      }
      if (lane * 4 < uint32_t(dh)) *reinterpret_cast<f4*>(xs + nq + 2 * dh + lane * 4) = lane * 4 < half ? cv : sv;
  }
  return true;
}

}  // namespace mk
