// mk_batch.hip — the batched persistent megakernel (B <= 8 sequences per step)
// for the parallel-block mixture-of-experts decoder.
//
// Cohere's decode megakernel write-up (airebao.com) is the model: attention
// and the MoE branch read one RMSNorm output and meet in one residual add
// («快在哪里» item 1); the router weights are small and sit in front of the
// experts («快在哪里» item 3); every weight byte that is streamed is applied to
// all sequences of the batch that need it («为什么值得做»).
//
// Same workgroup shape as the one-sequence kernel (2 loader + 6 compute waves,
// one workgroup per CU, counters in global memory), with a different LDS
// layout: the staged GEMV input holds every sequence's vector ([B][K] fp32),
// and the page ring has five pages.
//  * OP_BGEMV: a row pair per compute-wave item; each weight element read from
//    LDS once is multiplied into all B staged vectors (fp32 FMAs), and the
//    2 x B partial sums are reduced across the wave with one butterfly.
//  * OP_EGU / OP_EDN: every CU holds a slice of every expert (gate/up pairs,
//    down-projection rows), so the work per CU is the same whatever the router
//    picks.  The loader waves read the router logits, take the top-k of every
//    sequence and stream only the selected experts' slices, straight from the
//    expert tensors; the compute waves apply each slice to the sequences routed
//    to that expert.
//  * The down projection keeps, per (sequence, top-k slot, row), the dot of its
//    expert and sums the slots in order with the softmax weights, then adds the
//    residual (the O-projection output): x_{l+1} = x_l + attn + MoE.
#include <type_traits>

#include "mk_dev.h"

namespace mk {

// --------------------------------------------------------- routing tables
// One table per layer parity at lb::kRoute, written by the leader wave at the
// first expert instruction of a layer and read by every compute wave.
enum : int {
  RT_MASK = 0,     // u64 selected-expert mask (union over the batch)
  RT_NSEL = 8,     // u32 number of selected experts
  RT_NPAIR = 12,   // u32 routed (expert, sequence) pairs = B * top_k
  RT_TOK = 16,     // u8 [64] sequences routed to expert e (bit b)
  RT_LIST = 80,    // u8 [64] selected experts in increasing id order
  RT_SLOT = 144,   // u8 [64][8] top-k slot of expert e for sequence b
  RT_WT = 656,     // f32 [8][8] softmax weight of sequence b's slot s
  RT_PBASE = 912,  // u8 [64] first pair index of the selected expert of each rank
  RT_PAIR = 976,   // u16 [64] pair index -> expert | sequence << 6 | slot << 9
  RT_PRANK = 1104, // u8 [64] pair index -> rank of its expert
  RT_END = 1168,
};
static_assert(RT_END <= lb::kRouteBytes, "routing table size");

DEV int rt_base(uint32_t layer) { return lb::kRoute + int(layer & 1) * lb::kRouteBytes; }
DEV uint32_t rt_u8(int base, int off) { return *reinterpret_cast<const uint8_t*>(lds + base + off); }
DEV void rt_st8(int base, int off, uint32_t v) { *reinterpret_cast<uint8_t*>(lds + base + off) = uint8_t(v); }

// The layer's down projections are cut into units of Rb consecutive rows of
// one selected expert; the U = (selected experts) x (units per expert) units,
// in expert order, go to the CUs in even contiguous ranges.  Loader and
// compute waves take the same range from the same routing decision.
// All units, or with a ready queue (row0 = q > 0) all but a 1/q share, go to
// the CUs in even contiguous ranges; the rest wait in the queue: chunks of uc
// units handed out at run time by a per-layer counter, each to whichever CU
// asks first, so that CUs that finish early take the tail.
constexpr uint32_t kDynMax = 512;  // queue entries per layer parity in LDS
struct EdnSplit {
  uint32_t T, Ts, uc, n_dyn;  // units, static units, units per chunk, chunks
};
DEV EdnSplit edn_split(uint32_t nsel, uint32_t nb, uint32_t queue) {
  EdnSplit e;
  e.T = nsel * nb;
  e.Ts = queue ? e.T - e.T / queue : e.T;
  const uint32_t rest = e.T - e.Ts;
  e.uc = max(2u, (rest + kDynMax - 2) / (kDynMax - 1));
  e.n_dyn = (rest + e.uc - 1) / e.uc;
  return e;
}
DEV void edn_range(uint32_t U, uint32_t n_cus, uint32_t cu, uint32_t& lo, uint32_t& hi) {
  lo = uint32_t(uint64_t(U) * cu / n_cus);
  hi = uint32_t(uint64_t(U) * (cu + 1) / n_cus);
}
// Queue entry k of the layer's parity: (layer + 1) << 16 | chunk, written by
// the first loader wave after it took the chunk from the counter.
DEV int dyn_slot(uint32_t layer, uint32_t k) { return lb::kMfma + 4 * int((layer & 1) * kDynMax + k); }
// wait for entry k of this layer; false = abort or watchdog
DEV bool dyn_entry(uint32_t layer, uint32_t k, uint32_t& chunk) {
  Watch t0;
  for (;;) {
    const uint32_t e = lds_ld(dyn_slot(layer, k));
    if ((e >> 16) == layer + 1) {
      chunk = e & 0xFFFFu;
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
// Tag of the expert outputs y: the step and the layer (one buffer serves
// every layer; a reader must not take the previous layer's values).
DEV uint32_t y_tag(uint32_t ep, uint32_t layer) { return (ep << 7) | (layer & 127u); }

// Reductions over aligned groups of 8 lanes (every lane of the group gets
// the result): xor 1, xor 2, then the half-row mirror pairs the two quads.
template <class T, class Op>
DEV T group8(T v, Op op) {
  auto sh = [](T x, auto ctrl) {
    return __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), decltype(ctrl)::value,
                                                             0xF, 0xF, false));
  };
  v = op(v, sh(v, std::integral_constant<int, 0xB1>{}));
  v = op(v, sh(v, std::integral_constant<int, 0x4E>{}));
  v = op(v, sh(v, std::integral_constant<int, 0x141>{}));
  return v;
}

// Top-k of every sequence's router logits, all sequences at once: the 8 lanes
// of group b hold sequence b's logits (lane s: experts 8s .. 8s+7).  Each of
// the k rounds takes the group maximum and the lowest expert id holding it
// (ties go to the lower id).  Returns the union of the selections; with
// table >= 0 the leader also records the per-expert sequence masks and slots,
// the softmax weights over each sequence's k selected logits (top-k first,
// then softmax over those k), the selected experts in order and their first
// pair index.  false = abort or watchdog while waiting for fresh logits.
DEV bool route_topk(const KArgs& a, InstrCP I, uint64_t& mask, int table, uint32_t& retries) {
  const uint32_t lane = threadIdx.x & 63, b = lane >> 3, s = lane & 7;
  const uint32_t E = uint32_t(a.n_experts), k = uint32_t(a.top_k), nB = uint32_t(a.batch);
  const __amdgpu_buffer_rsrc_t r = act_rsrc(reinterpret_cast<const void*>(I->seg_ptr[0]), nB * E * kActBytes);
  const uint32_t live = (b < nB && 8 * s < E) ? min(8u, E - 8 * s) : 0u;
  uint2 t[8];
  auto off = [&](int, int j) -> uint32_t { return (b * E + 8 * s + uint32_t(j)) * kActBytes; };
#pragma unroll
  for (int j = 0; j < 8; j++) reload(t[j], r, off(0, j));
  if (!wait_fresh(t, live, r, off, 0, in_tag(a.epoch, I), retries)) return false;
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const float x = __uint_as_float(t[j].x);
    v[j] = (uint32_t(j) < live && x == x) ? x : -__builtin_inff();
  }
  uint32_t taken = 0, slot[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float myv = -__builtin_inff();  // lane s of a group: the value of round s
  auto fmax_ = [](float x, float y) { return fmaxf(x, y); };
  auto umin_ = [](uint32_t x, uint32_t y) { return min(x, y); };
  for (uint32_t rd = 0; rd < k; rd++) {
    float lm = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < 8; j++) lm = fmaxf(lm, ((taken >> j) & 1) ? -__builtin_inff() : v[j]);
    const float gm = group8(lm, fmax_);
    uint32_t ci = 0xFFu;
#pragma unroll
    for (int j = 7; j >= 0; j--)
      if (!((taken >> j) & 1) && uint32_t(j) < live && v[j] == gm) ci = 8 * s + uint32_t(j);
    const uint32_t ge = group8(ci, umin_);
    if (ge != 0xFFu && (ge >> 3) == s) {
      taken |= 1u << (ge & 7);
#pragma unroll
      for (int j = 0; j < 8; j++)
        if (uint32_t(j) == (ge & 7)) slot[j] = rd;
    }
    if (s == rd) myv = gm;
  }
  // union over the sequences: expert 8s + j is selected if a group took it
  uint64_t ball[8];
  mask = 0;
#pragma unroll
  for (int j = 0; j < 8; j++) {
    ball[j] = __builtin_amdgcn_ballot_w64((taken >> j) & 1);
    uint64_t m8 = ball[j];
    m8 |= m8 >> 32;
    m8 |= m8 >> 16;
    m8 |= m8 >> 8;
    for (uint32_t ss = 0; ss < 8; ss++)
      if ((m8 >> ss) & 1) mask |= 1ull << (8 * ss + uint32_t(j));
  }
  if (table < 0) return true;
  // slots of the taken experts; softmax weights of the k selected logits
#pragma unroll
  for (int j = 0; j < 8; j++)
    if ((taken >> j) & 1) rt_st8(table, RT_SLOT + int((8 * s + uint32_t(j)) * 8 + b), slot[j]);
  const float top = group8(myv, fmax_);
  const float ex = (s < k && b < nB) ? __expf(myv - top) : 0.f;
  const float den = group8(ex, [](float x, float y) { return x + y; });
  if (b < nB) *reinterpret_cast<float*>(lds + table + RT_WT + int(b * 8 + s) * 4) = ex / den;
  // lane e: the sequences routed to expert e
  {
    const uint32_t e = lane, je = e & 7, se = e >> 3;
    uint64_t bj = 0;
#pragma unroll
    for (int j = 0; j < 8; j++)
      if (uint32_t(j) == je) bj = ball[j];
    uint32_t tok = 0;
    for (uint32_t bb = 0; bb < nB; bb++) tok |= uint32_t((bj >> (8 * bb + se)) & 1) << bb;
    const bool sel = (mask >> e) & 1;
    const uint32_t rank = __builtin_popcountll(mask & ((1ull << e) - 1));
    // exclusive prefix sum of the selected experts' pair counts, in rank order
    uint32_t pc = sel ? __builtin_popcount(tok) : 0, inc = pc;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t up = __shfl_up(inc, d, 64);
      if (lane >= uint32_t(d)) inc += up;
    }
    if (e < E) rt_st8(table, RT_TOK + int(e), tok);
    if (sel) {
      rt_st8(table, RT_LIST + int(rank), e);
      rt_st8(table, RT_PBASE + int(rank), inc - pc);
      // the expert's pairs, in sequence order (slots were stored above by
      // the lanes that took them; one wave's LDS accesses are in order)
      uint32_t pi = inc - pc;
      for (uint32_t bits = tok; bits; bits &= bits - 1, pi++) {
        const uint32_t bb = __builtin_ctz(bits);
        const uint32_t sl = rt_u8(table, RT_SLOT + int(e * 8 + bb));
        *reinterpret_cast<uint16_t*>(lds + table + RT_PAIR + int(pi) * 2) = uint16_t(e | bb << 6 | sl << 9);
        rt_st8(table, RT_PRANK + int(pi), rank);
      }
    }
  }
  if (lane == 0) {
    *reinterpret_cast<uint64_t*>(lds + table + RT_MASK) = mask;
    *lw(table + RT_NSEL) = uint32_t(__builtin_popcountll(mask));
    *lw(table + RT_NPAIR) = nB * k;
  }
  return true;
}

// --------------------------------------------------------------- loader
// Two runs of four 1 KiB units into one half page: src_a's four units at M0,
// src_b's at M0 + 4 KiB (the gate and up rows of one pair when rows are 4 KiB),
// non-temporal, each DMA followed by the deep in-flight throttle.
#define MK_DMA44(T)                                                                                 \
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\t"                                                   \
               "global_load_lds_dwordx4 %1, %2 nt\n\ts_waitcnt vmcnt(" MK_STR(T) ")\n\t"              \
               "global_load_lds_dwordx4 %1, %2 offset:1024 nt\n\ts_waitcnt vmcnt(" MK_STR(T) ")\n\t"  \
               "global_load_lds_dwordx4 %1, %2 offset:2048 nt\n\ts_waitcnt vmcnt(" MK_STR(T) ")\n\t"  \
               "global_load_lds_dwordx4 %1, %2 offset:3072 nt\n\ts_waitcnt vmcnt(" MK_STR(T) ")\n\t"  \
               "s_add_u32 m0, %0, 0x1000\n\ts_nop 0\n\t"                                              \
               "global_load_lds_dwordx4 %1, %3 nt\n\ts_waitcnt vmcnt(" MK_STR(T) ")\n\t"              \
               "global_load_lds_dwordx4 %1, %3 offset:1024 nt\n\ts_waitcnt vmcnt(" MK_STR(T) ")\n\t"  \
               "global_load_lds_dwordx4 %1, %3 offset:2048 nt\n\ts_waitcnt vmcnt(" MK_STR(T) ")\n\t"  \
               "global_load_lds_dwordx4 %1, %3 offset:3072 nt\n\ts_waitcnt vmcnt(" MK_STR(T) ")"        \
               :                                                                                    \
               : "s"(lds_addr), "v"(voff), "s"(src_a), "s"(src_b)                                   \
               : "memory", "m0")
DEV void dma_44(uint32_t lds_addr, uint64_t src_a, uint64_t src_b, uint32_t voff) {
  lds_addr = uni(lds_addr);
  src_a = uni64(src_a);
  src_b = uni64(src_b);
  MK_DMA44(MK_VMT_DEEP);
}

// This loader wave's half page (units u0 .. u0+7) of an expert's gate/up
// region: pair q occupies units [2q*nit, 2q*nit + 2*nit), its gate row first.
// Units past the CU's npu pairs read the zero page.
DEV void issue_gate_up(const KArgs& a, uint32_t dst, uint64_t gate, uint64_t up, uint32_t u0, uint32_t npu,
                       uint32_t nit, uint32_t rb, uint32_t voff, uint32_t voff4k, uint32_t& nd) {
  const uint64_t zero = uint64_t(a.zero_page);
  if (nit == 4 || nit == 8) {
    const uint32_t q = u0 / (2 * nit);
    if (q >= npu) {
      dma_run8(dst, zero, voff, voff4k, true);
    } else if (nit == 4) {
      dma_44(dst, gate + uint64_t(q) * rb, up + uint64_t(q) * rb, voff);
    } else {
      dma_run8(dst, ((u0 / nit) & 1 ? up : gate) + uint64_t(q) * rb, voff, voff4k, true);
    }
    nd += kDmaPerPage;
    return;
  }
  for (uint32_t j = 0; j < kDmaPerPage; j++) {
    const uint32_t u = u0 + j, q = u / (2 * nit), jj = u % nit;
    const uint64_t src = q < npu ? ((u / nit) & 1 ? up : gate) + uint64_t(q) * rb + jj * kUnit : zero;
    dma_uniform(uni(dst + j * kUnit), uni64(src), voff);
    vm_throttle(nd);
  }
}

// Same paging as the one-sequence loader, with a running page index: an
// expert instruction takes (selected experts) x (pages per expert) pages, a
// number known only once the loader has read the layer's router logits.
DEV void loader_b(const KArgs& a, InstrCP q, uint32_t n, int v, int cu) {
  const uint32_t voff = (threadIdx.x & 63) * 16, voff4k = voff + 4096;
  const uint32_t half = uint32_t(v) * kDmaPerPage;
  uint32_t nd = 0, g_issue = 0, g_pub = 0, min_rel = 0, pg = 0;
  uint32_t route_layer = 0xFFFFFFFFu;
  uint64_t mask = 0;
  uint32_t retries = 0;
  // the last expert down projection of each layer parity (its ready-queue
  // entries are reused two layers later)
  uint32_t dyn_prev[2] = {kNoCounter, kNoCounter};
  // the last expert sum of each layer parity (the last reader of that
  // parity's routing table)
  uint32_t rt_last[2] = {kNoCounter, kNoCounter};
  // wait for ring space for page g; false = abort
  auto acquire = [&](uint32_t g) -> bool {
    if (g < min_rel + lb::kPages) return true;
    Watch t0;
    for (;;) {
      min_rel = uni(min_released());
      if (g < min_rel + lb::kPages) return true;
      if (g_pub < g_issue) {
        wait_vm_pages(g_issue - g_pub - 1);
        publish(g_pub, g_pub + 1, v);
        continue;
      }
      if (aborted() || local_timeout(t0, local_limit())) {
        if (!aborted()) local_abort(STC_LOCAL_TIMEOUT);
        wait_vm0();
        return false;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  };
  auto after_issue = [&](uint32_t g, bool deep) {
    g_issue = g + 1;
    const uint32_t vmt = deep ? kVmTDeep : kVmT;
    if (nd > vmt) publish(g_pub, (nd - vmt) / kDmaPerPage, v);
  };
  for (uint32_t i = 0; i < n; i++) {
    InstrCP I = q + i;
    const uint32_t op = i_op(I);
    if (op == OP_ERD) {
      // the last reader of its layer's routing table slot
      rt_last[I->layer & 1] = i;
      continue;
    }
    if (op == OP_EGU || op == OP_EDN) {
      const uint32_t layer = I->layer;
      if (layer != route_layer) {
        // The routing decision, at the layer's first expert instruction: the
        // selected-expert union for the streaming, and (first loader wave)
        // the whole table for the compute waves, which then find it ready
        // instead of deciding it between their attention and gate/up work.
        // Every issued page is published before the waits.
        wait_vm0();
        publish(g_pub, g_issue, v);
        // the table slot of this parity was last read by the expert sum two
        // layers back
        const bool table = v == 0;
        bool ok = wait_counter(a, I->aux[0], a.epoch * I->aux[1], cu, i);
        if (ok && table && rt_last[layer & 1] != kNoCounter) ok = wait_all_ge(C_XCONS, rt_last[layer & 1] + 1);
        ok = ok && route_topk(a, I, mask, table ? rt_base(layer) : -1, retries);
        if (!ok) {
          if ((threadIdx.x & 63) == 0) lds_st(C_ABORT, 1);
          return;
        }
        mask = uni64(mask);
        route_layer = layer;
        if (table && (threadIdx.x & 63) == 0) {
          lds_st(C_RTOK, layer + 1);
          // CU 0 counts the layer's selected experts (bytes streamed per step)
          if (cu == 0)
            __hip_atomic_fetch_add(gp(a.route_stats) + layer, uint32_t(__builtin_popcountll(mask)),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      if (i_flags(I) & F_DIRECT) continue;
      const uint32_t ppe = I->aux[2], npu = I->aux[3], run = I->seg_rows[0], nit = i_nit(I), rb = I->row_bytes;
      const uint64_t stride = I->seg_stride[0];
      if (op == OP_EDN) {
        // this CU's units of the selected experts' down projections: its
        // static range, then the chunks it takes from the ready queue
        const uint32_t Rb = npu, nb = I->aux[4], d = uint32_t(a.hidden), layer = I->layer;
        const EdnSplit sp = edn_split(uint32_t(__builtin_popcountll(mask)), nb, I->row0);
        auto stream = [&](uint32_t lo, uint32_t hi) -> bool {
          for (uint32_t u = lo; u < hi; u++) {
            const uint32_t ue = u / nb, ub = u % nb;
            uint64_t m = mask;
            for (uint32_t er = 0; er < ue; er++) m &= m - 1;
            const uint32_t e = uint32_t(__builtin_ctzll(m));
            const uint64_t src = I->seg_ptr[1] + e * stride + uint64_t(ub) * run;
            const uint32_t valid = min(Rb, d - ub * Rb) * rb;
            for (uint32_t p = 0; p < ppe; p++) {
              const uint32_t g = pg++;
              if (!acquire(g)) return false;
              const uint32_t dst = uint32_t(size_t(lds)) + page_off<LayB>(g) + half * kUnit;
              issue_run(a, dst, src, (p * kUnitsPerPage + half) * kUnit, valid, voff, voff4k, nd, true);
              after_issue(g, true);
            }
          }
          return true;
        };
        uint32_t lo, hi;
        edn_range(sp.Ts, I->n_items, uint32_t(cu), lo, hi);
        if (!stream(lo, hi)) return;
        if (!I->row0) continue;
        // the queue entries of this parity were last read by the compute
        // waves in the expert down projection two layers back
        if (dyn_prev[layer & 1] != kNoCounter && !wait_all_ge(C_XCONS, dyn_prev[layer & 1] + 1)) {
          if ((threadIdx.x & 63) == 0) lds_st(C_ABORT, 1);
          return;
        }
        dyn_prev[layer & 1] = i;
        uint32_t* ctr = reinterpret_cast<uint32_t*>(I->res_ptr) + (a.epoch & 1);
        for (uint32_t k = 0;; k++) {
          uint32_t ch = 0;
          if (v == 0) {
            if ((threadIdx.x & 63) == 0)
              ch = __hip_atomic_fetch_add(gp(ctr), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ch = min(uni(ch), 0xFFFFu);
            if ((threadIdx.x & 63) == 0) lds_st(dyn_slot(layer, k), (layer + 1) << 16 | ch);
          } else if (!dyn_entry(layer, k, ch)) {
            return;
          }
          if (ch >= sp.n_dyn) break;
          const uint32_t u0 = sp.Ts + ch * sp.uc;
          if (!stream(u0, min(sp.T, u0 + sp.uc))) return;
        }
        continue;
      }
      for (uint64_t m = mask; m; m &= m - 1) {
        const uint32_t e = uint32_t(__builtin_ctzll(m));
        const uint64_t b0 = I->seg_ptr[1] + e * stride, b1 = I->seg_ptr[2] + e * stride;
        for (uint32_t p = 0; p < ppe; p++) {
          const uint32_t g = pg++;
          if (!acquire(g)) return;
          const uint32_t dst = uint32_t(size_t(lds)) + page_off<LayB>(g) + half * kUnit;
          issue_gate_up(a, dst, b0, b1, p * kUnitsPerPage + half, npu, nit, rb, voff, voff4k, nd);
          after_issue(g, true);
        }
      }
      continue;
    }
    LoadView L;
    load_view(a, I, L, a.pos);
    const uint32_t np = I->n_pages;
    for (uint32_t p = 0; p < np; p++) {
      const uint32_t g = pg++;
      if (!acquire(g)) return;
      issue_page<LayB>(a, L, p, g, v, voff, voff4k, nd);
      after_issue(g, L.deep);
    }
  }
  wait_vm0();
  publish(g_pub, g_issue, v);
}

// ------------------------------------------------------------- reductions
// Butterfly over 64 lanes of 16 values: afterwards lane l holds the sum over
// all lanes of v[l % 16].  Each stage pairs lanes (row mirror, half-row
// mirror, xor 2, xor 1), and the lane keeps one half of its values plus its
// partner's copy of that half; the 16-lane rows are then added with two
// exchanges.  Fixed order: deterministic.
template <int CTRL, int N>
DEV void bfly_stage(float (&v)[16], bool keep_lo) {
#pragma unroll
  for (int j = 0; j < N; j++) {
    const float send = keep_lo ? v[j + N] : v[j];
    const float keep = keep_lo ? v[j] : v[j + N];
    v[j] = keep + dpp<CTRL>(send);
  }
}
DEV float reduce16(float (&v)[16]) {
  const uint32_t l = threadIdx.x & 63;
  bfly_stage<0x140, 8>(v, (l & 15) < 8);  // row_mirror
  bfly_stage<0x141, 4>(v, (l & 7) < 4);   // row_half_mirror
  bfly_stage<0x4E, 2>(v, (l & 3) < 2);    // quad_perm [2,3,0,1]
  bfly_stage<0xB1, 1>(v, (l & 1) == 0);   // quad_perm [1,0,3,2]
  float r = v[0];
  r += __shfl_xor(r, 16, 64);
  r += __shfl_xor(r, 32, 64);
  return r;
}

// Sums over the wave of 32 values at once: after five exchange stages
// (mirrors inside 16-lane rows first, so that no stage's partner flips a lane
// bit an earlier stage has assigned, then xor 16) and a final xor-32 add,
// lane l holds the sum of v[idx(l)], idx(l) = l3 l2 l1 l0 l4 (bits, high to
// low).
template <int N, class X>
DEV void bfly_stage32(float (&v)[32], bool keep_lo, X xch) {
#pragma unroll
  for (int j = 0; j < N; j++) {
    const float send = keep_lo ? v[j + N] : v[j];
    const float keep = keep_lo ? v[j] : v[j + N];
    v[j] = keep + xch(send);
  }
}
DEV float reduce32(float (&v)[32]) {
  const uint32_t l = threadIdx.x & 63;
  bfly_stage32<16>(v, (l & 15) < 8, [](float x) { return dpp<0x140>(x); });  // row_mirror
  bfly_stage32<8>(v, (l & 7) < 4, [](float x) { return dpp<0x141>(x); });    // row_half_mirror
  bfly_stage32<4>(v, (l & 3) < 2, [](float x) { return dpp<0x4E>(x); });     // quad_perm [2,3,0,1]
  bfly_stage32<2>(v, (l & 1) == 0, [](float x) { return dpp<0xB1>(x); });    // quad_perm [1,0,3,2]
  bfly_stage32<1>(v, (l & 16) == 0, [](float x) { return __shfl_xor(x, 16, 64); });
  return v[0] + __shfl_xor(v[0], 32, 64);
}
DEV uint32_t reduce32_index(uint32_t l) {
  return (((l >> 3) & 1) << 4) | (((l >> 2) & 1) << 3) | (((l >> 1) & 1) << 2) | ((l & 1) << 1) | ((l >> 4) & 1);
}

DEV const float* res_slot_b(uint32_t i) {
  return reinterpret_cast<const float*>(lds + lb::kRes + (i & 1) * 4 * kMaxResRows);
}

// input token of sequence b, checked against the vocabulary
DEV uint32_t token_b(const KArgs& a, uint32_t b) {
  const int32_t t = gp(a.tokens)[b];
  if (t >= 0 && t < a.vocab) return uint32_t(t);
  __hip_atomic_store(gp(a.status) + ST_BADTOK, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return 0;
}

// Inverse RMS of every staged sequence (lane b holds sequence b's), from the
// per-chunk sums of squares; 1 without RMSNorm.
DEV float inv_rms(const KArgs& a, InstrCP I) {
  const uint32_t lane = threadIdx.x & 63;
  if (!(i_flags(I) & F_NORM)) return 1.f;
  const uint32_t K = I->k, per = K / 128;
  const float* ss = reinterpret_cast<const float*>(lds + lb::kSS);
  float s = 0.f;
  if (lane < uint32_t(a.batch))
    for (uint32_t j = 0; j < per; j++) s += ss[lane * per + j];
  return rsqrtf(s / float(K) + a.rms_eps);
}

// ----------------------------------------------------------------- staging
// Cooperative staging of a batched GEMV input [B][K] (tagged activations, or
// the bf16 embedding rows of the B tokens): wave w loads the 128-value chunks
// w, w + kNComp, ... (every load before the first wait), and once every wave
// has read the previous input writes g * x (the RMSNorm gain folded in; the
// inverse RMS is applied to the dot products) and each chunk's sum of squares.
// The leader also stages the residual rows of an EPI_RESID tile or of an
// expert down-projection: res[b][row0 .. row0 + n) for every sequence.
DEV bool stage_res_b(Comp& c, InstrCP I, uint32_t i, uint32_t n_rows, uint32_t rstride);

DEV bool coop_stage_b(Comp& c, InstrCP I, uint32_t i, bool stage_x) {
  const KArgs& a = *c.a;
  const uint32_t lane = c.lane;
  constexpr int NC = (lb::kXFloats / 128 + kNComp - 1) / kNComp;
  const uint32_t K = I->k, nB = uint32_t(a.batch), nch = nB * K / 128;
  const bool norm = i_flags(I) & F_NORM, embed = i_flags(I) & F_IN_EMBED;
  const __amdgpu_buffer_rsrc_t r =
      act_rsrc_u(reinterpret_cast<const void*>(I->in_ptr), (stage_x && !embed) ? nB * K * kActBytes : 0);
  const __amdgpu_buffer_rsrc_t rg = act_rsrc_u(reinterpret_cast<const void*>(I->gain_ptr), (stage_x && norm) ? K * 2 : 0);
  auto chunk = [&](int qq) -> uint32_t { return uint32_t(c.w) + kNComp * qq; };
  auto off = [&](int, int qq) -> uint32_t { return (chunk(qq) * 128 + 2 * lane) * kActBytes; };
  const uint32_t live = (stage_x && uint32_t(c.w) < nch) ? (nch - c.w + kNComp - 1) / kNComp : 0;
  u4 t[NC];
  uint32_t gw[NC], ew[NC];
  const int32_t tokv = (embed && stage_x && lane < nB) ? gp(a.tokens)[lane] : 0;
#pragma unroll
  for (int qq = 0; qq < NC; qq++) {
    const uint32_t flat = chunk(qq) * 128, kk = flat % K;
    t[qq] = ld_tag2(r, off(0, qq));
    gw[qq] = __builtin_amdgcn_raw_buffer_load_b32(rg, (kk + 2 * lane) * 2, 0, 0);
    ew[qq] = 0;
    if (embed && qq < int(live)) {
      int32_t tok = __builtin_amdgcn_readlane(tokv, int(flat / K));
      if (tok < 0 || tok >= a.vocab) {
        __hip_atomic_store(gp(a.status) + ST_BADTOK, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        tok = 0;
      }
      ew[qq] = *gp(reinterpret_cast<const uint32_t*>(I->in_ptr) + (size_t(tok) * K + kk) / 2 + lane);
    }
  }
  if (stage_x) {
    if (!embed && !wait_fresh(t, live, r, off, 0, in_tag(a.epoch, I), c.retries)) return false;
    if (!wait_all_ge(C_XCONS, i)) return false;
    float* xs = reinterpret_cast<float*>(lds + lb::kX);
    float* ss = reinterpret_cast<float*>(lds + lb::kSS);
#pragma unroll
    for (int qq = 0; qq < NC; qq++) {
      if (qq >= int(live)) continue;
      const uint32_t flat = chunk(qq) * 128 + 2 * lane;
      const float v0 = embed ? bf_lo(ew[qq]) : __uint_as_float(t[qq].x);
      const float v1 = embed ? bf_hi(ew[qq]) : __uint_as_float(t[qq].z);
      const float g0 = norm ? bf_lo(gw[qq]) : 1.f, g1 = norm ? bf_hi(gw[qq]) : 1.f;
      *reinterpret_cast<float2*>(xs + flat) = float2{g0 * v0, g1 * v1};
      if (norm) {
        const float s = sum64(fmaf(v0, v0, v1 * v1));
        if (lane == 0) ss[chunk(qq)] = s;
      }
    }
  }
  if (c.w == 0 && i_op(I) == OP_BGEMV && i_epi(I) == EPI_RESID)
    return stage_res_b(c, I, i, I->n_rows, I->aux[2]);
  return true;
}

// residual rows res[b][row0 + r] for r < n_rows, b < B (n_rows * B <= 128):
// tagged activations or, with F_RES_EMBED, the embedding rows of the tokens
DEV bool stage_res_b(Comp& c, InstrCP I, uint32_t i, uint32_t n_rows, uint32_t rstride) {
  const KArgs& a = *c.a;
  const uint32_t lane = c.lane, nB = uint32_t(a.batch), total = n_rows * nB;
  const bool embed = i_flags(I) & F_RES_EMBED;
  const uint32_t r0 = I->row0;
  const __amdgpu_buffer_rsrc_t rr = act_rsrc(reinterpret_cast<const void*>(I->res_ptr),
                                             embed ? 0 : nB * rstride * kActBytes);
  uint2 t[2];
  uint32_t eo[2] = {0, 0};
  uint32_t offs[2];
  for (int j = 0; j < 2; j++) {
    const uint32_t idx = 2 * lane + j, b = idx / n_rows, rr_ = idx % n_rows;
    offs[j] = (b * rstride + r0 + rr_) * kActBytes;
    reload(t[j], rr, offs[j]);
    if (embed && idx < total) {
      const uint32_t tok = token_b(a, b);
      eo[j] = *gp(reinterpret_cast<const uint16_t*>(I->res_ptr) + size_t(tok) * a.hidden + r0 + rr_);
    }
  }
  const uint32_t live = 2 * lane >= total ? 0 : (2 * lane + 1 < total ? 2 : 1);
  if (!embed && !wait_fresh(t, live, rr, [&](int, int j) { return offs[j]; }, 0, in_tag(a.epoch, I), c.retries))
    return false;
  float* rs = const_cast<float*>(res_slot_b(i));
  for (int j = 0; j < 2; j++)
    if (j < int(live)) rs[2 * lane + j] = embed ? __uint_as_float(eo[j] << 16) : __uint_as_float(t[j].x);
  return true;
}

// ------------------------------------------------------------- batched GEMV
// Unit u of the instruction's page stream (starting at page pg), this lane's
// 16 bytes.
DEV u4 unit_ld(uint32_t pg, uint32_t u, uint32_t lane) {
  return *reinterpret_cast<const u4*>(lds + page_off<LayB>(pg + u / kUnitsPerPage) + (u % kUnitsPerPage) * kUnit +
                                      lane * 16);
}
DEV void widen8(u4 w, float (&o)[8]) {
  o[0] = bf_lo(w.x); o[1] = bf_hi(w.x); o[2] = bf_lo(w.y); o[3] = bf_hi(w.y);
  o[4] = bf_lo(w.z); o[5] = bf_hi(w.z); o[6] = bf_lo(w.w); o[7] = bf_hi(w.w);
}
// the same sum as dot8, on widened weights
DEV float dot8f(const float (&w)[8], const float (&x)[8]) {
  float a = w[0] * x[0];
  a = fmaf(w[1], x[1], a);
  float b = w[2] * x[2];
  b = fmaf(w[3], x[3], b);
  a = fmaf(w[4], x[4], a);
  a = fmaf(w[5], x[5], a);
  b = fmaf(w[6], x[6], b);
  b = fmaf(w[7], x[7], b);
  return a + b;
}
DEV void x8_ld(const float* p, float (&o)[8]) {
  const f4 lo = *reinterpret_cast<const f4*>(p);
  const f4 hi = *reinterpret_cast<const f4*>(p + 4);
  o[0] = lo.x; o[1] = lo.y; o[2] = lo.z; o[3] = lo.w;
  o[4] = hi.x; o[5] = hi.y; o[6] = hi.z; o[7] = hi.w;
}

// acc[b] += row a . x_b and acc[8 + b] += row b . x_b over the K values of
// the staged inputs of the sequences in `tm`; rows are NIT units from unit ua
// and ub of the stream; x_b starts at xs + xoff(b).
template <class XOff>
DEV void dot_pair(uint32_t pg, uint32_t ua, uint32_t ub, uint32_t nit, uint32_t tm, XOff xoff,
                  float (&acc)[16]) {
  const uint32_t lane = threadIdx.x & 63;
  const float* xs = reinterpret_cast<const float*>(lds + lb::kX);
#pragma unroll
  for (int e = 0; e < 16; e++) acc[e] = 0.f;
  for (uint32_t j = 0; j < nit; j++) {
    // the weights widened once, then applied to every sequence
    float fa[8], fb[8];
    widen8(unit_ld(pg, ua + j, lane), fa);
    widen8(unit_ld(pg, ub + j, lane), fb);
#pragma unroll
    for (int b = 0; b < lb::kMaxB; b++) {
      if (!((tm >> b) & 1)) continue;
      float x[8];
      x8_ld(xs + xoff(b) + j * 512 + lane * 8, x);
      acc[b] += dot8f(fa, x);
      acc[8 + b] += dot8f(fb, x);
    }
  }
}

// acc[8 r + b] = row r . x_b for four consecutive rows (rows at or past
// nrows count as zero) and the sequences in `tm`; row r is NIT units from
// unit u0 + r * NIT.  Each sequence's input is read once for the four rows.
template <class XOff>
DEV void dot_rows4(uint32_t pg, uint32_t u0, uint32_t nit, uint32_t nrows, uint32_t tm, XOff xoff,
                   float (&acc)[32]) {
  const uint32_t lane = threadIdx.x & 63;
  const float* xs = reinterpret_cast<const float*>(lds + lb::kX);
#pragma unroll
  for (int e = 0; e < 32; e++) acc[e] = 0.f;
  for (uint32_t j = 0; j < nit; j++) {
    // the weights widened once, then applied to every sequence
    float w[4][8];
#pragma unroll
    for (int r = 0; r < 4; r++) widen8(uint32_t(r) < nrows ? unit_ld(pg, u0 + r * nit + j, lane) : u4{0, 0, 0, 0}, w[r]);
#pragma unroll
    for (int b = 0; b < lb::kMaxB; b++) {
      if (!((tm >> b) & 1)) continue;
      float x[8];
      x8_ld(xs + xoff(b) + j * 512 + lane * 8, x);
#pragma unroll
      for (int r = 0; r < 4; r++) acc[8 * r + b] += dot8f(w[r], x);
    }
  }
}

DEV bool bgemv(Comp& c, InstrCP I, uint32_t i, uint32_t pg) {
  const KArgs& a = *c.a;
  const uint32_t lane = c.lane, nB = uint32_t(a.batch), K = I->k, nit = i_nit(I);
  const uint32_t epi = i_epi(I), n_rows = I->n_rows, n_items = I->n_items, row0 = I->row0;
  const uint32_t ostride = I->aux[0];
  const uint32_t tm = (1u << nB) - 1;
  const float inv = inv_rms(a, I);
  const uint32_t li = lane & 15, ri = li >> 3, bb = li & 7;
  const float my_inv = __shfl(inv, int(bb), 64);
  uint64_t* out = reinterpret_cast<uint64_t*>(I->out_ptr);
  const float* res = res_slot_b(i);
  ArgBest best{-__builtin_inff(), 0xFFFFFFFFu};
  for (uint32_t t = c.w; t < n_items; t += kNComp) {
    const uint32_t u0 = t * 2 * nit;
    if (lane == 0) lds_st(C_RELEASED + 4 * c.w, pg + u0 / kUnitsPerPage);
    if (!wait_page(pg + (u0 + 2 * nit - 1) / kUnitsPerPage, c.fcache)) return false;
    float acc[16];
    dot_pair(pg, u0, u0 + nit, nit, tm, [&](int b) { return uint32_t(b) * K; }, acc);
    const float s = reduce16(acc) * my_inv;
    const uint32_t rl_ = 2 * t + ri;
    if (lane < 16 && bb < nB && rl_ < n_rows) {
      const uint32_t row = row0 + rl_;
      switch (epi) {
        case EPI_STORE:
          st_tag(out + size_t(bb) * ostride + row, s, a.epoch);
          break;
        case EPI_RESID:
          st_tag(out + size_t(bb) * ostride + row, res[bb * n_rows + rl_] + s, a.epoch);
          break;
        default:  // EPI_ARGMAX
          if (a.logits) gp(a.logits)[size_t(bb) * a.vocab + row] = s;
          if (s != s) __hip_atomic_store(gp(a.status) + ST_NAN, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          arg_update(best, s, row);
          break;
      }
    }
  }
  if (epi == EPI_ARGMAX) {
    // lanes b and b + 8 hold sequence b's best of even and odd rows
    const float ov = __shfl(best.v, int(lane + 8) & 63, 64);
    const uint32_t oi = __shfl(best.i, int(lane + 8) & 63, 64);
    arg_update(best, ov, oi);
    if (lane < 8) {
      *lw(lb::kArg + (c.w * 8 + int(lane)) * 8) = __float_as_uint(best.v);
      *lw(lb::kArg + (c.w * 8 + int(lane)) * 8 + 4) = best.i;
    }
  }
  if (lane == 0) {
    lds_st(C_RELEASED + 4 * c.w, pg + I->n_pages);
    lds_st(C_XCONS + 4 * c.w, i + 1);
  }
  return true;
}

// ---------------------------------------------- matrix-core batched GEMV
// F_MFMA tiles: items are blocks of 16 rows, streamed in fragment order (one
// 1 KiB unit per 32 columns); the B operand is the staged input, the B
// sequences' bf16 high parts in columns 0 .. 7 and their low parts in 8 .. 15,
// so that one v_mfma_f32_16x16x32_bf16 applies 32 columns of 16 rows to both.
// Every compute wave takes the column steps w, w + 6, ... of each block (all
// waves walk the same pages), adds its high and low columns, and leaves its
// [16 rows][8 sequences] partial in LDS; the wave that arrives last at a
// block adds the six partials in wave order and runs the epilogue.  mblk
// counts the blocks of all such instructions so far (every wave alike).
// The staged input (g * x, fp32 [B][K]) rewritten in the B operand order of
// the matrix-core GEMV: column step k / 32, lane 16 ((k % 32) / 8) + b for the
// bf16 high part of x_b[k] and lane 16 ((k % 32) / 8) + 8 + b for the low part
// (the rounding residue, so that high + low carries 16 significant bits),
// value k % 8 of the lane's 8.  Each wave reads its values, all waves meet,
// then write; one more meeting publishes the slot.
DEV bool mfma_order(Comp& c, InstrCP I) {
  constexpr int NC = (lb::kXFloats / 128 + kNComp - 1) / kNComp;
  const uint32_t lane = c.lane, K = I->k, nch = uint32_t(c.a->batch) * K / 128;
  const float* xs = reinterpret_cast<const float*>(lds + lb::kX);
  float2 v[NC];
#pragma unroll
  for (int qq = 0; qq < NC; qq++) {
    const uint32_t ch = uint32_t(c.w) + kNComp * qq;
    if (ch < nch) v[qq] = *reinterpret_cast<const float2*>(xs + ch * 128 + 2 * lane);
  }
  if (!comp_barrier()) return false;
#pragma unroll
  for (int qq = 0; qq < NC; qq++) {
    const uint32_t ch = uint32_t(c.w) + kNComp * qq;
    if (ch >= nch) continue;
    const uint32_t flat = ch * 128 + 2 * lane, b = flat / K, k = flat % K;
    const uint32_t h0 = f2bf(v[qq].x), h1 = f2bf(v[qq].y);
    const uint32_t l0 = f2bf(v[qq].x - __uint_as_float(h0 << 16)), l1 = f2bf(v[qq].y - __uint_as_float(h1 << 16));
    char* xb = lds + lb::kX + (k / 32) * 1024 + ((k % 32) / 8) * 256 + (k % 8) * 2;
    *reinterpret_cast<uint32_t*>(xb + b * 16) = h0 | h1 << 16;
    *reinterpret_cast<uint32_t*>(xb + (8 + b) * 16) = l0 | l1 << 16;
  }
  return comp_barrier();
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
DEV bool bgemv_mfma(Comp& c, InstrCP I, uint32_t i, uint32_t pg, uint32_t& mblk) {
  const KArgs& a = *c.a;
  const uint32_t lane = c.lane, nB = uint32_t(a.batch), ks = I->k / 32;
  const uint32_t epi = i_epi(I), n_rows = I->n_rows, n_blocks = I->n_items, row0 = I->row0;
  const uint32_t ostride = I->aux[0];
  const uint32_t n = lane & 15, q = lane >> 4;  // output column, row quad
  const bool live_col = (n & 7) < nB;
  const float inv = inv_rms(a, I);
  const float my_inv = __shfl(inv, int(n & 7), 64);
  const char* xb = lds + lb::kX;
  f4* part = reinterpret_cast<f4*>(lds + lb::kMfma);
  uint64_t* out = reinterpret_cast<uint64_t*>(I->out_ptr);
  const float* res = res_slot_b(i);
  ArgBest best{-__builtin_inff(), 0xFFFFFFFFu};
  for (uint32_t blk = 0; blk < n_blocks; blk++, mblk++) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (uint32_t st = uint32_t(c.w); st < ks; st += kNComp) {
      const uint32_t u = blk * ks + st;
      if (lane == 0) lds_st(C_RELEASED + 4 * c.w, pg + u / kUnitsPerPage);
      if (!wait_page(pg + u / kUnitsPerPage, c.fcache)) return false;
      const bf16x8 A = *reinterpret_cast<const bf16x8*>(lds + page_off<LayB>(pg + u / kUnitsPerPage) +
                                                       (u % kUnitsPerPage) * kUnit + lane * 16);
      bf16x8 B = *reinterpret_cast<const bf16x8*>(xb + st * 1024 + lane * 16);
      if (!live_col) B = bf16x8{};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc, 0, 0, 0);
    }
    // lane (q, n < 8): rows 4 q .. 4 q + 3 of sequence n, high + low parts
    f4 v;
    v.x = acc[0] + __shfl_down(acc[0], 8, 64);
    v.y = acc[1] + __shfl_down(acc[1], 8, 64);
    v.z = acc[2] + __shfl_down(acc[2], 8, 64);
    v.w = acc[3] + __shfl_down(acc[3], 8, 64);
    // the partial slots are free once the previous block has been reduced
    if (!wait_lds_ge(C_MRED, mblk)) return false;
    if (n < 8) part[c.w * 32 + q * 8 + n] = v;
    uint32_t prev = 0;
    if (lane == 0) prev = lds_add(C_MARR, 1);
    prev = uni(prev);
    if (prev + 1 != uint32_t(kNComp) * (mblk + 1)) continue;
    // last to arrive: the block's sums, the six partials in wave order
    if (n < 8) {
      f4 t = part[q * 8 + n];
#pragma unroll
      for (int w2 = 1; w2 < kNComp; w2++) {
        const f4 p2 = part[w2 * 32 + q * 8 + n];
        t.x += p2.x;
        t.y += p2.y;
        t.z += p2.z;
        t.w += p2.w;
      }
      const float tv[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const uint32_t rl = blk * 16 + q * 4 + uint32_t(r);
        if (rl >= n_rows || n >= nB) continue;
        const float sv = tv[r] * my_inv;
        const uint32_t row = row0 + rl;
        switch (epi) {
          case EPI_STORE:
            st_tag(out + size_t(n) * ostride + row, sv, c.ep);
            break;
          case EPI_RESID:
            st_tag(out + size_t(n) * ostride + row, res[n * n_rows + rl] + sv, c.ep);
            break;
          default:  // EPI_ARGMAX
            if (a.logits) gp(a.logits)[size_t(n) * a.vocab + row] = sv;
            if (sv != sv) __hip_atomic_store(gp(a.status) + ST_NAN, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            arg_update(best, sv, row);
            break;
        }
      }
    }
    if (lane == 0) lds_st(C_MRED, mblk + 1);
  }
  if (epi == EPI_ARGMAX) {
    // lanes n, n + 16, n + 32, n + 48 hold sequence n's best of their rows
#pragma unroll
    for (int m = 16; m < 64; m <<= 1) {
      const float ov = __shfl_xor(best.v, m, 64);
      const uint32_t oi = __shfl_xor(best.i, m, 64);
      arg_update(best, ov, oi);
    }
    if (lane < 8) {
      *lw(lb::kArg + (c.w * 8 + int(lane)) * 8) = __float_as_uint(best.v);
      *lw(lb::kArg + (c.w * 8 + int(lane)) * 8 + 4) = best.i;
    }
  }
  if (lane == 0) {
    lds_st(C_RELEASED + 4 * c.w, pg + I->n_pages);
    lds_st(C_XCONS + 4 * c.w, i + 1);
  }
  return true;
}

// ------------------------------------------------------ expert gate / up
// Items are (selected expert, pair of the CU's slice) in expert order; the
// loader lays each pair out as its gate row then its up row.  An item applies
// the two rows to the sequences routed to the expert and stores
// m = silu(gate) * up (fp32) at [b][slot of e in b's top-k][row].  The stores
// are plain device-scope stores: the instruction's counter moves only after
// every wave's stores have landed.
DEV bool egu(Comp& c, InstrCP I, uint32_t i, uint32_t pg) {
  const KArgs& a = *c.a;
  const uint32_t lane = c.lane, K = I->k, nit = i_nit(I);
  const int rt = rt_base(I->layer);
  const uint32_t nsel = *lw(rt + RT_NSEL), npu = I->aux[3], ppe = I->aux[2];
  const uint32_t Fe = uint32_t(a.expert_ffn), k = uint32_t(a.top_k);
  const float inv = inv_rms(a, I);
  const float my_inv = __shfl(inv, int(lane & 7), 64);
  float* out = reinterpret_cast<float*>(I->out_ptr);
  const uint32_t n_items = nsel * npu;
  for (uint32_t t = c.w; t < n_items; t += kNComp) {
    const uint32_t er = t / npu, p = t % npu;
    const uint32_t e = uni(rt_u8(rt, RT_LIST + int(er)));
    const uint32_t tm = uni(rt_u8(rt, RT_TOK + int(e)));
    const uint32_t ug = er * ppe * kUnitsPerPage + 2 * p * nit, uu = ug + nit;
    if (lane == 0) lds_st(C_RELEASED + 4 * c.w, pg + ug / kUnitsPerPage);
    if (!wait_page(pg + (uu + nit - 1) / kUnitsPerPage, c.fcache)) return false;
    float acc[16];
    dot_pair(pg, ug, uu, nit, tm, [&](int b) { return uint32_t(b) * K; }, acc);
    const float s = reduce16(acc);
    const float up = __shfl(s, int((lane & 7) + 8), 64);
    if (lane < 8 && ((tm >> lane) & 1)) {
      const uint32_t slot = rt_u8(rt, RT_SLOT + int(e * 8 + lane));
      const float m = silu(s * my_inv) * (up * my_inv);
      st_act(out + (size_t(lane) * k + slot) * Fe + I->row0 + p, m);
    }
  }
  if (lane == 0) {
    lds_st(C_RELEASED + 4 * c.w, pg + nsel * ppe);
    lds_st(C_XCONS + 4 * c.w, i + 1);
  }
  return true;
}

// Gate/up with the weight rows loaded by the compute waves themselves: each
// wave keeps the rows of its next D-1 items in flight in registers while it
// computes the current one (NIT 1 KiB units per row), so the loads of six
// waves cover the memory latency without the LDS ring; the loader meanwhile
// prefetches the following instructions' pages.
template <int NIT>
DEV bool egu_direct(Comp& c, InstrCP I, uint32_t i) {
  constexpr int D = 3;
  const KArgs& a = *c.a;
  const uint32_t lane = c.lane, K = I->k;
  const int rt = rt_base(I->layer);
  const uint32_t nsel = *lw(rt + RT_NSEL), npu = I->aux[3];
  const uint32_t Fe = uint32_t(a.expert_ffn), k = uint32_t(a.top_k), rb = I->row_bytes;
  const uint64_t stride = I->seg_stride[0];
  // row 0 of expert 0's gate and up matrices
  const uint64_t gate0 = I->seg_ptr[1] - uint64_t(I->row0) * rb, up0 = I->seg_ptr[2] - uint64_t(I->row0) * rb;
  const uint64_t zero = uint64_t(a.zero_page);
  const float inv = inv_rms(a, I);
  const float my_inv = __shfl(inv, int(lane & 7), 64);
  const float* xs = reinterpret_cast<const float*>(lds + lb::kX);
  float* out = reinterpret_cast<float*>(I->out_ptr);
  // n items of this wave, item j = (selected-expert rank, FFN row), with
  // the rows of the next D - 1 items in flight while one is computed
  auto run = [&](uint32_t n, auto item) {
    u4 wg[D][NIT], wu[D][NIT];
    // Every call issues the same loads (items past the end read the zero
    // page), so that the wait before an item's use counts exactly the loads
    // issued after it and the next items stay in flight.
    auto issue = [&](uint32_t j, u4 (&g)[NIT], u4 (&u)[NIT]) {
      uint64_t ga = zero, ua = zero;
      if (j < n) {
        uint32_t er, row;
        item(j, er, row);
        const uint32_t e = uni(rt_u8(rt, RT_LIST + int(er)));
        ga = gate0 + e * stride + uint64_t(row) * rb;
        ua = up0 + e * stride + uint64_t(row) * rb;
      }
      const u4* gs = reinterpret_cast<const u4*>(ga) + lane;
      const u4* us = reinterpret_cast<const u4*>(ua) + lane;
#pragma unroll
      for (int jj = 0; jj < NIT; jj++) {
        g[jj] = __builtin_nontemporal_load(gp(gs + 64 * jj));
        u[jj] = __builtin_nontemporal_load(gp(us + 64 * jj));
      }
    };
#pragma unroll
    for (int s = 0; s < D - 1; s++) issue(uint32_t(s), wg[s], wu[s]);
    for (uint32_t i0 = 0;; i0 += D) {
#pragma unroll
      for (int s = 0; s < D; s++) {
        const uint32_t j = i0 + uint32_t(s);
        if (j >= n) return;
        issue(j + D - 1, wg[(s + D - 1) % D], wu[(s + D - 1) % D]);
        uint32_t er, row;
        item(j, er, row);
        const uint32_t e = uni(rt_u8(rt, RT_LIST + int(er)));
        const uint32_t tm = uni(rt_u8(rt, RT_TOK + int(e)));
        float acc[16];
#pragma unroll
        for (int qq = 0; qq < 16; qq++) acc[qq] = 0.f;
#pragma unroll
        for (int jj = 0; jj < NIT; jj++) {
#pragma unroll
          for (int b = 0; b < lb::kMaxB; b++) {
            if (!((tm >> b) & 1)) continue;
            float x[8];
            x8_ld(xs + uint32_t(b) * K + jj * 512 + lane * 8, x);
            acc[b] += dot8(wg[s][jj], x);
            acc[8 + b] += dot8(wu[s][jj], x);
          }
        }
        const float sv = reduce16(acc);
        const float upv = __shfl(sv, int((lane & 7) + 8), 64);
        if (lane < 8 && ((tm >> lane) & 1)) {
          const uint32_t slot = rt_u8(rt, RT_SLOT + int(e * 8 + lane));
          const float m = silu(sv * my_inv) * (upv * my_inv);
          st_act(out + (size_t(lane) * k + slot) * Fe + row, m);
        }
      }
    }
  };
  if (i_flags(I) & F_SHARE) {
    // the CU's share [g0, g1) of the (rank, row) items in rank order; item
    // g0 + t goes to wave t mod kNComp
    const uint64_t T = uint64_t(nsel) * Fe;
    const uint32_t g0 = uint32_t((T * I->seg_rows[1]) >> 16), g1 = uint32_t((T * I->seg_rows[2]) >> 16);
    const uint32_t n_mine = g0 + uint32_t(c.w) < g1 ? (g1 - g0 - c.w + kNComp - 1) / kNComp : 0u;
    run(n_mine, [&](uint32_t j, uint32_t& er, uint32_t& row) {
      const uint32_t g = g0 + uint32_t(c.w) + kNComp * j;
      er = g / Fe;
      row = g % Fe;
    });
  } else {
    // the CU's slice of every expert: items t = w, w + kNComp, ... of
    // (rank, pair) in rank order
    const uint32_t n_static = nsel * npu;
    const uint32_t n_mine = uint32_t(c.w) < n_static ? (n_static - c.w + kNComp - 1) / kNComp : 0u;
    run(n_mine, [&](uint32_t j, uint32_t& er, uint32_t& row) {
      const uint32_t t = uint32_t(c.w) + kNComp * j;
      er = t / npu;
      row = I->row0 + t % npu;
    });
  }
  if (lane == 0) lds_st(C_XCONS + 4 * c.w, i + 1);
  return true;
}

// ---------------------------------------------------- expert down projection
// A CU's units touch one expert, or a few; only the routed sequences of
// those experts are staged: their intermediates m[b][slot] go into the x slot
// in groups of whole experts (at most cap = 16384 / Fe vectors; most CUs
// need one group).  Items are (unit,
// block of four rows); an item applies its rows to every sequence routed to
// the unit's expert and stores y[b][slot of the expert in b's top-k][row].
// The items of units [ua, ub) of an expert down projection, loaded by the
// compute waves themselves: item t = (unit, block of four rows) goes to wave
// t mod kNComp; its rows (DN 1 KiB units each) are loaded two items ahead.
// The routed sequences of the item's expert are taken four at a time (one
// pass covers the usual case); the experts' routed inputs are in the x slot
// from pair p0 on.
template <int DN>
DEV void edn_items_direct(Comp& c, InstrCP I, uint32_t ua, uint32_t ub, uint32_t p0, const float* xs,
                          uint64_t* yout, uint32_t ytag) {
  constexpr int D = 3;
  const KArgs& a = *c.a;
  const uint32_t lane = c.lane, K = I->k, Rb = I->aux[3], nb = I->aux[4], d = uint32_t(a.hidden);
  const uint32_t k = uint32_t(a.top_k), rbytes = I->row_bytes;
  const uint64_t stride = I->seg_stride[0], w0 = I->seg_ptr[1];
  const int rt = rt_base(I->layer);
  const uint32_t nrb = (Rb + 3) / 4, n_items = (ub - ua) * nrb;
  const uint32_t n = uint32_t(c.w) < n_items ? (n_items - uint32_t(c.w) + kNComp - 1) / kNComp : 0u;
  // Every call issues the same loads (items past the end read the zero
  // page, a row past the unit's last re-reads that row, its sums unused), so
  // that the wait before an item's use counts exactly the loads issued after
  // it and the next items stay in flight.
  const uint64_t zero = uint64_t(a.zero_page);
  u4 wr[D][4][DN];
  // (selects, not branches: the loads must not sit in conditional blocks)
  auto issue = [&](uint32_t j, u4 (&w)[4][DN]) {
    const bool ok = j < n;
    const uint32_t it = uint32_t(c.w) + kNComp * (ok ? j : 0u);
    const uint32_t u = ua + it / nrb, r0 = 4 * (it % nrb), rb = u % nb;
    const uint32_t er = ok ? u / nb : 0u, rows = min(Rb, d - rb * Rb);
    const uint32_t e = uni(rt_u8(rt, RT_LIST + int(er)));
    const uint64_t src = ok ? w0 + e * stride + uint64_t(rb * Rb) * rbytes : zero;
    const uint32_t step = ok ? rbytes : 0u;
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const uint64_t rs = src + uint64_t(min(r0 + uint32_t(r), rows - 1) * step);
#pragma unroll
      for (int jj = 0; jj < DN; jj++) w[r][jj] = __builtin_nontemporal_load(gp(reinterpret_cast<const u4*>(rs) + lane + 64 * jj));
    }
  };
#pragma unroll
  for (int s = 0; s < D - 1; s++) issue(uint32_t(s), wr[s]);
  for (uint32_t i0 = 0;; i0 += D) {
#pragma unroll
    for (int s = 0; s < D; s++) {
      const uint32_t j = i0 + uint32_t(s);
      if (j >= n) return;
      issue(j + D - 1, wr[(s + D - 1) % D]);
      const uint32_t it = uint32_t(c.w) + kNComp * j;
      const uint32_t u = ua + it / nrb, r0 = 4 * (it % nrb), er = u / nb, rb = u % nb;
      const uint32_t rows = min(Rb, d - rb * Rb);
      const uint32_t e = uni(rt_u8(rt, RT_LIST + int(er)));
      const uint32_t tok = uni(rt_u8(rt, RT_TOK + int(e)));
      const uint32_t base = uni(rt_u8(rt, RT_PBASE + int(er))) - p0;
      const uint32_t nt = uint32_t(__builtin_popcount(tok));
      for (uint32_t p = 0; p < nt; p += 4) {
        // acc[4 r + q] = row r . x of the routed sequence of rank p + q
        float acc[16];
#pragma unroll
        for (int q = 0; q < 16; q++) acc[q] = 0.f;
#pragma unroll
        for (int jj = 0; jj < DN; jj++) {
#pragma unroll
          for (int q = 0; q < 4; q++) {
            if (p + q >= nt) continue;
            float x[8];
            x8_ld(xs + (base + p + uint32_t(q)) * K + jj * 512 + lane * 8, x);
#pragma unroll
            for (int r = 0; r < 4; r++) acc[4 * r + q] += dot8(wr[s][r][jj], x);
          }
        }
        // lane l < 16 holds the sum of acc[l]: row l / 4, rank p + l % 4
        const float sdot = reduce16(acc);
        const uint32_t rr = lane >> 2, rank = p + (lane & 3);
        if (lane < 16 && rank < nt && r0 + rr < rows) {
          uint32_t m = tok;
          for (uint32_t t = 0; t < rank; t++) m &= m - 1;
          const uint32_t bb = uint32_t(__builtin_ctz(m));
          const uint32_t slot = rt_u8(rt, RT_SLOT + int(e * 8 + bb));
          st_tag(yout + size_t(bb * k + slot) * d + rb * Rb + r0 + rr, sdot, ytag);
        }
      }
    }
  }
}

// DN = 0: the loader streams the units through the page ring; DN = 1, 2
// (F_DIRECT, DN = 1 KiB units per row): each compute wave loads its own
// rows, three items in flight, and wave 0 takes the ready-queue chunks.
template <int DN>
DEV bool edn(Comp& c, InstrCP I, uint32_t i, uint32_t pg, uint32_t& np) {
  const KArgs& a = *c.a;
  const uint32_t lane = c.lane, K = I->k, nit = i_nit(I), nB = uint32_t(a.batch);
  const int rt = rt_base(I->layer);
  const uint32_t nsel = *lw(rt + RT_NSEL);
  const uint32_t ppu = I->aux[2], Rb = I->aux[3], nb = I->aux[4], d = uint32_t(a.hidden);
  const uint32_t k = uint32_t(a.top_k), Fe = uint32_t(a.expert_ffn);
  const uint32_t cap = uint32_t(lb::kXFloats) / K;  // staged vectors per group
  const EdnSplit sp = edn_split(nsel, nb, I->row0);
  const uint32_t ytag = y_tag(c.ep, I->layer);
  float* xs = reinterpret_cast<float*>(lds + lb::kX);
  uint64_t* yout = reinterpret_cast<uint64_t*>(I->out_ptr);
  const bool trl = a.trace && c.w == 0 && lane == 0;
  const __amdgpu_buffer_rsrc_t rm = act_rsrc(reinterpret_cast<const void*>(I->in_ptr), nB * k * Fe * 4);
  auto n_pairs = [&](uint32_t er) -> uint32_t {
    return uint32_t(__builtin_popcount(rt_u8(rt, RT_TOK + int(rt_u8(rt, RT_LIST + int(er))))));
  };
  // the intermediates of the pairs [p0, p0 + np) into the x slot, 256
  // values per wave and chunk, four chunks of a wave in flight at a time
  auto stage_group = [&](uint32_t p0, uint32_t npr) {
    const uint32_t nch = npr * K / 256;
    for (uint32_t c0 = uint32_t(c.w); c0 < nch; c0 += 4 * kNComp) {
      f4 t[4];
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const uint32_t ch = c0 + kNComp * j;
        uint32_t off = 0;
        if (ch < nch) {
          const uint32_t pi = p0 + ch * 256 / K, kk = ch * 256 % K;
          const uint32_t pr = *reinterpret_cast<const uint16_t*>(lds + rt + RT_PAIR + int(pi) * 2);
          const uint32_t b = (pr >> 6) & 7, sl = pr >> 9;
          off = ((b * k + sl) * Fe + kk + 4 * lane) * 4;
        }
        t[j] = ld_act4(rm, off);
      }
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const uint32_t ch = c0 + kNComp * j;
        if (ch < nch) *reinterpret_cast<f4*>(xs + ch * 256 + 4 * lane) = t[j];
      }
    }
  };
  const uint32_t nrb = (Rb + 3) / 4;
  bool staged_any = false;
  // Units [u_lo, u_hi), whose pages start pofs pages into the instruction's
  // stream: their experts' routed sequences are staged in groups of whole
  // experts (at most cap pairs); items are (unit, block of four rows).
  auto run_units = [&](uint32_t u_lo, uint32_t u_hi, uint32_t pofs) -> bool {
    const uint32_t er_last = (u_hi - 1) / nb;
    for (uint32_t g0 = u_lo / nb;;) {
      uint32_t g1 = g0, cnt = n_pairs(g0);
      while (g1 < er_last && cnt + n_pairs(g1 + 1) <= cap) cnt += n_pairs(++g1);
      const uint32_t p0 = rt_u8(rt, RT_PBASE + int(g0));
      const uint32_t npr = rt_u8(rt, RT_PBASE + int(g1)) + n_pairs(g1) - p0;
      // every wave has finished the previous group before its slot is rewritten
      if (staged_any && !comp_barrier()) return false;
      staged_any = true;
      stage_group(p0, npr);
      if (!comp_barrier()) return false;
      if (trl && pofs == 0 && g0 == u_lo / nb) {
        trace_put(a, c.cu, i, TR_STAGED, now32());
        trace_put(a, c.cu, i, TR_ITEM0, now32());
      }
      const uint32_t ua = max(u_lo, g0 * nb), ub = min(u_hi, (g1 + 1) * nb);
      const uint32_t n_items = (ub - ua) * nrb;
      if constexpr (DN > 0) {
        edn_items_direct<DN>(c, I, ua, ub, p0, xs, yout, ytag);
        if (g1 >= er_last) return true;
        g0 = g1 + 1;
        continue;
      }
      for (uint32_t it = c.w; it < n_items; it += kNComp) {
        const uint32_t u = ua + it / nrb, r0 = 4 * (it % nrb);
        const uint32_t er = u / nb, rb = u % nb;
        const uint32_t rows_u = min(Rb, d - rb * Rb);
        if (r0 >= rows_u) continue;
        const uint32_t e = uni(rt_u8(rt, RT_LIST + int(er)));
        const uint32_t tok = uni(rt_u8(rt, RT_TOK + int(e)));
        const uint32_t base = uni(rt_u8(rt, RT_PBASE + int(er))) - p0;
        const uint32_t nrows = min(4u, rows_u - r0);
        const uint32_t u0 = (pofs + (u - u_lo) * ppu) * kUnitsPerPage + r0 * nit;
        if (lane == 0) lds_st(C_RELEASED + 4 * c.w, pg + u0 / kUnitsPerPage);
        if (!wait_page(pg + (u0 + nrows * nit - 1) / kUnitsPerPage, c.fcache)) return false;
        float acc[32];
        dot_rows4(pg, u0, nit, nrows, tok,
                  [&](int b) { return (base + __builtin_popcount(tok & ((1u << b) - 1))) * K; }, acc);
        const float sdot = reduce32(acc);
        const uint32_t idx = reduce32_index(lane), rr = idx >> 3, bb = idx & 7;
        if (lane < 32 && ((tok >> bb) & 1) && rr < nrows) {
          const uint32_t slot = rt_u8(rt, RT_SLOT + int(e * 8 + bb));
          st_tag(yout + size_t(bb * k + slot) * d + rb * Rb + r0 + rr, sdot, ytag);
        }
      }
      // the next group starts at the unit after this group's last one
      if (lane == 0) lds_st(C_RELEASED + 4 * c.w, pg + pofs + (ub - u_lo) * ppu);
      if (g1 >= er_last) return true;
      g0 = g1 + 1;
    }
  };
  // every wave has left the previous input before the slot is rewritten
  if (!wait_all_ge(C_XCONS, i)) return false;
  if (trl) trace_put(a, c.cu, i, TR_XFREE, now32());
  uint32_t u_lo, u_hi, pofs = 0;
  edn_range(sp.Ts, I->n_items, uint32_t(c.cu), u_lo, u_hi);
  if (u_lo < u_hi) {
    if (!run_units(u_lo, u_hi, 0)) return false;
    pofs = (u_hi - u_lo) * ppu;
  }
  // then the chunks the loader (direct: compute wave 0) took from the ready
  // queue, in its order
  for (uint32_t q = 0; I->row0; q++) {
    uint32_t ch = 0;
    if (DN > 0 && c.w == 0) {
      if (lane == 0)
        ch = __hip_atomic_fetch_add(gp(reinterpret_cast<uint32_t*>(I->res_ptr)) + (c.ep & 1), 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
      ch = min(uni(ch), 0xFFFFu);
      if (lane == 0) lds_st(dyn_slot(I->layer, q), (I->layer + 1) << 16 | ch);
    } else if (!dyn_entry(I->layer, q, ch)) {
      return false;
    }
    if (ch >= sp.n_dyn) break;
    const uint32_t u0 = sp.Ts + ch * sp.uc, u1 = min(sp.T, u0 + sp.uc);
    if (!run_units(u0, u1, pofs)) return false;
    pofs += (u1 - u0) * ppu;
  }
  if (trl) trace_put(a, c.cu, i, TR_A_STATS, now32());
  if constexpr (DN > 0) pofs = 0;
  if (lane == 0) {
    lds_st(C_RELEASED + 4 * c.w, pg + pofs);
    lds_st(C_XCONS + 4 * c.w, i + 1);
  }
  np = pofs;
  return true;
}

// Expert sum: x_{l+1}[b][r] = h[b][r] + sum over the top-k slots s, in slot
// order, of w[b][s] * y[b][s][r] for the instruction's rows.  The outputs of
// the experts are polled by their tags (their writers are decided by the
// routing), the residual h by the step's tag.
DEV bool erd(Comp& c, InstrCP I, uint32_t i) {
  const KArgs& a = *c.a;
  const uint32_t lane = c.lane, nB = uint32_t(a.batch), k = uint32_t(a.top_k), d = uint32_t(a.hidden);
  const uint32_t nr = I->n_rows, r0 = I->row0, total = nB * nr;
  const int rt = rt_base(I->layer);
  const float* wt = reinterpret_cast<const float*>(lds + rt + RT_WT);
  const uint32_t htag = in_tag(c.ep, I), ytag = y_tag(htag, I->layer);
  const __amdgpu_buffer_rsrc_t ry = act_rsrc(reinterpret_cast<const void*>(I->in_ptr), nB * k * d * kActBytes);
  const __amdgpu_buffer_rsrc_t rh = act_rsrc(reinterpret_cast<const void*>(I->res_ptr), nB * d * kActBytes);
  uint64_t* out = reinterpret_cast<uint64_t*>(I->out_ptr);
  // one CU clears the layer's ready-queue counter of the next step (this
  // step's expert down projections use the other one)
  if (I->seg_ptr[0] && c.w == 0 && lane == 0)
    __hip_atomic_store(gp(reinterpret_cast<uint32_t*>(I->seg_ptr[0])) + ((c.ep + 1) & 1), 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  for (uint32_t base = uint32_t(c.w) * 64; base < total; base += 64 * kNComp) {
    const uint32_t idx = base + lane, on = idx < total;
    const uint32_t b = on ? idx / nr : 0, r = on ? idx % nr : 0, row = r0 + r;
    auto yoff = [&](int, int s) -> uint32_t { return ((b * k + uint32_t(s)) * d + row) * kActBytes; };
    uint2 ty[lb::kMaxTopK], th[1];
#pragma unroll
    for (int s = 0; s < lb::kMaxTopK; s++)
      if (uint32_t(s) < k) reload(ty[s], ry, yoff(0, s));
    reload(th[0], rh, (b * d + row) * kActBytes);
    if (!wait_fresh(ty, on ? k : 0, ry, yoff, 0, ytag, c.retries)) return false;
    if (!wait_fresh(th, on, rh, [&](int, int) { return (b * d + row) * kActBytes; }, 0, htag, c.retries))
      return false;
    if (a.trace && c.w == 0 && lane == 0 && base == 0) trace_put(a, c.cu, i, TR_STAGED, now32());
    float y = 0.f;
#pragma unroll
    for (int s = 0; s < lb::kMaxTopK; s++)
      if (uint32_t(s) < k) y = fmaf(wt[b * 8 + uint32_t(s)], __uint_as_float(ty[s].x), y);
    if (on) st_tag(out + size_t(b) * d + row, __uint_as_float(th[0].x) + y, c.ep);
  }
  if (lane == 0) lds_st(C_XCONS + 4 * c.w, i + 1);
  return true;
}

// LM head: per sequence, combine the waves' bests, publish the CU's slot,
// take a ticket; the last CU reduces every sequence's slots (lowest index
// wins ties) and writes the tokens.
DEV void lm_finish_b(Comp& c, InstrCP I) {
  const KArgs& a = *c.a;
  const uint32_t lane = c.lane, nB = uint32_t(a.batch);
  const uint32_t tile = I->aux[1], n_tiles = I->aux[3];
  if (lane < nB) {
    ArgBest b{-__builtin_inff(), 0xFFFFFFFFu};
    for (int w = 0; w < kNComp; w++)
      arg_update(b, __uint_as_float(*lw(lb::kArg + (w * 8 + int(lane)) * 8)), *lw(lb::kArg + (w * 8 + int(lane)) * 8 + 4));
    st_act(a.lm_slots + (size_t(tile) * lb::kMaxB + lane) * 2, b.v);
    st_act(a.lm_slots + (size_t(tile) * lb::kMaxB + lane) * 2 + 1, __uint_as_float(b.i));
  }
  uint32_t old = 0;
  if (lane == 0) old = ctr_release(ctr_line(a, I->sig_ctr, 0));
  old = uni(old);
  if (old + 1 != a.epoch * n_tiles) return;
  ctr_acquire();
  for (uint32_t b = 0; b < nB; b++) {
    ArgBest all{-__builtin_inff(), 0xFFFFFFFFu};
    for (uint32_t t = lane; t < n_tiles; t += 64)
      arg_update(all, ld_act(a.lm_slots + (size_t(t) * lb::kMaxB + b) * 2),
                 __float_as_uint(ld_act(a.lm_slots + (size_t(t) * lb::kMaxB + b) * 2 + 1)));
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const float ov = __shfl_xor(all.v, m, 64);
      const uint32_t oi = __shfl_xor(all.i, m, 64);
      arg_update(all, ov, oi);
    }
    if (lane == 0) gp(a.next)[b] = int32_t(all.i);
  }
}

// ---------------------------------------------------------------- variants
// GeoB: attention tile shape (query heads per tile, head dimension) compiled
// for one shape; GeoBAny dispatches it per instruction.
// MF: the kernel also runs matrix-core GEMV tiles (F_MFMA); compiled into a
// variant of its own, so that the other variants keep their register
// allocation.
template <int H, int D, bool MF>
struct GeoB {
  static constexpr bool any = false, mf = MF;
  static constexpr int hpt = H, dh = D;
};
struct GeoBAny {
  static constexpr bool any = true, mf = true;
};

template <class G>
DEV bool run_attn_b(Comp& c, InstrCP I, uint32_t i, uint32_t pg) {
  if constexpr (!G::any) {
    return attn<G::hpt, G::dh, LayB>(c, I, i, pg);
  } else {
    const uint32_t hpt = I->n_items;
    if (c.a->head_dim == 64) {
      switch (hpt) {
        case 1: return attn<1, 64, LayB>(c, I, i, pg);
        case 2: return attn<2, 64, LayB>(c, I, i, pg);
        case 4: return attn<4, 64, LayB>(c, I, i, pg);
        default: return attn<8, 64, LayB>(c, I, i, pg);
      }
    }
    switch (hpt) {
      case 1: return attn<1, 128, LayB>(c, I, i, pg);
      case 2: return attn<2, 128, LayB>(c, I, i, pg);
      default: return attn<4, 128, LayB>(c, I, i, pg);
    }
  }
}
template <class G>
DEV void run_merge_b(Comp& c, InstrCP I) {
  if constexpr (!G::any) {
    attn_merge<G::hpt, G::dh>(c, I);
  } else {
    const uint32_t hpt = I->n_items;
    if (c.a->head_dim == 64) {
      switch (hpt) {
        case 1: return attn_merge<1, 64>(c, I);
        case 2: return attn_merge<2, 64>(c, I);
        case 4: return attn_merge<4, 64>(c, I);
        default: return attn_merge<8, 64>(c, I);
      }
    }
    switch (hpt) {
      case 1: return attn_merge<1, 128>(c, I);
      case 2: return attn_merge<2, 128>(c, I);
      default: return attn_merge<4, 128>(c, I);
    }
  }
}

template <class G>
DEV void compute_b(const KArgs& a, InstrCP q, uint32_t n, int w, int cu) {
  Comp c{&a, cu, w, uint32_t(threadIdx.x & 63), 0, 0, 0, a.epoch, a.pos, 0, 0};
  const bool tr = a.trace != nullptr;
  // the instruction whose input the x slot holds (kNoCounter: none); its
  // record is re-read to decide whether a later instruction can reuse it
  uint32_t staged = kNoCounter;
  // the last instruction at which the compute waves synchronised
  uint32_t last_sync = 0;
  // matrix-core GEMV blocks of the launch so far
  uint32_t mblk = 0;
  uint32_t seen_ctr = kNoCounter, seen_val = 0;
  uint32_t pg = 0;
  for (uint32_t i = 0; i < n; i++) {
    InstrCP I = q + i;
    const uint32_t op = i_op(I);
    if (w == 0) {
      if (tr && c.lane == 0) {
        trace_put(a, cu, i, TR_START, now32());
        trace_put(a, cu, i, TR_HW0, hw0(I));
        trace_put(a, cu, i, TR_HW1, hw1(I));
      }
      c.retries = 0;
      bool ok = true;
      // Only the expert down projection waits on counters: its input (the
      // expert intermediates) is untagged fp32 behind release increments.
      // Every other input is tagged per element with the step, and staging
      // polls those tags instead, starting while the producers' last rows
      // are still in flight.
      for (int k = 0; k < 2 && ok && op == OP_EDN; k++) {
        if (!I->wait_cnt[k]) continue;
        const uint32_t ctr = I->wait_ctr[k], target = a.epoch * I->wait_cnt[k];
        if (ctr == seen_ctr && int32_t(seen_val - target) >= 0) continue;
        ok = wait_counter(a, ctr, target, cu, i);
        seen_ctr = ctr;
        seen_val = target;
      }
      if (ok && (i_flags(I) & F_ROUTE)) {
        // the first loader wave has written the layer's routing table
        if (tr && c.lane == 0) trace_put(a, cu, i, TR_A_PASS1, now32());
        ok = wait_lds_ge(C_RTOK, I->layer + 1);
        if (tr && c.lane == 0) trace_put(a, cu, i, TR_A_PASS3, now32());
      }
      if (!ok) {
        if (c.lane == 0) lds_st(C_ABORT, 1);
        return;
      }
      if (c.lane == 0) lds_st(C_DEPOK, i + 1);
      if (tr && c.lane == 0) trace_put(a, cu, i, TR_DEPS, now32());
    }
    if (op == OP_ATTN) {
      if (w == 0) {
        if (!wait_all_ge(C_XCONS, i) || !stage_attn<LayB>(c, I)) {
          if (c.lane == 0) lds_st(C_ABORT, 1);
          return;
        }
        if (c.lane == 0) lds_st(C_XOK, i + 1);
      } else if (!wait_lds_ge(C_XOK, i + 1)) {
        return;
      }
    } else if (w != 0 && !wait_lds_ge(C_DEPOK, i + 1)) {
      return;
    }
    uint32_t np = I->n_pages;
    if (op == OP_EGU) np = *lw(rt_base(I->layer) + RT_NSEL) * I->aux[2];

    if (i_flags(I) & F_DIRECT) np = 0;
    bool ok = true;
    if (op == OP_BGEMV || op == OP_EGU) {
      const uint32_t fl = i_flags(I) & (F_IN_EMBED | F_NORM | F_MFMA);
      InstrCP S = q + (staged == kNoCounter ? i : staged);
      const bool reuse = staged != kNoCounter && I->in_ptr == S->in_ptr &&
                         fl == (i_flags(S) & (F_IN_EMBED | F_NORM | F_MFMA)) && I->k == S->k &&
                         (!(fl & F_NORM) || I->gain_ptr == S->gain_ptr);
      const bool res = op == OP_BGEMV && i_epi(I) == EPI_RESID;
      if (!reuse || res) {
        if (!coop_stage_b(c, I, i, !reuse)) {
          if (c.lane == 0) lds_st(C_ABORT, 1);
          return;
        }
        if (!comp_barrier()) return;
        if constexpr (G::mf) {
          if ((i_flags(I) & F_MFMA) && !reuse && !mfma_order(c, I)) return;
        }
        last_sync = i;
      } else if (!done_slot_free(i, last_sync)) {
        if (c.lane == 0) lds_st(C_ABORT, 1);
        return;
      }
      if (tr && w == 0 && c.lane == 0) {
        trace_put(a, cu, i, TR_STAGED, now32());
        trace_put(a, cu, i, TR_RETRY, c.retries);
      }
      if (!reuse) staged = i;
      if (op == OP_BGEMV) {
        if constexpr (G::mf) {
          ok = (i_flags(I) & F_MFMA) ? bgemv_mfma(c, I, i, pg, mblk) : bgemv(c, I, i, pg);
        } else {
          ok = bgemv(c, I, i, pg);
        }
      } else if (i_flags(I) & F_DIRECT) {
        const uint32_t nit = i_nit(I);
        ok = nit == 4 ? egu_direct<4>(c, I, i) : nit == 2 ? egu_direct<2>(c, I, i) : egu_direct<1>(c, I, i);
      } else {
        ok = egu(c, I, i, pg);
      }
    } else if (op == OP_ERD) {
      ok = done_slot_free(i, last_sync) && erd(c, I, i);
    } else {
      // attention and the expert down projection wait for every wave to
      // have read the previous instruction's inputs
      staged = kNoCounter;
      last_sync = i;
      if (op == OP_EDN)
        ok = !(i_flags(I) & F_DIRECT) ? edn<0>(c, I, i, pg, np)
                                       : i_nit(I) == 2 ? edn<2>(c, I, i, pg, np) : edn<1>(c, I, i, pg, np);
      else
        ok = run_attn_b<G>(c, I, i, pg);
    }
    if (!ok) {
      if (c.lane == 0) lds_st(C_ABORT, 1);
      return;
    }
    pg += np;
    if (tr && w == 0 && c.lane == 0) trace_put(a, cu, i, TR_ITEMS, now32());
    const bool lm = op == OP_BGEMV && i_epi(I) == EPI_ARGMAX;
    const bool ticket = op == OP_ATTN && I->aux[3] > 1;
    // untagged data behind a counter (argmax slots, attention partials, the
    // expert intermediates) lands before the counter moves
    if (lm || ticket || op == OP_EGU) wait_vm0();
    uint32_t prev = 0;
    if (c.lane == 0) prev = lds_add(C_DONE + 4 * (i % kDoneRing), 1);
    prev = uni(prev);
    if (prev != kNComp - 1) continue;
    if (c.lane == 0) lds_st(C_DONE + 4 * (i % kDoneRing), 0);
    if (lm) {
      lm_finish_b(c, I);
      continue;
    }
    if (ticket) {
      uint32_t old = 0;
      if (c.lane == 0) old = ctr_release(ctr_line(a, I->seg_rows[0], 0));
      old = uni(old);
      if (old + 1 != a.epoch * I->aux[3]) continue;
      ctr_acquire();
      run_merge_b<G>(c, I);
    }
    if ((i_flags(I) & F_SIGNAL) && c.lane == 0) ctr_signal(ctr_line(a, I->sig_ctr, uint32_t(cu) % kCtrSpread));
    if (tr && c.lane == 0) trace_put(a, cu, i, TR_SIGNAL, now32());
  }
}

template <class G>
__global__ __launch_bounds__(kThreads, 1) void mk_megakernel_b(KArgs a) {
  for (int o = threadIdx.x * 4; o < C_CTRL_END; o += kThreads * 4) *lw(o) = 0;
  // the expert down projection's ready-queue entries (tagged by layer)
  for (int o = threadIdx.x * 4; o < 4 * int(2 * kDynMax); o += kThreads * 4) *lw(lb::kMfma + o) = 0;
  __syncthreads();
  if (threadIdx.x == 0) {
    *lw(C_STATUS_LO) = uint32_t(uint64_t(a.status));
    *lw(C_STATUS_HI) = uint32_t(uint64_t(a.status) >> 32);
    *lw(C_LIMIT_LO) = uint32_t(a.watchdog_ticks);
    *lw(C_LIMIT_HI) = uint32_t(a.watchdog_ticks >> 32);
  }
  __syncthreads();
  const int cu = blockIdx.x;
  const uint32_t beg = a.q_off[cu], end = a.q_off[cu + 1];
  InstrCP q = (InstrCP)(a.instrs + beg);
  const int wave = int(uni(threadIdx.x >> 6));
  if (wave < kNLoad)
    loader_b(a, q, end - beg, wave, cu);
  else
    compute_b<G>(a, q, end - beg, wave - kNLoad, cu);
}

}  // namespace mk

namespace {
struct BVariant {
  int hpt, dh;  // 0 = generic
  bool mf;      // runs matrix-core GEMV tiles
  const void* fn;
};
const BVariant kBVariants[] = {
    {0, 0, true, reinterpret_cast<const void*>(&mk::mk_megakernel_b<mk::GeoBAny>)},
    {4, 128, false, reinterpret_cast<const void*>(&mk::mk_megakernel_b<mk::GeoB<4, 128, false>>)},
    {4, 128, true, reinterpret_cast<const void*>(&mk::mk_megakernel_b<mk::GeoB<4, 128, true>>)},
};
constexpr int kNumBVariants = sizeof(kBVariants) / sizeof(kBVariants[0]);
bool g_battr_set[kNumBVariants] = {};
}  // namespace

// Index of the batched kernel built for this attention tile shape (with or
// without matrix-core GEMV tiles), or 0.
extern "C" int mk_pick_batched(int hpt, int dh, int mfma) {
  for (int v = 1; v < kNumBVariants; v++)
    if (kBVariants[v].hpt == hpt && kBVariants[v].dh == dh && kBVariants[v].mf == (mfma != 0)) return v;
  return 0;
}

extern "C" hipError_t mk_launch_batched(const mk::KArgs* args, int n_cus, hipStream_t stream, int cooperative,
                                        int variant) {
  if (variant < 0 || variant >= kNumBVariants) return hipErrorInvalidValue;
  const void* fn = kBVariants[variant].fn;
  if (!g_battr_set[variant]) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, mk::lb::kTotal);
    if (e != hipSuccess) return e;
    g_battr_set[variant] = true;
  }
  mk::KArgs a = *args;
  void* params[] = {&a};
  if (cooperative)
    return hipLaunchCooperativeKernel(fn, dim3(n_cus), dim3(mk::kThreads), params, mk::lb::kTotal, stream);
  return hipLaunchKernel(fn, dim3(n_cus), dim3(mk::kThreads), params, mk::lb::kTotal, stream);
}
