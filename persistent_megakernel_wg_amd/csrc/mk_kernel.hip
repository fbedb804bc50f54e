// mk_kernel.hip — the persistent decode megakernel for gfx950 (MI355X).
//
// One workgroup per CU interprets its queue of tile instructions (the on-GPU
// interpreter of the Llama-1B megakernel write-up, rocketrecap.com summary,
// "Fusing Operations with an On-GPU Interpreter"; Cohere's resident
// one-block-per-SM task list, airebao.com «Megakernel 是什么»).
//
// Workgroup = 2 loader waves + 6 compute waves (512 threads, 1 WG/CU, two
// waves per SIMD so each wave may hold up to 256 VGPRs).
//  * Loader waves walk the queue ahead of the compute waves and copy each
//    instruction's weight (or KV-cache) stream into a ring of 8 x 16 KiB LDS
//    pages with global_load_lds_dwordx4 (the shared-memory paging of the
//    write-up, "Efficient Shared Memory Management"; weights are immutable, so
//    they are fetched before the activation dependency is met, as in Cohere's
//    «三点关键差异» item 3 and «快在哪里» item 3).  Loaders never wait on
//    global counters; they track their own DMA with vmcnt and publish each
//    page through an LDS word.
//  * The compute waves stage the instruction's input vector into LDS (the
//    leader alone for attention's q/k/v and the embedding row), polling the
//    step tag every activation element carries until the producers' values
//    are there; then all compute waves run the op from the LDS pages.  The
//    last wave to finish an instruction increments its counter or takes its
//    ticket (the counter system of the write-up, "Custom Synchronization
//    Mechanism", kept for the data that carries no tag).
#include "mk_dev.h"

namespace mk {

// Pages of a CU's queue are numbered over the launch: step s's instruction i
// takes pages s * P + page0(i) ..., where P is the pages of one step.
DEV uint32_t step_pages(InstrCP q, uint32_t n) { return n ? q[n - 1].page0 + q[n - 1].n_pages : 0; }

// Prefetch cursor of a loader wave: the next page (instruction of the launch,
// step * n + i, and page of it) whose lines it has not yet touched.
struct PfCursor {
  uint32_t ig, p;
};

// Touch this wave's half of the next page after the DMA cursor (instruction
// ig of the launch, page p, ring index g) not yet touched, if it lies less
// than kPfPages past g.  Only GEMV weight streams are touched; attention pages
// (the KV cache) are skipped.  Returns false when no page is due.
DEV bool prefetch_next(InstrCP q, uint32_t n, uint32_t n_total, uint32_t P, uint32_t ig, uint32_t p, uint32_t g,
                       int v, PfCursor& c, uint32_t sink, uint32_t voff128) {
  if (c.ig < ig || (c.ig == ig && c.p < p)) c = {ig, p};
  while (c.ig < n_total && c.p >= q[c.ig % n].n_pages) c = {c.ig + 1, 0};
  if (c.ig >= n_total) return false;
  InstrCP I = q + c.ig % n;
  if ((c.ig / n) * P + I->page0 + c.p >= g + kPfPages) return false;
  if (i_op(I) == OP_GEMV) {
    const uint32_t u0 = c.p * kUnitsPerPage + uint32_t(v) * kDmaPerPage;
    const uint32_t units = (I->n_rows * I->row_bytes + kUnit - 1) / kUnit;
    // the DMA reads the same half page (the stream is padded to it)
    if (u0 < units) l2_touch(sink, uni64(I->src_ptr + uint64_t(u0) * kUnit), voff128);
  }
  c.p++;
  return true;
}

// The loader waves walk the launch's steps back to back: the weights of the
// next step are streamed (and touched ahead) while the current step's last
// instructions still run, since they do not depend on its results.
DEV void loader(const KArgs& a, InstrCP q, uint32_t n, int v) {
  const uint32_t voff = (threadIdx.x & 63) * 16, voff4k = voff + 4096;
  const uint32_t voff128 = (threadIdx.x & 63) * 128, sink = uint32_t(size_t(lds)) + kLdsPf;
  const uint32_t P = step_pages(q, n), n_total = n * a.n_steps;
  uint32_t nd = 0;       // DMAs issued by this wave (kDmaPerPage per page)
  uint32_t g_issue = 0;  // pages issued
  uint32_t g_pub = 0;    // pages published
  uint32_t min_rel = 0;  // oldest page a compute wave may still read
  PfCursor pf{0, 0};
  for (uint32_t ig = 0; ig < n_total; ig++) {
    const uint32_t step = ig / n;
    InstrCP I = q + (ig - step * n);
    LoadView L;
    load_view(a, I, L, a.pos + int32_t(step));
    const uint32_t np = I->n_pages, page0 = step * P + I->page0;
    for (uint32_t p = 0; p < np; p++) {
      const uint32_t g = page0 + p;
      if (g >= min_rel + kPages) {
        Watch t0;
        for (;;) {
          min_rel = uni(min_released());
          if (g < min_rel + kPages) break;
          if (g_pub < g_issue) {  // nothing free yet: complete the oldest page
            wait_vm_pages(g_issue - g_pub - 1);
            publish(g_pub, g_pub + 1, v);
            continue;
          }
          // (every DMA is published here, so the loads below are the
          // newest and no page's completion waits on them)
          if (kPfPages && prefetch_next(q, n, n_total, P, ig, p, g, v, pf, sink, voff128)) continue;
          if (aborted() || local_timeout(t0, local_limit())) {
            if (!aborted()) local_abort(STC_LOCAL_TIMEOUT);
            wait_vm0();
            return;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      issue_page<LayA>(a, L, p, g, v, voff, voff4k, nd);
      g_issue = g + 1;
      // pages whose DMAs all precede the last T (the throttle just applied)
      // are complete
      const uint32_t vmt = L.deep ? kVmTDeep : kVmT;
      if (nd > vmt) publish(g_pub, (nd - vmt) / kDmaPerPage, v);
    }
  }
  wait_vm0();
  publish(g_pub, g_issue, v);
}

DEV const float* res_slot(uint32_t i) {
  return reinterpret_cast<const float*>(lds + kLdsRes + (i & 1) * 4 * kMaxResRows);
}

// instruction fields of the epilogue, read once per instruction
struct EpiCtx {
  uint64_t* out;
  uint32_t epi, acc0, row0;
  uint32_t gn, gstride;  // gate/up over every chunk: pairs per chunk here, pairs per chunk
};
DEV EpiCtx epi_of(InstrCP I) {
  const bool all = i_flags(I) & F_GU_ALL;
  return EpiCtx{reinterpret_cast<uint64_t*>(I->out_ptr), i_epi(I), I->aux[0], I->row0,
                all ? I->aux[1] : 0u, all ? I->aux[2] : 0u};
}
// OP: the kernel variant also runs split-K O tiles (EPI_OPART)
template <bool OP>
DEV void epi_row(Comp& c, const EpiCtx& E, uint32_t i, uint32_t t_row, float v, ArgBest& best) {
  const KArgs& a = *c.a;
  uint64_t* out = E.out;
  const uint32_t row = E.row0 + t_row;
  if constexpr (OP) {
    if (E.epi == EPI_OPART) {
      // the group's partial row (untagged fp32, published by the ticket)
      st_act(reinterpret_cast<float*>(out) + row, v);
      return;
    }
  }
  switch (E.epi) {
    case EPI_SWIGLU:
      if (E.gn) {
        // item t of a gate/up instruction over every chunk: pair t % n of
        // chunk t / n
        const uint32_t ch = t_row / E.gn;
        st_tag(out + E.row0 + ch * E.gstride + (t_row - ch * E.gn), v, c.ep);
        break;
      }
      st_tag(out + row, v, c.ep);
      break;
    case EPI_STORE:
      st_tag(out + row, v, c.ep);
      break;
    case EPI_RESID:
    case EPI_ACC_ONLY:
      st_tag(out + row, res_slot(i)[t_row] + v, c.ep);
      break;
    case EPI_ACC_FIRST:
      reinterpret_cast<float*>(lds + kLdsAcc)[E.acc0 + t_row] = res_slot(i)[t_row] + v;
      break;
    case EPI_ACC_MID:
      reinterpret_cast<float*>(lds + kLdsAcc)[E.acc0 + t_row] += v;
      break;
    case EPI_ACC_LAST:
      st_tag(out + row, reinterpret_cast<float*>(lds + kLdsAcc)[E.acc0 + t_row] + v, c.ep);
      break;
    case EPI_ARGMAX:
      if (a.logits) gp(a.logits)[size_t(c.step) * uint32_t(a.vocab) + row] = v;
      if (v != v) __hip_atomic_store(gp(a.status) + ST_NAN, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      arg_update(best, v, row);
      break;
  }
}

template <int NIT, int RPU, bool OP = false>
DEV bool gemv(Comp& c, InstrCP I, uint32_t i) {
  constexpr int LPR = 64 / RPU;
  const KArgs& a = *c.a;
  const uint32_t lane = c.lane;
  const float* xs = reinterpret_cast<const float*>(lds + kLdsX);
  float xv[NIT][8];
#pragma unroll
  for (int j = 0; j < NIT; j++) {
    const uint32_t col = RPU == 1 ? j * 512 + lane * 8 : (lane % LPR) * 8;
    const f4 lo = *reinterpret_cast<const f4*>(xs + col);
    const f4 hi = *reinterpret_cast<const f4*>(xs + col + 4);
    xv[j][0] = lo.x; xv[j][1] = lo.y; xv[j][2] = lo.z; xv[j][3] = lo.w;
    xv[j][4] = hi.x; xv[j][5] = hi.y; xv[j][6] = hi.z; xv[j][7] = hi.w;
  }
  if (lane == 0) lds_st(C_XCONS + 4 * c.w, i + 1);
  // RMSNorm: the staged input is x * gain, and its row sums are scaled by
  // 1 / rms(x), from the staged shares of the sum of squares
  float inv = 1.f;
  if (i_flags(I) & F_NORM) {
    float ss = 0.f;
#pragma unroll
    for (int w = 0; w < kNComp; w++) ss += *reinterpret_cast<const float*>(lds + kLdsSS + 4 * w);
    inv = rsqrtf(ss / float(I->k) + a.rms_eps);
  }
  const bool trl = c.a->trace && c.w == 0 && lane == 0;
  if (trl) trace_put(a, c.cu, i, TR_XREADY, now32());

  const uint32_t n_items = I->n_items, page0 = c.pbase + I->page0;
  const bool pair = i_epi(I) == EPI_SWIGLU;
  const EpiCtx E = epi_of(I);
  ArgBest best{-__builtin_inff(), 0xFFFFFFFFu};
  if constexpr (RPU == 1) {
    // Whole rows.  The wave's items are t = w, w + kNComp, ...; it takes two
    // at a time, with the loads of both issued before the first product
    // (one row, or one row of each pair, at a time for the widest inputs),
    // and reduces them together.
    auto rows = [&](auto pair_c) -> bool {
      constexpr int RU = decltype(pair_c)::value ? 2 : 1;  // rows per item
      constexpr uint32_t UPI = RU * NIT;                    // units per item
      constexpr int RL = 2 * RU * NIT <= 16 ? RU : 1;       // rows loaded together
      // the units an iteration spans must fit in the page ring, or the wave
      // would wait for a page that only its own release can free
      static_assert((kNComp + 1) * UPI <= uint32_t(kPages * kUnitsPerPage), "an iteration's rows exceed the page ring");
      for (uint32_t t = c.w; t < n_items; t += 2 * kNComp) {
        const uint32_t tb = t + kNComp;
        const bool two = tb < n_items;
        const uint32_t ua = t * UPI, ub = (two ? tb : t) * UPI;
        if (lane == 0) lds_st(C_RELEASED + 4 * c.w, page0 + ua / kUnitsPerPage);
        {
          const uint32_t tw = trl ? now32() : 0;
          if (!wait_page(page0 + (ub + UPI - 1) / kUnitsPerPage, c.fcache)) return false;
          if (trl) c.pagewait += now32() - tw;
          if (trl && t == 0) trace_put(a, c.cu, i, TR_A_PASS1, now32());  // first pages ready
        }
        float sum[2][RU];
#pragma unroll
        for (int r0 = 0; r0 < RU; r0 += RL) {
          u4 wr[2][RL][NIT];
#pragma unroll
          for (int s2 = 0; s2 < 2; s2++)
#pragma unroll
            for (int r = 0; r < RL; r++)
#pragma unroll
              for (int j = 0; j < NIT; j++) {
                const uint32_t u = (s2 ? ub : ua) + (r0 + r) * NIT + j;
                wr[s2][r][j] = *reinterpret_cast<const u4*>(lds + page_off<LayA>(page0 + u / kUnitsPerPage) +
                                                            (u % kUnitsPerPage) * kUnit + lane * 16);
              }
#pragma unroll
          for (int r = 0; r < RL; r++) {
            float acc[2];
#pragma unroll
            for (int s2 = 0; s2 < 2; s2++) {
              acc[s2] = 0.f;
#pragma unroll
              for (int j = 0; j < NIT; j++) acc[s2] += dot8(wr[s2][r][j], xv[j]);
            }
            sum64x2(acc[0], acc[1], sum[0][r0 + r], sum[1][r0 + r]);
          }
        }
        if (trl && t == 0) trace_put(a, c.cu, i, TR_A_STATS, now32());  // first sums reduced
        if (lane == 0) {
          const float a0 = sum[0][0] * inv, b0 = sum[1][0] * inv;
          epi_row<OP>(c, E, i, t, RU == 2 ? silu(a0) * (sum[0][RU - 1] * inv) : a0, best);
          if (two) epi_row<OP>(c, E, i, tb, RU == 2 ? silu(b0) * (sum[1][RU - 1] * inv) : b0, best);
        }
        if (trl && t == 0) trace_put(a, c.cu, i, TR_ITEM0, now32());
      }
      return true;
    };
    if (!(pair ? rows(std::true_type{}) : rows(std::false_type{}))) return false;
  } else {
    // half-wave rows of 512 B (K = 256): one unit holds two rows (or a pair)
    for (uint32_t t = c.w; t < n_items; t += kNComp) {
      const uint32_t u0 = t;
      if (lane == 0) lds_st(C_RELEASED + 4 * c.w, page0 + u0 / kUnitsPerPage);
      {
        const uint32_t tw = trl ? now32() : 0;
        if (!wait_page(page0 + u0 / kUnitsPerPage, c.fcache)) return false;
        if (trl) c.pagewait += now32() - tw;
      }
      const u4 wa = *reinterpret_cast<const u4*>(lds + page_off<LayA>(page0 + u0 / kUnitsPerPage) +
                                                 (u0 % kUnitsPerPage) * kUnit + lane * 16);
      float lo, hi;
      sum32x2(dot8(wa, xv[0]), lo, hi);
      lo *= inv;
      hi *= inv;
      if (pair) {
        if (lane == 0) epi_row<OP>(c, E, i, t, silu(lo) * hi, best);
      } else if ((lane & 31) == 0) {
        epi_row<OP>(c, E, i, 2 * t + (lane >> 5), lane ? hi : lo, best);
      }
      if (trl && t == 0) trace_put(a, c.cu, i, TR_ITEM0, now32());
    }
  }
  if (i_epi(I) == EPI_ARGMAX) {
    // combine lanes 0 and 32 (512 B rows) and publish the wave's best
    float ov = __shfl(best.v, 32, 64);
    uint32_t oi = __shfl(best.i, 32, 64);
    if (RPU == 2) arg_update(best, ov, oi);
    if (lane == 0) {
      *lw(C_ARGV + 4 * c.w) = __float_as_uint(best.v);
      *lw(C_ARGI + 4 * c.w) = best.i;
    }
  }
  if (lane == 0) lds_st(C_RELEASED + 4 * c.w, page0 + I->n_pages);
  return true;
}

// rows of the residual an epilogue adds (staged with the inputs)
DEV bool needs_res(InstrCP I) {
  const uint32_t e = i_epi(I);
  return i_op(I) == OP_GEMV && (e == EPI_RESID || e == EPI_ACC_ONLY || e == EPI_ACC_FIRST);
}
DEV uint32_t out_rows(InstrCP I) {
  return (i_rpu(I) == 2 && i_epi(I) != EPI_SWIGLU) ? 2 * I->n_items : I->n_items;
}

// Leader staging (attention and the embedding input of the first layer):
// for a GEMV, the input times its RMSNorm gain into the x slot and the sum of
// squares of the input (the GEMV scales its row sums by 1 / rms).  For attention: the group's
// q, k, v and the position's cos, sin.  Every load is issued before the first
// is waited for: one memory round trip.  false = abort or watchdog.
DEV bool stage_leader(Comp& c, InstrCP I, uint32_t i) {
  const KArgs& a = *c.a;
  const uint32_t lane = c.lane;
  float* xs = reinterpret_cast<float*>(lds + kLdsX);
  if (i_op(I) == OP_GEMV) {
    // bf16 embedding row of the token (8 values per lane per 512) and the gain
    constexpr int NE = kMaxK / 512;
    const uint32_t K = I->k;
    const bool norm = i_flags(I) & F_NORM;
    const uint16_t* e = reinterpret_cast<const uint16_t*>(I->in_ptr) + size_t(token_of(a, c.step, c.ep)) * K;
    const __amdgpu_buffer_rsrc_t r = act_rsrc(e, K * 2);
    const __amdgpu_buffer_rsrc_t rg = act_rsrc(reinterpret_cast<const void*>(I->gain_ptr), norm ? K * 2 : 0);
    u4 raw[NE], gw[NE];
#pragma unroll
    for (int j = 0; j < NE; j++) {
      raw[j] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, (lane * 8 + 512 * j) * 2, 0, 0));
      gw[j] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rg, (lane * 8 + 512 * j) * 2, 0, 0));
    }
    // x * gain into the x slot (the GEMV applies 1 / rms to its row sums)
    // and the sum of squares of x
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NE; j++) {
      const uint32_t o = lane * 8 + 512 * j;
      const uint32_t xw[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
      const uint32_t gg[4] = {gw[j].x, gw[j].y, gw[j].z, gw[j].w};
      float v[8];
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const float x0 = bf_lo(xw[e]), x1 = bf_hi(xw[e]);
        ss = fmaf(x0, x0, fmaf(x1, x1, ss));
        v[2 * e] = norm ? x0 * bf_lo(gg[e]) : x0;
        v[2 * e + 1] = norm ? x1 * bf_hi(gg[e]) : x1;
      }
      if (o < K) {
        *reinterpret_cast<f4*>(xs + o) = f4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f4*>(xs + o + 4) = f4{v[4], v[5], v[6], v[7]};
      }
    }
    if (norm) {
      ss = sum64(ss);
      if (lane < uint32_t(kNComp)) *reinterpret_cast<float*>(lds + kLdsSS + 4 * lane) = lane == 0 ? ss : 0.f;
    }
  } else {
    return stage_attn<LayA>(c, I);
  }
  return true;
}

// Cooperative staging of a GEMV's tagged input: wave w loads the chunks of
// 128 values j = w, w + kNComp, ... (every load before the first wait: one
// round trip per wave, all waves in parallel), re-reads stale ones, and
// writes them times their RMSNorm gains to the x slot, with the wave's share
// of the sum of squares, once every wave has read the previous input.  The
// leader also stages the epilogue's residual rows.  A barrier of the compute
// waves follows.  The loads can be issued early (stage_issue, while the
// previous instruction's items run) and completed later (stage_finish).
constexpr int kStageNC = (kMaxK / 128 + kNComp - 1) / kNComp;
struct StageIn {
  u4 t[kStageNC];        // value | tag pairs of the wave's chunks
  uint32_t gw[kStageNC]; // their RMSNorm gains (bf16 pairs)
  uint2 res_t[2];        // leader: tagged residual rows
  uint16_t res_e[2];     // leader: residual rows from the embedding
};
struct StageGeo {
  __amdgpu_buffer_rsrc_t r, rg, rr;
  uint32_t nch;
  bool norm, has_res, res_embed;
};
DEV StageGeo stage_geo(Comp& c, InstrCP I, bool stage_x) {
  StageGeo g;
  const uint32_t K = I->k;
  g.nch = K / 128;
  g.norm = i_flags(I) & F_NORM;
  g.r = act_rsrc_u(reinterpret_cast<const void*>(I->in_ptr), stage_x ? K * kActBytes : 0);
  g.rg = act_rsrc_u(reinterpret_cast<const void*>(I->gain_ptr), (stage_x && g.norm) ? K * 2 : 0);
  g.has_res = c.w == 0 && needs_res(I);
  g.res_embed = g.has_res && (i_flags(I) & F_RES_EMBED);
  const uint32_t n_res = g.has_res ? out_rows(I) : 0;
  g.rr = act_rsrc_u(reinterpret_cast<const char*>(I->res_ptr) + size_t(I->row0) * kActBytes,
                  (g.has_res && !g.res_embed) ? n_res * kActBytes : 0);
  return g;
}
DEV uint32_t stage_off(const Comp& c, int q) { return ((uint32_t(c.w) + kNComp * q) * 128 + 2 * c.lane) * kActBytes; }

DEV void stage_issue(Comp& c, InstrCP I, bool stage_x, StageIn& S) {
  static_assert(kMaxResRows == 128, "residual staging takes two rows per lane");
  const uint32_t lane = c.lane;
  const StageGeo g = stage_geo(c, I, stage_x);
#pragma unroll
  for (int q = 0; q < kStageNC; q++) {
    S.t[q] = ld_tag2(g.r, stage_off(c, q));
    S.gw[q] = __builtin_amdgcn_raw_buffer_load_b32(g.rg, ((uint32_t(c.w) + kNComp * q) * 128 + 2 * lane) * 2, 0, 0);
  }
  // residual rows r0 + 2*lane + {0,1} (leader): tagged elements, or the bf16
  // row of the token's embedding (per-element loads: a resource of n_res
  // elements reads zero past the tile)
  reload(S.res_t[0], g.rr, 2 * lane * kActBytes);
  reload(S.res_t[1], g.rr, (2 * lane + 1) * kActBytes);
  S.res_e[0] = S.res_e[1] = 0;
  if (g.res_embed) {
    const KArgs& a = *c.a;
    const uint32_t n_res = out_rows(I);
    const uint16_t* e =
        reinterpret_cast<const uint16_t*>(I->res_ptr) + size_t(token_of(a, c.step, c.ep)) * a.hidden + I->row0;
    const __amdgpu_buffer_rsrc_t re = act_rsrc_u(e, n_res * 2);
    S.res_e[0] = __builtin_amdgcn_raw_buffer_load_b16(re, 4 * lane, 0, 0);
    S.res_e[1] = __builtin_amdgcn_raw_buffer_load_b16(re, 4 * lane + 2, 0, 0);
  }
}

// false = abort or watchdog
DEV bool stage_finish(Comp& c, InstrCP I, uint32_t i, bool stage_x, StageIn& S) {
  const uint32_t lane = c.lane;
  const uint32_t tag = in_tag(c.ep, I);
  const StageGeo g = stage_geo(c, I, stage_x);
  const uint32_t n_res = g.has_res ? out_rows(I) : 0;
  const uint32_t res_live = 2 * lane >= n_res ? 0 : (2 * lane + 1 < n_res ? 2 : 1);
  if (stage_x) {
    const uint32_t live = uint32_t(c.w) < g.nch ? (g.nch - c.w + kNComp - 1) / kNComp : 0;
    if (!wait_fresh(S.t, live, g.r, [&](int, int q) { return stage_off(c, q); }, 0, tag, c.retries)) return false;
    // every wave has read the previous input out of the x slot
    if (!wait_all_ge(C_XCONS, i)) return false;
    float* xs = reinterpret_cast<float*>(lds + kLdsX);
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < kStageNC; q++) {
      if (q >= int(live)) continue;
      const uint32_t o = (uint32_t(c.w) + kNComp * q) * 128 + 2 * lane;
      const float v0 = __uint_as_float(S.t[q].x), v1 = __uint_as_float(S.t[q].z);
      if (g.norm) {
        *reinterpret_cast<float2*>(xs + o) = float2{v0 * bf_lo(S.gw[q]), v1 * bf_hi(S.gw[q])};
        ss = fmaf(v0, v0, fmaf(v1, v1, ss));
      } else {
        *reinterpret_cast<float2*>(xs + o) = float2{v0, v1};
      }
    }
    // this wave's share of the sum of squares (gemv adds the kNComp shares)
    if (g.norm) {
      ss = sum64(ss);
      if (lane == 0) *reinterpret_cast<float*>(lds + kLdsSS + 4 * c.w) = ss;
    }
  }
  if (g.has_res) {
    float* rs = const_cast<float*>(res_slot(i));
    const uint32_t res_off[2] = {2 * lane * kActBytes, (2 * lane + 1) * kActBytes};
    if (!g.res_embed && !wait_fresh(S.res_t, res_live, g.rr, [&](int, int j) { return res_off[j]; }, 0, tag, c.retries))
      return false;
#pragma unroll
    for (int j = 0; j < 2; j++)
      if (j < int(res_live))
        rs[2 * lane + j] = g.res_embed ? __uint_as_float(uint32_t(S.res_e[j]) << 16) : __uint_as_float(S.res_t[j].x);
  }
  return true;
}

// ---- kernel variants
// GeoAny: one kernel for every supported shape; the GEMV width, the KV
// group size and the head dimension are dispatched per instruction.
// GeoFix: the kernel for one shape.  Only the code paths that shape uses are
// compiled, which keeps the kernel inside the register file (the generic
// kernel spills) and its code small.  The runtime picks a GeoFix kernel when
// every instruction of the plan matches it.
struct GeoAny {
  static constexpr bool any = true, os = true;
};
// H = query heads per attention tile, D = head dimension
// OS: the O projection is split per KV group (its tiles and merges are
// compiled only into these variants)
template <int ND, int RD, int NQ, int RQ, int NF, int RF, int H, int D, bool OS>
struct GeoFix {
  static constexpr bool any = false, os = OS;
  static constexpr int nd = ND, rd = RD, nq = NQ, rq = RQ, nf = NF, rf = RF, hpt = H, dh = D;
};

template <class G>
DEV bool run_gemv(Comp& c, InstrCP I, uint32_t i) {
  if constexpr (!G::any) {
    const uint32_t nit = i_nit(I), rpu = i_rpu(I);
    if (nit == uint32_t(G::nd) && rpu == uint32_t(G::rd)) return gemv<G::nd, G::rd>(c, I, i);
    if (nit == uint32_t(G::nq) && rpu == uint32_t(G::rq)) return gemv<G::nq, G::rq, G::os>(c, I, i);
    return gemv<G::nf, G::rf>(c, I, i);
  } else {
    if (i_rpu(I) == 2) return gemv<1, 2, true>(c, I, i);
    switch (i_nit(I)) {
      case 1: return gemv<1, 1, true>(c, I, i);
      case 2: return gemv<2, 1, true>(c, I, i);
      case 3: return gemv<3, 1>(c, I, i);
      case 4: return gemv<4, 1, true>(c, I, i);
      case 5: return gemv<5, 1>(c, I, i);
      case 6: return gemv<6, 1>(c, I, i);
      case 7: return gemv<7, 1>(c, I, i);
      default: return gemv<8, 1>(c, I, i);
    }
  }
}

template <class G>
DEV bool run_attn(Comp& c, InstrCP I, uint32_t i) {
  if constexpr (!G::any) {
    return attn<G::hpt, G::dh, LayA>(c, I, i, c.pbase + I->page0);
  } else {
    const uint32_t hpt = I->n_items;
    if (c.a->head_dim == 64) {
      switch (hpt) {
        case 1: return attn<1, 64, LayA>(c, I, i, c.pbase + I->page0);
        case 2: return attn<2, 64, LayA>(c, I, i, c.pbase + I->page0);
        case 4: return attn<4, 64, LayA>(c, I, i, c.pbase + I->page0);
        default: return attn<8, 64, LayA>(c, I, i, c.pbase + I->page0);
      }
    }
    switch (hpt) {
      case 1: return attn<1, 128, LayA>(c, I, i, c.pbase + I->page0);
      case 2: return attn<2, 128, LayA>(c, I, i, c.pbase + I->page0);
      default: return attn<4, 128, LayA>(c, I, i, c.pbase + I->page0);
    }
  }
}

template <class G>
DEV void run_merge(Comp& c, InstrCP I) {
  if constexpr (!G::any) {
    // the kernels built for one shape issue the loads of up to 32 blocks
    // (16 for 8 outputs per lane) before using any: one memory round trip
    // for the long-context tiles instead of one per 8 blocks
    constexpr int PER = G::hpt * G::dh / 64;
    attn_merge<G::hpt, G::dh, (PER <= 2 ? 32 : PER == 4 ? 16 : 8)>(c, I);
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

// Split-K O projection, by the tile that took its row block's last ticket:
// h_l[r] = x_l[r] + part[0][r] + ... + part[G-1][r], in group order, for the
// block's rows (x_l tagged, or the token's embedding row in the first layer).
DEV bool o_merge(Comp& c, InstrCP I) {
  const KArgs& a = *c.a;
  const uint32_t lane = c.lane, d = uint32_t(a.hidden), G = I->aux[3], n = out_rows(I), r0 = I->row0;
  const float* part = reinterpret_cast<const float*>(I->out_ptr) - size_t(I->aux[1]) * d;
  uint64_t* h = reinterpret_cast<uint64_t*>(I->seg_ptr[2]);
  const bool embed = i_flags(I) & F_RES_EMBED;
  const uint16_t* e = embed ? reinterpret_cast<const uint16_t*>(I->res_ptr) + size_t(token_of(a, c.step, c.ep)) * d
                            : nullptr;
  const __amdgpu_buffer_rsrc_t rx =
      act_rsrc_u(reinterpret_cast<const void*>(I->res_ptr), embed ? 0 : (r0 + n) * kActBytes);
  for (uint32_t b0 = 0; b0 < n; b0 += 64) {
    const uint32_t r = r0 + b0 + lane, on = b0 + lane < n;
    uint2 t[1];
    reload(t[0], rx, r * kActBytes);
    if (!embed && !wait_fresh(t, on, rx, [&](int, int) { return r * kActBytes; }, 0, in_tag(c.ep, I), c.retries))
      return false;
    float v = 0.f;
    if (on) {
      v = embed ? __uint_as_float(uint32_t(e[r]) << 16) : __uint_as_float(t[0].x);
      for (uint32_t g = 0; g < G; g++) v += ld_act(part + size_t(g) * d + r);
      st_tag(h + r, v, c.ep);
    }
  }
  return true;
}

// LM head: combine the per-wave bests, publish the CU's slot, take a ticket;
// the last CU reduces all slots (lowest index wins ties) and writes the token.
DEV void lm_finish(Comp& c, InstrCP I) {
  const KArgs& a = *c.a;
  const uint32_t lane = c.lane;
  ArgBest b{-__builtin_inff(), 0xFFFFFFFFu};
  for (int w = 0; w < kNComp; w++) arg_update(b, __uint_as_float(*lw(C_ARGV + 4 * w)), *lw(C_ARGI + 4 * w));
  const uint32_t tile = I->aux[1], n_tiles = I->aux[3];
  if (lane == 0) {
    st_act(a.lm_slots + 2 * tile, b.v);
    st_act(a.lm_slots + 2 * tile + 1, __uint_as_float(b.i));
  }
  uint32_t old = 0;
  if (lane == 0) old = ctr_release(ctr_line(a, I->sig_ctr, 0));
  old = uni(old);
  if (old + 1 != c.ep * n_tiles) return;
  ctr_acquire();
  ArgBest all{-__builtin_inff(), 0xFFFFFFFFu};
  for (uint32_t t = lane; t < n_tiles; t += 64)
    arg_update(all, ld_act(a.lm_slots + 2 * t), __float_as_uint(ld_act(a.lm_slots + 2 * t + 1)));
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const float ov = __shfl_xor(all.v, m, 64);
    const uint32_t oi = __shfl_xor(all.i, m, 64);
    arg_update(all, ov, oi);
  }
  if (lane == 0) {
    gp(a.next)[c.step] = int32_t(all.i);
    // the next step of the launch takes its input token from here
    if (c.step + 1 < a.n_steps) st_tag(a.tok_tag, __uint_as_float(all.i), c.ep);
  }
}

template <class G>
DEV void compute(const KArgs& a, InstrCP q, uint32_t n, int w, int cu) {
  Comp c{&a, cu, w, uint32_t(threadIdx.x & 63), 0, 0, 0, a.epoch, a.pos, 0, 0};
  const bool tr = a.trace != nullptr;
  const uint32_t P = step_pages(q, n), n_total = n * a.n_steps;
  // input currently in the x slot (every wave tracks it, so all take the
  // same staging decision)
  uint64_t staged_in = 0;
  uint32_t staged_flags = 0, staged_k = 0;
  uint64_t staged_gain = 0;
  // the staged input of the previous GEMV can be reused as is
  auto reuses = [&](InstrCP I) {
    return i_op(I) == OP_GEMV && I->in_ptr == staged_in &&
           (i_flags(I) & (F_IN_EMBED | F_NORM)) == staged_flags && I->k == staged_k &&
           (!(i_flags(I) & F_NORM) || I->gain_ptr == staged_gain);
  };
  // tagged GEMV inputs are staged by all compute waves together; the
  // embedding input and attention inputs by the leader
  auto is_coop = [](InstrCP I) { return i_op(I) == OP_GEMV && !(i_flags(I) & F_IN_EMBED); };
  // loads of the next instruction's input, issued while this one's items run
  StageIn pre;
  uint32_t pre_i = 0xFFFFFFFFu;
  // the last instruction at which the compute waves synchronised
  uint32_t last_sync = 0;
  // The launch runs a.n_steps steps back to back.  Instruction i of step s is
  // instruction ig = s * n + i of the launch: the LDS words that order the
  // waves count instructions and pages of the launch, and each step carries
  // its own epoch (the activation tag and counter target), position and
  // page base.  The trace keeps the first step of a launch.
  for (uint32_t ig = 0; ig < n_total; ig++) {
    const uint32_t step = ig / n, i = ig - step * n;
    const uint32_t ti = step == 0 ? i : 0xFFFFFFFFu;  // trace slot
    if (i == 0) {
      c.ep = a.epoch + step;
      c.pos = a.pos + int32_t(step);
      c.step = step;
      c.pbase = step * P;
      staged_in = 0;
    }
    InstrCP I = q + i;
    const bool is_gemv = i_op(I) == OP_GEMV;
    const bool reuse = reuses(I);
    const bool coop = is_coop(I);
    if (w == 0) {
      if (tr && c.lane == 0) {
        trace_put(a, cu, ti, TR_START, now32());
        trace_put(a, cu, ti, TR_HW0, hw0(I));
        trace_put(a, cu, ti, TR_HW1, hw1(I));
      }
      c.pagewait = 0;
      c.retries = 0;
      // No counter wait: every input of this kernel behind a producer is
      // tagged per element with the step (activations) or sits behind a
      // ticket (attention partials, argmax slots), and every activation
      // buffer is written once per step.  Staging polls the tags of the
      // elements it reads and re-reads only the stale ones, so it starts
      // while the producers' last rows are still in flight instead of a
      // counter round trip after the last of them.
      if (tr && c.lane == 0) trace_put(a, cu, ti, TR_DEPS, now32());
    }
    if (coop) {
      // every wave stages its share; a barrier publishes the x slot.  An
      // instruction that reuses the slot takes the barrier only after a run
      // of such instructions long enough to wrap the completion-counter
      // ring (a fast wave must not add to a slot whose previous instruction
      // a slow wave has not finished)
      const bool stage = !reuse || needs_res(I);
      if (stage || ig - last_sync >= uint32_t(kDoneRing - 1)) {
        if (stage) {
          if (pre_i != ig) stage_issue(c, I, !reuse, pre);
          if (!stage_finish(c, I, ig, !reuse, pre)) {
            if (c.lane == 0) lds_st(C_ABORT, 1);
            return;
          }
        }
        // the leader's own share staged (the barrier then waits for the others)
        if (tr && w == 0 && c.lane == 0) trace_put(a, cu, ti, TR_XFREE, now32());
        if (!comp_barrier()) return;
        last_sync = ig;
      }
      if (tr && w == 0 && c.lane == 0) {
        trace_put(a, cu, ti, TR_STAGED, now32());
        trace_put(a, cu, ti, TR_RETRY, c.retries);
      }
    } else if (w == 0) {
      // every compute wave has read the previous instruction's staged inputs
      if (!wait_all_ge(C_XCONS, ig)) {
        if (c.lane == 0) lds_st(C_ABORT, 1);
        return;
      }
      if (tr && c.lane == 0) {
        trace_put(a, cu, ti, TR_XFREE, now32());
        *lw(C_TR_LOOP) = 0xFFFFFFFFu;  // the attention loops' end stamps
        *lw(C_TR_LOOP + 4) = 0u;
      }
      if (!stage_leader(c, I, ig)) {
        if (c.lane == 0) lds_st(C_ABORT, 1);
        return;
      }
      if (c.lane == 0) lds_st(C_XOK, ig + 1);
      if (tr && c.lane == 0) {
        trace_put(a, cu, ti, TR_STAGED, now32());
        trace_put(a, cu, ti, TR_RETRY, c.retries);
      }
    } else if (!wait_lds_ge(C_XOK, ig + 1)) {
      return;
    }
    if (!coop) last_sync = ig;
    if (is_gemv) {
      staged_in = I->in_ptr;
      staged_flags = i_flags(I) & (F_IN_EMBED | F_NORM);
      staged_k = I->k;
      staged_gain = I->gain_ptr;
      // A down-projection chunk reads the gate/up output of a chunk that
      // every CU finished before its previous instruction began, so its
      // input is usually complete by now: issue its loads while this
      // instruction's items run, and staging it later costs only the
      // re-reads of what was still stale.  (The other inputs are written by
      // the stage that runs at the same time, and early loads of them would
      // only be read twice.)
      // Not during a gate/up instruction over every chunk: the first
      // chunk's pairs are written by its own items on every CU.
      const uint32_t ne = i + 1 < n ? i_epi(I + 1) : 0u;
      if (i + 1 < n && is_coop(I + 1) && !(i_flags(I) & F_GU_ALL) &&
          (ne == EPI_ACC_FIRST || ne == EPI_ACC_MID || ne == EPI_ACC_LAST)) {
        const bool nreuse = reuses(I + 1);
        if (!nreuse || needs_res(I + 1)) {
          stage_issue(c, I + 1, !nreuse, pre);
          pre_i = ig + 1;
        }
      }
    } else {
      staged_in = 0;
    }
    bool ok = i_op(I) == OP_GEMV ? run_gemv<G>(c, I, ig) : run_attn<G>(c, I, ig);
    if (!ok) return;
    if (tr && w == 0 && c.lane == 0) {
      trace_put(a, cu, ti, TR_ITEMS, now32());
      trace_put(a, cu, ti, TR_PAGEWAIT, c.pagewait);
    }
    // completion: the last wave signals.  Tagged outputs need no wait; the
    // untagged data behind a ticket (argmax slots, attention partials) must
    // have landed before the ticket moves.
    const bool opart = G::os && i_op(I) == OP_GEMV && i_epi(I) == EPI_OPART;
    const bool release = (i_op(I) == OP_GEMV && i_epi(I) == EPI_ARGMAX) ||
                         (i_op(I) == OP_ATTN && I->aux[3] > 1) || opart;
    if (release) wait_vm0();
    if (tr && w == 0 && c.lane == 0) trace_put(a, cu, ti, TR_VISIBLE, now32());
    uint32_t prev = 0;
    if (c.lane == 0) prev = lds_add(C_DONE + 4 * (ig % kDoneRing), 1);
    prev = uni(prev);
    if (prev != kNComp - 1) continue;
    if (c.lane == 0) lds_st(C_DONE + 4 * (ig % kDoneRing), 0);
    if (i_op(I) == OP_GEMV && i_epi(I) == EPI_ARGMAX) {
      lm_finish(c, I);
      continue;
    }
    if (i_op(I) == OP_ATTN && I->aux[3] > 1) {
      uint32_t old = 0;
      if (c.lane == 0) old = ctr_release(ctr_line(a, I->seg_rows[0], 0));
      old = uni(old);
      if (old + 1 != c.ep * I->aux[3]) continue;
      ctr_acquire();
      run_merge<G>(c, I);
    }
    if constexpr (G::os) {
      if (opart) {
        uint32_t old = 0;
        if (c.lane == 0) old = ctr_release(ctr_line(a, I->aux[2], 0));
        old = uni(old);
        if (old + 1 != c.ep * I->aux[3]) continue;
        ctr_acquire();
        if (!o_merge(c, I)) {
          if (c.lane == 0) lds_st(C_ABORT, 1);
          return;
        }
      }
    }
    if ((i_flags(I) & F_SIGNAL) && c.lane == 0) ctr_signal(ctr_line(a, I->sig_ctr, uint32_t(cu) % kCtrSpread));
    if (tr && c.lane == 0) trace_put(a, cu, ti, TR_SIGNAL, now32());
  }
}

template <class G>
__global__ __launch_bounds__(kThreads, 1) void mk_megakernel(KArgs a) {
  for (int o = threadIdx.x * 4; o < C_CTRL_END; o += kThreads * 4) *lw(o) = 0;
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
    loader(a, q, end - beg, wave);
  else
    compute<G>(a, q, end - beg, wave - kNLoad, cu);
}

// Plan-time fill of the packed weight stream: one workgroup column per copy,
// 16-byte loads and stores, rows split over gridDim.y.
__global__ void __launch_bounds__(256) mk_pack_kernel(const PackCopy* copies, uint32_t n,
                                                       uint8_t* base) {
  for (uint32_t c = blockIdx.x; c < n; c += gridDim.x) {
    const PackCopy cp = copies[c];
    const uint32_t per_row = cp.row_bytes / 16;
    const uint64_t total = uint64_t(cp.rows) * per_row;
    for (uint64_t t = threadIdx.x + uint64_t(blockIdx.y) * blockDim.x; t < total;
         t += uint64_t(blockDim.x) * gridDim.y) {
      const uint64_t r = t / per_row, k = t - r * per_row;
      const u4 v = *reinterpret_cast<const u4*>(cp.src + r * cp.src_stride + k * 16);
      // fragment order: block r / 16, column step k / 4, lane (k % 4) * 16 + r % 16
      const uint64_t o = cp.frag ? (r / 16) * 16 * cp.row_bytes + (k / 4) * 1024 + ((k % 4) * 16 + r % 16) * 16
                                 : r * cp.dst_stride + k * 16;
      *reinterpret_cast<u4*>(base + cp.dst + o) = v;
    }
  }
}

}  // namespace mk

extern "C" hipError_t mk_launch_pack(const mk::PackCopy* copies, uint32_t n, void* base,
                                     hipStream_t stream) {
  const uint32_t gx = n < 65535u ? n : 65535u;
  hipLaunchKernelGGL(mk::mk_pack_kernel, dim3(gx, 16), dim3(256), 0, stream, copies, n,
                     static_cast<uint8_t*>(base));
  return hipGetLastError();
}

// ---- kernel table (used by the runtime; not part of the public ABI)
namespace {
struct Variant {
  int nd, rd, nq, rq, nf, rf, hpt, dh;  // 0 = generic
  bool os;                              // split-K O projection
  const void* fn;
};
#define MK_VARIANT(ND, RD, NQ, RQ, NF, RF, H, D, OS) \
  {ND, RD, NQ, RQ, NF, RF, H, D, OS,                 \
   reinterpret_cast<const void*>(&mk::mk_megakernel<mk::GeoFix<ND, RD, NQ, RQ, NF, RF, H, D, OS>>)}
// Shapes with their own kernel: the Llama-3.2-1B shape (MLP in two chunks;
// one query head per attention tile at short contexts, the whole KV group at
// long ones), the Llama-3-8B shape (four chunks) and the small test decoder.
const Variant kVariants[] = {
    {0, 0, 0, 0, 0, 0, 0, 0, true, reinterpret_cast<const void*>(&mk::mk_megakernel<mk::GeoAny>)},
    MK_VARIANT(4, 1, 4, 1, 8, 1, 1, 64, false),
    MK_VARIANT(4, 1, 4, 1, 8, 1, 4, 64, false),
    MK_VARIANT(8, 1, 8, 1, 7, 1, 4, 128, false),
    MK_VARIANT(1, 2, 1, 2, 2, 1, 1, 64, false),
    // the same shapes with the O projection split per KV group
    MK_VARIANT(4, 1, 1, 2, 8, 1, 1, 64, true),
    MK_VARIANT(4, 1, 1, 2, 8, 1, 4, 64, true),
    MK_VARIANT(8, 1, 1, 1, 7, 1, 4, 128, true),
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);
bool g_attr_set[kNumVariants] = {};
}  // namespace

// Index of the kernel built for this geometry, or 0 (the generic kernel).
extern "C" int mk_pick_variant(int nd, int rd, int nq, int rq, int nf, int rf, int hpt, int dh, int os) {
  for (int v = 1; v < kNumVariants; v++) {
    const Variant& k = kVariants[v];
    if (k.nd == nd && k.rd == rd && k.nq == nq && k.rq == rq && k.nf == nf && k.rf == rf && k.hpt == hpt &&
        k.dh == dh && k.os == (os != 0))
      return v;
  }
  return 0;
}

extern "C" hipError_t mk_launch_megakernel(const mk::KArgs* args, int n_cus, hipStream_t stream,
                                           int cooperative, int variant) {
  if (variant < 0 || variant >= kNumVariants) return hipErrorInvalidValue;
  const void* fn = kVariants[variant].fn;
  if (!g_attr_set[variant]) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, mk::kLdsTotal);
    if (e != hipSuccess) return e;
    g_attr_set[variant] = true;
  }
  mk::KArgs a = *args;
  void* params[] = {&a};
  if (cooperative)
    return hipLaunchCooperativeKernel(fn, dim3(n_cus), dim3(mk::kThreads), params, mk::kLdsTotal, stream);
  return hipLaunchKernel(fn, dim3(n_cus), dim3(mk::kThreads), params, mk::kLdsTotal, stream);
}
