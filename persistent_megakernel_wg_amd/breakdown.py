"""Per-stage time breakdown of one decode step from the kernel's own trace.

    python -m persistent_megakernel_wg_amd.breakdown [--workload llama1b_ctx128]
        [--steps 4] [--json out.json] [--o-split 1] [--mfma 1] [--egu-balance 1]

Runs a few steps of the workload on the GPU with the per-instruction trace
switched on (mk_trace_enable: s_memrealtime stamps, 100 MHz, written by each
CU's leader wave), and prints where the last traced step's time goes, in the
shape of the runtime breakdown the Llama-1B megakernel write-up gives for its
B200 step (rocketrecap.com summary, "Detailed Runtime Breakdown"): for every
stage kind the wall time it holds on the step's critical path, split into

  * hand-over: from the last producer of the previous stage finishing to the
    median CU having its inputs staged (signal visibility, tag polling and
    the cross-CU load of the input vector), and
  * work: from the median CU's inputs staged to the stage's last CU finishing
    (items, page waits on weights that did not stream ahead, the tail of the
    slowest CU, the epilogue).

Stages follow each other strictly within a layer (QKV -> attention -> O ->
gate/up chunks -> down chunks, then the next layer), so the per-stage spans
add up to the step.  The trace costs a few stores per instruction, so a
traced step runs a little slower than an untraced one.
"""
from __future__ import annotations

import argparse
import json
import sys
from collections import defaultdict

import numpy as np

TR = dict(START=0, DEPS=1, STAGED=2, ITEMS=3, SIGNAL=4, PAGEWAIT=5, HW0=6, HW1=7,
          XREADY=8, ITEM0=9, VISIBLE=10, XFREE=11, A_PASS1=12, A_STATS=13, A_PASS3=14, RETRY=15)
OP_GEMV, OP_ATTN, OP_BGEMV, OP_EGU, OP_EDN, OP_ERD = 1, 2, 3, 4, 5, 6
EPI_NAMES = {0: "qkv", 1: "o", 2: "gate_up", 3: "down", 4: "down", 5: "down", 6: "down",
             7: "lm_head", 8: "o"}
TICK_US = 0.01  # s_memrealtime runs at 100 MHz


def stage_of(hw0: int, batched: bool) -> str:
    op, epi = hw0 & 0xFF, (hw0 >> 8) & 0xFF
    if op == OP_ATTN:
        return "attention"
    if op == OP_EGU:
        return "expert_gate_up"
    if op == OP_EDN:
        return "expert_down"
    if op == OP_ERD:
        return "expert_sum"
    if op == OP_BGEMV and epi == 0:
        return "qkv_router"
    return EPI_NAMES.get(epi, "op%d" % op)


def analyse(tr: np.ndarray, batched: bool = False) -> dict:
    """tr: uint32 [n_cus, stride, 16] of one step.  Returns the breakdown."""
    n_cus, stride, _ = tr.shape
    valid = tr[:, :, TR["HW0"]] != 0
    # the 32-bit stamps wrap every 43 s: take differences to one stamp as
    # signed 32-bit values, then start the step at the earliest
    ref = int(tr[:, :, TR["START"]][valid][0])

    def signed(v):
        return ((np.asarray(v).astype(np.int64) - ref + (1 << 31)) & 0xFFFFFFFF) - (1 << 31)

    t0 = int(np.min(signed(tr[:, :, TR["START"]][valid])))

    def rel(v):
        return (signed(v) - t0) * TICK_US

    # per (layer, stage, occurrence on the CU) -> lists over CUs
    rec = defaultdict(lambda: defaultdict(list))
    for cu in range(n_cus):
        seen = defaultdict(int)
        for i in range(stride):
            if not valid[cu, i]:
                continue
            w = tr[cu, i]
            layer = int(w[TR["HW1"]] >> 16)
            st = stage_of(int(w[TR["HW0"]]), batched)
            k = seen[(layer, st)]
            seen[(layer, st)] += 1
            end = w[TR["SIGNAL"]] if w[TR["SIGNAL"]] else w[TR["ITEMS"]]
            r = rec[(layer, st, k)]
            r["start"].append(rel(np.array(w[TR["START"]])))
            # instructions without a staging stamp (attention tiles, CUs
            # with no expert units) count as staged once their waits passed
            staged = w[TR["STAGED"]] or w[TR["DEPS"]] or w[TR["START"]]
            r["staged"].append(rel(np.array(staged)))
            r["end"].append(rel(np.array(end)))
            r["pagewait"].append(int(w[TR["PAGEWAIT"]]) * TICK_US)
            # phases inside the instruction, per CU (leader's stamps)
            for name in ("XREADY", "ITEM0", "ITEMS", "VISIBLE", "A_PASS1", "A_STATS", "A_PASS3", "XFREE"):
                r[name.lower()].append(rel(np.array(w[TR[name]])) if w[TR[name]] else np.nan)
    order = sorted(rec.keys(), key=lambda k: (k[0], float(np.median(rec[k]["start"])), k[2]))
    rows = []
    prev_end = 0.0
    for key in order:
        r = rec[key]
        staged = np.array(r["staged"], dtype=np.float64)
        end = np.array(r["end"], dtype=np.float64)
        end_max = float(np.max(end))
        st_med = float(np.median(staged))
        handover = max(0.0, min(st_med, end_max) - prev_end)
        work = max(0.0, end_max - max(prev_end, min(st_med, end_max)))
        def med(a, b):
            d = np.array(r[a], dtype=np.float64) - np.array(r[b], dtype=np.float64)
            d = d[np.isfinite(d)]
            return float(np.median(d)) if d.size else float("nan")
        phases = {"staged_to_xready_us": med("xready", "staged"),
                  "xready_to_item0_us": med("item0", "xready"),
                  "item0_to_items_us": med("items", "item0"),
                  "items_to_end_us": med("end", "items"),
                  "staged_to_end_us": med("end", "staged"),
                  "start_to_staged_us": med("staged", "start"),
                  # one-sequence GEMV rows: the first iteration of wave 0
                  # one-sequence GEMV rows: the leader's own staging, then
                  # the barrier of the staging waves
                  "start_to_ownstage_us": med("xfree", "start"),
                  "ownstage_to_staged_us": med("staged", "xfree"),
                  "xready_to_page_us": med("a_pass1", "xready"),
                  "page_to_sums_us": med("a_stats", "a_pass1"),
                  "sums_to_item0_us": med("item0", "a_stats"),
                  # attention tiles: wave 0's pass to the barrier after the
                  # lane-group merge, then the wave merge and the stores
                  "item0_to_wavemerge_us": med("a_pass3", "item0"),
                  "wavemerge_to_items_us": med("items", "a_pass3"),
                  # one-sequence attention tiles: the waves' loop ends
                  # (earliest, latest) against wave 0's and the barrier
                  "loop_spread_us": med("a_stats", "a_pass1"),
                  "lastloop_to_wavemerge_us": med("a_pass3", "a_stats")}
        rows.append({"layer": key[0], "stage": key[1], "part": key[2], "cus": len(end), **phases,
                     "staged_median_us": st_med, "end_median_us": float(np.median(end)),
                     "end_max_us": end_max, "handover_us": handover, "work_us": work,
                     "pagewait_median_us": float(np.median(r["pagewait"]))})
        prev_end = max(prev_end, end_max)
    total = prev_end
    kinds = defaultdict(lambda: [0.0, 0.0])
    for r in rows:
        kinds[r["stage"]][0] += r["handover_us"]
        kinds[r["stage"]][1] += r["work_us"]
    return {"step_us": total, "rows": rows, "batched": bool(batched),
            "by_stage": {k: {"handover_us": v[0], "work_us": v[1], "total_us": v[0] + v[1]}
                         for k, v in kinds.items()}}


def report(res: dict, title: str) -> str:
    out = ["## %s" % title, "",
           "Traced step: %.1f us (first instruction start to last stage end)." % res["step_us"], "",
           "| stage | hand-over (us) | work (us) | total (us) | share |",
           "|---|---|---|---|---|"]
    tot = res["step_us"] or 1.0
    for k, v in sorted(res["by_stage"].items(), key=lambda kv: -kv[1]["total_us"]):
        out.append("| %s | %.1f | %.1f | %.1f | %.1f %% |" % (
            k, v["handover_us"], v["work_us"], v["total_us"], 100 * v["total_us"] / tot))
    out += ["", "Per stage of a middle layer (medians over CUs, us from the step start):", "",
            "| layer | stage | part | CUs | staged (median) | end (median) | end (last CU) | page wait (median) |",
            "|---|---|---|---|---|---|---|---|"]
    layers = sorted({r["layer"] for r in res["rows"]})
    mid = layers[len(layers) // 2] if layers else 0
    for r in res["rows"]:
        if r["layer"] == mid or r["stage"] == "lm_head":
            out.append("| %d | %s | %d | %d | %.2f | %.2f | %.2f | %.2f |" % (
                r["layer"], r["stage"], r["part"], r["cus"], r["staged_median_us"],
                r["end_median_us"], r["end_max_us"], r["pagewait_median_us"]))
    out += ["", "Inside one instruction of the same layer (medians over CUs of per-CU differences, us):", "",
            "| stage | part | start->staged | staged->x ready | x ready->first item | first item->items done "
            "| items done->end | staged->end |", "|---|---|---|---|---|---|---|---|"]
    for r in res["rows"]:
        if r["layer"] == mid or r["stage"] == "lm_head":
            out.append("| %s | %d | %.2f | %.2f | %.2f | %.2f | %.2f | %.2f |" % (
                r["stage"], r["part"], r["start_to_staged_us"], r["staged_to_xready_us"],
                r["xready_to_item0_us"], r["item0_to_items_us"], r["items_to_end_us"],
                r["staged_to_end_us"]))
    gem = [r for r in res["rows"] if not res.get("batched") and (r["layer"] == mid or r["stage"] == "lm_head")
           and r["stage"] != "attention" and np.isfinite(r.get("page_to_sums_us", np.nan))]
    if gem:
        out += ["", "The first item of wave 0 in the same GEMV instructions (medians, us):", "",
                "| stage | part | start->leader's share staged | ->barrier passed | x ready->pages ready "
                "| pages ready->sums reduced | sums reduced->first item done |",
                "|---|---|---|---|---|---|---|"]
        for r in gem:
            out.append("| %s | %d | %.2f | %.2f | %.2f | %.2f | %.2f |" % (
                r["stage"], r["part"], r["start_to_ownstage_us"], r["ownstage_to_staged_us"],
                r["xready_to_page_us"], r["page_to_sums_us"], r["sums_to_item0_us"]))
    att = [r for r in res["rows"] if r["layer"] == mid and r["stage"] == "attention"
           and np.isfinite(r.get("item0_to_wavemerge_us", np.nan))]
    if att:
        out += ["", "After the position loop of wave 0 in the attention tiles of the same layer (medians, us):", "",
                "| part | loop end->lane groups merged, records written, barrier | ->waves merged, outputs stored, barrier |",
                "|---|---|---|"]
        for r in att:
            out.append("| %d | %.2f | %.2f |" % (r["part"], r["item0_to_wavemerge_us"], r["wavemerge_to_items_us"]))
        if not res.get("batched"):
            out += ["", "| part | first to last wave's loop end | last loop end->lane groups merged, barrier |",
                    "|---|---|---|"]
            for r in att:
                out.append("| %d | %.2f | %.2f |" % (r["part"], r["loop_spread_us"], r["lastloop_to_wavemerge_us"]))
    return "\n".join(out)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="llama1b_ctx128")
    ap.add_argument("--steps", type=int, default=4)
    ap.add_argument("--json", default="")
    ap.add_argument("--o-split", type=int, default=0,
                    help="1: O projection split per KV group; -1: whole rows; 0: the plan's default")
    ap.add_argument("--egu-balance", type=int, default=0,
                    help="MoE decoder: 1: weighted gate/up shares; -1: even row slices")
    ap.add_argument("--mfma", type=int, default=0,
                    help="batched decoder: 1: LM head on matrix cores; -1: vector ALUs; 0: default")
    args = ap.parse_args()
    from . import binding as B
    from . import synth
    from .engine import Engine
    s = synth.SHAPES[args.workload]
    w = synth.make_weights(s)
    kc, vc = synth.make_kv_cache(s)
    tok = synth.make_tokens(s)
    opts = (B.plan_opts(o_split=args.o_split, mfma=args.mfma, egu_balance=args.egu_balance)
            if (args.o_split or args.mfma or args.egu_balance) else None)
    eng = Engine(s, w, kc, vc, plan=opts)
    try:
        info = eng.plan_info()
        B.mk_trace_enable(eng.ctx, True)
        eng.tokens.copy_(eng.torch.from_numpy(tok))
        for i in range(args.steps):
            eng.launch(s.prefill + i)
            eng.sync()
        tr = B.mk_trace_read(eng.ctx, info["n_cus"], info["max_queue"])
    finally:
        eng.close()
    res = analyse(tr, batched=s.is_moe)
    print(report(res, "%s, step %d (traced)" % (s.name, args.steps)), flush=True)
    if args.json:
        with open(args.json, "w") as fh:
            json.dump({"workload": s.name, **res}, fh, indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
