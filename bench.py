#!/usr/bin/env python3
"""Benchmark of the decode megakernel on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama1b_ctx128]

A step is one whole decode step (every stage of the hot path, one launch) of
the Llama-3.2-1B-shaped decoder at batch 1 over synthetic bf16 weights, with
the greedy token chained on the device.  W warm-up steps run from the
pre-filled context, then the position is reset and exactly K steps are timed,
bracketed by device synchronisation.  Prints ONE JSON line.

--workload moe_b8_ctx2048 runs the batch-8 parallel-block MoE decoder instead
(a separate line, not the headline metric); its weight bytes per step count
the experts the router selected in the timed steps.

roofline.achieved = algorithmic bytes of one launch (every weight once, the
KV rows [0, pos) read and the new row written) / the average kernel duration
measured with HIP events recorded around every launch on its stream.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs per decode step @batch1 (Llama-1B shape); achieved HBM GB/s vs peak"
PEAK_HBM = 8.0e12  # MI355X published HBM3E bandwidth, bytes/s


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("mk_kernel.hip", "mk_dev.h", "mk_isa.h", "mk_batch.hip"):
        with open(os.path.join(ROOT, "persistent_megakernel_wg_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str):
    """HBM bytes per decode step measured with rocprofv3 counters, if they were
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch") / rec.get("steps_per_launch", 1)


def host_info():
    """Host CPU model, logical cores and the BLAS thread count numpy uses."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = None
    return {"cpu_model": model, "host_cores": os.cpu_count(), "blas_threads": blas}


def _one_thread():
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=1)
    except Exception:
        import contextlib
        return contextlib.nullcontext()


def cpu_baseline_moe(shape, weights, kc, vc, tokens):
    """Time the float64 CPU oracle on one sequence of one step of the batched
    workload (the sequences of a step are independent) and scale it to the
    batch."""
    import numpy as np
    from oracle import DecoderOracle
    hi = host_info()
    orc = DecoderOracle(shape, weights, keep_f64=False)
    k, v = kc.copy(), vc.copy()
    t0 = time.perf_counter()
    orc.step(np.asarray(tokens), shape.prefill, k, v, seqs=[0])
    one = time.perf_counter() - t0
    return {"value": round(1e6 * one * shape.batch, 1), "unit": "us/step",
            "cores": hi["blas_threads"] or hi["host_cores"], "kind": "oracle",
            "oracle": "float64 (bf16 weights widened exactly per use)", **hi,
            "sample": "%s: sequence 0 of one float64 decode step at position %d (%.1f s, weights "
                      "widened per use), times %d sequences" % (shape.name, shape.prefill, one,
                                                                shape.batch)}


def cpu_baseline(shape, weights, kc, vc, tokens, budget_s: float = 20.0):
    """Time the float64 CPU oracle on a bounded sample of the same workload:
    with numpy's BLAS on all its threads, then on one thread."""
    import numpy as np
    from oracle import DecoderOracle
    hi = host_info()
    orc = DecoderOracle(shape, weights)
    k, v = kc.copy(), vc.copy()
    tok = np.asarray(tokens)
    t0 = time.perf_counter()
    _, tok = orc.step(tok, shape.prefill, k, v)       # warm-up: widens the weights
    warm = time.perf_counter() - t0
    times = []
    pos = shape.prefill + 1
    while sum(times) < budget_s and pos < shape.max_seq and len(times) < shape.steps:
        t0 = time.perf_counter()
        _, tok = orc.step(tok, pos, k, v)
        times.append(time.perf_counter() - t0)
        pos += 1
    us = 1e6 * sum(times) / len(times)
    # the same oracle on one thread, for a few steps of the budget
    t1 = []
    with _one_thread():
        while sum(t1) < budget_s / 4 and pos < shape.max_seq and len(t1) < 8:
            t0 = time.perf_counter()
            _, tok = orc.step(tok, pos, k, v)
            t1.append(time.perf_counter() - t0)
            pos += 1
    return {"value": round(us, 1), "unit": "us/step", "cores": hi["blas_threads"] or hi["host_cores"],
            "kind": "oracle", "oracle": "float64 (bf16 weights widened exactly once)", **hi,
            "value_1thread": round(1e6 * sum(t1) / max(1, len(t1)), 1) if t1 else None,
            "sample": "%s: %d float64 decode steps at positions %d..%d after one warm-up step "
                      "(%.1f s, weight widening) with BLAS on %s threads, then %d steps on one "
                      "thread" % (shape.name, len(times), shape.prefill + 1,
                                  shape.prefill + len(times), warm, hi["blas_threads"], len(t1))}


def stream_read_calibration(nbytes: int, dev, stream, reps: int = 5):
    """Achievable streaming read rate: a plain read of nbytes of device memory
    (the step's algorithmic bytes) with the library's calibration kernel,
    timed with HIP events on the launch stream (best block count of a few)."""
    import numpy as np
    import torch
    from persistent_megakernel_wg_amd import binding as B
    nbytes -= nbytes % 16
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    best = None
    for blocks in (1024, 2048, 4096, 8192):
        sink = torch.empty(blocks, dtype=torch.int32, device=dev)
        for _ in range(2):
            B.mk_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), blocks, stream.cuda_stream)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            B.mk_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), blocks, stream.cuda_stream)
            b.record(stream)
        torch.cuda.synchronize(dev)
        us = 1e3 * float(np.mean([a.elapsed_time(b) for a, b in ev]))
        gbps = nbytes / (us * 1e-6) / 1e9
        if best is None or gbps > best["stream_read_GBps"]:
            best = {"stream_read_GBps": round(gbps, 1), "bytes": nbytes, "blocks": blocks,
                    "us": round(us, 2), "kernel": "mk_stream_read (16 B non-temporal loads)"}
    del buf
    return best


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama1b_ctx128")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--n-cus", type=int, default=0)
    ap.add_argument("--attn-block", type=int, default=0)
    ap.add_argument("--mlp-chunks", type=int, default=0)
    ap.add_argument("--mfma", type=int, default=0,
                    help="batched decoder: 1: LM head on matrix cores; -1: vector ALUs; 0: default")
    ap.add_argument("--edn-queue", type=int, default=0,
                    help="MoE decoder: q > 1: a 1/q share of the expert down-projection units in a ready queue")
    ap.add_argument("--egu-balance", type=int, default=0,
                    help="MoE decoder: 1: gate/up shares weighted by each CU's earlier work; -1: even row slices")
    ap.add_argument("--o-split", type=int, default=0,
                    help="1: O projection split per KV group; -1: whole rows; 0: the plan's default")
    ap.add_argument("--attn-heads", type=int, default=0,
                    help="query heads per attention tile (0: the plan's default)")
    ap.add_argument("--gu-all", type=int, default=0,
                    help="1: gate/up of every MLP chunk in one instruction per CU; -1: one per chunk; "
                         "0: the plan's default")
    ap.add_argument("--launch", choices=("resident", "single"), default="resident",
                    help="resident: the K timed steps run in one launch (mk_decode_steps); "
                         "single: one launch per step, chained on the device")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode megakernel runs on a single device "
              "(--gpus %d is not supported)" % args.gpus, file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from persistent_megakernel_wg_amd import binding as B
    from persistent_megakernel_wg_amd import synth
    from persistent_megakernel_wg_amd.engine import Engine

    shape = synth.SHAPES[args.workload]
    t0 = time.perf_counter()
    weights = synth.make_weights(shape)
    kc, vc = synth.make_kv_cache(shape)
    tokens = synth.make_tokens(shape)
    t_gen = time.perf_counter() - t0
    print("[bench] inputs generated in %.1f s" % t_gen, file=sys.stderr, flush=True)

    eng = Engine(shape, weights, kc, vc,
                 plan=B.plan_opts(n_cus=args.n_cus, attn_block=args.attn_block,
                                  mlp_chunks=args.mlp_chunks, o_split=args.o_split, mfma=args.mfma,
                                  attn_heads=args.attn_heads,
                                  edn_queue=args.edn_queue,
                                  egu_balance=args.egu_balance, gu_all=args.gu_all))
    info = eng.plan_info()
    dev = eng.dev
    stream = torch.cuda.current_stream(dev)
    span = shape.max_seq - shape.prefill
    K, W = args.steps, args.warmup
    bufs = [torch.zeros(shape.batch, dtype=torch.int32, device=dev) for _ in range(K + W + 1)]
    bufs[0].copy_(torch.from_numpy(tokens))

    def pos_of(i):
        return shape.prefill + (i % span)

    resident = args.launch == "resident"
    if resident and (K > span or W > span):
        print("bench.py: --steps and --warmup must fit the cache (%d positions after the "
              "pre-filled ones) with --launch resident" % span, file=sys.stderr)
        return 2
    # warm-up from the initial state, then restart at the pre-filled position
    if resident:
        warm_out = torch.zeros(max(W, 1), shape.batch, dtype=torch.int32, device=dev)
        if W:
            B.mk_decode_steps(eng.ctx, bufs[0].data_ptr(), shape.prefill, W, warm_out.data_ptr(), 0,
                              stream.cuda_stream)
    else:
        for i in range(W):
            eng.launch(pos_of(i), tokens=bufs[i], next_out=bufs[i + 1], stream=stream)
    eng.sync()
    bufs[W].copy_(bufs[0])
    n_launch = 1 if resident else K
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_launch)]
    if shape.is_moe:
        B.mk_route_stats(eng.ctx, shape.n_layers, reset=True)
    out_k = torch.zeros(K, shape.batch, dtype=torch.int32, device=dev)
    torch.cuda.synchronize(dev)
    t_start = time.perf_counter()
    if resident:
        # K greedy steps in one launch; the events bracket the launch
        ev[0][0].record(stream)
        B.mk_decode_steps(eng.ctx, bufs[W].data_ptr(), shape.prefill, K, out_k.data_ptr(), 0,
                          stream.cuda_stream)
        ev[0][1].record(stream)
    else:
        for i in range(K):
            ev[i][0].record(stream)
            eng.launch(pos_of(i), tokens=bufs[W + i], next_out=bufs[W + i + 1], stream=stream)
            ev[i][1].record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t_start
    eng.sync()
    # per-step kernel time: launch durations divided by the steps they ran
    kern_ms = [a.elapsed_time(b) / (K if resident else 1) for a, b in ev]
    avg_kernel_s = float(np.mean(kern_ms)) / 1e3
    ms_per_step = 1e3 * wall / K

    if shape.is_moe:
        # fixed part (attention, router, LM head, norms, embedding rows) + the
        # selected experts' gate, up and down rows, averaged over the K steps
        sel = B.mk_route_stats(eng.ctx, shape.n_layers)
        wbytes = info["weight_bytes"] + 6.0 * shape.hidden * shape.expert_ffn * sum(sel) / K
        experts_per_layer = sum(sel) / (K * shape.n_layers)
    else:
        wbytes = synth.weight_bytes_per_step(shape)
        experts_per_layer = None
    kvb = [synth.kv_bytes_per_step(shape, pos_of(i)) for i in range(K)]
    alg_bytes = wbytes + float(np.mean(kvb))
    achieved = alg_bytes / avg_kernel_s
    traffic = traffic_from_profiles(shape.name)
    if traffic is not None:
        traffic = int(traffic * (K if resident else 1))  # per launch, like achieved

    calib = stream_read_calibration(int(alg_bytes), dev, stream)

    metric = METRIC if not shape.is_moe else \
        "µs per decode step @batch%d (parallel-block MoE shape); achieved HBM GB/s vs peak" % shape.batch
    out = {
        "metric": metric,
        "value": round(ms_per_step * 1e3, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "precision": "bf16 weights and KV cache, fp32 arithmetic",
        "data": "synthetic",
        "config": {"workload": shape.name, "layers": shape.n_layers, "hidden": shape.hidden,
                   "q_heads": shape.n_q_heads, "kv_heads": shape.n_kv_heads,
                   "head_dim": shape.head_dim, "ffn": shape.ffn, "vocab": shape.vocab,
                   "batch": shape.batch, "context": shape.prefill, "weights": "bf16",
                   "kv_cache": "bf16", "n_cus": info["n_cus"], "attn_block": info["attn_block"],
                   "mlp_chunks": info["mlp_chunks"]},
        "tokens_per_step": shape.batch,
        "launch": ("one launch of %d steps (mk_decode_steps)" % K) if resident else "one launch per step",
        "kernel_us_per_step": round(avg_kernel_s * 1e6, 2),
        "kernel_us_median": round(float(np.median(kern_ms)) * 1e3, 2),
        "kernel_us_p90": round(float(np.percentile(kern_ms, 90)) * 1e3, 2),
        "tok_per_s": round(shape.batch / (ms_per_step / 1e3), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved / 1e9, 1), "peak": PEAK_HBM / 1e9,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM, 4),
                     "traffic": traffic, "alg_bytes_per_step": int(alg_bytes),
                     "alg_bytes_per_launch": int(alg_bytes * (K if resident else 1))},
        "cpu_baseline": None,
        "calibration": calib,
    }
    if calib:
        out["roofline"]["frac_of_stream_read"] = round(achieved / (calib["stream_read_GBps"] * 1e9), 4)
    if shape.is_moe:
        out["config"].update({"experts": shape.n_experts, "top_k": shape.top_k,
                              "expert_ffn": shape.expert_ffn, "parallel_block": True})
        out["experts_selected_per_layer"] = round(experts_per_layer, 2)
    eng.close()
    del eng
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle (bounded sample)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = (cpu_baseline_moe(shape, weights, kc, vc, tokens) if shape.is_moe else
                               cpu_baseline(shape, weights, kc, vc, tokens, args.cpu_budget))
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
