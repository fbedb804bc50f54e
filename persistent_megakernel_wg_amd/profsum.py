"""Summaries of rocprofv3 runs of the decode megakernel, for the profiles/ folder.

    python -m persistent_megakernel_wg_amd.profsum stats <kernel_stats.csv> <workload> <command...>
    python -m persistent_megakernel_wg_amd.profsum traffic <workload> <fetch.csv> <write.csv> \\
        <copy_fetch.csv> <copy_write.csv> <alg_bytes_per_launch> [--steps-per-launch N]

`stats` prints a Markdown table of the kernel-duration summary
(`rocprofv3 --kernel-trace --stats`) with the command that produced it.

`traffic` turns two `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` passes over the
decode step, and the same two passes over a device copy of known size
(`python -m persistent_megakernel_wg_amd.profcopy`), into HBM bytes per launch:
the counters report KiB per dispatch; the copy's ratio of known bytes to
counted bytes scales them.  It writes a JSON record keyed by the hash of the
kernel sources (bench.py reports the traffic only while that hash matches).
"""
from __future__ import annotations

import csv
import json
import sys


def _rows(path):
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def _key(row, *names):
    for n in names:
        for k in row:
            if k.lower().replace("_", "") == n.lower().replace("_", ""):
                return row[k]
    raise KeyError(names)


def stats_table(path: str, command: str) -> str:
    rows = _rows(path)
    out = ["Command (from the repository root):", "", "```", command, "```", "",
           "| kernel | calls | average ns | min ns | max ns |", "|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(_key(r, "TotalDurationNs"))):
        out.append("| `%s` | %s | %.0f | %s | %s |" % (
            _key(r, "Name", "KernelName"), _key(r, "Calls"), float(_key(r, "AverageNs")),
            _key(r, "MinNs"), _key(r, "MaxNs")))
    return "\n".join(out)


def counter_per_dispatch(path: str, counter: str, kernel_sub: str):
    """Mean of `counter` over dispatches whose kernel name contains kernel_sub
    (summed over the rows a dispatch reports), and the dispatch count."""
    per = {}
    matched = None  # name of the counted kernel (the last matching row's)
    for r in _rows(path):
        name = _key(r, "Kernel_Name", "KernelName")
        if kernel_sub not in name or _key(r, "Counter_Name", "CounterName") != counter:
            continue
        matched = name
        d = _key(r, "Dispatch_Id", "DispatchId")
        per[d] = per.get(d, 0.0) + float(_key(r, "Counter_Value", "CounterValue"))
    if not per:
        raise SystemExit("no %s rows for a kernel containing %r in %s" % (counter, kernel_sub, path))
    vals = [per[k] for k in sorted(per, key=lambda x: int(x))]
    return vals, matched


def traffic(workload, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, alg_bytes, steps_per_launch=1):
    sys.path.insert(0, __file__.rsplit("/", 2)[0])
    import bench
    f_vals, kname = counter_per_dispatch(fetch_csv, "FETCH_SIZE", "mk_megakernel")
    w_vals, _ = counter_per_dispatch(write_csv, "WRITE_SIZE", "mk_megakernel")
    cf, _ = counter_per_dispatch(copy_fetch_csv, "FETCH_SIZE", "")
    cw, _ = counter_per_dispatch(copy_write_csv, "WRITE_SIZE", "")
    copy_bytes = 1 << 30
    # the copy dispatches of profcopy: the largest counts are the 1 GiB copies
    cf_kib, cw_kib = max(cf), max(cw)
    ff, wf = copy_bytes / 1024.0 / cf_kib, copy_bytes / 1024.0 / cw_kib
    # skip the first (warm-up) dispatch of the step when there are several
    fs = f_vals[1:] if len(f_vals) > 1 else f_vals
    ws = w_vals[1:] if len(w_vals) > 1 else w_vals
    f_kib, w_kib = sum(fs) / len(fs), sum(ws) / len(ws)
    rd, wr = f_kib * 1024 * ff, w_kib * 1024 * wf
    return {
        "workload": workload, "kernel": kname, "kernel_hash": bench.kernel_source_hash(),
        "steps_per_launch": steps_per_launch,
        "fetch_size_kib_per_dispatch": round(f_kib, 1), "write_size_kib_per_dispatch": round(w_kib, 1),
        "copy_calibration": {"bytes_read_and_written_per_dispatch": copy_bytes, "fetch_size_kib": cf_kib,
                             "write_size_kib": cw_kib, "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)},
        "hbm_read_bytes_per_launch": int(rd), "hbm_write_bytes_per_launch": int(wr),
        "hbm_bytes_per_launch": int(rd + wr), "alg_bytes_per_launch": int(alg_bytes),
        "traffic_over_algorithmic": round((rd + wr) / alg_bytes, 4),
    }


def main(argv) -> int:
    if len(argv) >= 3 and argv[0] == "stats":
        print(stats_table(argv[1], " ".join(argv[3:])))
        return 0
    if len(argv) >= 7 and argv[0] == "traffic":
        spl = 1
        if "--steps-per-launch" in argv:
            spl = int(argv[argv.index("--steps-per-launch") + 1])
        rec = traffic(argv[1], argv[2], argv[3], argv[4], argv[5], float(argv[6]), spl)
        print(json.dumps(rec, indent=1))
        return 0
    print(__doc__)
    return 2


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
