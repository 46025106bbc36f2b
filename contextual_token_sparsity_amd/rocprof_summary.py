"""Turns rocprofv3 CSV output into the short summaries kept under profiles/.

    # kernel durations (rocprofv3 --kernel-trace --stats ... -o trace); with the
    # per-dispatch trace beside STATS_CSV, the exact-score launches in detail
    python -m contextual_token_sparsity_amd.rocprof_summary trace STATS_CSV OUT_TXT "COMMAND" [TIMED_STEPS]

    # HBM bytes per launch of the exact-score kernel from two counter runs
    # (rocprofv3 --pmc FETCH_SIZE / --pmc WRITE_SIZE of `bench.py --copy-probe`)
    python -m contextual_token_sparsity_amd.rocprof_summary traffic FETCH_CSV WRITE_CSV OUT_JSON OUT_TXT "COMMANDS"

The counters are calibrated on the plain 1 GiB device-to-device copy that
`bench.py --copy-probe` issues: the ratio of its known bytes to what each
counter reports scales the exact-score kernel's readings.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 1 << 30
# the benchmark's exact-score launch: head_dim 128, PAPER head reduction,
# blocks of 64, whole blocks (diagonal-only exclusions; template value 0);
# the causal launch (value 2) is reported beside it
SCORE_KERNEL = "k_block_scores<128, 0, 64, 0>"
CAUSAL_KERNEL = "k_block_scores<128, 0, 64, 2>"


def kernel_source_hash() -> str:
    p = os.path.join(PKG, "csrc", "block_scores.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def _score_launches(trace_csv: str, timed_steps: int):
    """Per-dispatch durations (us) of the benchmark's exact-score launches,
    in dispatch order, from the kernel-trace CSV.  Only dispatches of at
    least half the longest one count (a much smaller launch of the same
    instantiation would otherwise dilute the average).  The bench times
    `timed_steps` steps right before its first causal launch."""
    rows = list(csv.DictReader(open(trace_csv)))
    seq = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]) for r in rows)
    full = [(s, (e - s) / 1e3) for s, e, n in seq if SCORE_KERNEL in n]
    causal = [(s, (e - s) / 1e3) for s, e, n in seq if CAUSAL_KERNEL in n]
    if not full:
        return []
    top = max(d for _, d in full)
    many = [(s, d) for s, d in full if d >= 0.5 * top]
    first_causal = causal[0][0] if causal else None
    timed = [d for s, d in many if first_causal is None or s < first_causal][-timed_steps:]
    lines = ["", f"{SCORE_KERNEL}, 32-head launches only ({len(full) - len(many)} much smaller launches left "
             f"out): {len(many)} launches, avg {sum(d for _, d in many) / len(many):.1f} us "
             "(includes the clock-settle launches)",
             f"  the {len(timed)} launches just before the first causal launch (the bench's timed steps): "
             f"avg {sum(timed) / max(len(timed), 1):.1f} us"]
    if causal:
        ds = [d for _, d in causal]
        lines.append(f"{CAUSAL_KERNEL}: {len(ds)} launches, avg {sum(ds) / len(ds):.1f} us; "
                     f"the last {min(10, len(ds))}: avg {sum(ds[-10:]) / len(ds[-10:]):.1f} us")
    return lines


def trace(stats_csv: str, out_txt: str, command: str, timed_steps: int = 10) -> None:
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# rocprofv3 kernel statistics", f"# command: {command}", "",
             f"{'kernel':<72} {'calls':>6} {'avg us':>10} {'min us':>10} {'max us':>10} {'% time':>7}"]
    for r in rows:
        name = r["Name"]
        short = name if len(name) <= 72 else name[:69] + "..."
        lines.append(f"{short:<72} {r['Calls']:>6} {float(r['AverageNs']) / 1e3:>10.1f} "
                     f"{float(r['MinNs']) / 1e3:>10.1f} {float(r['MaxNs']) / 1e3:>10.1f} "
                     f"{float(r['Percentage']):>7.2f}")
    trace_csv = stats_csv.replace("_kernel_stats.csv", "_kernel_trace.csv")
    if trace_csv != stats_csv and os.path.exists(trace_csv):
        lines += _score_launches(trace_csv, int(timed_steps))
    with open(out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")


def _per_kernel(counter_csv: str):
    rows = list(csv.DictReader(open(counter_csv)))
    vals = defaultdict(list)
    copies = []
    for r in rows:
        v = float(r["Counter_Value"])
        name = r["Kernel_Name"]
        if SCORE_KERNEL in name:
            vals["score"].append(v)
        elif CAUSAL_KERNEL in name:
            vals["causal"].append(v)
        elif "copyBuffer" in name:
            copies.append((v, int(r["Grid_Size"])))
    return vals["score"], vals["causal"], copies


def _many_heads(vals):
    """Only the benchmark's 32-head launches: a launch of the same
    instantiation on a much smaller problem would fetch a few percent of
    theirs, so keep the dispatches within half of the largest."""
    top = max(vals)
    return [v for v in vals if v >= 0.5 * top]


def traffic(fetch_csv: str, write_csv: str, out_json: str, out_txt: str, commands: str) -> None:
    f_all, f_causal, f_copy = _per_kernel(fetch_csv)
    w_score, w_causal, w_copy = _per_kernel(write_csv)
    if not (f_all and w_score and f_copy and w_copy):
        raise SystemExit("missing score-kernel or copy-probe dispatches in the counter files")
    # fetch: the 32-head launches only; write (M, 256 KiB) is averaged over
    # every launch of the instantiation
    f_score = _many_heads(f_all)
    # the copy probe is the copyBuffer dispatch with the largest reading
    # (uploads of the inputs are host-to-device and smaller)
    f_ref = max(f_copy)[0]
    w_ref = max(w_copy)[0]
    f_scale = COPY_BYTES / (f_ref * 1024.0)
    w_scale = COPY_BYTES / (w_ref * 1024.0)
    fetch_b = sum(f_score) / len(f_score) * 1024.0 * f_scale
    write_b = sum(w_score) / len(w_score) * 1024.0 * w_scale
    causal = None
    if f_causal and w_causal:
        cf = sum(f_causal) / len(f_causal) * 1024.0 * f_scale
        cw = sum(w_causal) / len(w_causal) * 1024.0 * w_scale
        causal = {"kernel": CAUSAL_KERNEL, "fetch_bytes_per_launch": cf, "write_bytes_per_launch": cw,
                  "hbm_bytes_per_launch": cf + cw, "launches": len(f_causal)}
    rec = {
        "kernel": SCORE_KERNEL,
        "kernel_source_sha256_16": kernel_source_hash(),
        "fetch_bytes_per_launch": fetch_b,
        "write_bytes_per_launch": write_b,
        "hbm_bytes_per_launch": fetch_b + write_b,
        "fetch_scale": f_scale,
        "write_scale": w_scale,
        "launches": len(f_score),
        "one_head_launches_left_out": len(f_all) - len(f_score),
        "causal": causal,
        "commands": commands,
    }
    with open(out_json, "w") as f:
        json.dump(rec, f, indent=1)
    with open(out_txt, "w") as f:
        f.write("# HBM traffic of the exact-score kernel (rocprofv3 counters)\n")
        f.write(f"# commands: {commands}\n\n")
        f.write(f"copy probe (1 GiB device copy): FETCH_SIZE {f_ref:.0f} KiB, WRITE_SIZE {w_ref:.0f} KiB\n")
        f.write(f"  -> scale factors: fetch x{f_scale:.3f}, write x{w_scale:.3f}\n")
        f.write(f"{SCORE_KERNEL}: {len(f_score)} launches, FETCH_SIZE avg {sum(f_score) / len(f_score):.0f} KiB, "
                f"WRITE_SIZE avg {sum(w_score) / len(w_score):.0f} KiB\n")
        f.write(f"  -> HBM bytes per launch: read {fetch_b / 1e9:.3f} GB, write {write_b / 1e9:.4f} GB, "
                f"total {(fetch_b + write_b) / 1e9:.3f} GB\n")
        f.write(f"  ({len(f_all) - len(f_score)} much smaller launches of the same instantiation left out of the "
                f"fetch average)\n")
        if causal:
            f.write(f"{CAUSAL_KERNEL}: {causal['launches']} launches -> HBM bytes per launch: read "
                    f"{causal['fetch_bytes_per_launch'] / 1e9:.3f} GB, write "
                    f"{causal['write_bytes_per_launch'] / 1e9:.4f} GB\n")
        f.write(f"kernel source sha256[:16]: {kernel_source_hash()}\n")


if __name__ == "__main__":
    cmd = sys.argv[1] if len(sys.argv) > 1 else ""
    if cmd == "trace" and len(sys.argv) in (5, 6):
        trace(*sys.argv[2:])
    elif cmd == "traffic" and len(sys.argv) == 7:
        traffic(*sys.argv[2:7])
    else:
        print(__doc__)
        sys.exit(2)
