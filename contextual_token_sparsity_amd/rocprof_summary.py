"""Turns rocprofv3 CSV output into the short summaries kept under profiles/.

    # kernel durations (rocprofv3 --kernel-trace --stats ... -o trace); with the
    # per-dispatch trace beside STATS_CSV, the exact-score launches in detail
    python -m contextual_token_sparsity_amd.rocprof_summary trace STATS_CSV OUT_TXT "COMMAND" [TIMED_STEPS]

    # HBM bytes per launch of the exact-score kernel from two counter runs
    # (rocprofv3 --pmc FETCH_SIZE / --pmc WRITE_SIZE of `bench.py --copy-probe`)
    python -m contextual_token_sparsity_amd.rocprof_summary traffic FETCH_CSV WRITE_CSV OUT_JSON OUT_TXT "COMMANDS"

    # where the exact-score kernel's cycles go, from two counter runs of
    # `bench.py` (SQ/GRBM/TCP counters listed in BUSY_PASSES)
    python -m contextual_token_sparsity_amd.rocprof_summary busy PASS1_CSV PASS2_CSV OUT_TXT "COMMANDS"

    # HBM bytes per launch of the movement and pooling kernels, split by grid
    # (two counter runs with --copy-probe, and a kernel trace of the same command)
    python -m contextual_token_sparsity_amd.rocprof_summary movement FETCH_CSV WRITE_CSV TRACE_CSV OUT_TXT "COMMANDS"

The traffic counters are calibrated on the plain 1 GiB device-to-device copy that
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
# blocks of 64, no causal mask (the eight-wave kernel); the causal launch of
# the same kernel is reported beside it
SCORE_KERNEL = "k_block_scores_pp<128, 0, 64, false>"
CAUSAL_KERNEL = "k_block_scores_pp<128, 0, 64, true>"


def kernel_source_hash() -> str:
    p = os.path.join(PKG, "csrc", "block_scores.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def _score_launches(trace_csv: str, timed_steps: int):
    """Per-dispatch durations (us) of the benchmark's exact-score launches,
    in dispatch order, from the kernel-trace CSV.  Only dispatches of at
    least half the longest one count (a much smaller launch of the same
    instantiation would otherwise dilute the average).  The bench runs its
    `timed_steps` timed steps, then as many steps again with an event after
    every stage (the stage breakdown), right before its first causal launch."""
    rows = list(csv.DictReader(open(trace_csv)))
    seq = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]) for r in rows)
    full = [(s, (e - s) / 1e3) for s, e, n in seq if SCORE_KERNEL in n]
    causal = [(s, (e - s) / 1e3) for s, e, n in seq if CAUSAL_KERNEL in n]
    if not full:
        return []
    top = max(d for _, d in full)
    many = [(s, d) for s, d in full if d >= 0.5 * top]
    first_causal = causal[0][0] if causal else None
    before = [d for s, d in many if first_causal is None or s < first_causal]
    timed = before[-2 * timed_steps:-timed_steps] if len(before) >= 2 * timed_steps else []
    staged = before[-timed_steps:]
    lines = ["", f"{SCORE_KERNEL}, 32-head launches only ({len(full) - len(many)} much smaller launches left "
             f"out): {len(many)} launches, avg {sum(d for _, d in many) / len(many):.1f} us "
             "(includes the clock-settle launches)",
             f"  the bench's {len(timed)} timed steps: avg {sum(timed) / max(len(timed), 1):.1f} us; the "
             f"{len(staged)} steps of the stage breakdown after them: avg {sum(staged) / max(len(staged), 1):.1f} us"]
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


# counter passes for `busy` (each within one run's per-block limits: at most
# 8 SQ counters; GRBM_GUI_ACTIVE in both, since it times each dispatch)
BUSY_PASSES = (
    "GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS SQ_WAVE_CYCLES "
    "SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_BUSY_CU_CYCLES",
    "GRBM_GUI_ACTIVE SQ_INSTS_VMEM SQ_INSTS_VALU SQ_VALU_MFMA_COEXEC_CYCLES SQ_LDS_BANK_CONFLICT "
    "TCP_PENDING_STALL_CYCLES_sum",
)
N_XCD, N_CU, N_SIMD = 8, 256, 1024


def _dispatch_counters(counter_csv: str):
    """{dispatch id: (duration s, {counter: value})} of the exact-score
    kernel's 32-head launches."""
    per = defaultdict(dict)
    dur = {}
    for r in csv.DictReader(open(counter_csv)):
        if SCORE_KERNEL not in r["Kernel_Name"]:
            continue
        d = int(r["Dispatch_Id"])
        per[d][r["Counter_Name"]] = float(r["Counter_Value"])
        dur[d] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    if not per:
        raise SystemExit(f"no {SCORE_KERNEL} dispatches in {counter_csv}")
    top = max(v.get("GRBM_GUI_ACTIVE", 0.0) for v in per.values())
    return {d: (dur[d], v) for d, v in per.items() if v.get("GRBM_GUI_ACTIVE", 0.0) >= 0.5 * top}


def busy(pass1_csv: str, pass2_csv: str, out_txt: str, commands: str) -> None:
    """Cycle-level figures of the exact-score kernel.  GRBM_GUI_ACTIVE is
    summed over the 8 XCDs, so a launch takes GRBM/8 shader cycles and
    GRBM/8/duration is the clock it ran at; SQ_VALU_MFMA_BUSY_CYCLES is
    summed over the 1024 SIMDs."""
    p1, p2 = _dispatch_counters(pass1_csv), _dispatch_counters(pass2_csv)

    def avg(p, name):
        vals = [v[name] for _, v in p.values() if name in v]
        return sum(vals) / len(vals) if vals else float("nan")

    cyc1 = avg(p1, "GRBM_GUI_ACTIVE") / N_XCD
    cyc2 = avg(p2, "GRBM_GUI_ACTIVE") / N_XCD
    # the clock of the last launches of the first pass (the earliest run
    # while the clock is still rising)
    last = sorted(p1)[-10:]
    clocks = [p1[d][1]["GRBM_GUI_ACTIVE"] / N_XCD / p1[d][0] for d in last]
    clock = sum(clocks) / len(clocks)
    mfma_busy = avg(p1, "SQ_VALU_MFMA_BUSY_CYCLES") / N_SIMD
    n_mfma = avg(p1, "SQ_INSTS_MFMA")
    lds_active = avg(p1, "SQ_LDS_IDX_ACTIVE") / N_CU
    n_lds = avg(p1, "SQ_INSTS_LDS")
    wave_cyc = avg(p1, "SQ_WAVE_CYCLES") * 4           # the SQ wave counters tick every 4 cycles
    wait_any = avg(p1, "SQ_WAIT_ANY") * 4
    wait_inst = avg(p1, "SQ_WAIT_INST_ANY") * 4
    n_vmem = avg(p2, "SQ_INSTS_VMEM")
    n_valu = avg(p2, "SQ_INSTS_VALU")
    coexec = avg(p2, "SQ_VALU_MFMA_COEXEC_CYCLES") / N_SIMD
    conflicts = avg(p2, "SQ_LDS_BANK_CONFLICT")
    tcp_pending = avg(p2, "TCP_PENDING_STALL_CYCLES_sum") / N_CU
    lines = [
        "# where the exact-score kernel's cycles go (rocprofv3 counters)",
        f"# commands: {commands}",
        "",
        f"{SCORE_KERNEL}: {len(p1)} + {len(p2)} launches (32-head launches of the two passes)",
        f"cycles per launch (GRBM_GUI_ACTIVE / 8 XCDs): {cyc1:.4g} (pass 1), {cyc2:.4g} (pass 2)",
        f"clock under this load (cycles / launch duration, last {len(last)} launches of pass 1): "
        f"{clock / 1e9:.2f} GHz",
        f"MFMA instructions per launch: {n_mfma:.4g}; busy cycles per SIMD: {mfma_busy:.4g} "
        f"({mfma_busy / cyc1:.1%} of the launch's cycles)",
        f"  -> at {clock / 1e9:.2f} GHz that is {mfma_busy / cyc1 * clock / 2.4e9:.1%} of the dense bf16 peak "
        "quoted at 2.4 GHz",
        f"LDS: {n_lds:.4g} instructions, index-active {lds_active:.4g} cycles per CU "
        f"({lds_active / cyc1:.1%} of the cycles), {lds_active * N_CU / max(n_lds, 1):.2f} cycles per instruction, "
        f"bank conflicts {conflicts:.4g}",
        f"waves: {wave_cyc:.4g} wave-cycles, waiting on anything {wait_any / wave_cyc:.1%}, "
        f"waiting to issue {wait_inst / wave_cyc:.1%}",
        f"VMEM (direct-to-LDS refills): {n_vmem:.4g} instructions; vector L1 stalled on pending L2 data "
        f"{tcp_pending:.4g} cycles per CU ({tcp_pending / cyc2:.1%})",
        f"VALU: {n_valu:.4g} instructions (MFMA included); MFMA busy while a VALU op issued: "
        f"{coexec:.4g} cycles per SIMD",
        f"kernel source sha256[:16]: {kernel_source_hash()}",
    ]
    with open(out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")


MOVEMENT_KERNELS = ("k_gather", "k_scatter", "k_pool")


def _short(name: str) -> str:
    for k in MOVEMENT_KERNELS:
        if f"::{k}" in name or name.startswith(k):
            return k + ("<sub>" if "k_scatter<true" in name else "")
    return ""


def _copy_scale(counter_csv: str) -> float:
    """Bytes per counted KiB, from the largest copyBuffer dispatch (the 1 GiB copy probe)."""
    best = 0.0
    for r in csv.DictReader(open(counter_csv)):
        if "copyBuffer" in r["Kernel_Name"]:
            best = max(best, float(r["Counter_Value"]))
    if not best:
        raise SystemExit(f"no copy-probe dispatch in {counter_csv}")
    return COPY_BYTES / best


def _by_grid(counter_csv: str):
    out = defaultdict(list)
    for r in csv.DictReader(open(counter_csv)):
        k = _short(r["Kernel_Name"])
        if k:
            out[(k, int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
    return out


def movement(fetch_csv: str, write_csv: str, trace_csv: str, out_txt: str, commands: str) -> None:
    """Per launch of each movement / pooling kernel, grouped by grid size
    (one group per call site in a run of bench.py that names only the
    sections it needs): HBM bytes read and written (FETCH_SIZE, WRITE_SIZE,
    each scaled by what it reads for the 1 GiB copy probe) and the median
    kernel-trace duration, hence the HBM rate the counters imply."""
    fs, ws = _copy_scale(fetch_csv), _copy_scale(write_csv)
    f, w = _by_grid(fetch_csv), _by_grid(write_csv)
    durs = defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        k = _short(r["Kernel_Name"])
        if k:
            g = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            durs[(k, g)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["# HBM traffic of the movement and pooling kernels (rocprofv3 counters), by grid size",
             f"# commands: {commands}", "",
             f"copy probe scale: FETCH_SIZE x{fs / 1024:.3f} bytes per counted byte, "
             f"WRITE_SIZE x{ws / 1024:.3f}", "",
             f"{'kernel':<14} {'grid (work-items)':>18} {'launches':>8} {'read MB':>9} {'write MB':>9} "
             f"{'med us':>8} {'GB/s':>8} {'of 8 TB/s':>9}"]
    for key in sorted(set(f) | set(w)):
        fv, wv = f.get(key, []), w.get(key, [])
        rd = sum(fv) / len(fv) * fs if fv else float("nan")
        wr = sum(wv) / len(wv) * ws if wv else float("nan")
        dl = sorted(durs.get(key, []))
        med = dl[len(dl) // 2] if dl else float("nan")
        rate = (rd + wr) / (med * 1e-6) / 1e9 if dl else float("nan")
        lines.append(f"{key[0]:<14} {key[1]:>18} {len(fv):>8} {rd / 1e6:>9.1f} {wr / 1e6:>9.1f} {med:>8.1f} "
                     f"{rate:>8.0f} {rate / 8000:>9.1%}")
    with open(out_txt, "w") as fo:
        fo.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    cmd = sys.argv[1] if len(sys.argv) > 1 else ""
    if cmd == "trace" and len(sys.argv) in (5, 6):
        trace(*sys.argv[2:])
    elif cmd == "traffic" and len(sys.argv) == 7:
        traffic(*sys.argv[2:7])
    elif cmd == "busy" and len(sys.argv) == 6:
        busy(*sys.argv[2:6])
    elif cmd == "movement" and len(sys.argv) == 7:
        movement(*sys.argv[2:7])
    else:
        print(__doc__)
        sys.exit(2)
