"""The profile summariser on small synthetic rocprofv3 CSV files (host logic
only): calibration of the traffic counters on the copy probe, and the cycle
figures of the exact-score kernel."""
import csv
import json

import pytest

from contextual_token_sparsity_amd import rocprof_summary as R

COUNTER_FIELDS = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value",
                  "Start_Timestamp", "End_Timestamp"]
SCORE = f"void (anonymous namespace)::{R.SCORE_KERNEL}(unsigned short const*, ...)"
CAUSAL = f"void (anonymous namespace)::{R.CAUSAL_KERNEL}(unsigned short const*, ...)"


def write_counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COUNTER_FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(COUNTER_FIELDS, r)))


def test_traffic_calibrates_on_the_copy_probe(tmp_path):
    # the copy probe reads half its bytes on FETCH_SIZE and all of them on
    # WRITE_SIZE; score launches of 1 MiB read and 4 KiB written (counter
    # units) scale by the same factors; a much smaller launch is left out
    fetch = [(1, "copyBuffer", 1, "FETCH_SIZE", 524288, 0, 1),
             (2, SCORE, 1, "FETCH_SIZE", 1024, 0, 1),
             (3, SCORE, 1, "FETCH_SIZE", 1024, 0, 1),
             (4, SCORE, 1, "FETCH_SIZE", 10, 0, 1),
             (5, CAUSAL, 1, "FETCH_SIZE", 512, 0, 1)]
    write = [(1, "copyBuffer", 1, "WRITE_SIZE", 1048576, 0, 1),
             (2, SCORE, 1, "WRITE_SIZE", 4, 0, 1),
             (3, SCORE, 1, "WRITE_SIZE", 4, 0, 1),
             (5, CAUSAL, 1, "WRITE_SIZE", 2, 0, 1)]
    fc, wc = tmp_path / "f.csv", tmp_path / "w.csv"
    write_counters(fc, fetch)
    write_counters(wc, write)
    out_json, out_txt = tmp_path / "t.json", tmp_path / "t.txt"
    R.traffic(str(fc), str(wc), str(out_json), str(out_txt), "cmd")
    rec = json.load(open(out_json))
    assert rec["fetch_scale"] == pytest.approx(2.0)
    assert rec["write_scale"] == pytest.approx(1.0)
    assert rec["launches"] == 2 and rec["one_head_launches_left_out"] == 1
    assert rec["fetch_bytes_per_launch"] == pytest.approx(1024 * 1024 * 2.0)
    assert rec["write_bytes_per_launch"] == pytest.approx(4 * 1024)
    assert rec["causal"]["hbm_bytes_per_launch"] == pytest.approx(512 * 1024 * 2.0 + 2 * 1024)
    assert rec["kernel_source_sha256_16"] == R.kernel_source_hash()


def test_traffic_needs_the_copy_probe(tmp_path):
    fc, wc = tmp_path / "f.csv", tmp_path / "w.csv"
    write_counters(fc, [(2, SCORE, 1, "FETCH_SIZE", 1024, 0, 1)])
    write_counters(wc, [(2, SCORE, 1, "WRITE_SIZE", 4, 0, 1)])
    with pytest.raises(SystemExit):
        R.traffic(str(fc), str(wc), str(tmp_path / "t.json"), str(tmp_path / "t.txt"), "cmd")


def test_busy_clock_and_mfma_share(tmp_path):
    # two launches of 10^6 cycles per XCD (GRBM summed over 8 XCDs) in 0.5 ms:
    # 2 GHz; MFMA busy 6 x 10^5 cycles per SIMD: 60% of the cycles, 50% of
    # the peak quoted at 2.4 GHz; LDS 4 cycles per instruction
    cyc = 1_000_000
    p1, p2 = [], []
    for d in (10, 11):
        t0, t1 = d * 10**7, d * 10**7 + 500_000          # ns
        common = (SCORE, 1)
        p1 += [(d, *common, "GRBM_GUI_ACTIVE", 8 * cyc, t0, t1),
               (d, *common, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 600_000, t0, t1),
               (d, *common, "SQ_INSTS_MFMA", 1024 * 600_000 / 32, t0, t1),
               (d, *common, "SQ_LDS_IDX_ACTIVE", 256 * 400_000, t0, t1),
               (d, *common, "SQ_INSTS_LDS", 256 * 100_000, t0, t1),
               (d, *common, "SQ_WAVE_CYCLES", 1000, t0, t1),
               (d, *common, "SQ_WAIT_ANY", 100, t0, t1),
               (d, *common, "SQ_WAIT_INST_ANY", 500, t0, t1)]
        p2 += [(d, *common, "GRBM_GUI_ACTIVE", 8 * cyc, t0, t1),
               (d, *common, "SQ_INSTS_VMEM", 1000, t0, t1),
               (d, *common, "SQ_INSTS_VALU", 2000, t0, t1),
               (d, *common, "SQ_VALU_MFMA_COEXEC_CYCLES", 1024 * 1000, t0, t1),
               (d, *common, "SQ_LDS_BANK_CONFLICT", 0, t0, t1),
               (d, *common, "TCP_PENDING_STALL_CYCLES_sum", 256 * 250_000, t0, t1)]
    # a much smaller launch of the same instantiation is left out
    p1.append((12, SCORE, 1, "GRBM_GUI_ACTIVE", 8 * 1000, 0, 1000))
    c1, c2 = tmp_path / "p1.csv", tmp_path / "p2.csv"
    write_counters(c1, p1)
    write_counters(c2, p2)
    out = tmp_path / "busy.txt"
    R.busy(str(c1), str(c2), str(out), "cmd")
    text = open(out).read()
    assert "2 + 2 launches" in text
    assert "2.00 GHz" in text
    assert "(60.0% of the launch's cycles)" in text
    assert "50.0% of the dense bf16 peak" in text
    assert "4.00 cycles per instruction" in text
    assert "waiting on anything 10.0%" in text and "waiting to issue 50.0%" in text
    assert "(25.0%)" in text


def test_busy_needs_score_dispatches(tmp_path):
    c1 = tmp_path / "p1.csv"
    write_counters(c1, [(1, "copyBuffer", 1, "GRBM_GUI_ACTIVE", 8, 0, 1)])
    with pytest.raises(SystemExit):
        R.busy(str(c1), str(c1), str(tmp_path / "o.txt"), "cmd")


def test_movement_groups_by_grid(tmp_path):
    """Movement kernels grouped by grid size: counter readings scaled by the
    copy probe, durations from the kernel trace, the scatter's subtraction
    variant kept apart."""
    G = "(anonymous namespace)::k_gather((anonymous namespace)::GatherArgs, int, ...)"
    S = "void (anonymous namespace)::k_scatter<false>(unsigned short*, int, ...)"
    SUB = "void (anonymous namespace)::k_scatter<true>(unsigned short*, int, ...)"
    fetch = [(1, "copyBuffer", 1, "FETCH_SIZE", 524288, 0, 1),
             (2, G, 100, "FETCH_SIZE", 1000, 0, 1), (3, G, 100, "FETCH_SIZE", 3000, 0, 1),
             (4, G, 200, "FETCH_SIZE", 500, 0, 1), (5, S, 100, "FETCH_SIZE", 7000, 0, 1),
             (6, SUB, 100, "FETCH_SIZE", 9000, 0, 1), (7, "other_kernel", 100, "FETCH_SIZE", 1, 0, 1)]
    write = [(1, "copyBuffer", 1, "WRITE_SIZE", 1048576, 0, 1),
             (2, G, 100, "WRITE_SIZE", 4000, 0, 1), (3, G, 100, "WRITE_SIZE", 4000, 0, 1),
             (4, G, 200, "WRITE_SIZE", 2000, 0, 1), (5, S, 100, "WRITE_SIZE", 3000, 0, 1),
             (6, SUB, 100, "WRITE_SIZE", 3000, 0, 1)]
    fc, wc, tc, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "t.csv", tmp_path / "o.txt"
    write_counters(fc, fetch)
    write_counters(wc, write)
    with open(tc, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z",
                                          "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for name, gx, gy, t in ((G, 50, 2, 2000), (G, 50, 2, 4000), (G, 50, 2, 3000), (G, 200, 1, 1000),
                                (S, 100, 1, 5000)):
            w.writerow({"Kernel_Name": name, "Grid_Size_X": gx, "Grid_Size_Y": gy, "Grid_Size_Z": 1,
                        "Start_Timestamp": 0, "End_Timestamp": t})
    R.movement(str(fc), str(wc), str(tc), str(out), "cmd")
    lines = open(out).read().splitlines()
    row = lambda k, g: next(l for l in lines if l.split()[:2] == [k, str(g)])
    # gather at grid 100: fetch avg 2000 KiB-units x 2048 B = 4.096 MB read; write 4000 x 1024 = 4.096 MB;
    # median duration 3 us -> 8.192 MB / 3 us = 2731 GB/s
    r = row("k_gather", 100).split()
    assert r[2] == "2" and r[3] == "4.1" and r[4] == "4.1" and r[5] == "3.0" and r[6] == "2731"
    assert row("k_gather", 200).split()[3] == "1.0"
    assert row("k_scatter", 100).split()[3] == "14.3"
    assert row("k_scatter<sub>", 100).split()[3] == "18.4"
    assert not any(l.startswith("other_kernel") for l in lines)


def test_trace_separates_timed_and_staged_score_launches(tmp_path):
    """Kernel-trace summary: the exact-score launches of the bench's timed steps
    and of the stage-breakdown steps after them are averaged apart, both taken
    right before the first causal launch; much smaller launches of the same
    instantiation are left out."""
    stats = tmp_path / "trace_kernel_stats.csv"
    trace_csv = tmp_path / "trace_kernel_trace.csv"
    out = tmp_path / "o.txt"
    with open(stats, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"])
        w.writeheader()
        w.writerow({"Name": SCORE, "Calls": 9, "AverageNs": 1, "MinNs": 1, "MaxNs": 1, "Percentage": 1})
    # (start, duration ns, kernel): 3 settle launches, 2 timed, 2 staged, a small
    # one-head launch of the same instantiation, then the causal launch and
    # another full launch after it
    seq = [(0, 5000, SCORE), (10, 5000, SCORE), (20, 5000, SCORE), (30, 4000, SCORE), (40, 6000, SCORE),
           (50, 100, SCORE), (60, 5000, SCORE), (70, 7000, SCORE), (80, 7000, CAUSAL), (90, 5000, SCORE)]
    with open(trace_csv, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for s, d, n in seq:
            w.writerow({"Kernel_Name": n, "Start_Timestamp": s * 1000, "End_Timestamp": s * 1000 + d})
    R.trace(str(stats), str(out), "cmd", 2)
    text = open(out).read()
    assert "1 much smaller launches left out" in text
    assert "the bench's 2 timed steps: avg 5.0 us" in text          # 4000 and 6000 ns
    assert "the 2 steps of the stage breakdown after them: avg 6.0 us" in text   # 5000 and 7000 ns
