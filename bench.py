#!/usr/bin/env python3
"""Benchmark of the token-elimination hot path on one MI355X.

One step = one pass of every stage of the hot path over one synthetic
Llama2-7B-shaped layer at N = 16384 tokens (d = 4096, 32 heads of 128,
block 64, predictor rank 128, MLP width 11008), all on one stream with no
host synchronisation inside the step:
  1. lemo_block_scores     exact block scores of Q K^T (Eq. 2 head reduction)
  2. lemo_predict_scores   predicted block scores from X (Eq. 3)
  3. lemo_select_mask      mean threshold on the predicted scores (Alg. 1 step 1)
  4. lemo_gather_pad_multi kept rows of X and of the MLP activation (one launch), padded to 256
  5. lemo_scatter_residual layer output of the kept rows added into the residual
Inputs are generated (seeded, synthetic) and resident in device memory before
the timed region.  Reported value: tokens scored + eliminated per second.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens/s scored+eliminated per layer at Llama2-7B N=16K; % MFMA / HBM peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
WORKLOAD = "llama2-7b-n16k"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "block_scores_llama2-7b-n16k_traffic.json")
CLOCK_SETTLE_S = 0.3
SECTIONS = ("c4", "movement", "copy", "chain", "select", "causal", "headmax", "mlp", "recompute", "token", "fused",
            "other_configs", "gemm_ceiling")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-full", action="store_true",
                    help="time the oracle's exact scores over every query block (minutes) instead of a sample")
    ap.add_argument("--head-reduce", choices=["paper", "headmax"], default="paper")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the exact scores at the smaller configurations (they launch the same kernel "
                         "instantiation as the step, which would mix into a profiler's per-kernel average)")
    ap.add_argument("--sections", default=",".join(SECTIONS),
                    help="comma-separated supplementary sections to run after the step (default: all of "
                         + ", ".join(SECTIONS) + "); profiled runs name only the ones they need so that each "
                         "kernel's launches come from one call site")
    args = ap.parse_args()
    args.sections = [x for x in args.sections.split(",") if x]
    unknown = set(args.sections) - set(SECTIONS)
    if unknown:
        ap.error(f"unknown sections {sorted(unknown)}")
    if args.no_other_configs and "other_configs" in args.sections:
        args.sections.remove("other_configs")
    return args


def load_traffic(causal=False):
    """HBM bytes per launch of the exact-score kernel (PAPER head reduction;
    the full-attention launch, or the causal one) from committed counter
    runs, only if they were taken on the current kernel source."""
    from contextual_token_sparsity_amd.rocprof_summary import kernel_source_hash
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    if causal:
        return (rec.get("causal") or {}).get("hbm_bytes_per_launch")
    return rec.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); sharding the path over "
              "several GPUs is a design note, not a measured configuration", file=sys.stderr)
        sys.exit(2)
    import torch
    from contextual_token_sparsity_amd import lemo, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    lemo.lib()
    w = synth.WORKLOADS[WORKLOAD]
    N, d, H, hd, b, r, wm = w.n_tokens, w.d_model, w.n_heads, w.head_dim, w.block, w.rank, w.mlp_width
    nb = N // b
    mode = lemo.REDUCE_PAPER if args.head_reduce == "paper" else lemo.REDUCE_HEADMAX
    print(f"[bench] generating {WORKLOAD} inputs", file=sys.stderr, flush=True)
    L = synth.make_layer(N, d, b, w.seed, n_heads=H, head_dim=hd, rank=r, mlp_width=wm,
                         planted_frac=w.planted_frac, proj_device="cuda")
    dev = torch.device("cuda:0")

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    q, k, x, act = up(L.q), up(L.k), up(L.x), up(L.act)
    uq, vq, uk, vk = up(L.u_q), up(L.v_q), up(L.u_k), up(L.v_k)
    resid = x.clone()
    cap = N                                        # worst case: every block kept
    y = up(synth.random_bf16(np.random.default_rng(w.seed + 7), (cap, d)))
    xk = torch.empty((cap, d), dtype=torch.int16, device=dev)
    ak = torch.empty((cap, wm), dtype=torch.int16, device=dev)
    I_exact = torch.empty(nb, dtype=torch.float32, device=dev)
    I_pred = torch.empty(nb, dtype=torch.float32, device=dev)
    ws_exact = torch.empty(lemo.lemo_block_scores_workspace(N, b), dtype=torch.uint8, device=dev)
    ws_pred = torch.empty(lemo.lemo_predict_scores_workspace(N, d, b, r), dtype=torch.uint8, device=dev)
    mask = torch.empty(nb, dtype=torch.uint8, device=dev)
    kept = torch.empty(nb, dtype=torch.int32, device=dev)
    n_kept = torch.empty(1, dtype=torch.int32, device=dev)
    theta = torch.empty(1, dtype=torch.float32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    ev = {}

    def mark(name):
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        ev.setdefault(name, []).append(e)

    # marks: 0 none, 1 around the exact scores only (the timed steps: the
    # roofline's launch duration), 2 after every stage (the stage breakdown)
    def step(marks):
        if marks:
            mark("scores0" if marks == 1 else "s_scores0")
        lemo.lemo_block_scores(q, k, H, hd, b, mode, scores=I_exact, workspace=ws_exact)
        if marks:
            mark("scores1" if marks == 1 else "scores1_staged")
        lemo.lemo_predict_scores(x, uq, vq, uk, vk, b, scores=I_pred, workspace=ws_pred)
        if marks == 2:
            mark("predict1")
        lemo.lemo_select_mask(I_pred, lemo.SELECT_MEAN, mask=mask, kept_blocks=kept, n_kept=n_kept,
                              threshold_used=theta, dev_status=status)
        if marks == 2:
            mark("select1")
        lemo.lemo_gather_pad_multi([x, act], [xk, ak], b, kept, n_kept, pad_multiple=256, dev_status=status)
        if marks == 2:
            mark("gather1")
        lemo.lemo_scatter_residual(resid, b, kept, n_kept, y, dev_status=status)
        if marks == 2:
            mark("scatter1")

    # The GPU clock ramps up under sustained load; run untimed steps for at
    # least CLOCK_SETTLE_S first so the timed steps see the steady-state clock.
    print(f"[bench] clock settle {CLOCK_SETTLE_S} s, then warmup {args.warmup}", file=sys.stderr, flush=True)
    t_settle = time.perf_counter()
    settle_steps = 0
    while time.perf_counter() - t_settle < CLOCK_SETTLE_S:
        step(0)
        torch.cuda.synchronize()
        settle_steps += 1
    for _ in range(args.warmup):
        step(0)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    host0 = time.perf_counter()
    for _ in range(args.steps):
        step(1)
    t1.record(stream)
    torch.cuda.synchronize()
    host_s = time.perf_counter() - host0
    total_ms = t0.elapsed_time(t1)
    ms_step = total_ms / args.steps
    # the other stages' times from a second pass of the same number of steps
    # with an event between stages (kept out of the timed steps above: each
    # event record adds a small gap to the stream)
    for _ in range(args.steps):
        step(2)
    torch.cuda.synchronize()

    def avg(a, b_):
        return float(np.mean([x.elapsed_time(y_) for x, y_ in zip(ev[a], ev[b_])]))

    stages = {
        "block_scores": avg("scores0", "scores1"),
        "predict_scores": avg("scores1_staged", "predict1"),
        "select_mask": avg("predict1", "select1"),
        "gather_pad_x_and_act": avg("select1", "gather1"),
        "scatter_residual": avg("gather1", "scatter1"),
    }
    nk = int(n_kept.item())
    st = int(status.item())
    flops = 2.0 * N * N * hd * H
    t_scores_s = stages["block_scores"] * 1e-3
    achieved = flops / t_scores_s / 1e12
    R = nk * b
    Rp = -(-R // 256) * 256
    # algorithmic bytes: a gathered row is read and written once, a pad row
    # written once; a scattered row reads residual and y and writes residual
    bytes_gx = 2 * R * d * 2 + (Rp - R) * d * 2
    bytes_ga = 2 * R * wm * 2 + (Rp - R) * wm * 2
    bytes_sc = 3 * R * d * 2
    move_bytes = bytes_gx + bytes_ga + bytes_sc
    warm_ms = {"gather_x_and_act": stages["gather_pad_x_and_act"], "scatter": stages["scatter_residual"]}
    out = {
        "metric": METRIC,
        "value": N * args.steps / (total_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "Llama2-7B-shaped layer, N=16384, d=4096, 32 heads x 128, block 64: exact block "
                        "scores + predictor (rank 128) + mean-threshold select + gather of X and of the MLP "
                        "activation (11008) padded to 256 + in-place residual add",
            "n_tokens": N, "d_model": d, "n_heads": H, "head_dim": hd, "block": b, "rank": r,
            "mlp_width": wm, "head_reduce": args.head_reduce, "select": "mean",
        },
        "roofline": {
            "kernel": "lemo_block_scores (k_block_scores_pp + column sum)",
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": load_traffic() if mode == lemo.REDUCE_PAPER else None,
        },
        "stages_ms": stages,
        "n_kept_blocks": nk,
        "movement_GBps": move_bytes / ((stages["gather_pad_x_and_act"] + stages["scatter_residual"]) * 1e-3) / 1e9,
        "movement_in_step": {
            "gather_x_and_act": {"bytes": bytes_gx + bytes_ga,
                                 "GBps": (bytes_gx + bytes_ga) / (warm_ms["gather_x_and_act"] * 1e-3) / 1e9},
            "scatter": {"bytes": bytes_sc, "GBps": bytes_sc / (warm_ms["scatter"] * 1e-3) / 1e9}},
        "predictor_path_tokens_per_s": N / (sum(v for kk, v in stages.items() if kk != "block_scores") * 1e-3),
        "device": {"name": torch.cuda.get_device_name(dev),
                   "compute_units": torch.cuda.get_device_properties(dev).multi_processor_count},
        "dev_status": st,
        "host_wall_s": host_s,
        "clock_settle_steps": settle_steps,
    }
    sec = args.sections
    if "movement" in sec or "copy" in sec:
        out["movement"] = movement_streaming(x, act, y, kept, n_kept, nk, N, d, wm, b, stream, dev,
                                             calls=("movement" in sec, "copy" in sec))
    if "chain" in sec:
        out["chain_13b"] = chain_13b(stream, dev)
    if "select" in sec:
        out["select_topk"] = select_latency(stream, dev, "topk")
        out["select_mean"] = select_latency(stream, dev, "mean")
    if "causal" in sec:
        out["causal_scores"] = causal_scores(q, k, N, H, hd, b, mode, stream, dev)
    if "headmax" in sec:
        out["other_head_reduce"] = other_head_reduce(q, k, N, H, hd, b, mode, stream, dev)
    if "mlp" in sec:
        out["mlp_scores"] = mlp_scores(act, N, wm, b, stream, dev)
    if "recompute" in sec:
        out["residual_recompute"] = recompute(resid, y, kept, n_kept, nk, d, b, stream)
    if "c4" in sec:
        out["c4_predictor_path"] = c4_predictor_path(
            x, act, (uq, vq, uk, vk), resid, y, (xk, ak), (I_pred, ws_pred, mask, kept, n_kept, theta, status),
            N, b, stream, dev)
    if "token" in sec:
        out["token_predictor"] = token_predictor(x, uq, vq, uk, vk, N, d, b, r, stream, dev)
    if "fused" in sec:
        out["fused_movement"] = fused_movement(x, resid, kept, n_kept, nk, N, d, b, stream, dev)
    if "other_configs" in sec:
        out["exact_scores_other_configs"] = exact_scores_other_configs(mode, stream, dev)
    if "gemm_ceiling" in sec:
        out["library_gemm_ceiling"] = library_gemm_ceiling(stream, dev)
        # the exact-score kernel's rate against the vendor GEMM's on the same box
        out["block_scores_vs_library_gemm"] = achieved / out["library_gemm_ceiling"]["TFLOPs"]
    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        dst.copy_(src)
        c1.record(stream)
        torch.cuda.synchronize()
        out["copy_probe_GBps"] = 2.0 * (1 << 30) / (c0.elapsed_time(c1) * 1e-3) / 1e9
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(L, w, full=args.cpu_full)
    print(json.dumps(out), flush=True)


SECTION_SETTLE_S = 0.15


def _settle(fn):
    """Runs `fn` for SECTION_SETTLE_S seconds before a section is timed, so
    that every figure is taken at the clock the chip holds under that
    section's own sustained load (a short burst after the host-side gaps
    between sections runs at a different clock)."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < SECTION_SETTLE_S:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


def causal_scores(q, k, N, H, hd, b, mode, stream, dev, reps=10):
    """The causal variant of the exact scores on the same Q and K
    (lemo_block_scores_batched with the causal flag: only the tiles on or
    below the diagonal are launched).  Algorithmic work: the N (N - 1) / 2
    pairs j < i, 2 hd flops per pair and head.  Mean event times over `reps`
    calls after 3 warm-up calls."""
    import torch
    from contextual_token_sparsity_amd import lemo
    nb = N // b
    I = torch.empty((1, nb), dtype=torch.float32, device=dev)
    ws = torch.empty(lemo.lemo_block_scores_batched_workspace(1, N, b), dtype=torch.uint8, device=dev)
    _settle(lambda: lemo.lemo_block_scores_batched(q, k, H, hd, b, mode, causal=True, scores=I, workspace=ws))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps + 3)]
    for i in range(reps + 3):
        ev[i][0].record(stream)
        lemo.lemo_block_scores_batched(q, k, H, hd, b, mode, causal=True, scores=I, workspace=ws)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    t = float(np.mean([e[0].elapsed_time(e[1]) for e in ev[3:]]))
    flops = 2.0 * hd * H * N * (N - 1) / 2
    tf = flops / (t * 1e-3) / 1e12
    return {"ms": t, "TFLOPs": tf, "frac": tf / PEAK_BF16_TFLOPS, "tokens_per_s": N / (t * 1e-3),
            "traffic": load_traffic(causal=True) if mode == lemo.REDUCE_PAPER else None}


def other_head_reduce(q, k, N, H, hd, b, mode, stream, dev):
    """The exact scores with the other head reduction (HEADMAX when the step
    uses PAPER, and the reverse) on the same Q and K: mean event time of 10
    calls after a clock-settle phase, TFLOP/s and fraction of the bf16 peak."""
    import torch
    from contextual_token_sparsity_amd import lemo
    other = lemo.REDUCE_HEADMAX if mode == lemo.REDUCE_PAPER else lemo.REDUCE_PAPER
    I = torch.empty(N // b, dtype=torch.float32, device=dev)
    ws = torch.empty(lemo.lemo_block_scores_workspace(N, b), dtype=torch.uint8, device=dev)
    t = _mean_ms(lambda: lemo.lemo_block_scores(q, k, H, hd, b, other, scores=I, workspace=ws), stream)
    tf = 2.0 * N * N * hd * H / (t * 1e-3) / 1e12
    return {"head_reduce": "headmax" if other == lemo.REDUCE_HEADMAX else "paper", "ms": t, "TFLOPs": tf,
            "frac": tf / PEAK_BF16_TFLOPS, "tokens_per_s": N / (t * 1e-3)}


def exact_scores_other_configs(mode, stream, dev):
    """The exact scores at the two smaller exact-scoring configurations
    (Llama2-7B at N = 8192, and OPT-1.3B at N = 4096 with 32 heads of 64),
    on seeded random bf16 Q and K of those shapes (the work does not depend on
    the values): mean event time of 10 calls after a clock-settle phase, flops
    2 N^2 hd H, and the fraction of the bf16 peak."""
    import torch
    from contextual_token_sparsity_amd import lemo, synth
    res = {}
    for name in ("llama2-7b-n8k-exact", "opt1.3b-n4k"):
        w = synth.WORKLOADS[name]
        N, H, hd, b = w.n_tokens, w.n_heads, w.head_dim, w.block
        g = torch.Generator(device=dev).manual_seed(w.seed)
        q = torch.randn(N, H * hd, device=dev, generator=g).to(torch.bfloat16)
        k = torch.randn(N, H * hd, device=dev, generator=g).to(torch.bfloat16)
        I = torch.empty(N // b, dtype=torch.float32, device=dev)
        ws = torch.empty(lemo.lemo_block_scores_workspace(N, b), dtype=torch.uint8, device=dev)
        t = _mean_ms(lambda: lemo.lemo_block_scores(q, k, H, hd, b, mode, scores=I, workspace=ws), stream)
        tf = 2.0 * N * N * hd * H / (t * 1e-3) / 1e12
        res[name] = {"n_tokens": N, "n_heads": H, "head_dim": hd, "block": b, "ms": t, "TFLOPs": tf,
                     "frac": tf / PEAK_BF16_TFLOPS, "tokens_per_s": N / (t * 1e-3)}
        del q, k, ws
    return res


def _mean_ms(fn, stream, reps=10, warm=3):
    import torch
    _settle(fn)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps + warm)]
    for e in ev:
        e[0].record(stream)
        fn()
        e[1].record(stream)
    torch.cuda.synchronize()
    return float(np.mean([e[0].elapsed_time(e[1]) for e in ev[warm:]]))


def mlp_scores(act, N, wm, b, stream, dev):
    """MLP-block token scores on the layer's MLP activation [N][wm] (one pass
    over it), and the SiLU-gated form from a gate and an up projection of the
    same shape (two passes' worth of bytes).  Algorithmic bytes: every
    activation element read once, 2 B each."""
    import torch
    from contextual_token_sparsity_amd import lemo, synth
    I = torch.empty(-(-N // b), dtype=torch.float32, device=dev)
    ws = torch.empty(lemo.lemo_mlp_block_scores_workspace(N, wm, b), dtype=torch.uint8, device=dev)
    upj = torch.from_numpy(synth.random_bf16(np.random.default_rng(99), (N, wm)).view(np.int16)).to(dev)
    t = _mean_ms(lambda: lemo.lemo_mlp_block_scores(act, b, scores=I, workspace=ws), stream)
    tg = _mean_ms(lambda: lemo.lemo_mlp_block_scores_gated(act, upj, b, scores=I, workspace=ws), stream)
    by = 2.0 * N * wm
    return {"ms": t, "GBps": by / (t * 1e-3) / 1e9, "frac": by / (t * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "gated_ms": tg, "gated_GBps": 2 * by / (tg * 1e-3) / 1e9,
            "gated_frac": 2 * by / (tg * 1e-3) / 1e9 / PEAK_HBM_GBS}


def recompute(resid, y, kept, n_kept, nk, d, b, stream):
    """Backward recompute of the layer input on the step's mask (the kept
    rows of the residual minus the layer output), the mirror of the in-place
    addition: 3 w 2 B per kept row."""
    from contextual_token_sparsity_amd import lemo
    t = _mean_ms(lambda: lemo.lemo_residual_recompute(resid, b, kept, n_kept, y), stream)
    by = 3.0 * nk * b * d * 2
    return {"ms": t, "GBps": by / (t * 1e-3) / 1e9, "frac": by / (t * 1e-3) / 1e9 / PEAK_HBM_GBS}


def c4_predictor_path(x, act, wts, resid, y, outs, bufs, N, b, stream, dev, iters=100, warm=10):
    """The online layer the predictor drives (predicted scores -> MEAN select
    -> gather of X and of the MLP activation in one launch -> in-place
    addition), timed as one event pair around the whole sequence with no host
    synchronisation inside, per iteration: `warm` untimed iterations, then
    `iters` timed ones; median and minimum.  "warm": back to back; "cold": the
    256 MB Infinity Cache is flushed before each iteration by writing a
    512 MiB scratch buffer (outside the event pair).  Also without the
    MLP-activation gather (X only).  tokens/s = N / time."""
    import torch
    from contextual_token_sparsity_amd import lemo
    uq, vq, uk, vk = wts
    xk, ak = outs
    I_pred, ws_pred, mask, kept, n_kept, theta, status = bufs
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def seq(with_act):
        lemo.lemo_predict_scores(x, uq, vq, uk, vk, b, scores=I_pred, workspace=ws_pred)
        lemo.lemo_select_mask(I_pred, lemo.SELECT_MEAN, mask=mask, kept_blocks=kept, n_kept=n_kept,
                              threshold_used=theta, dev_status=status)
        if with_act:
            lemo.lemo_gather_pad_multi([x, act], [xk, ak], b, kept, n_kept, pad_multiple=256, dev_status=status)
        else:
            lemo.lemo_gather_pad(x, b, kept, n_kept, xk, pad_multiple=256, dev_status=status)
        lemo.lemo_scatter_residual(resid, b, kept, n_kept, y, dev_status=status)

    res = {"iters": iters}
    for with_act in (True, False):
        for cold in (False, True):
            for _ in range(warm):
                if cold:
                    scratch.zero_()
                seq(with_act)
            evs = []
            for _ in range(iters):
                if cold:
                    scratch.zero_()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                seq(with_act)
                e1.record(stream)
                evs.append((e0, e1))
            torch.cuda.synchronize()
            t = np.array([a.elapsed_time(b_) for a, b_ in evs]) * 1e3      # us
            key = ("with" if with_act else "without") + "_mlp_gather_" + ("cold" if cold else "warm")
            res[key] = {"median_us": float(np.median(t)), "min_us": float(t.min()),
                        "tokens_per_s_median": N / (float(np.median(t)) * 1e-6)}
    del scratch
    return res


def token_predictor(x, uq, vq, uk, vk, N, d, b, r, stream, dev, reps=10):
    """The per-token predictor variant on the same layer: embeddings of every
    token (lemo_token_embeddings) scored by the exact-score kernel as one head
    of width r.  Mean event times over `reps` calls after 3 warm-up calls."""
    import torch
    from contextual_token_sparsity_amd import lemo
    nb = N // b
    q_hat = torch.empty((N, r), dtype=torch.int16, device=dev)
    k_hat = torch.empty((N, r), dtype=torch.int16, device=dev)
    ws = torch.empty(lemo.lemo_token_embeddings_workspace(N, d, r), dtype=torch.uint8, device=dev)
    I = torch.empty(nb, dtype=torch.float32, device=dev)
    ws_s = torch.empty(lemo.lemo_block_scores_workspace(N, b), dtype=torch.uint8, device=dev)

    def both():
        lemo.lemo_token_embeddings(x, uq, vq, uk, vk, q_hat=q_hat, k_hat=k_hat, workspace=ws)
        lemo.lemo_block_scores(q_hat, k_hat, 1, r, b, lemo.REDUCE_PAPER, scores=I, workspace=ws_s)
    _settle(both)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps + 3)]
    for i in range(reps + 3):
        ev[i][0].record(stream)
        lemo.lemo_token_embeddings(x, uq, vq, uk, vk, q_hat=q_hat, k_hat=k_hat, workspace=ws)
        ev[i][1].record(stream)
        lemo.lemo_block_scores(q_hat, k_hat, 1, r, b, lemo.REDUCE_PAPER, scores=I, workspace=ws_s)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    t_e = float(np.mean([e[0].elapsed_time(e[1]) for e in ev[3:]]))
    t_s = float(np.mean([e[1].elapsed_time(e[2]) for e in ev[3:]]))
    f_e = 2.0 * N * d * 2 * r + 2.0 * 2 * N * r * r
    f_s = 2.0 * N * N * r
    return {"embeddings_ms": t_e, "scores_ms": t_s,
            "embeddings_TFLOPs": f_e / (t_e * 1e-3) / 1e12, "scores_TFLOPs": f_s / (t_s * 1e-3) / 1e12,
            "tokens_per_s": N / ((t_e + t_s) * 1e-3)}


def library_gemm_ceiling(stream, dev, n=8192, reps=10):
    """The vendor library's bf16 product (torch.mm, hipBLASLt) on random
    normal operands at n x n x n: what a tuned dense kernel sustains on this
    part once real data drives the matrix units and the clock settles under
    that load (a reference point for the MFMA kernels' fractions, not part of
    the path).  Mean event time over `reps` calls after a 0.3 s settle."""
    import torch
    g = torch.Generator(device=dev).manual_seed(321)
    a = torch.randn(n, n, device=dev, generator=g).to(torch.bfloat16)
    b_ = torch.randn(n, n, device=dev, generator=g).to(torch.bfloat16)
    c = torch.empty(n, n, dtype=torch.bfloat16, device=dev)
    t = time.perf_counter()
    while time.perf_counter() - t < CLOCK_SETTLE_S:
        torch.mm(a, b_, out=c)
        torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        torch.mm(a, b_, out=c)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    return {"shape": [n, n, n], "ms": ms, "TFLOPs": tf, "frac": tf / PEAK_BF16_TFLOPS}


def fused_movement(x, resid, kept, n_kept, nk, N, d, b, stream, dev, reps=10):
    """Token movement fused into the layer's products on the same layer and
    mask: the kept-row gather feeding a d x d projection (lemo_gather_linear)
    and a d x d projection added back into the residual stream
    (lemo_linear_scatter), each against the stand-alone movement call plus the
    same product, and the gather against the stand-alone gather plus the vendor
    library's product (torch.mm, hipBLASLt) as a reference point.  Mean event
    times over `reps` calls after a clock-settle phase."""
    import torch
    from contextual_token_sparsity_amd import lemo
    R = nk * b
    cap = -(-R // 256) * 256
    g = torch.Generator(device=dev).manual_seed(123)
    w = (torch.randn(d, d, device=dev, generator=g) / d ** 0.5).to(torch.bfloat16)
    a = torch.randn(cap, d, device=dev, generator=g).to(torch.bfloat16)
    y = torch.empty((cap, d), dtype=torch.int16, device=dev)
    xg = torch.empty((cap, d), dtype=torch.int16, device=dev)
    y2 = torch.empty((R, d), dtype=torch.int16, device=dev)
    ident = torch.arange(cap // b, dtype=torch.int32, device=dev)

    def gather_fused():
        lemo.lemo_gather_linear(x, b, kept, n_kept, w, y, pad_multiple=256)

    def gather_unfused():
        lemo.lemo_gather_pad(x, b, kept, n_kept, xg, pad_multiple=256)
        lemo.lemo_gather_linear(xg, b, ident, n_kept, w, y, pad_multiple=256, n_tokens=cap)

    xgb = xg.view(torch.bfloat16)
    yb = torch.empty((cap, d), dtype=torch.bfloat16, device=dev)
    wt = w.t().contiguous()                     # [in][out]: a plain row-major product

    def gather_then_library():
        lemo.lemo_gather_pad(x, b, kept, n_kept, xg, pad_multiple=256)
        torch.mm(xgb, wt, out=yb)

    def scatter_fused():
        lemo.lemo_linear_scatter(a[:R], w, resid, b, kept, n_kept)

    def scatter_unfused():
        lemo.lemo_gather_linear(a[:R], b, ident, n_kept, w, y2, n_tokens=R)
        lemo.lemo_scatter_residual(resid, b, kept, n_kept, y2)

    res = {}
    for name, fn in (("gather_linear", gather_fused), ("gather_then_linear", gather_unfused),
                     ("gather_then_library_linear", gather_then_library),
                     ("linear_scatter", scatter_fused), ("linear_then_scatter", scatter_unfused)):
        _settle(fn)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name + "_ms"] = e0.elapsed_time(e1) / reps
    flops = 2.0 * R * d * d
    res["kept_rows"] = R
    res["gather_linear_TFLOPs"] = flops / (res["gather_linear_ms"] * 1e-3) / 1e12
    res["linear_scatter_TFLOPs"] = flops / (res["linear_scatter_ms"] * 1e-3) / 1e12
    return res


def movement_streaming(x, act, y, kept, n_kept, nk, N, d, wm, b, stream, dev, reps=30, calls=(True, True)):
    """Each movement call on the step's mask, launched back to back `reps`
    times with the source rotated over three copies (so every launch reads
    data it last touched two launches earlier, more than the 256 MB Infinity
    Cache ago: the reads stream from HBM).  Mean event time per call;
    algorithmic bytes as in the step (a gathered row read and written once, a
    pad row written once, a scattered row read twice and written once).
    `copy_ceiling` is the same gather kernel on a keep-all list: a plain
    contiguous copy of X, the streaming-copy rate this part reaches with these
    kernels, beside torch's device-to-device copy of the same bytes."""
    import torch
    from contextual_token_sparsity_amd import lemo
    R = nk * b
    Rp = -(-R // 256) * 256
    xs = [x] + [x.clone() for _ in range(2)]
    acts = [act] + [act.clone() for _ in range(2)]
    res = [x.clone() for _ in range(3)]
    xk = torch.empty((Rp, d), dtype=torch.int16, device=dev)
    ak = torch.empty((Rp, wm), dtype=torch.int16, device=dev)
    want_moves, want_copy = calls
    calls = {} if not want_moves else {
        "gather_x": (2 * R * d * 2 + (Rp - R) * d * 2,
                     lambda c: lemo.lemo_gather_pad(xs[c], b, kept, n_kept, xk, pad_multiple=256)),
        "gather_act": (2 * R * wm * 2 + (Rp - R) * wm * 2,
                       lambda c: lemo.lemo_gather_pad(acts[c], b, kept, n_kept, ak, pad_multiple=256)),
        "gather_x_and_act": (2 * R * (d + wm) * 2 + (Rp - R) * (d + wm) * 2,
                             lambda c: lemo.lemo_gather_pad_multi([xs[c], acts[c]], [xk, ak], b, kept, n_kept,
                                                                  pad_multiple=256)),
        "scatter": (3 * R * d * 2, lambda c: lemo.lemo_scatter_residual(res[c], b, kept, n_kept, y)),
    }
    all_kept = torch.arange(N // b, dtype=torch.int32, device=dev)
    n_all = torch.tensor([N // b], dtype=torch.int32, device=dev)
    xcopy = torch.empty_like(x)
    if want_copy:
        calls["copy_ceiling"] = (2 * N * d * 2, lambda c: lemo.lemo_gather_pad(xs[c], b, all_kept, n_all, xcopy))
        calls["torch_copy"] = (2 * N * d * 2, lambda c: xcopy.copy_(xs[c]))
    out = {}
    for name, (by, fn) in calls.items():
        for c in range(6):
            fn(c % 3)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            fn(i % 3)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        gbps = by / (ms * 1e-3) / 1e9
        out[name] = {"bytes": int(by), "us": ms * 1e3, "GBps": gbps, "frac": gbps / PEAK_HBM_GBS}
    del xs, acts, res, xcopy
    return out


def chain_13b(stream, dev, reps=5):
    """The Llama2-13B-shaped four-layer chain (N = 32768, d = 5120, blocks of
    128, predictor rank 256) on one stream with no host synchronisation: per
    layer, predicted scores of the current residual stream, top-k select
    (keep 60 / 45 / 35 / 25 %), gather of the kept rows (the layer's input),
    and in-place addition of a stand-in layer output.  Inputs are seeded
    Gaussian tensors drawn on the device (the work does not depend on the
    values: top-k fixes the kept count).  The chain time is the event time of
    `reps` chains without events between stages; per-layer stage times are
    mean event times over `reps` further chains with an event after each stage
    (`chain_us_with_stage_events` is their sum); algorithmic bytes: the predictor reads X
    once (plus its weights), the gather moves 2 R d 2 B, the scatter 3 R d 2 B;
    the ideal time is the total at 8 TB/s."""
    import torch
    from contextual_token_sparsity_amd import lemo, synth
    w = synth.WORKLOADS["llama2-13b-n32k-4layer"]
    N, d, b, r = w.n_tokens, w.d_model, w.block, w.rank
    nb = N // b
    g = torch.Generator(device=dev).manual_seed(w.seed)
    resid = torch.randn(N, d, device=dev, generator=g).to(torch.bfloat16)
    layers = []
    for _ in w.keep_pct:
        wt = [(torch.randn(*s_, device=dev, generator=g) / s_[0] ** 0.5).to(torch.bfloat16)
              for s_ in ((d, r), (r, r), (d, r), (r, r))]
        yl = torch.randn(N, d, device=dev, generator=g).to(torch.bfloat16)
        layers.append((wt, yl))
    I = torch.empty(nb, dtype=torch.float32, device=dev)
    ws = torch.empty(lemo.lemo_predict_scores_workspace(N, d, b, r), dtype=torch.uint8, device=dev)
    mask = torch.empty(nb, dtype=torch.uint8, device=dev)
    kept = torch.empty(nb, dtype=torch.int32, device=dev)
    n_kept = torch.empty(1, dtype=torch.int32, device=dev)
    theta = torch.empty(1, dtype=torch.float32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    xin = torch.empty((N, d), dtype=torch.bfloat16, device=dev)
    ks = [synth.keep_count(p, nb) for p in w.keep_pct]
    ev = {}

    def mark(key):
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        ev.setdefault(key, []).append(e)

    def chain(timed):
        if timed:
            mark("start")
        for li, ((wt, yl), k) in enumerate(zip(layers, ks)):
            lemo.lemo_predict_scores(resid, *wt, b, scores=I, workspace=ws)
            if timed:
                mark((li, "predict"))
            lemo.lemo_select_mask(I, lemo.SELECT_TOPK, keep_blocks=k, mask=mask, kept_blocks=kept, n_kept=n_kept,
                                  threshold_used=theta, dev_status=status)
            if timed:
                mark((li, "select"))
            lemo.lemo_gather_pad(resid, b, kept, n_kept, xin, dev_status=status)
            if timed:
                mark((li, "gather"))
            lemo.lemo_scatter_residual(resid, b, kept, n_kept, yl, dev_status=status)
            if timed:
                mark((li, "scatter"))

    _settle(lambda: chain(False))
    # the whole chain without events between its stages, then the same number
    # of chains with them for the per-stage times
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(reps):
        chain(False)
    c1.record(stream)
    for _ in range(reps):
        chain(True)
    torch.cuda.synchronize()
    chain_ms = c0.elapsed_time(c1) / reps

    def span(a, b_):
        return float(np.mean([x_.elapsed_time(y_) for x_, y_ in zip(ev[a], ev[b_])]))

    prev = "start"
    layers_out = []
    total_bytes = 0
    weights_bytes = 2 * (2 * d * r + 2 * r * r)
    for li, k in enumerate(ks):
        R = k * b
        by = {"predict": N * d * 2 + weights_bytes, "gather": 2 * R * d * 2, "scatter": 3 * R * d * 2}
        t = {}
        for st_ in ("predict", "select", "gather", "scatter"):
            t[st_] = span(prev, (li, st_))
            prev = (li, st_)
        total_bytes += sum(by.values())
        layers_out.append({
            "keep_pct": w.keep_pct[li], "kept_blocks": k, "us": {kk: v * 1e3 for kk, v in t.items()},
            "GBps": {kk: by[kk] / (t[kk] * 1e-3) / 1e9 for kk in by},
            "frac": {kk: by[kk] / (t[kk] * 1e-3) / 1e9 / PEAK_HBM_GBS for kk in by}})
    staged_ms = span("start", (len(ks) - 1, "scatter"))
    ideal_us = total_bytes / (PEAK_HBM_GBS * 1e9) * 1e6
    st = int(status.item())
    del layers, resid, xin
    return {"workload": "Llama2-13B-shaped, 4 layers: N=32768, d=5120, block 128, rank 256, top-k 60/45/35/25%",
            "chain_us": chain_ms * 1e3, "chain_us_with_stage_events": staged_ms * 1e3, "bytes": int(total_bytes),
            "ideal_us_at_8TBps": ideal_us, "frac_of_ideal": ideal_us / (chain_ms * 1e3),
            "token_layers_per_s": 4 * N / (chain_ms * 1e-3), "layers": layers_out, "dev_status": st}


def select_latency(stream, dev, mode):
    """Latency of the select at 256 and 8192 blocks on seeded random scores:
    top-k keeping 30 %, or the mean threshold; mean event time of 20 calls
    after a settle phase."""
    import torch
    from contextual_token_sparsity_amd import lemo, synth
    out = {}
    for nb in (256, 8192):
        g = torch.Generator(device=dev).manual_seed(nb)
        s_ = torch.rand(nb, device=dev, generator=g)
        bufs = (torch.empty(nb, dtype=torch.uint8, device=dev), torch.empty(nb, dtype=torch.int32, device=dev),
                torch.empty(1, dtype=torch.int32, device=dev), torch.empty(1, dtype=torch.float32, device=dev))
        if mode == "topk":
            sel, kw = lemo.SELECT_TOPK, {"keep_blocks": synth.keep_count(30, nb)}
        else:
            sel, kw = lemo.SELECT_MEAN, {}
        t = _mean_ms(lambda: lemo.lemo_select_mask(s_, sel, mask=bufs[0], kept_blocks=bufs[1], n_kept=bufs[2],
                                                   threshold_used=bufs[3], **kw),
                     stream, reps=20)
        out[f"nb{nb}_us"] = t * 1e3
    return out


def cpu_baseline(L, w, full=False):
    """The oracle on the host cores, timed per stage at the step's boundaries
    on a bounded sample of one step: exact scores for `s` of the nb query
    blocks against every key block (one run, scaled up by nb / s; with
    `full`, all of them once), then the full predictor, select, gather of X,
    gather of the MLP activation and scatter (median of 3 runs each).  Beside it, the whole exact-score oracle at
    the two smaller exact configurations (1024 tokens: median of 3 runs;
    OPT-1.3B at 4096 tokens: one run)."""
    from oracle import lemo_oracle as O
    from contextual_token_sparsity_amd import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [os.cpu_count()])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    nb = w.n_blocks
    s = nb if full else 8
    print(f"[bench] cpu baseline: oracle on {s}/{nb} query blocks + full predictor/movement", file=sys.stderr,
          flush=True)
    stages = {}

    def timed(name, fn, scale=1.0, runs=3):
        ts = []
        for _ in range(runs):
            t = time.perf_counter()
            r = fn()
            ts.append(time.perf_counter() - t)
        stages[name] = float(np.median(ts)) * scale
        return r

    timed("exact_scores", lambda: O.exact_block_scores(L.q, L.k, w.n_heads, w.head_dim, w.block, O.REDUCE_PAPER,
                                                        query_blocks=list(range(0, nb, nb // s))[:s]),
          nb / s, runs=1)
    _, I_hat, _, _ = timed("predict_scores", lambda: O.predict_scores(L.x, L.u_q, L.v_q, L.u_k, L.v_k, w.block))
    _, kept, nk, _ = timed("select_mask", lambda: O.select_mask(I_hat.astype(np.float32), O.SELECT_MEAN))
    R = nk * w.block
    cap = -(-R // 256) * 256
    timed("gather_x", lambda: O.gather_pad(L.x, w.block, kept, nk, np.zeros((cap, w.d_model), np.uint16), 256))
    timed("gather_act", lambda: O.gather_pad(L.act, w.block, kept, nk, np.zeros((cap, w.mlp_width), np.uint16), 256))
    y = L.y[O.kept_token_rows(kept, nk, w.block)]
    timed("scatter_residual", lambda: O.scatter_residual(L.x, w.block, kept, nk, y))
    t_step = sum(stages.values())
    small = {}
    for name, runs in (("tiny", 3), ("opt1.3b-n4k", 1)):
        sw = synth.WORKLOADS[name]
        Ls = synth.make_layer(sw.n_tokens, sw.d_model, sw.block, sw.seed, n_heads=sw.n_heads,
                              head_dim=sw.head_dim, planted_frac=sw.planted_frac, with_y=False)
        ts = []
        for _ in range(runs):
            t = time.perf_counter()
            O.exact_block_scores(Ls.q, Ls.k, sw.n_heads, sw.head_dim, sw.block, O.REDUCE_PAPER)
            ts.append(time.perf_counter() - t)
        med = float(np.median(ts))
        small[name] = {"exact_scores_s": med, "runs": runs, "tokens_per_s": sw.n_tokens / med}
    return {
        "value": w.n_tokens / t_step,
        "unit": "tokens/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"exact scores of {s} of {nb} query blocks" + (f" (x{nb // s})" if s < nb else "") +
                   f" + full predictor, mean select, gathers and scatter; est. step {t_step:.1f} s"),
        "stages_s": stages,
        "exact_scores_small_configs": small,
    }


if __name__ == "__main__":
    main()
