#!/usr/bin/env python3
"""Benchmark of the token-elimination hot path on one MI355X.

One step = one pass of every stage of the hot path over one synthetic
Llama2-7B-shaped layer at N = 16384 tokens (d = 4096, 32 heads of 128,
block 64, predictor rank 128, MLP width 11008), all on one stream with no
host synchronisation inside the step:
  1. lemo_block_scores     exact block scores of Q K^T (Eq. 2 head reduction)
  2. lemo_predict_scores   predicted block scores from X (Eq. 3)
  3. lemo_select_mask      mean threshold on the predicted scores (Alg. 1 step 1)
  4. lemo_gather_pad x2    kept rows of X and of the MLP activation, padded to 256
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--head-reduce", choices=["paper", "headmax"], default="paper")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the exact scores at the smaller configurations (they launch the same kernel "
                         "instantiation as the step, which would mix into a profiler's per-kernel average)")
    return ap.parse_args()


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

    def step(timed):
        if timed:
            mark("scores0")
        lemo.lemo_block_scores(q, k, H, hd, b, mode, scores=I_exact, workspace=ws_exact)
        if timed:
            mark("scores1")
        lemo.lemo_predict_scores(x, uq, vq, uk, vk, b, scores=I_pred, workspace=ws_pred)
        if timed:
            mark("predict1")
        lemo.lemo_select_mask(I_pred, lemo.SELECT_MEAN, mask=mask, kept_blocks=kept, n_kept=n_kept,
                              threshold_used=theta, dev_status=status)
        if timed:
            mark("select1")
        lemo.lemo_gather_pad(x, b, kept, n_kept, xk, pad_multiple=256, dev_status=status)
        if timed:
            mark("gatherx1")
        lemo.lemo_gather_pad(act, b, kept, n_kept, ak, pad_multiple=256, dev_status=status)
        if timed:
            mark("gather1")
        lemo.lemo_scatter_residual(resid, b, kept, n_kept, y, dev_status=status)
        if timed:
            mark("scatter1")

    # The GPU clock ramps up under sustained load; run untimed steps for at
    # least CLOCK_SETTLE_S first so the timed steps see the steady-state clock.
    print(f"[bench] clock settle {CLOCK_SETTLE_S} s, then warmup {args.warmup}", file=sys.stderr, flush=True)
    t_settle = time.perf_counter()
    settle_steps = 0
    while time.perf_counter() - t_settle < CLOCK_SETTLE_S:
        step(False)
        torch.cuda.synchronize()
        settle_steps += 1
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    host0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    t1.record(stream)
    torch.cuda.synchronize()
    host_s = time.perf_counter() - host0
    total_ms = t0.elapsed_time(t1)
    ms_step = total_ms / args.steps

    def avg(a, b_):
        return float(np.mean([x.elapsed_time(y_) for x, y_ in zip(ev[a], ev[b_])]))

    stages = {
        "block_scores": avg("scores0", "scores1"),
        "predict_scores": avg("scores1", "predict1"),
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
    warm_ms = {"gather_x": avg("select1", "gatherx1"), "gather_act": avg("gatherx1", "gather1"),
               "scatter": stages["scatter_residual"]}
    cold_ms = movement_cold(lambda: lemo.lemo_gather_pad(x, b, kept, n_kept, xk, pad_multiple=256),
                            lambda: lemo.lemo_gather_pad(act, b, kept, n_kept, ak, pad_multiple=256),
                            lambda: lemo.lemo_scatter_residual(resid, b, kept, n_kept, y), stream, dev)
    move_bytes_k = {"gather_x": bytes_gx, "gather_act": bytes_ga, "scatter": bytes_sc}
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
            "kernel": "lemo_block_scores (k_block_scores + column sum)",
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
        "movement": {
            kname: {"bytes": move_bytes_k[kname],
                    "warm_GBps": move_bytes_k[kname] / (warm_ms[kname] * 1e-3) / 1e9,
                    "cold_GBps": move_bytes_k[kname] / (cold_ms[kname] * 1e-3) / 1e9,
                    "cold_frac": move_bytes_k[kname] / (cold_ms[kname] * 1e-3) / 1e9 / PEAK_HBM_GBS}
            for kname in ("gather_x", "gather_act", "scatter")},
        "predictor_path_tokens_per_s": N / (sum(v for kk, v in stages.items() if kk != "block_scores") * 1e-3),
        "tokens_per_s_without_mlp_gather": N / ((ms_step - warm_ms["gather_act"]) * 1e-3),
        "dev_status": st,
        "host_wall_s": host_s,
        "clock_settle_steps": settle_steps,
    }
    out["causal_scores"] = causal_scores(q, k, N, H, hd, b, mode, stream, dev)
    out["other_head_reduce"] = other_head_reduce(q, k, N, H, hd, b, mode, stream, dev)
    out["mlp_scores"] = mlp_scores(act, N, wm, b, stream, dev)
    out["residual_recompute"] = recompute(resid, y, kept, n_kept, nk, d, b, stream)
    out["token_predictor"] = token_predictor(x, uq, vq, uk, vk, N, d, b, r, stream, dev)
    out["fused_movement"] = fused_movement(x, resid, kept, n_kept, nk, N, d, b, stream, dev)
    if not args.no_other_configs:
        out["exact_scores_other_configs"] = exact_scores_other_configs(mode, stream, dev)
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
        out["cpu_baseline"] = cpu_baseline(L, w)
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


def movement_cold(gx, ga, sc, stream, dev, reps=5):
    """Median time (ms) of each movement call with the 256 MB Infinity Cache
    flushed first: a 512 MiB buffer is read (not written, so no dirty lines
    are left to be written back during the timed call) before every launch."""
    import torch
    flush = torch.zeros(512 << 20, dtype=torch.uint8, device=dev).view(torch.int64)
    res = {}
    for name, fn in (("gather_x", gx), ("gather_act", ga), ("scatter", sc)):
        ts = []
        for i in range(reps):
            flush.sum()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        res[name] = float(np.median(ts))
    return res


def cpu_baseline(L, w):
    """The oracle on the host cores, on a bounded sample of one step: exact
    scores for `s` of the nb query blocks against every key block (scaled up by
    nb / s), plus the full predictor, select, gather of X and of the MLP
    activation, and scatter."""
    from oracle import lemo_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [os.cpu_count()])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    nb = w.n_blocks
    s = 8
    print(f"[bench] cpu baseline: oracle on {s}/{nb} query blocks + full predictor/movement", file=sys.stderr,
          flush=True)
    t = time.perf_counter()
    O.exact_block_scores(L.q, L.k, w.n_heads, w.head_dim, w.block, O.REDUCE_PAPER,
                         query_blocks=list(range(0, nb, nb // s))[:s])
    t_exact = (time.perf_counter() - t) * nb / s
    t = time.perf_counter()
    _, I_hat, _, _ = O.predict_scores(L.x, L.u_q, L.v_q, L.u_k, L.v_k, w.block)
    _, kept, nk, _ = O.select_mask(I_hat.astype(np.float32), O.SELECT_MEAN)
    R = nk * w.block
    cap = -(-R // 256) * 256
    O.gather_pad(L.x, w.block, kept, nk, np.zeros((cap, w.d_model), np.uint16), 256)
    O.gather_pad(L.act, w.block, kept, nk, np.zeros((cap, w.mlp_width), np.uint16), 256)
    O.scatter_residual(L.x, w.block, kept, nk, L.y[O.kept_token_rows(kept, nk, w.block)])
    t_rest = time.perf_counter() - t
    t_step = t_exact + t_rest
    return {
        "value": w.n_tokens / t_step,
        "unit": "tokens/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"exact scores of {s} of {nb} query blocks (x{nb // s}) + full predictor, mean select, "
                  f"gathers and scatter; est. step {t_step:.1f} s",
    }


if __name__ == "__main__":
    main()
