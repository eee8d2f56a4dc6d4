"""Benchmark of the VLA scan on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
the penalty-direction projection u = normalize(W_u k_raw) followed by the
scan (inverse tracking, coefficient, state update, cap, readout), with inputs
already resident in HBM.  The workload is the long-context configuration
(B=2, H=8, T=65536, d=64, r=1, bf16 storage, fp32 state, nudge every 1024
tokens, Frobenius cap 1e3).

Prints one JSON line.  ``value`` is tokens*heads per second of the whole step.
``roofline`` reports the scan kernel (the dominant one) against the fp32
vector ALU peak, with algorithmic flops 2*(2r+3)*d^2 per token*head.
``cpu_baseline`` times the fp64 CPU oracle on a bounded prefix of the same
workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "VLA scan tokens·heads/sec at d=64 + % of fp32 VALU peak (1 MI355X)"
FP32_VECTOR_PEAK_TFLOPS = 157.3   # 256 CU x 4 SIMD x 16 lanes x 2 (dual fp32) x 2 flop x 2.4 GHz
HBM_PEAK_GBS = 8000.0


def alg_flops_per_token_head(d: int, r: int) -> int:
    return 2 * (2 * r + 3) * d * d


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="long")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not supported "
              "(chains are independent, so more GPUs would each run their own share)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from recurrent_inverse_scan_amd import CONFIGS, make_inputs, project_u, scan_forward, workspace_size

    cfg = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    x = make_inputs(cfg, seed=0)
    q, k, v = x["q"].to(dev), x["k"].to(dev), x["v"].to(dev)
    W, kr = x["W_u"].to(dev), x["k_raw"].to(dev)
    B, H, T, d, r = cfg.B, cfg.H, cfg.T, cfg.d, cfg.r
    u = torch.empty((B, H, T, r, d), device=dev, dtype=q.dtype)
    outs = (torch.empty_like(q), torch.empty((B, H, d, d), device=dev), torch.empty((B, H, d, d), device=dev),
            torch.empty((B, H, d), device=dev), torch.empty((B, H, 4), device=dev, dtype=torch.int32))
    ws_bytes = workspace_size(B, H, T, d, r, q.dtype, nudge_period=cfg.nudge_period, s_cap=cfg.s_cap)
    schedule = "chunked" if ws_bytes > 0 else "sequential"
    ws = torch.empty(max(ws_bytes, 1), device=dev, dtype=torch.uint8)
    torch.cuda.synchronize()

    def step(ev=None):
        project_u(W, kr, out=u)
        if ev is not None:
            ev[0].record()
        scan_forward(q, k, v, u, nudge_period=cfg.nudge_period, s_cap=cfg.s_cap, out=outs, workspace=ws)
        if ev is not None:
            ev[1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(evs[i])
        print(f"[bench] step {i + 1}/{args.steps} enqueued", file=sys.stderr, flush=True)
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    scan_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    ms_per_step = total_ms / args.steps

    tok_heads = B * H * T
    value = tok_heads / (ms_per_step * 1e-3)
    flops = alg_flops_per_token_head(d, r) * tok_heads
    scan_tflops = flops / (scan_ms * 1e-3) / 1e12
    es = 2 if cfg.in_dtype == "bf16" else 4
    scan_bytes = tok_heads * d * es * (4 + r) + 2 * B * H * (2 * d * d + d) * 4   # q,k,v,u in, o out, state
    stats = outs[4].cpu().numpy()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, x, args.cpu_baseline_seconds)

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens*heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: VLA scan B={B} H={H} T={T} d={d} r={r}, {cfg.in_dtype} storage, "
                               f"f32 state, nudge every {cfg.nudge_period}, Frobenius cap {cfg.s_cap}",
                   "B": B, "H": H, "T": T, "d": d, "r": r, "storage": cfg.in_dtype,
                   "nudge_period": cfg.nudge_period, "s_cap": cfg.s_cap, "schedule": schedule,
                   "workspace_bytes": ws_bytes},
        "roofline": {"bound": "alu", "achieved": scan_tflops, "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": scan_tflops / FP32_VECTOR_PEAK_TFLOPS, "traffic": None},
        "scan_ms": scan_ms,
        "projection_ms": ms_per_step - scan_ms,
        "scan_hbm_gbs": scan_bytes / (scan_ms * 1e-3) / 1e9,
        "guard_fires": int(stats[..., 0].sum()),
        "cap_fires": int(stats[..., 1].sum()),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def cpu_baseline(cfg, x, budget_s: float):
    """Time the fp64 oracle on all chains over a bounded prefix of the tokens."""
    import numpy as np

    from oracle.vla_oracle import oracle_project_u, oracle_scan

    C, d, r = cfg.B * cfg.H, cfg.d, cfg.r

    def run(n_tok):
        kr = x["k_raw"].reshape(C, cfg.T, d)[:, :n_tok]
        t0 = time.perf_counter()
        u = oracle_project_u(x["W_u"], kr.reshape(-1, d)).reshape(C, n_tok, r, d)
        oracle_scan(x["q"].reshape(C, cfg.T, d)[:, :n_tok], x["k"].reshape(C, cfg.T, d)[:, :n_tok],
                    x["v"].reshape(C, cfg.T, d)[:, :n_tok], u, nudge_period=cfg.nudge_period, s_cap=cfg.s_cap)
        return time.perf_counter() - t0

    probe = min(cfg.T, 256)
    dt = run(probe)
    n_tok = int(min(cfg.T, max(probe, probe * budget_s / max(dt, 1e-6))))
    dt = run(n_tok)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {"value": C * n_tok / dt, "unit": "tokens*heads/s", "cores": 1, "kind": "oracle",
            "sample": f"all {C} chains, first {n_tok} of {cfg.T} tokens (projection + scan), fp64 NumPy, "
                      f"{dt:.1f} s wall; single-threaded loops ({cores} cores visible)"}


if __name__ == "__main__":
    sys.exit(main())
