"""Benchmark of the VLA scan on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
the penalty-direction projection u = normalize(W_u k_raw) followed by the
scan (inverse tracking, coefficient, state update, cap, readout), with inputs
already resident in HBM.  The workload is the long-context configuration
(B=2, H=8, T=65536, d=64, r=1, bf16 storage, fp32 state, nudge every 1024
tokens, Frobenius cap 1e3).

Prints one JSON line.  ``value`` is tokens*heads per second of the whole step.
``roofline`` reports the dominant kernel, the state-chain kernel of the
chunked schedule (the sequential S/cap recursion, launched once per segment
of the sequence): its algorithmic flops per launch are those of the memory
update and the cap's norm, 2 d^2 + 2 d^2 per token*head of the launch's
segment, over the launch's mean duration from HIP events the library records
on the kernel's own stream during the timed steps; ``traffic`` is its HBM
bytes per launch from rocprofv3 counters
(profiles/state_chain_long_traffic.md), or null when the kernel sources have
changed since they were taken.  ``scan_valu_frac`` is the
whole scan's algorithmic flops 2 (2r+3) d^2 per token*head against the fp32
vector peak.  ``cpu_baseline`` times the fp64 CPU oracle on a bounded prefix
of the same workload.

``--update residual`` times the residual (delta-rule) update on the same
workload instead (its chunked schedule's dominant kernel is the residual
chain kernel); the headline line is the default additive update.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "VLA scan tokens·heads/sec at d=64 + % of fp32 VALU peak (1 MI355X)"
FP32_VECTOR_PEAK_TFLOPS = 157.3   # 256 CU x 4 SIMD x 16 lanes x 2 (dual fp32) x 2 flop x 2.4 GHz
HBM_PEAK_GBS = 8000.0


# The dominant kernel of each update's chunked schedule, the sources it is
# built from, and the committed counter summary of its HBM traffic.
CHAIN = {
    "additive": ("vla_state_chain_kernel",
                 ("state_pass.hip", "vla_common.h", "vla_kernels.h", "vla_mfma.h", "vla_seq.h"),
                 os.path.join(ROOT, "profiles", "state_chain_long_traffic.md")),
    "residual": ("vla_res_chain_kernel",
                 ("residual_pass.hip", "vla_residual.h", "vla_common.h", "vla_kernels.h", "vla_mfma.h", "vla_seq.h"),
                 os.path.join(ROOT, "profiles", "residual_chain_long_traffic.md")),
}


def chunked_kernel_name(d: int) -> str:
    """The dominant kernel of the time-parallel schedule: the state-chain
    kernel at d = 64; at d = 128 (no cap, linear state pass) the blocked
    inverse pass over spans of chunks."""
    return "vla_state_chain_kernel" if d == 64 else "vla_inverse_wy128_kernel (blocked inverse pass)"


def seq_kernel_name(d: int, T: int) -> str:
    """The kernel the sequential schedule launches: calls longer than 16 tokens
    at d <= 64 run the two-wave kernel, T = 1 at d = 64 the decode kernel."""
    if T == 1 and d == 64:
        return "vla_decode_kernel"
    return "vla_scan_split_kernel" if (d <= 64 and T > 16) else "vla_scan_seq_kernel"


def alg_flops_per_token_head(d: int, r: int, update: str = "additive") -> int:
    """2 (2r + 3) d^2: r rank-1 updates (product and update, 2 d^2 each), the
    coefficient A k, the state update and the readout; the residual update
    adds the prediction S k_hat (one more d^2 product)."""
    return 2 * (2 * r + 3 + (1 if update == "residual" else 0)) * d * d


def chain_flops_per_token_head(d: int, cap_on: bool, update: str = "additive") -> int:
    """The state recurrence the chain kernel carries: additive, the memory
    update S += v alpha^T (d^2 FMA) plus the cap's |S|^2 (d^2 FMA); residual,
    the prediction S k_hat and the update (2 d^2 FMA; its cap test runs in
    the readout)."""
    if update == "residual":
        return 4 * d * d
    return 2 * d * d + (2 * d * d if cap_on else 0)


def chain_source_sha(update: str = "additive") -> str:
    h = hashlib.sha256()
    for name in CHAIN[update][1]:
        with open(os.path.join(ROOT, "recurrent_inverse_scan_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(update: str = "additive"):
    """HBM bytes per launch of the chain kernel from the committed counter
    summary, if it was taken on the current kernel sources."""
    try:
        text = open(CHAIN[update][2]).read()
    except OSError:
        return None
    vals = dict(re.findall(r"^([a-z_0-9]+):\s*(\S+)\s*$", text, flags=re.M))
    if vals.get("source_sha256") != chain_source_sha(update):
        return None
    try:
        return float(vals["fetch_bytes_per_launch"]) + float(vals["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="long")
    ap.add_argument("--update", default="additive", choices=("additive", "residual"),
                    help="state update of the timed scan (the headline is the additive update)")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=20.0,
                    help="approximate CPU time budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the secondary measurements (residual update, decode step)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the run, one device-to-device copy of this many MiB (a known-size kernel "
                         "for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE counters)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not supported "
              "(chains are independent, so more GPUs would each run their own share)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from recurrent_inverse_scan_amd import (CONFIGS, make_inputs, project_u, scan_forward, timing_collect,
                                            timing_enable, workspace_size)

    cfg = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    x = make_inputs(cfg, seed=0)
    q, k, v = x["q"].to(dev), x["k"].to(dev), x["v"].to(dev)
    W, kr = x["W_u"].to(dev), x["k_raw"].to(dev)
    B, H, T, d, r = cfg.B, cfg.H, cfg.T, cfg.d, cfg.r
    u = torch.empty((B, H, T, r, d), device=dev, dtype=q.dtype)
    outs = (torch.empty_like(q), torch.empty((B, H, d, d), device=dev), torch.empty((B, H, d, d), device=dev),
            torch.empty((B, H, d), device=dev), torch.empty((B, H, 4), device=dev, dtype=torch.int32))
    upd = args.update
    ws_bytes = workspace_size(B, H, T, d, r, q.dtype, nudge_period=cfg.nudge_period, s_cap=cfg.s_cap, update=upd)
    schedule = "chunked" if ws_bytes > 0 else "sequential"
    ws = torch.empty(max(ws_bytes, 1), device=dev, dtype=torch.uint8)
    torch.cuda.synchronize()

    def step(ev=None):
        project_u(W, kr, out=u)
        if ev is not None:
            ev[0].record()
        scan_forward(q, k, v, u, nudge_period=cfg.nudge_period, s_cap=cfg.s_cap, out=outs, workspace=ws, update=upd)
        if ev is not None:
            ev[1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    timing_enable(True)   # the library records HIP events around the chain kernel on its stream
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(evs[i])
        print(f"[bench] step {i + 1}/{args.steps} enqueued", file=sys.stderr, flush=True)
    t_end.record()
    torch.cuda.synchronize()
    chain_ms_all = timing_collect()
    timing_enable(False)
    total_ms = t_start.elapsed_time(t_end)
    scan_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    ms_per_step = total_ms / args.steps
    # The chunked schedule runs the chain kernel as a few pipelined segment
    # launches per scan: its time per step is the sum over those launches.
    chain_ms = sum(chain_ms_all) / args.steps if chain_ms_all else None
    chain_launches = len(chain_ms_all) // args.steps if chain_ms_all else 0
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, device=dev, dtype=torch.float32)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: {args.copy_calibration_mib} MiB read and written", file=sys.stderr,
              flush=True)
        del src, dst

    tok_heads = B * H * T
    value = tok_heads / (ms_per_step * 1e-3)
    flops = alg_flops_per_token_head(d, r, upd) * tok_heads
    scan_tflops = flops / (scan_ms * 1e-3) / 1e12
    cap_on = cfg.s_cap is not None and cfg.s_cap > 0
    chain_flops = chain_flops_per_token_head(d, cap_on, upd) * tok_heads
    if chain_ms:
        launch_ms = chain_ms / chain_launches   # mean launch: the segments differ in length
        launch_flops = chain_flops / chain_launches
        roofline = {"bound": "alu", "achieved": launch_flops / (launch_ms * 1e-3) / 1e12,
                    "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": launch_flops / (launch_ms * 1e-3) / 1e12 / FP32_VECTOR_PEAK_TFLOPS,
                    "traffic": measured_traffic(upd),
                    "kernel": CHAIN[upd][0], "kernel_ms": launch_ms, "flops_per_launch": launch_flops,
                    "launches_per_step": chain_launches, "kernel_ms_per_step": chain_ms}
    else:   # no chain kernel (the sequential schedule; d = 128): the whole scan against the peak
        roofline = {"bound": "alu", "achieved": scan_tflops, "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": scan_tflops / FP32_VECTOR_PEAK_TFLOPS, "traffic": None,
                    "kernel": (f"whole scan (dominant: {chunked_kernel_name(d)})" if schedule == "chunked"
                               else seq_kernel_name(d, T)),
                    "kernel_ms": scan_ms, "launches_per_step": 1, "flops_per_step": flops}
    es = 2 if cfg.in_dtype == "bf16" else 4
    scan_bytes = tok_heads * d * es * (4 + r) + 2 * B * H * (2 * d * d + d) * 4   # q,k,v,u in, o out, state
    stats = outs[4].cpu().numpy()

    extra = None if (args.no_extra or upd != "additive") else extra_measurements(CONFIGS, dev)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, x, args.cpu_baseline_seconds, upd)

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
                               f"f32 state, nudge every {cfg.nudge_period}, Frobenius cap {cfg.s_cap}"
                               + ("" if upd == "additive" else f", {upd} update"),
                   "update": upd,
                   "B": B, "H": H, "T": T, "d": d, "r": r, "storage": cfg.in_dtype,
                   "nudge_period": cfg.nudge_period, "s_cap": cfg.s_cap, "schedule": schedule,
                   "workspace_bytes": ws_bytes},
        "roofline": roofline,
        "scan_ms": scan_ms,
        "scan_tflops": scan_tflops,
        "scan_valu_frac": scan_tflops / FP32_VECTOR_PEAK_TFLOPS,
        "projection_ms": ms_per_step - scan_ms,
        "scan_hbm_gbs": scan_bytes / (scan_ms * 1e-3) / 1e9,
        "guard_fires": int(stats[..., 0].sum()),
        "cap_fires": int(stats[..., 1].sum()),
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)
    return 0


def _time_ms(fn, reps: int, warmup: int = 2) -> float:
    """Mean milliseconds of fn() over reps calls, from events on torch's
    current stream (the sequential schedule launches only there)."""
    import torch

    for _ in range(warmup):
        fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def extra_measurements(CONFIGS, dev):
    """Secondary workloads, each timed on its own with inputs resident:

    * residual: the residual (delta-rule) update, on the 512-chain recall
      workload (sequential schedule) and on the long workload (time-parallel
      schedule); algorithmic
      flops 2 (2r+4) d^2 per token*head (one more d^2 sweep than additive);
    * the other workloads (tiny, base, recall, wide) with the additive update,
      each on the schedule the library picks for it;
    * decode: one token per call (T = 1) for 4096 chains with the state read
      from and written back to HBM in place; its bound is HBM, with
      algorithmic bytes per chain of A, S (read and written, fp32), n, and
      the token's q, k, v, u in and o out.
    """
    import torch

    from recurrent_inverse_scan_amd import make_inputs, project_u, scan_forward, workspace_size

    out = {}
    for name, reps in (("recall", 20), ("long", 2)):
        cfg = CONFIGS[name]
        x = make_inputs(cfg, seed=0)
        q, k, v = x["q"].to(dev), x["k"].to(dev), x["v"].to(dev)
        u = project_u(x["W_u"].to(dev), x["k_raw"].to(dev))
        B, H, T, d, r = cfg.B, cfg.H, cfg.T, cfg.d, cfg.r
        o = (torch.empty_like(q), torch.empty((B, H, d, d), device=dev), torch.empty((B, H, d, d), device=dev),
             torch.empty((B, H, d), device=dev), torch.empty((B, H, 4), device=dev, dtype=torch.int32))
        ws_bytes = workspace_size(B, H, T, d, r, q.dtype, nudge_period=cfg.nudge_period, s_cap=cfg.s_cap,
                                  update="residual")
        sched = "chunked" if ws_bytes > 0 else "sequential"
        ws = torch.empty(max(ws_bytes, 1), device=dev, dtype=torch.uint8)
        fn = lambda: scan_forward(q, k, v, u, nudge_period=cfg.nudge_period, s_cap=cfg.s_cap, update="residual",
                                  out=o, workspace=ws)
        ms = _time_ms(fn, reps, warmup=1)
        th = B * H * T
        tfl = 2 * (2 * r + 4) * d * d * th / (ms * 1e-3) / 1e12
        out[f"residual_{name}"] = {
            "workload": f"{name}: residual update, B={B} H={H} T={T} d={d} r={r}, {cfg.in_dtype} storage, "
                        f"{sched} schedule", "ms": ms, "tokens_heads_per_s": th / (ms * 1e-3),
            "alg_tflops": tfl, "valu_frac": tfl / FP32_VECTOR_PEAK_TFLOPS,
            "kernel": "vla_res_chain_kernel" if sched == "chunked" else seq_kernel_name(d, T)}
        del q, k, v, u, o, x, ws

    # The other workloads (additive update), each on the schedule the library
    # picks for it.
    for name, reps in (("tiny", 20), ("base", 20), ("recall", 20), ("wide", 2)):
        cfg = CONFIGS[name]
        x = make_inputs(cfg, seed=0)
        q, k, v = x["q"].to(dev), x["k"].to(dev), x["v"].to(dev)
        u = project_u(x["W_u"].to(dev), x["k_raw"].to(dev))
        B, H, T, d, r = cfg.B, cfg.H, cfg.T, cfg.d, cfg.r
        o = (torch.empty_like(q), torch.empty((B, H, d, d), device=dev), torch.empty((B, H, d, d), device=dev),
             torch.empty((B, H, d), device=dev), torch.empty((B, H, 4), device=dev, dtype=torch.int32))
        ws_bytes = workspace_size(B, H, T, d, r, q.dtype, nudge_period=cfg.nudge_period, s_cap=cfg.s_cap)
        sched = "chunked" if ws_bytes > 0 else "sequential"
        ws = torch.empty(max(ws_bytes, 1), device=dev, dtype=torch.uint8)
        fn = lambda: scan_forward(q, k, v, u, nudge_period=cfg.nudge_period, s_cap=cfg.s_cap, out=o, workspace=ws)
        ms = _time_ms(fn, reps, warmup=1)
        th = B * H * T
        tfl = 2 * (2 * r + 3) * d * d * th / (ms * 1e-3) / 1e12
        out[f"additive_{name}"] = {
            "workload": f"{name}: additive update, B={B} H={H} T={T} d={d} r={r}, {cfg.in_dtype} storage, "
                        f"{sched} schedule", "ms": ms, "tokens_heads_per_s": th / (ms * 1e-3),
            "alg_tflops": tfl, "valu_frac": tfl / FP32_VECTOR_PEAK_TFLOPS,
            "kernel": chunked_kernel_name(d) if sched == "chunked" else seq_kernel_name(d, T)}
        del q, k, v, u, o, x, ws

    # Backward pass (additive update, sequential per chain): the recall and
    # base workloads.  Algorithmic work of the reverse recurrence, 2 (5r + 10)
    # d^2 flops per token*head: per rank-1 step (G + G^T) z, the gA and
    # A^T gz products and rebuilding A_before (5 d^2 FMA); per token the
    # readout's S q, S^T g_o and g_o q^T, the state step's gX alpha_hat and
    # gX^T v, the coefficient's g_alpha k^T and A^T g_alpha, and the
    # recomputed S (10 d^2 FMA).  The forward pass that records the tape is
    # a recomputation and is not counted.
    from recurrent_inverse_scan_amd import scan_backward

    for name, reps in (("recall", 3), ("base", 2)):
        cfg = CONFIGS[name]
        x = make_inputs(cfg, seed=0)
        q, k, v = x["q"].to(dev), x["k"].to(dev), x["v"].to(dev)
        u = project_u(x["W_u"].to(dev), x["k_raw"].to(dev))
        B, H, T, d, r = cfg.B, cfg.H, cfg.T, cfg.d, cfg.r
        go = torch.randn(B, H, T, d, device=dev)
        fn = lambda: scan_backward(q, k, v, u, g_o=go, nudge_period=cfg.nudge_period, s_cap=cfg.s_cap)
        ms = _time_ms(fn, reps, warmup=1)
        th = B * H * T
        tfl = 2 * (5 * r + 10) * d * d * th / (ms * 1e-3) / 1e12
        out[f"backward_{name}"] = {
            "workload": f"{name}: backward of the additive scan, B={B} H={H} T={T} d={d} r={r}, "
                        f"{cfg.in_dtype} storage, float32 gradients", "ms": ms,
            "tokens_heads_per_s": th / (ms * 1e-3), "alg_tflops": tfl, "valu_frac": tfl / FP32_VECTOR_PEAK_TFLOPS,
            "kernel": "vla_bwd_tape_kernel + vla_bwd_reverse_kernel"}
        del q, k, v, u, x, go

    # Fused prologue: the scan from raw q, k and W_u (features and u built by
    # the library), against the unfused projection + scan on the same data.
    from recurrent_inverse_scan_amd import fused_workspace_size, scan_forward_fused

    for name, reps in (("recall", 20), ("long", 3), ("wide", 2)):
        cfg = CONFIGS[name]
        x = make_inputs(cfg, seed=0)
        qr, kr, v, W = x["q_raw"].to(dev), x["k_raw"].to(dev), x["v"].to(dev), x["W_u"].to(dev)
        q, k = x["q"].to(dev), x["k"].to(dev)
        B, H, T, d, r = cfg.B, cfg.H, cfg.T, cfg.d, cfg.r
        o = (torch.empty_like(q), torch.empty((B, H, d, d), device=dev), torch.empty((B, H, d, d), device=dev),
             torch.empty((B, H, d), device=dev), torch.empty((B, H, 4), device=dev, dtype=torch.int32))
        fws = fused_workspace_size(B, H, T, d, r, q.dtype, nudge_period=cfg.nudge_period, s_cap=cfg.s_cap)
        wsf = torch.empty(max(fws, 1), device=dev, dtype=torch.uint8)
        fn = lambda: scan_forward_fused(qr, kr, v, W, nudge_period=cfg.nudge_period, s_cap=cfg.s_cap, out=o,
                                        workspace=wsf)
        ms = _time_ms(fn, reps, warmup=1)
        u = torch.empty((B, H, T, r, d), device=dev, dtype=q.dtype)
        ws_bytes = workspace_size(B, H, T, d, r, q.dtype, nudge_period=cfg.nudge_period, s_cap=cfg.s_cap)
        ws = torch.empty(max(ws_bytes, 1), device=dev, dtype=torch.uint8)

        def unfused():
            project_u(W, kr, out=u)
            scan_forward(q, k, v, u, nudge_period=cfg.nudge_period, s_cap=cfg.s_cap, out=o, workspace=ws)

        ms_u = _time_ms(unfused, reps, warmup=1)
        th = B * H * T
        tfl = 2 * (2 * r + 3) * d * d * th / (ms * 1e-3) / 1e12
        out[f"fused_{name}"] = {
            "workload": f"{name}: fused feature map + projection + scan (additive), B={B} H={H} T={T} d={d} r={r}, "
                        f"{cfg.in_dtype} storage, "
                        + ("prologue in the scan kernel (u never in HBM)" if fws == 0 else
                           "prologue pass into the workspace"),
            "ms": ms, "unfused_projection_plus_scan_ms": ms_u, "tokens_heads_per_s": th / (ms * 1e-3),
            "alg_tflops": tfl, "valu_frac": tfl / FP32_VECTOR_PEAK_TFLOPS,
            "kernel": "vla_scan_split_kernel (fused)" if fws == 0 else "feature map + projection + scan"}
        del qr, kr, v, W, q, k, o, x, ws, wsf, u

    # Decode: 4096 chains, one token per call, state carried in place.
    B, H, d, r = 256, 16, 64, 1
    g = torch.Generator(device="cpu").manual_seed(0)
    elu1 = lambda z: torch.nn.functional.elu(z) + 1.0
    q = elu1(torch.randn(B, H, 1, d, generator=g)).to(torch.bfloat16).to(dev)
    k = elu1(torch.randn(B, H, 1, d, generator=g)).to(torch.bfloat16).to(dev)
    v = torch.randn(B, H, 1, d, generator=g).to(torch.bfloat16).to(dev)
    uu = torch.randn(B, H, 1, r, d, generator=g)
    u = (uu / uu.norm(dim=-1, keepdim=True)).to(torch.bfloat16).to(dev)
    A = torch.eye(d, device=dev).expand(B, H, d, d).contiguous()
    S = torch.zeros(B, H, d, d, device=dev)
    n = torch.zeros(B, H, d, device=dev)
    o = torch.empty_like(q)
    st = torch.empty(B, H, 4, device=dev, dtype=torch.int32)
    for upd in ("additive", "residual"):
        fn = lambda: scan_forward(q, k, v, u, A, S, n, nudge_period=1024, s_cap=1e3, update=upd,
                                  out=(o, A, S, n, st))
        ms = _time_ms(fn, 50, warmup=5)
        chains = B * H
        alg_bytes = chains * (2 * (2 * d * d + d) * 4 + (4 + r) * d * 2)
        gbs = alg_bytes / (ms * 1e-3) / 1e9
        out[f"decode_{upd}"] = {
            "workload": f"decode: {upd} update, T=1 per call, B={B} H={H} d={d} r={r}, bf16 "
                        f"token storage, f32 state in HBM carried in place", "ms": ms,
            "tokens_heads_per_s": chains / (ms * 1e-3), "alg_bytes": alg_bytes, "hbm_gbs": gbs,
            "hbm_frac": gbs / HBM_PEAK_GBS, "kernel": seq_kernel_name(d, 1)}
    return out


def cpu_baseline(cfg, x, budget_s: float, update: str = "additive"):
    """Time the fp64 oracle on all chains over a bounded prefix of the tokens,
    with its BLAS held to one thread (the oracle's loops are single-threaded)."""
    from threadpoolctl import threadpool_limits

    from oracle.vla_oracle import oracle_project_u, oracle_scan

    C, d, r = cfg.B * cfg.H, cfg.d, cfg.r

    def run(n_tok):
        kr = x["k_raw"].reshape(C, cfg.T, d)[:, :n_tok]
        t0 = time.perf_counter()
        u = oracle_project_u(x["W_u"], kr.reshape(-1, d)).reshape(C, n_tok, r, d)
        oracle_scan(x["q"].reshape(C, cfg.T, d)[:, :n_tok], x["k"].reshape(C, cfg.T, d)[:, :n_tok],
                    x["v"].reshape(C, cfg.T, d)[:, :n_tok], u, nudge_period=cfg.nudge_period, s_cap=cfg.s_cap,
                    update=update)
        return time.perf_counter() - t0

    with threadpool_limits(limits=1):
        probe = min(cfg.T, 512)
        dt = run(probe)
        n_tok = int(min(cfg.T, max(probe, probe * budget_s / max(dt, 1e-6))))
        if n_tok > probe:
            dt = run(n_tok)
    try:
        visible = len(os.sched_getaffinity(0))
    except AttributeError:
        visible = os.cpu_count()
    cpu_model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    import numpy

    return {"value": C * n_tok / dt, "unit": "tokens*heads/s", "cores": 1, "kind": "oracle",
            "sample": f"all {C} chains, first {n_tok} of {cfg.T} tokens (projection + scan), fp64 NumPy, "
                      f"{dt:.1f} s wall on 1 thread (BLAS limited to 1; {visible} cores visible)",
            "cpu_model": cpu_model, "numpy": numpy.__version__}


if __name__ == "__main__":
    sys.exit(main())
