"""Benchmark of the per-sample gradient-norm hot path on one MI355X.

One step = one grouped Hutchinson call over the Llama-3.2-1B-shaped stack
(16 decoder layers x {q, k, v, o, gate, up, down}, B = 4, T = 4096, k = 32,
bf16 inputs, fp32 accumulation, an independent P per projection): G P, the
split-free A^T (G P) contraction with its squared Frobenius norm, the
per-sample layer sum over all 112 projections and the clip factors at C = 1.
Inputs are synthetic, seeded, and resident in HBM before timing starts.

Prints one JSON line with the throughput (samples * tokens / s), the roofline
of the dominant kernel (per-launch durations from HIP events the library
records between its launches, on the stream the kernels run on) and the CPU
oracle timed on a bounded sample of the same workload.
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

HBM_PEAK_GBS = 8000.0
METRIC = "per-sample norm-est samples·tokens/s (k=32, 1B-shape layers); % peak HBM BW"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=4, help="decoder layers in the oracle's sample")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 1 GiB device-to-device copy first (reference for hardware byte counters)")
    return ap.parse_args()


def cpu_baseline(layers, B, T, n_layers_total, n_sample_layers):
    """The fp64 oracle on sample 0 of the first `n_sample_layers` decoder
    layers (7 projections each), scaled to the whole step."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1
    sub = layers[: 7 * n_sample_layers]
    host = [(A[:1].cpu(), G[:1].cpu(), P.cpu()) for (A, G, P) in sub]
    host = [(oracle.to_f64(A), oracle.to_f64(G), oracle.to_f64(P)) for (A, G, P) in host]
    t0 = time.perf_counter()
    parts = [oracle.hutch(A, G, P) for (A, G, P) in host]
    tot = oracle.layer_sum(parts)
    oracle.clip_factors(tot, 1.0)
    dt = time.perf_counter() - t0
    # one sample over n_sample_layers of the n_layers_total decoder layers
    step_s = dt * B * (n_layers_total / n_sample_layers)
    return {"value": B * T / step_s, "unit": "samples·tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 numpy oracle, sample 0 of {n_sample_layers} decoder layer(s) x 7 projections "
                      f"(T={T}), {dt:.2f} s, scaled x{B * n_layers_total // n_sample_layers} to the step"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs on one GPU only (the per-sample norm path needs no collectives); "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import sample_grad_norms_amd as dp
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, T, k = 4, 4096, 32
    projs = [workloads.config3_projection(j, device=dev) for j in range(112)]
    layers = [(q.A, q.G, q.P) for q in projs]
    ws_bytes = dp.hutch_grouped_workspace(layers, torch.bfloat16, B, T, k)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    n = torch.empty(B, dtype=torch.float32, device=dev)
    c = torch.empty(B, dtype=torch.float32, device=dev)
    bytes_A = sum(A.numel() * A.element_size() for (A, _, _) in layers)
    bytes_G = sum(G.numel() * G.element_size() for (_, G, _) in layers)
    bytes_P = sum(P.numel() * P.element_size() for (_, _, P) in layers)
    alg_bytes = bytes_A + bytes_G + bytes_P
    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    torch.cuda.synchronize()

    def step(timer=None):
        dp.hutch_grouped(layers, out=n, C_clip=1.0, clip_out=c, workspace=ws, timer=timer)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps

    # per-launch durations from the library's events (separate, traced steps)
    timer = dp.KernelTimer(64)
    per_kind = {}
    n_trace = max(3, min(args.steps, 10))
    for _ in range(n_trace):
        step(timer)
        for kind, ms in timer.last():
            per_kind.setdefault(kind, []).append(ms)
    avg = {kk: sum(v) / n_trace for kk, v in per_kind.items()}  # per step (prepare may run several times)
    dom = max(("rowproj", "tcontract"), key=lambda kk: avg.get(kk, 0.0))
    dom_bytes = bytes_G if dom == "rowproj" else bytes_A
    achieved = dom_bytes / (avg[dom] * 1e-3) / 1e9
    value = B * T / (ms_step * 1e-3)

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "samples·tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Llama-3.2-1B-shaped linear stack, Hutchinson + layer sum + clip",
                   "layers": 16, "projections": 112, "B": B, "T": T, "k": k, "C": 1.0,
                   "algorithmic_bytes": alg_bytes},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None},
        "step_hbm_gbs": alg_bytes / (ms_step * 1e-3) / 1e9,
        "step_hbm_frac": alg_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "kernel_ms": avg,
        "kernel_gbs": {"rowproj": bytes_G / (avg["rowproj"] * 1e-3) / 1e9,
                       "tcontract": bytes_A / (avg["tcontract"] * 1e-3) / 1e9},
        "clip_fraction": float((c < 1.0).float().mean().item()),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(layers, B, T, 16, args.cpu_layers)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
