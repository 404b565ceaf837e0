"""Benchmark of the per-sample gradient-norm hot path on one MI355X.

One step = one grouped Hutchinson call over the Llama-3.2-1B-shaped stack
(16 decoder layers x {q, k, v, o, gate, up, down}, B = 4, T = 4096, k = 32,
bf16 inputs, fp32 accumulation, an independent P per projection): G P, the
A^T (G P) contraction with its squared Frobenius norm, the per-sample layer
sum over all 112 projections and the clip factors at C = 1. Inputs are
synthetic, seeded, and resident in HBM before timing starts.

Prints one JSON line: the throughput (samples * tokens / s), the roofline of
the dominant kernel (per-launch durations from HIP events the library records
between its launches, on the stream the kernels run on; HBM traffic from the
committed rocprofv3 counter summary when it matches the current sources),
the fp64 CPU oracle timed on the host over the same workload, and the other
workloads (Hutch++, the exact comparator, single layers) under "extras".
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
METRIC = "per-sample norm-est samples·tokens/s (k=32, 1B-shape layers); % peak HBM BW"
PROFILE = os.path.join(ROOT, "profiles", "rowproj_tcontract_llama1b_stack_B4_T4096_k32.md")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=16, help="decoder layers the CPU oracle runs over")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 1 GiB device-to-device copy first (reference for hardware byte counters)")
    return ap.parse_args()


def timed(fn, steps, warmup):
    """Mean milliseconds per call of fn over `steps` calls after `warmup`."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def cpu_baseline(layers, B, T, n_layers):
    """The fp64 oracle over the first `n_layers` decoder layers (7 projections
    each, all B samples), one projection at a time; only the oracle's own
    arithmetic is timed, the device-to-host copies and fp64 conversions are
    not. Scaled to the 16-layer step when n_layers < 16."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1
    spent = copy_s = 0.0
    parts = []
    for (A, G, P) in layers[: 7 * n_layers]:
        t0 = time.perf_counter()
        a, g, p = oracle.to_f64(A), oracle.to_f64(G), oracle.to_f64(P)
        copy_s += time.perf_counter() - t0
        t0 = time.perf_counter()
        parts.append(oracle.hutch(a, g, p))
        spent += time.perf_counter() - t0
        del a, g, p
    t0 = time.perf_counter()
    oracle.clip_factors(oracle.layer_sum(parts), 1.0)
    spent += time.perf_counter() - t0
    step_s = spent * 16 / n_layers
    return {"value": B * T / step_s, "unit": "samples·tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 numpy oracle over {n_layers} decoder layer(s) x 7 projections, all {B} samples, "
                      f"T={T}: {spent:.2f} s of oracle arithmetic"
                      + ("" if n_layers == 16 else f", scaled x{16 / n_layers:g} to the step")
                      + f" (device-to-host copies and fp64 conversion, untimed in the rate: {copy_s:.2f} s)",
            "host": host_cpu()}


def oracle_per_config():
    """The fp64 oracle on the other workloads, each once on its full inputs
    (copied to the host and converted to float64 first; only the oracle's
    arithmetic is timed): the tiny fp32 layer (Hutchinson, exact, clip), the
    single layer (Hutchinson; the exact norm by the Gram route), Hutch++ and
    the long-context layer (Hutchinson; the exact norm by the explicit route,
    about 1.1 TFLOP of fp64). Rates in samples * tokens / s of that work."""
    import oracle
    import torch
    import workloads
    dev = torch.device("cuda:0")

    def run(name, B, T, parts):
        out = {}
        for what, fn in parts:
            t0 = time.perf_counter()
            fn()
            out[what] = time.perf_counter() - t0
        total = sum(out.values())
        return {"value": B * T / total, "unit": "samples·tokens/s", "seconds": out, "workload": name}

    res = {}
    pr = workloads.config1(device=dev)
    A, G, P = oracle.to_f64(pr.A), oracle.to_f64(pr.G), oracle.to_f64(pr.P)
    res["tiny_fp32_B2_T128_d64_p64_k8"] = run(pr.name, 2, 128, [
        ("hutch", lambda: oracle.hutch(A, G, P)), ("exact_explicit", lambda: oracle.exact_explicit(A, G)),
        ("clip", lambda: oracle.clip_factors(oracle.hutch(A, G, P), 1.0))])
    pr = workloads.config2(device=dev)
    A, G, P = oracle.to_f64(pr.A), oracle.to_f64(pr.G), oracle.to_f64(pr.P)
    res["single_layer_B8_T1024_d2048_p2048_k32"] = run(pr.name, 8, 1024, [
        ("hutch", lambda: oracle.hutch(A, G, P)), ("exact_gram", lambda: oracle.exact_gram(A, G))])
    pr = workloads.config4(device=dev)
    A, G, S, P = oracle.to_f64(pr.A), oracle.to_f64(pr.G), oracle.to_f64(pr.S), oracle.to_f64(pr.P)
    res["hutchpp_B4_T4096_d2048_p2048_k32"] = run(pr.name, 4, 4096, [("hutchpp", lambda: oracle.hutchpp(A, G, S, P))])
    del A, G, S, P
    pr = workloads.config5(device=dev)
    A, G, P = oracle.to_f64(pr.A), oracle.to_f64(pr.G), oracle.to_f64(pr.P)
    del pr
    res["long_context_B1_T32768_d2048_p8192_k32"] = run("config5_bf16_B1_T32768_d2048_p8192_k32", 1, 32768, [
        ("hutch", lambda: oracle.hutch(A, G, P)), ("exact_explicit", lambda: oracle.exact_explicit(A, G))])
    del A, G, P
    return res


def host_cpu() -> str:
    """The host's CPU model and logical CPU count (from /proc/cpuinfo)."""
    model, n = "unknown", 0
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    n += 1
                    model = line.split(":", 1)[1].strip()
    except OSError:
        pass
    return f"{model}, {n or os.cpu_count()} logical CPUs"


def rotated(make, copies):
    """`copies` independent input sets so that repeated calls stream from HBM
    rather than from the 256 MB last-level cache."""
    return [make(r) for r in range(copies)]


def hbm_calibration(dev):
    """The device's memory clock and bus width (HIP device attributes 60 and
    59: hipDeviceAttributeMemoryClockRate in kHz, hipDeviceAttributeMemoryBusWidth
    in bits) with the double-data-rate peak they imply, and the rate of a
    read-only stream over 16 GiB with the stage kernels' load path."""
    import ctypes
    import torch
    import sample_grad_norms_amd as dp
    out = {"spec_gbs": HBM_PEAK_GBS}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        clk, bus = ctypes.c_int(0), ctypes.c_int(0)
        idx = dev.index or 0
        if hip.hipDeviceGetAttribute(ctypes.byref(clk), 60, idx) == 0 and \
                hip.hipDeviceGetAttribute(ctypes.byref(bus), 59, idx) == 0:
            out["memory_clock_khz"] = clk.value
            out["bus_width_bits"] = bus.value
            out["ddr_formula_gbs"] = 2.0 * clk.value * 1e3 * bus.value / 8 / 1e9
    except OSError:
        pass
    buf = torch.empty(16 << 30, dtype=torch.uint8, device=dev)
    ms = timed(lambda: dp.read_probe(buf), 5, 2)
    out["read_probe_16GiB_gbs"] = buf.numel() / (ms * 1e-3) / 1e9
    out["note"] = ("percentages of peak in this record use spec_gbs; ddr_formula_gbs (2 x memory clock x bus "
                   "width / 8 from the device attributes) counts two transfers per reported clock, which is "
                   "below what HBM3E delivers here (the read probe exceeds it)")
    del buf
    return out


def shared_input_stack(args):
    """The Llama-3.2-1B-shaped stack with inputs shared as in the real model
    (q, k, v read one activation tensor, gate and up another): projections on
    one input share one pass over it."""
    import torch
    import sample_grad_norms_amd as dp
    import workloads
    dev = torch.device("cuda:0")
    B, T, k = 4, 4096, 32
    layers = workloads.shared_input_stack(device=dev, B=B, T=T, k=k)
    ws = torch.empty(dp.hutch_grouped_workspace(layers, torch.bfloat16, B, T, k), dtype=torch.uint8, device=dev)
    n = torch.empty(B, dtype=torch.float32, device=dev)
    c = torch.empty(B, dtype=torch.float32, device=dev)

    def step(timer=None):
        dp.hutch_grouped(layers, out=n, C_clip=1.0, clip_out=c, workspace=ws, timer=timer)
    ms = timed(step, args.steps, args.warmup)
    timer = dp.KernelTimer(64)
    per_kind = {}
    for _ in range(3):
        step(timer)
        for kind, t in timer.last():
            per_kind[kind] = per_kind.get(kind, 0.0) + t / 3
    inputs = {A.data_ptr(): A for (A, _, _) in layers}
    bytes_A = sum(A.numel() * A.element_size() for A in inputs.values())
    bytes_GP = sum(G.numel() * G.element_size() + P.numel() * P.element_size() for (_, G, P) in layers)
    out = {"ms_per_step": ms, "samples_tokens_per_s": B * T / (ms * 1e-3), "algorithmic_bytes": bytes_A + bytes_GP,
           "hbm_gbs": (bytes_A + bytes_GP) / (ms * 1e-3) / 1e9, "kernel_ms": per_kind,
           "tcontract_gbs": bytes_A / (per_kind["tcontract"] * 1e-3) / 1e9}
    del layers, ws
    return out


def dpsgd_rc_step(args):
    """One DP-SGD-RC training step (forward, backward 1, norm path, clip,
    backward 2, noise, Adam) on a randomly initialised Llama-shaped stack at
    Llama-3.2-1B widths (2 decoder layers, B=4, T=2048, bf16; attention in
    float32), with a non-private step (forward, one backward, Adam) on the
    same model beside it."""
    import torch
    import sample_grad_norms_amd as dp
    from sample_grad_norms_amd.dpsgd_rc import RandomizedClipping
    from workloads import llama_block as lb
    dev = torch.device("cuda:0")
    shape = dict(layers=2, dim=2048, heads=32, kv_heads=8, hidden=8192, vocab=2048)
    B, T = 4, 2048
    model = lb.build(90, device=dev, dtype=torch.bfloat16, **shape)
    x, y = lb.batch(91, B, T, shape["dim"], shape["vocab"], device=dev, dtype=torch.bfloat16)
    timer = dp.KernelTimer(64)
    rc = RandomizedClipping(model, C=1.0, noise_multiplier=1.0, k=32, timer=timer)
    opt = torch.optim.Adam(rc.params, lr=1e-5)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    parts = {"forward": 0.0, "backward1_and_norms": 0.0, "backward2": 0.0, "noise_and_adam": 0.0}
    norm_ms, reps = 0.0, 3
    for r in range(reps + 1):
        ev[0].record()
        with rc.capture():
            losses = lb.per_sample_loss(model(x), y)
        ev[1].record()
        n, c = rc.clip_factors(losses)
        ev[2].record()
        rc.clipped_backward(losses, c)
        ev[3].record()
        rc.add_noise()
        opt.step()
        opt.zero_grad(set_to_none=True)
        ev[4].record()
        torch.cuda.synchronize()
        if r == 0:
            continue
        for j, key in enumerate(parts):
            parts[key] += ev[j].elapsed_time(ev[j + 1]) / reps
        norm_ms += sum(ms for _, ms in timer.last()) / reps
    del losses, n, c

    def plain():
        loss = lb.per_sample_loss(model(x), y).mean()
        loss.backward()
        opt.step()
        opt.zero_grad(set_to_none=True)
    plain_ms = timed(plain, reps, 1)
    step_ms = sum(parts.values())
    rc.remove()
    return {"model": "random-init Llama-3.2-1B-width stack, 2 decoder layers + output projection (vocab 2048)",
            "B": B, "T": T, "dtype": "bf16", "k": 32, "step_ms": step_ms, "parts_ms": parts,
            "norm_path_kernels_ms": norm_ms, "norm_path_share": norm_ms / step_ms,
            "nonprivate_step_ms": plain_ms, "dpsgd_rc_over_nonprivate": step_ms / plain_ms}


def sign_projection_stack(args, layers):
    """The Llama-3.2-1B-shaped stack with +-1 projections stored as bits
    (dpnorm_hutch_sign_grouped) in place of the bf16 Gaussian P."""
    import torch
    import sample_grad_norms_amd as dp
    dev = torch.device("cuda:0")
    B, T, k = 4, 4096, 32
    g = torch.Generator(device=dev)
    g.manual_seed(2024)
    triples = [(A, G, dp.random_signs(G.shape[2], k, device=dev, generator=g)) for (A, G, _) in layers]
    ws = torch.empty(dp.hutch_grouped_workspace(layers, torch.bfloat16, B, T, k), dtype=torch.uint8, device=dev)
    n = torch.empty(B, dtype=torch.float32, device=dev)
    c = torch.empty(B, dtype=torch.float32, device=dev)
    ms = timed(lambda: dp.hutch_sign_grouped(triples, k, out=n, C_clip=1.0, clip_out=c, workspace=ws),
               args.steps, args.warmup)
    return {"ms_per_step": ms, "samples_tokens_per_s": B * T / (ms * 1e-3),
            "projection_bytes_sign": sum(S.numel() * 4 for (_, _, S) in triples),
            "projection_bytes_bf16": sum(P.numel() * 2 for (_, _, P) in layers)}


def lora_stack(args):
    """LoRA factors (rank 16) of every projection of the Llama-3.2-1B-shaped
    stack (224 factors, B=4, T=4096): the routed call (exact norms, since
    every factor's narrow side is 16 <= k = 32) against the Hutchinson
    estimate with k = 32 on the same factors and against dpnorm_exact called
    per factor."""
    import torch
    import sample_grad_norms_amd as dp
    import workloads
    dev = torch.device("cuda:0")
    B, T, k = 4, 4096, 32
    layers = workloads.lora_stack(device=dev, B=B, T=T, k=k)
    inputs = {}
    for (A, G, _) in layers:
        inputs[A.data_ptr()] = A.numel() * A.element_size()
        inputs[G.data_ptr()] = G.numel() * G.element_size()
    alg = sum(inputs.values())
    n = torch.empty(B, dtype=torch.float32, device=dev)
    routed = [(A, G, None) for (A, G, _) in layers]
    ms_routed = timed(lambda: dp.norms_routed(routed, k, out=n), args.steps, args.warmup)
    ms_hutch = timed(lambda: dp.hutch_grouped(layers, out=n), args.steps, args.warmup)
    ws = torch.empty(max(dp.exact_workspace(torch.bfloat16, B, T, A.shape[2], G.shape[2]) for (A, G, _) in layers),
                     dtype=torch.uint8, device=dev)

    def exact_each():
        for j, (A, G, _) in enumerate(layers):
            dp.exact(A, G, out=n, accumulate=j > 0, workspace=ws)
    ms_exact = timed(exact_each, max(2, args.steps // 4), 1)
    out = {"factors": len(layers), "rank": 16, "algorithmic_bytes": alg,
           "routed_exact_ms": ms_routed, "routed_samples_tokens_per_s": B * T / (ms_routed * 1e-3),
           "routed_hbm_gbs": alg / (ms_routed * 1e-3) / 1e9, "hutch_k32_ms": ms_hutch,
           "exact_call_per_factor_ms": ms_exact}
    del layers, routed
    return out


def estimator_variance(pr, ws, wsh, draws=200):
    """Relative variance of n_hat / n over `draws` fresh draws of (S, P) for
    Hutch++ and of P for Hutchinson at the same budget k on the Hutch++
    workload (n from dpnorm_exact), and their ratio per sample."""
    import math
    import torch
    import sample_grad_norms_amd as dp
    dev = pr.A.device
    B, T, d = pr.A.shape
    p, k = pr.G.shape[2], pr.k
    ms_, mt = dp.hutchpp_split(k)
    n = dp.exact(pr.A, pr.G).double()
    gen = torch.Generator(device=dev)
    gen.manual_seed(4_000_999)
    hu = torch.empty(draws, B, device=dev)
    hp = torch.empty(draws, B, device=dev)
    for r in range(draws):
        P = (torch.randn(p, k, generator=gen, device=dev) / math.sqrt(k)).to(torch.bfloat16)
        S = torch.randn(p, ms_, generator=gen, device=dev).to(torch.bfloat16)
        Pt = (torch.randn(p, mt, generator=gen, device=dev) / math.sqrt(mt)).to(torch.bfloat16)
        dp.hutch(pr.A, pr.G, P, out=hu[r], workspace=wsh)
        dp.hutchpp(pr.A, pr.G, S, Pt, k=k, out=hp[r], workspace=ws)
    torch.cuda.synchronize()
    vu = (hu.double() / n).var(dim=0)
    vp = (hp.double() / n).var(dim=0)
    return {"draws": draws, "hutch_rel_var": vu.tolist(), "hutchpp_rel_var": vp.tolist(),
            "hutch_over_hutchpp": (vu / vp).tolist()}


def extras(args):
    """Other workloads: single-layer Hutchinson, Hutch++ and the exact
    comparator, each timed the same way."""
    import torch
    import sample_grad_norms_amd as dp
    import workloads
    dev = torch.device("cuda:0")
    out = {}
    steps, warm = max(5, args.steps // 2), 2
    # calls well under a millisecond: enough of them that the launch latency at
    # the start of the timed region and the clock's ramp from idle (several us
    # each) vanish in the mean; still only milliseconds of GPU time
    small_steps, small_warm = max(100, 10 * args.steps), 20

    # single layer, bf16, B=8 T=1024 d=p=2048 k=32 (67 MB: rotate 6 copies)
    sets = []
    for r in range(6):
        pr = workloads.config2(device=dev)
        if r:
            pr.A.copy_(torch.roll(pr.A, r, 1))
            pr.G.copy_(torch.roll(pr.G, r, 1))
        sets.append(pr)
    B, T, d, p = 8, 1024, 2048, 2048
    ws = torch.empty(dp.hutch_workspace(torch.bfloat16, B, T, d, p, 32), dtype=torch.uint8, device=dev)
    wse = torch.empty(dp.exact_workspace(torch.bfloat16, B, T, d, p), dtype=torch.uint8, device=dev)
    cyc = {"j": 0}

    def h2():
        pr = sets[cyc["j"] % len(sets)]
        cyc["j"] += 1
        dp.hutch(pr.A, pr.G, pr.P, workspace=ws)

    def e2():
        pr = sets[cyc["j"] % len(sets)]
        cyc["j"] += 1
        dp.exact(pr.A, pr.G, workspace=wse)
    byt = B * T * (d + p) * 2
    ms = timed(h2, small_steps, small_warm)
    mse = timed(e2, 20, 30)   # MFMA-bound: untimed calls first, until the clock has settled (about 30 calls)
    out["single_layer_B8_T1024_d2048_p2048_k32"] = {
        "hutch_ms": ms, "hutch_samples_tokens_per_s": B * T / (ms * 1e-3), "hutch_hbm_gbs": byt / ms / 1e6,
        "exact_gram_ms": mse, "exact_gram_tflops": 2 * B * T * T * (d + p) / 2 / (mse * 1e-3) / 1e12}
    del sets, ws, wse

    # Hutch++ single layer, B=4 T=4096 d=p=2048, budget 32 (11/11/10); 134 MB: rotate 4 copies
    sets = [workloads.config4(device=dev)]
    for r in range(1, 4):
        base = sets[0]
        sets.append(workloads.Problem(torch.roll(base.A, r, 1).contiguous(), torch.roll(base.G, r, 1).contiguous(),
                                      base.P, S=base.S, k=base.k))
    B, T, d, p, k = 4, 4096, 2048, 2048, 32
    ws = torch.empty(dp.hutchpp_workspace(torch.bfloat16, B, T, d, p, k), dtype=torch.uint8, device=dev)
    wsh = torch.empty(dp.hutch_workspace(torch.bfloat16, B, T, d, p, k), dtype=torch.uint8, device=dev)
    Pk = workloads.projection(p, k, 12345, dev, torch.bfloat16)

    def h4():
        pr = sets[cyc["j"] % len(sets)]
        cyc["j"] += 1
        dp.hutchpp(pr.A, pr.G, pr.S, pr.P, k=k, workspace=ws)

    def h4h():
        pr = sets[cyc["j"] % len(sets)]
        cyc["j"] += 1
        dp.hutch(pr.A, pr.G, Pk, workspace=wsh)
    ms = timed(h4, small_steps, small_warm)
    msh = timed(h4h, small_steps, small_warm)
    byt = 3 * B * T * (d + p) * 2
    out["hutchpp_B4_T4096_d2048_p2048_k32"] = {
        "hutchpp_ms": ms, "hutchpp_samples_tokens_per_s": B * T / (ms * 1e-3),
        "hutchpp_hbm_gbs_3_streams": byt / ms / 1e6, "hutch_same_inputs_ms": msh,
        "hutchpp_over_hutch_time": ms / msh,
        "variance_over_draws": estimator_variance(sets[0], ws, wsh)}
    # the ghost-clipping (Gram) route on the same T = 4096 inputs, beside Hutchinson
    wsg = torch.empty(dp.exact_workspace(torch.bfloat16, B, T, d, p, "gram"), dtype=torch.uint8, device=dev)
    msg = timed(lambda: dp.exact(sets[0].A, sets[0].G, route="gram", workspace=wsg), 10, 10)
    gram_over_hutch = msg / msh
    del sets, ws, wsh, wsg

    # the pages' relative figures (context, on their hardware where they name one), beside ours
    Bm, Tm, dm, pm, km = 4, 4096, 8192, 2048, 32   # the largest Llama-3.2-1B layer (down), T = 4096, k = 32
    ws_big = dp.hutch_workspace(torch.bfloat16, Bm, Tm, dm, pm, km)
    grads = Bm * dm * pm * 4                       # fp32 per-sample gradients, materialised
    out["pages_figures_beside_ours"] = {
        "hutch_vs_hutchpp_time": {"pages": "Hutch about 3x faster than Hutch++ (A100 80GB)",
                                  "ours": ms / msh, "workload": "B=4, T=4096, d=p=2048, budget 32"},
        "hutch_vs_ghost_clipping": {"pages": "128x fewer FLOPs at T=4096, k=32",
                                    "flop_ratio_full_gram": Tm / km,            # 2 T^2 (d+p) against 2 T k (d+p)
                                    "flop_ratio_gram_route_with_symmetry": Tm / (2 * km),
                                    "measured_time_ratio": gram_over_hutch, "ghost_gram_ms": msg,
                                    "workload": "B=4, T=4096, d=p=2048, the Gram route against Hutchinson"},
        "hutch_vs_explicit_flop_saving_largest_layer": {"pages": "98.05 %",
                                                        "closed_form": 1 - km * (dm + pm) / (dm * pm)},
        "memory_saving_excl_inputs_largest_layer": {"pages": "99.22 %", "closed_form": 1 - Tm * km / (dm * pm),
                                                    "ours_workspace_bytes": ws_big,
                                                    "ours_vs_fp32_per_sample_gradients": 1 - ws_big / grads}}

    # long context, B=1 T=32768 d=2048 p=8192: Hutchinson and the exact (explicit) comparator side by side
    pr = workloads.config5(device=dev)
    B, T, d, p = 1, 32768, 2048, 8192
    ws = torch.empty(dp.hutch_workspace(torch.bfloat16, B, T, d, p, 32), dtype=torch.uint8, device=dev)
    wse = torch.empty(dp.exact_workspace(torch.bfloat16, B, T, d, p), dtype=torch.uint8, device=dev)
    ms = timed(lambda: dp.hutch(pr.A, pr.G, pr.P, workspace=ws), small_steps, small_warm)
    mse = timed(lambda: dp.exact(pr.A, pr.G, workspace=wse), 20, 30)   # as above
    fl = 2 * T * d * p
    out["long_context_B1_T32768_d2048_p8192_k32"] = {
        "hutch_ms": ms, "hutch_samples_tokens_per_s": B * T / (ms * 1e-3),
        "hutch_hbm_gbs": B * T * (d + p) * 2 / ms / 1e6, "exact_explicit_ms": mse,
        "exact_explicit_tflops": fl / (mse * 1e-3) / 1e12,
        "exact_explicit_mfma_frac": fl / (mse * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "exact_over_hutch_time": mse / ms}
    del pr, ws, wse

    # tiny fp32 layer (latency)
    pr = workloads.config1(device=dev)
    ms = timed(lambda: dp.hutch_grouped([(pr.A, pr.G, pr.P)], C_clip=1.0), small_steps, small_warm)
    mse = timed(lambda: dp.exact(pr.A, pr.G), small_steps, small_warm)
    out["tiny_fp32_B2_T128_d64_p64_k8"] = {"hutch_clip_ms": ms, "exact_ms": mse}
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures a single GPU (the per-sample norm path needs no exchange between GPUs); "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import sample_grad_norms_amd as dp
    from sample_grad_norms_amd import profiling
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, T, k = 4, 4096, 32
    projs = [workloads.config3_projection(j, device=dev) for j in range(112)]
    layers = [(q.A, q.G, q.P) for q in projs]
    ws = torch.empty(dp.hutch_grouped_workspace(layers, torch.bfloat16, B, T, k), dtype=torch.uint8, device=dev)
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

    ms_step = timed(step, args.steps, args.warmup)

    # per-launch durations from the library's events (separate, traced steps)
    timer = dp.KernelTimer(64)
    per_kind = {}
    n_trace = max(3, min(args.steps, 10))
    for _ in range(n_trace):
        step(timer)
        for kind, ms in timer.last():
            per_kind[kind] = per_kind.get(kind, 0.0) + ms
    avg = {kk: v / n_trace for kk, v in per_kind.items()}  # per step (prepare runs several times per step)
    alg = {"rowproj": bytes_G + bytes_P, "tcontract": bytes_A}
    dom = max(alg, key=lambda kk: avg.get(kk, 0.0))
    achieved = alg[dom] / (avg[dom] * 1e-3) / 1e9
    traffic = profiling.read_traffic(PROFILE, "k_" + dom)
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
        "config": {"workload": "Llama-3.2-1B-shaped linear stack: Hutchinson per-sample norms, layer sum, clip",
                   "layers": 16, "projections": 112, "B": B, "T": T, "k": k, "C": 1.0,
                   "algorithmic_bytes": alg_bytes},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic},
        "step_hbm_gbs": alg_bytes / (ms_step * 1e-3) / 1e9,
        "step_hbm_frac": alg_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "kernel_ms": avg,
        "kernel_gbs": {kk: alg[kk] / (avg[kk] * 1e-3) / 1e9 for kk in alg if kk in avg},
        "clip_fraction": float((c < 1.0).float().mean().item()),
    }
    if not args.no_extras:
        rec["extras"] = {"hbm_calibration": hbm_calibration(dev),
                         "llama_shared_inputs_B4_T4096_k32": shared_input_stack(args),
                         "llama_stack_sign_projections_B4_T4096_k32": sign_projection_stack(args, layers),
                         "lora_r16_llama1b_B4_T4096": lora_stack(args),
                         "dpsgd_rc_step_llama1b_width_2layers_B4_T2048": dpsgd_rc_step(args)}
        rec["extras"].update(extras(args))
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(layers, B, T, max(1, min(16, args.cpu_layers)))
        del layers, projs, ws
        rec["cpu_baseline"]["per_config"] = oracle_per_config()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
