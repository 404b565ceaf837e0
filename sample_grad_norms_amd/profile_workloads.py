"""Runs one named single-layer workload a few times, for profiling with
rocprofv3 (the 112-projection stack is profiled through bench.py).

    python sample_grad_norms_amd/profile_workloads.py NAME [--reps R] [--calib-copy]

NAME is one of:
  long_context_hutch  Hutchinson, B=1, T=32768, d=2048, p=8192, k=32
  long_context_exact  the exact explicit route on the same inputs
  hutchpp             Hutch++, B=4, T=4096, d=p=2048, budget 32
  single_layer        Hutchinson, B=8, T=1024, d=p=2048, k=32
  single_layer_gram   the exact Gram route on the same inputs
--calib-copy first runs one 1 GiB device-to-device copy, the reference the
counter summaries scale FETCH_SIZE and WRITE_SIZE by.
"""
from __future__ import annotations

import argparse
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

NAMES = ("long_context_hutch", "long_context_exact", "hutchpp", "single_layer", "single_layer_gram")


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("name", choices=NAMES)
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--calib-copy", action="store_true")
    a = ap.parse_args()
    import torch
    import sample_grad_norms_amd as dp
    import workloads
    dev = torch.device("cuda:0")
    if a.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src
    if a.name.startswith("long_context"):
        pr = workloads.config5(device=dev)
        fn = (lambda: dp.hutch(pr.A, pr.G, pr.P)) if a.name.endswith("hutch") else (lambda: dp.exact(pr.A, pr.G))
    elif a.name == "hutchpp":
        pr = workloads.config4(device=dev)
        fn = lambda: dp.hutchpp(pr.A, pr.G, pr.S, pr.P, k=pr.k)
    else:
        pr = workloads.config2(device=dev)
        fn = (lambda: dp.exact(pr.A, pr.G, route="gram")) if a.name.endswith("gram") else (lambda: dp.hutch(pr.A, pr.G, pr.P))
    for _ in range(a.reps):
        fn()
    torch.cuda.synchronize()
    print(f"{a.name}: {a.reps} calls done", flush=True)


if __name__ == "__main__":
    main()
