"""GPU parity of the one-launch Hutchinson call (one bf16 layer, P read in
place, k = 16 or 32, B a multiple of 8, a small call) against the fp64 CPU
oracle. In that call sample i is handled by the work groups of XCD i % 8:
stage 1 and stage 2 of the sample hand over through that XCD's L2, and the
last stage-2 item of a sample sums the items' sums and writes n (and c).

Shapes are ragged in T (against the 32-row stage-1 items and the four
quarters of stage 2), in d (against the 64-column stage-2 items) and in p
(against the 64-column chunks of stage 1). Also: accumulation, the clip
factors of the one-layer grouped call, bitwise repeatability, and the bounded
wait of a stage-2 item (forced to give up from the host: every sample is then
either the right value or NaN).
"""
import math
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skip(reason="the one-launch path is switched off: its first GPU runs did not finish within 120 s "
                            "(cause not established); these tests stay for when it is fixed"),
]

TOL = 1e-3


def dev():
    return torch.device("cuda:0")


def check(got, want, what):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want) / np.abs(want)
    print(f"{what}: max rel err {err.max():.3e}", flush=True)
    assert np.all(err <= TOL), f"{what}: rel err {err} > {TOL}"


@pytest.mark.parametrize("B,T,d,p,k", [(8, 1024, 2048, 2048, 32), (8, 1000, 1000, 520, 32), (16, 77, 136, 264, 16),
                                       (24, 300, 2056, 64, 32), (8, 2048, 64, 4096, 16), (16, 33, 8192, 8, 32)])
def test_one_launch_shapes(B, T, d, p, k):
    import sample_grad_norms_amd as dp
    pr = workloads.random_problem(B, T, d, p, k, seed=B + T + d, device=dev(), dtype=torch.bfloat16)
    n = dp.hutch(pr.A, pr.G, pr.P)
    torch.cuda.synchronize()
    check(n.cpu(), oracle.hutch(pr.A, pr.G, pr.P), f"one launch B{B} T{T} d{d} p{p} k{k}")


def test_one_launch_accumulates_clips_and_repeats_bitwise():
    import sample_grad_norms_amd as dp
    B, T, d, p, k = 16, 512, 1032, 520, 32
    pr = workloads.random_problem(B, T, d, p, k, seed=81, device=dev(), dtype=torch.bfloat16)
    want = oracle.hutch(pr.A, pr.G, pr.P)
    base = torch.linspace(1.0, 2.0, B, device=dev())
    n = base.clone()
    dp.hutch(pr.A, pr.G, pr.P, out=n, accumulate=True)
    torch.cuda.synchronize()
    check(n.cpu() - base.cpu(), want, "accumulated")
    C = float(np.sqrt(np.median(want)))
    c = torch.empty(B, device=dev())
    n2 = dp.hutch_grouped([(pr.A, pr.G, pr.P)], C_clip=C, clip_out=c)
    torch.cuda.synchronize()
    check(n2.cpu(), want, "grouped, one layer")
    cw = oracle.clip_factors(want, C)
    assert np.all(np.abs(c.cpu().numpy() - cw) <= TOL * cw)
    outs = [dp.hutch(pr.A, pr.G, pr.P) for _ in range(5)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


_CHILD = r'''
import sys
sys.path.insert(0, sys.argv[1])
import numpy as np, torch
import sample_grad_norms_amd as dp, workloads, oracle
pr = workloads.random_problem(8, 1024, 2048, 2048, 32, seed=83, device=torch.device("cuda:0"), dtype=torch.bfloat16)
want = oracle.hutch(pr.A, pr.G, pr.P)
for rep in range(5):
    n = dp.hutch(pr.A, pr.G, pr.P).cpu().numpy().astype(np.float64)
    ok = np.isnan(n) | (np.abs(n - want) <= 1e-3 * want)
    print("rep", rep, "nan", int(np.isnan(n).sum()), "ok", bool(ok.all()), flush=True)
    assert ok.all(), (n, want)
print("done", flush=True)
'''


def test_one_launch_wait_gives_up_with_nan():
    """With a spin limit of zero a stage-2 item that finds its sample's stage
    1 unfinished gives up at once: that sample's n is NaN, the others are
    right, and the kernel ends (run in a child process with the limit set)."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, DPNORM_XCD_SPIN_LIMIT="0")
    res = subprocess.run([sys.executable, "-c", _CHILD, root], capture_output=True, text=True, timeout=300, env=env,
                         cwd=root)
    print(res.stdout.strip(), flush=True)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert "done" in res.stdout
