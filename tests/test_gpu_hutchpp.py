"""GPU parity of Hutch++ against the fp64 CPU oracle (same A, G, S, P).

The estimate must match the oracle ('Efficient DP-SGD for LLMs with
Randomized Clipping', papernotes.org note, 关键设计 › Hutch++) within 1e-3
relative for bf16 inputs and 1e-5 for fp32. Where the oracle's sketch has
full rank m_s < p, the exact head ||A^T G Q||^2 and the Hutchinson tail
||A^T G (I - QQ^T) P||^2 are each held to that tolerance of their own value
(a tail below 1e-4 of the estimate, which is rounding on both sides, to that
tolerance of the estimate), the kept rank exactly, and the residuals that
decided it to the oracle's (tests/hutchpp_parity.py states the rule).
"""
import math

import numpy as np
import pytest
import torch

import hutchpp_parity
import oracle
import workloads

pytestmark = pytest.mark.gpu


def dev():
    return torch.device("cuda:0")


def rel(got, want):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    return np.abs(got - want) / np.maximum(np.abs(want), 1e-300)


def run(prob_A, prob_G, S, P, tol, what):
    import sample_grad_norms_amd as dp
    n, head, tail, rank, resid = dp.hutchpp(prob_A, prob_G, S, P, return_parts=True, return_residuals=True)
    torch.cuda.synchronize()
    want = oracle.hutchpp(prob_A, prob_G, S, P)
    print(hutchpp_parity.check(prob_A, prob_G, S, (n, head, tail, rank), want, tol, what, resid=resid), flush=True)
    return n, head, tail, resid


@pytest.mark.parametrize("dtype,tol", [(torch.bfloat16, 1e-3), (torch.float32, 1e-5)])
@pytest.mark.parametrize("B,T,d,p,k", [(2, 300, 264, 136, 32), (3, 77, 64, 520, 3), (1, 1000, 1032, 64, 96),
                                       (2, 129, 8, 16, 12),
                                       # sketches of lower rank than m_s (T = 2; d = 16 < m_s = 32): the
                                       # dependent columns' residuals are rounding, far below the threshold
                                       (7, 2, 1000, 480, 32), (3, 1500, 16, 88, 96)])
def test_hutchpp_shapes(dtype, tol, B, T, d, p, k):
    ms, mt = oracle.hutchpp_split(k)
    pr = workloads.random_problem(B, T, d, p, k, seed=T + d + k, device=dev(), dtype=dtype)
    S = workloads.gaussian((p, ms), 1.0, 900 + k, dev(), dtype)
    P = workloads.projection(p, mt, 901 + k, dev(), dtype)
    run(pr.A, pr.G, S, P, tol, f"{dtype} B{B} T{T} d{d} p{p} k{k}")


def test_hutchpp_low_rank_is_exact_and_zero_sample():
    """G of rank <= m_s: the head captures everything, the tail vanishes and
    the estimate equals the exact norm; a zero sample gives rank 0 and 0."""
    import sample_grad_norms_amd as dp
    B, T, d, p, k = 3, 256, 128, 96, 24
    ms, mt = oracle.hutchpp_split(k)
    g = torch.Generator().manual_seed(5)
    A = torch.randn(B, T, d, generator=g)
    U = torch.randn(B, T, 3, generator=g)
    V = torch.randn(B, 3, p, generator=g)
    G = U @ V
    G[2].zero_()
    A, G = A.to(dev()), G.to(dev())
    S = workloads.gaussian((p, ms), 1.0, 17, dev())
    P = workloads.projection(p, mt, 18, dev())
    n, head, tail, rank = dp.hutchpp(A, G, S, P, return_parts=True)
    torch.cuda.synchronize()
    exact = oracle.exact_explicit(A, G)
    assert rank.cpu().tolist() == [3, 3, 0]
    assert np.all(rel(n.cpu()[:2], exact[:2]) <= 1e-5)
    assert float(tail[:2].abs().max()) <= 1e-5 * float(n[:2].min())
    assert n[2].item() == 0.0 and head[2].item() == 0.0 and tail[2].item() == 0.0


def test_config4_full_size():
    prob = workloads.config4(device=dev())
    n, head, tail, resid = run(prob.A, prob.G, prob.S, prob.P, 1e-3, prob.name)
    # the structured workload puts almost all of the norm in the head
    assert float((tail / n).max()) < 0.05
    # Every sketch column is kept on both sides, by a margin that rounding
    # cannot close. The kernel's residuals carry the rounding of its fp32
    # sketch of bf16 data, at most about 1e-5 of the largest column norm
    # (0.1 tau): each side must clear the threshold by twice that, and the
    # two sides must agree to well within it.
    wres = hutchpp_parity.oracle_residuals(prob.A, prob.G, prob.S)
    for side, r in (("kernel", resid), ("oracle", wres)):
        kept_min, dropped_max = hutchpp_parity.margins(r)
        print(f"{side}: smallest kept residual {kept_min:.3f} tau, largest dropped {dropped_max:.2f} tau", flush=True)
        assert kept_min >= 1.2 and dropped_max <= 0.8
    diff = float(np.abs(resid.cpu().double().numpy() - wres).max())
    print(f"largest residual difference kernel - oracle: {diff / oracle.RANK_TAU:.4f} tau", flush=True)
    assert diff <= 0.05 * oracle.RANK_TAU


def test_hutchpp_accumulates():
    import sample_grad_norms_amd as dp
    pr = workloads.random_problem(2, 200, 136, 64, 32, seed=3, device=dev(), dtype=torch.bfloat16)
    ms, mt = oracle.hutchpp_split(32)
    S = workloads.gaussian((64, ms), 1.0, 4, dev(), torch.bfloat16)
    P = workloads.projection(64, mt, 5, dev(), torch.bfloat16)
    base = torch.full((2,), 3.0, device=dev())
    dp.hutchpp(pr.A, pr.G, S, P, out=base, accumulate=True)
    torch.cuda.synchronize()
    want = oracle.hutchpp(pr.A, pr.G, S, P)[0] + 3.0
    assert np.all(rel(base.cpu(), want) <= 1e-3)


def test_hutchpp_is_bitwise_deterministic():
    """Every work group of the apply kernel forms its sample's basis itself;
    they must agree, and repeated calls must give the same bits."""
    import sample_grad_norms_amd as dp
    B, T, d, p, k = 3, 600, 264, 520, 32
    ms, mt = oracle.hutchpp_split(k)
    pr = workloads.random_problem(B, T, d, p, k, seed=21, device=dev(), dtype=torch.bfloat16)
    S = workloads.gaussian((p, ms), 1.0, 22, dev(), torch.bfloat16)
    P = workloads.projection(p, mt, 23, dev(), torch.bfloat16)
    runs = [tuple(t.clone() for t in dp.hutchpp(pr.A, pr.G, S, P, return_parts=True)) for _ in range(3)]
    torch.cuda.synchronize()
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert torch.equal(a, b)
