"""GPU parity of the exact per-sample norm ||A_i^T G_i||_F^2 (explicit and
Gram routes) against the fp64 CPU oracle ('Efficient DP-SGD for LLMs with
Randomized Clipping', papernotes.org note, 研究背景与动机: explicit
per-sample gradients versus ghost clipping)."""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu


def dev():
    return torch.device("cuda:0")


def rel(got, want):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    return np.abs(got - want) / np.maximum(np.abs(want), 1e-300)


def check(got, want, tol, what):
    e = rel(got, want)
    print(f"{what}: max rel err {e.max():.3e}", flush=True)
    assert np.all(e <= tol), e


def test_config1_fp32_exact():
    import sample_grad_norms_amd as dp
    prob = workloads.config1(device=dev())
    got = {r: dp.exact(prob.A, prob.G, route=r) for r in ("auto", "explicit", "gram")}
    torch.cuda.synchronize()
    want = oracle.exact_explicit(prob.A, prob.G)
    for r, v in got.items():
        check(v.cpu(), want, 1e-5, f"config1 exact {r}")


@pytest.mark.parametrize("dtype,tol", [(torch.bfloat16, 1e-3), (torch.float32, 1e-5)])
@pytest.mark.parametrize("B,T,d,p", [(2, 333, 264, 136), (1, 1, 8, 8), (3, 260, 1032, 520), (2, 40, 200, 72),
                                     (1, 777, 96, 40)])
@pytest.mark.parametrize("route", ["explicit", "gram"])
def test_exact_shapes(dtype, tol, B, T, d, p, route):
    import sample_grad_norms_amd as dp
    pr = workloads.random_problem(B, T, d, p, 8, seed=B + T + d, device=dev(), dtype=dtype)
    n = dp.exact(pr.A, pr.G, route=route)
    torch.cuda.synchronize()
    check(n.cpu(), oracle.exact_explicit(pr.A, pr.G), tol, f"{dtype} {route} B{B} T{T} d{d} p{p}")


def test_exact_accumulate_and_zero():
    import sample_grad_norms_amd as dp
    pr = workloads.random_problem(2, 100, 64, 32, 8, seed=1, device=dev(), dtype=torch.bfloat16)
    pr.A[1].zero_()
    base = torch.full((2,), 2.0, device=dev())
    dp.exact(pr.A, pr.G, out=base, accumulate=True)
    torch.cuda.synchronize()
    want = oracle.exact_explicit(pr.A, pr.G) + 2.0
    check(base.cpu(), want, 1e-3, "exact accumulate")
    assert base[1].item() == 2.0


def test_config2_full_size_gram():
    import sample_grad_norms_amd as dp
    prob = workloads.config2(device=dev())
    n = dp.exact(prob.A, prob.G)  # d p > T^2: the Gram route
    torch.cuda.synchronize()
    check(n.cpu(), oracle.exact_gram(prob.A, prob.G), 1e-3, "config2 exact (gram)")


def test_config5_full_size_explicit():
    import sample_grad_norms_amd as dp
    prob = workloads.config5(device=dev())
    n = dp.exact(prob.A, prob.G)  # d p <= T^2: the explicit route
    torch.cuda.synchronize()
    check(n.cpu(), oracle.exact_explicit(prob.A, prob.G), 1e-3, "config5 exact (explicit)")


@pytest.mark.parametrize("route", ["explicit", "gram"])
def test_exact_is_bitwise_deterministic(route):
    import sample_grad_norms_amd as dp
    pr = workloads.random_problem(3, 777, 264, 136, 8, seed=11, device=dev(), dtype=torch.bfloat16)
    runs = [dp.exact(pr.A, pr.G, route=route).clone() for _ in range(3)]
    torch.cuda.synchronize()
    assert all(torch.equal(runs[0], r) for r in runs[1:])
