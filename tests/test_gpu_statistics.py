"""Statistics of the GPU estimators over many random projections.

'Efficient DP-SGD for LLMs with Randomized Clipping' (papernotes.org note):
关键设计 › Hutchinson (P with N(0, 1/k) entries gives an unbiased estimate
that concentrates within (1 +- alpha) at k = O(log(1/beta) / alpha^2)),
› Hutch++ (the exact head removes the dominant directions), and 实验关键数据 ›
关键发现 (Hutch++ about an order of magnitude more accurate than Hutchinson).

Each draw is one call of the HIP path with a fresh projection drawn on the
device; the exact norms come from dpnorm_exact, itself checked against the
fp64 oracle here. Checks:
  * unbiasedness: the mean over S draws is within 4 sd / sqrt(S) of n;
  * variance: Hutchinson's sample variance lies in the chi-square 99.9 %
    interval around the closed form 2 ||O||_F^2 / k (O = G^T A A^T G);
  * Hutch++ against Hutchinson at equal budget on the structured Hutch++
    workload (rank-8 G with halving singular values over a noise floor):
    variance at least ten times lower;
  * the law: for one token (W = a g^T of rank 1), n_hat / n is distributed
    as chi^2(k) / k exactly (Kolmogorov-Smirnov, p > 1e-3);
  * (1 +- alpha) concentration: the miss fraction stays below the chi-square
    Chernoff bound, which holds for every spectrum.
"""
import math

import numpy as np
import pytest
import torch
from scipy import stats

import oracle
import workloads

pytestmark = pytest.mark.gpu

DRAWS = 200


def dev():
    return torch.device("cuda:0")


def chernoff_miss_bound(k, alpha):
    """P(|chi^2(k)/k - 1| >= alpha) <= exp(-k/2 (a - ln(1+a))) + exp(-k/2 (-a - ln(1-a)))."""
    up = math.exp(-0.5 * k * (alpha - math.log1p(alpha)))
    down = math.exp(-0.5 * k * (-alpha - math.log1p(-alpha))) if alpha < 1 else 0.0
    return up + down


def frob2_of_O(A, G):
    """||O_i||_F^2 = ||W_i^T W_i||_F^2 with W_i = A_i^T G_i, fp64 on the host."""
    A, G = oracle.to_f64(A), oracle.to_f64(G)
    out = np.empty(A.shape[0])
    for i in range(A.shape[0]):
        W = A[i].T @ G[i]
        M = W.T @ W
        out[i] = float(np.sum(M * M))
    return out


def test_hutch_and_hutchpp_over_draws_on_the_hutchpp_workload():
    import sample_grad_norms_amd as dp
    prob = workloads.config4(device=dev())
    B, T, d, p = prob.shape
    k = prob.k
    ms, mt = oracle.hutchpp_split(k)
    n_exact = dp.exact(prob.A, prob.G)
    torch.cuda.synchronize()
    ne = n_exact.cpu().double().numpy()
    want = oracle.exact_explicit(prob.A, prob.G)
    assert np.all(np.abs(ne - want) <= 1e-3 * want)
    gen = torch.Generator(device=dev()).manual_seed(4_000_777)
    hu = torch.empty(DRAWS, B, device=dev())
    hp = torch.empty(DRAWS, B, device=dev())
    ws_h = torch.empty(dp.hutch_workspace(torch.bfloat16, B, T, d, p, k), dtype=torch.uint8, device=dev())
    ws_p = torch.empty(dp.hutchpp_workspace(torch.bfloat16, B, T, d, p, k), dtype=torch.uint8, device=dev())
    for r in range(DRAWS):
        P = (torch.randn(p, k, generator=gen, device=dev()) / math.sqrt(k)).to(torch.bfloat16)
        S = torch.randn(p, ms, generator=gen, device=dev()).to(torch.bfloat16)
        Pt = (torch.randn(p, mt, generator=gen, device=dev()) / math.sqrt(mt)).to(torch.bfloat16)
        dp.hutch(prob.A, prob.G, P, out=hu[r], workspace=ws_h)
        dp.hutchpp(prob.A, prob.G, S, Pt, out=hp[r], workspace=ws_p)
    torch.cuda.synchronize()
    hu, hp = hu.cpu().double().numpy() / ne, hp.cpu().double().numpy() / ne
    sd_closed = np.sqrt(2.0 * frob2_of_O(prob.A, prob.G) / k) / ne
    var_u, var_p = hu.var(axis=0, ddof=1), hp.var(axis=0, ddof=1)
    print(f"hutch: mean n_hat/n {hu.mean(0).round(4).tolist()} sd {np.sqrt(var_u).round(4).tolist()} "
          f"(closed form {sd_closed.round(4).tolist()})", flush=True)
    print(f"hutch++: mean n_hat/n {hp.mean(0).round(6).tolist()} sd {np.sqrt(var_p).round(6).tolist()}; "
          f"variance ratio hutch / hutch++ {(var_u / var_p).round(1).tolist()}", flush=True)
    # unbiased
    assert np.all(np.abs(hu.mean(0) - 1.0) <= 4.0 * sd_closed / math.sqrt(DRAWS))
    assert np.all(np.abs(hp.mean(0) - 1.0) <= 4.0 * np.sqrt(var_p) / math.sqrt(DRAWS))
    # Hutchinson's variance against the closed form (99.9 % chi-square interval)
    lo, hi = (stats.chi2.ppf(q, DRAWS - 1) / (DRAWS - 1) for q in (0.0005, 0.9995))
    assert np.all((var_u / sd_closed ** 2 >= lo) & (var_u / sd_closed ** 2 <= hi))
    # Hutch++ an order of magnitude (in variance) more accurate at equal budget
    assert np.all(var_u >= 10.0 * var_p)
    # (1 +- alpha) concentration of Hutchinson at alpha = 0.75
    bound = chernoff_miss_bound(k, 0.75)
    miss = np.mean(np.abs(hu - 1.0) >= 0.75, axis=0)
    assert np.all(miss <= bound + 3.0 * math.sqrt(bound / DRAWS))


def test_hutch_variance_matches_the_closed_form_on_a_flat_spectrum():
    """Gaussian A and G (no dominant direction): the sample variance of
    n_hat over 2000 draws against 2 ||O||_F^2 / k, and the mean against n."""
    import sample_grad_norms_amd as dp
    B, T, d, p, k, draws = 2, 96, 64, 72, 16, 2000
    pr = workloads.random_problem(B, T, d, p, k, seed=41, device=dev(), dtype=torch.bfloat16)
    ne = oracle.exact_explicit(pr.A, pr.G)
    sd = np.sqrt(2.0 * frob2_of_O(pr.A, pr.G) / k)
    gen = torch.Generator(device=dev()).manual_seed(42)
    est = torch.empty(draws, B, device=dev())
    ws = torch.empty(dp.hutch_workspace(torch.bfloat16, B, T, d, p, k), dtype=torch.uint8, device=dev())
    for r in range(draws):
        P = (torch.randn(p, k, generator=gen, device=dev()) / math.sqrt(k)).to(torch.bfloat16)
        dp.hutch(pr.A, pr.G, P, out=est[r], workspace=ws)
    torch.cuda.synchronize()
    e = est.cpu().double().numpy()
    var = e.var(axis=0, ddof=1)
    print(f"flat spectrum: mean/n {(e.mean(0) / ne).round(4).tolist()} var/closed form {(var / sd ** 2).round(3).tolist()}",
          flush=True)
    assert np.all(np.abs(e.mean(0) - ne) <= 4.0 * sd / math.sqrt(draws))
    lo, hi = (stats.chi2.ppf(q, draws - 1) / (draws - 1) for q in (0.0005, 0.9995))
    assert np.all((var / sd ** 2 >= lo) & (var / sd ** 2 <= hi))


def test_rank_one_estimate_is_chi_square_over_k():
    """One token: n = ||a||^2 ||g||^2 and n_hat / n = ||P^T g||^2 / ||g||^2,
    a sum of k squares of N(0, 1/k) variables, whatever a and g are."""
    import sample_grad_norms_amd as dp
    d, p, k, draws = 256, 256, 32, 2000
    pr = workloads.random_problem(1, 1, d, p, k, seed=43, device=dev(), dtype=torch.bfloat16)
    a, g = oracle.to_f64(pr.A)[0, 0], oracle.to_f64(pr.G)[0, 0]
    n = float(a @ a) * float(g @ g)
    gen = torch.Generator(device=dev()).manual_seed(44)
    est = torch.empty(draws, 1, device=dev())
    ws = torch.empty(dp.hutch_workspace(torch.bfloat16, 1, 1, d, p, k), dtype=torch.uint8, device=dev())
    for r in range(draws):
        P = (torch.randn(p, k, generator=gen, device=dev()) / math.sqrt(k)).to(torch.bfloat16)
        dp.hutch(pr.A, pr.G, P, out=est[r], workspace=ws)
    torch.cuda.synchronize()
    ratio = est.cpu().double().numpy()[:, 0] / n
    ks = stats.kstest(ratio, stats.chi2(k, scale=1.0 / k).cdf)
    print(f"rank 1: mean {ratio.mean():.4f} var {ratio.var():.4f} (chi2/k: 1, {2 / k:.4f}); KS p = {ks.pvalue:.3g}",
          flush=True)
    assert ks.pvalue > 1e-3
