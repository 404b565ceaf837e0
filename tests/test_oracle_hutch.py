"""Pins of the oracle's Hutchinson estimate.

The estimate is n_hat = ||A^T (G P)||_F^2 = trace(P^T O P), O = G^T A A^T G,
P with i.i.d. N(0, 1/k) entries ('Efficient DP-SGD for LLMs with Randomized
Clipping', papernotes.org note, 关键设计 › Hutchinson 随机投影估范数). Pins:
hand-worked values, P = I (the estimate is then exact), T = 1 closed form,
column additivity and scaling, the trace form, and its law: with
lambda = eigenvalues of W^T W (W = A^T G), n_hat = sum_m lambda_m chi2_m(k)/k,
so E n_hat = n and Var n_hat = 2 ||lambda||_2^2 / k; for rank-one W the ratio
n_hat / n is exactly chi2(k)/k (the law of Z^2 in the note's f-DP section),
and the (1 +- alpha) miss probability obeys the chi2(k)/k Chernoff bound for
every spectrum.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy import stats

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _case(name):
    with open(GOLDEN) as f:
        return {c["name"]: c for c in json.load(f)["cases"]}[name]


@pytest.mark.parametrize("name", ["exact_and_hutch_nonsymmetric", "exact_rectangular"])
def test_hand_examples(name):
    c = _case(name)
    got = oracle.hutch(np.array([c["A"]], float), np.array([c["G"]], float), np.array(c["P"], float))
    assert got[0] == c["n_hutch"]


def test_identity_projection_is_exact():
    rng = np.random.default_rng(11)
    A = rng.standard_normal((3, 9, 5))
    G = rng.standard_normal((3, 9, 6))
    np.testing.assert_allclose(oracle.hutch(A, G, np.eye(6)), oracle.exact_explicit(A, G), rtol=1e-12)


def test_single_token_closed_form():
    rng = np.random.default_rng(12)
    a, g = rng.standard_normal(7), rng.standard_normal(5)
    P = rng.standard_normal((5, 3))
    ptg = [sum(P[v][j] * g[v] for v in range(5)) for j in range(3)]
    want = sum(x * x for x in a) * sum(y * y for y in ptg)
    got = oracle.hutch(a.reshape(1, 1, 7), g.reshape(1, 1, 5), P)[0]
    assert math.isclose(got, want, rel_tol=1e-12)


def test_column_additivity_scaling_trace_form():
    rng = np.random.default_rng(13)
    A = rng.standard_normal((2, 10, 4))
    G = rng.standard_normal((2, 10, 6))
    P = rng.standard_normal((6, 5))
    n = oracle.hutch(A, G, P)
    cols = sum(oracle.hutch(A, G, P[:, j:j + 1]) for j in range(5))
    np.testing.assert_allclose(cols, n, rtol=1e-12)
    np.testing.assert_allclose(oracle.hutch(A, G, 3.0 * P), 9.0 * n, rtol=1e-12)
    np.testing.assert_allclose(oracle.hutch_trace_form(A, G, P), n, rtol=1e-11)


def _spectrum(A, G):
    W = A.T @ G
    s = np.linalg.svd(W, compute_uv=False)
    return s ** 2


def _draws(A, G, k, S, seed):
    rng = np.random.default_rng(seed)
    out = np.empty(S)
    for r in range(S):
        P = rng.standard_normal((G.shape[1], k)) / math.sqrt(k)
        out[r] = oracle.hutch(A[None], G[None], P)[0]
    return out


def test_unbiased_with_closed_form_variance():
    rng = np.random.default_rng(14)
    A = rng.standard_normal((6, 5))
    G = rng.standard_normal((6, 4)) * np.array([3.0, 1.0, 0.5, 0.2])
    lam = _spectrum(A, G)
    n = float(lam.sum())
    assert math.isclose(n, oracle.exact_explicit(A[None], G[None])[0], rel_tol=1e-12)
    k, S = 8, 4000
    x = _draws(A, G, k, S, 99) / n
    sd = math.sqrt(2.0 * float(np.sum(lam ** 2)) / k) / n
    assert abs(x.mean() - 1.0) <= 4.0 * sd / math.sqrt(S)
    assert abs(x.var(ddof=1) / sd ** 2 - 1.0) < 0.15


def test_rank_one_law_is_chi2_over_k():
    rng = np.random.default_rng(15)
    a, g = rng.standard_normal((1, 6)), rng.standard_normal((1, 5))  # T = 1
    n = oracle.exact_explicit(a[None], g[None])[0]
    k, S = 8, 10000
    x = _draws(a, g, k, S, 7) / n
    res = stats.kstest(x, stats.chi2(df=k, scale=1.0 / k).cdf)
    assert res.pvalue > 1e-3, res


def _chernoff(k, alpha):
    up = math.exp(-(k / 2.0) * (alpha - math.log1p(alpha)))
    lo = math.exp(-(k / 2.0) * (-alpha - math.log1p(-alpha)))
    return up + lo


@pytest.mark.parametrize("k,alpha", [(32, 0.5), (8, 0.75)])
def test_concentration_within_chernoff_bound(k, alpha):
    rng = np.random.default_rng(16)
    A = rng.standard_normal((5, 4))
    G = rng.standard_normal((5, 3))
    S = 3000
    x = _draws(A, G, k, S, 5) / oracle.exact_explicit(A[None], G[None])[0]
    miss = float(np.mean(np.abs(x - 1.0) >= alpha))
    bound = _chernoff(k, alpha)
    assert miss <= bound + 3.0 * math.sqrt(bound / S)


def test_rank_one_miss_rate_matches_chi2():
    # rank one is the extreme spectrum: the miss rate is the chi2(k)/k tail
    a, g = np.ones((1, 3)), np.ones((1, 2))
    k, alpha, S = 32, 0.5, 6000
    x = _draws(a, g, k, S, 8) / 6.0
    miss = float(np.mean(np.abs(x - 1.0) >= alpha))
    d = stats.chi2(df=k, scale=1.0 / k)
    want = d.sf(1 + alpha) + d.cdf(1 - alpha)
    assert abs(miss - want) <= 4.0 * math.sqrt(want * (1 - want) / S)
    assert want <= _chernoff(k, alpha)
