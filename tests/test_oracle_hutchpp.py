"""Pins of the oracle's Hutch++ estimate.

Hutch++ ('Efficient DP-SGD for LLMs with Randomized Clipping', papernotes.org
note, 关键设计 › Hutch++ 头-尾分解; gist.science/nl summary, Kernmechanisme):
an orthonormal Q spanning Col(O S) gives an exact head trace(Q^T O Q) and a
Hutchinson tail on (I - Q Q^T). Pins: a hand-worked example, the orthonormal
basis against a library rank and projector check, exactness when O has rank
at most m_s, invariance to the choice of basis, unbiasedness over the tail
projection with the closed-form variance 2 ||Pi O Pi||_F^2 / m_t, the m_s = 0
reduction to Hutchinson, and the budget split.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def test_hand_example():
    with open(GOLDEN) as f:
        c = {x["name"]: x for x in json.load(f)["cases"]}["hutchpp_diagonal"]
    A, G = np.array([c["A"]], float), np.array([c["G"]], float)
    n, head, tail, rank = oracle.hutchpp(A, G, np.array(c["S"], float), np.array(c["P"], float))
    assert head[0] == c["head"] and tail[0] == c["tail"] and n[0] == c["n_hutchpp"]
    assert rank[0] == 1
    assert oracle.exact_explicit(A, G)[0] == c["n_exact"]
    n2, _, t2, _ = oracle.hutchpp(A, G, np.array(c["S"], float), np.array([[1.0], [1.0]]))
    assert t2[0] == 1.0 and n2[0] == c["n_exact"]


def _golden(name):
    with open(GOLDEN) as f:
        return {x["name"]: x for x in json.load(f)["cases"]}[name]


def _frac(x):
    return x[0] / x[1]


@pytest.mark.parametrize("name", ["hutchpp_sketch_direction", "hutchpp_sketch_rectangular"])
def test_hand_examples_where_the_sketch_direction_depends_on_O(name):
    """S is not an eigenvector of O, so the basis direction, and with it the
    head, depends on every factor of O S = G^T A A^T G S: a sketch that drops
    A A^T, works in d-space or transposes G gives another head (the hand
    derivations list them)."""
    c = _golden(name)
    A, G = np.array([c["A"]], float), np.array([c["G"]], float)
    S, P = np.array(c["S"], float), np.array(c["P"], float)
    X = oracle.hutchpp_sketch(A[0], G[0], S)
    np.testing.assert_allclose(X, np.array(c["sketch"], float), rtol=0, atol=1e-12)
    n, head, tail, rank = oracle.hutchpp(A, G, S, P)
    assert math.isclose(head[0], _frac(c["head"]), rel_tol=1e-12)
    assert math.isclose(tail[0], _frac(c["tail"]), rel_tol=1e-12, abs_tol=1e-12)
    assert math.isclose(n[0], _frac(c["n_hutchpp"]), rel_tol=1e-12)
    assert rank[0] == 1
    assert oracle.exact_explicit(A, G)[0] == c["n_exact"]


def test_sketch_equals_O_times_S_with_O_built_entrywise():
    """X = O S with O[u][v] = sum_{t,s} G[t,u] (a_t . a_s) G[s,v], summed
    entry by entry in pure Python (T x T token similarities, no matrix
    product), on non-square inputs with p != d."""
    rng = np.random.default_rng(31)
    T, d, p, m = 5, 3, 4, 2
    A = rng.standard_normal((T, d))
    G = rng.standard_normal((T, p))
    S = rng.standard_normal((p, m))
    K = [[sum(A[t, u] * A[s, u] for u in range(d)) for s in range(T)] for t in range(T)]
    O = [[sum(G[t, u] * K[t][s] * G[s, v] for t in range(T) for s in range(T)) for v in range(p)]
         for u in range(p)]
    want = np.array([[sum(O[u][v] * S[v, j] for v in range(p)) for j in range(m)] for u in range(p)])
    got = oracle.hutchpp_sketch(A, G, S)
    assert got.shape == (p, m)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())
    # the head on the basis of that sketch is trace(Q^T O Q) with the same O
    Q = oracle.orthonormal_basis(got)
    head, _ = oracle.hutchpp_head_tail(A, G, Q, np.zeros((p, 1)))
    O = np.array(O)
    assert math.isclose(head, float(np.trace(Q.T @ O @ Q)), rel_tol=1e-12)


def test_budget_split():
    assert oracle.hutchpp_split(32) == (11, 10)
    assert oracle.hutchpp_split(96) == (32, 32)
    assert oracle.hutchpp_split(3) == (1, 1)
    assert oracle.hutchpp_split(4) == (2, 0)


def test_basis_orthonormal_and_spanning():
    rng = np.random.default_rng(21)
    X = rng.standard_normal((40, 7)) * np.logspace(0, 4, 7)
    Q = oracle.orthonormal_basis(X)
    assert Q.shape == (40, 7)
    np.testing.assert_allclose(Q.T @ Q, np.eye(7), atol=1e-12)
    assert np.linalg.norm(X - Q @ (Q.T @ X)) <= 1e-12 * np.linalg.norm(X)


def test_rank_threshold_is_relative_to_the_largest_column():
    """A column is kept iff its residual after the kept columns before it
    exceeds RANK_TAU times the largest column norm: residuals of 1.5 tau and
    tau / 6 of that norm fall on either side of the rule, at any overall
    scale."""
    tau = oracle.RANK_TAU
    for scale in (1e-3, 1.0, 1e5):
        e = np.eye(6)
        X = scale * np.stack([e[0], e[0] + 3 * tau * e[1], e[0] + tau / 3 * e[2], 2 * e[3], e[1]], axis=1)
        # largest column norm is 2 scale; residuals: 1 (e0), 3 tau, tau / 3, 2, then 0 after e0 and e1
        Q = oracle.orthonormal_basis(X)
        assert Q.shape[1] == 3, scale
        kept = np.abs(Q.T @ np.eye(6)) > 0.5
        assert kept[:, 0].any() and kept[:, 1].any() and kept[:, 3].any() and not kept[:, 2].any()
        # the residuals the rule compared, relative to that largest norm
        r = oracle.basis_residuals(X)
        want = np.array([1.0, 3 * tau, tau / 3, 2.0, 0.0]) / 2.0
        np.testing.assert_allclose(r, want, rtol=1e-6, atol=1e-15)
    assert np.all(oracle.basis_residuals(np.zeros((4, 3))) == 0.0)


def test_basis_rank_deficient():
    rng = np.random.default_rng(22)
    X = rng.standard_normal((30, 3)) @ rng.standard_normal((3, 8))
    X[:, 5] = 0.0
    Q = oracle.orthonormal_basis(X)
    assert Q.shape[1] == np.linalg.matrix_rank(X) == 3
    np.testing.assert_allclose(Q.T @ Q, np.eye(3), atol=1e-12)
    assert np.linalg.norm(X - Q @ (Q.T @ X)) <= 1e-12 * np.linalg.norm(X)
    assert oracle.orthonormal_basis(np.zeros((5, 3))).shape == (5, 0)


def test_exact_when_rank_at_most_sketch():
    rng = np.random.default_rng(23)
    T, d, p, r = 30, 12, 16, 3
    A = rng.standard_normal((2, T, d))
    G = np.stack([rng.standard_normal((T, r)) @ rng.standard_normal((r, p)) for _ in range(2)])
    S = rng.standard_normal((p, 5))
    P = rng.standard_normal((p, 4)) / 2.0
    n, head, tail, rank = oracle.hutchpp(A, G, S, P)
    exact = oracle.exact_explicit(A, G)
    np.testing.assert_allclose(n, exact, rtol=1e-10)
    np.testing.assert_allclose(head, exact, rtol=1e-10)
    assert np.all(tail <= 1e-10 * exact)
    assert np.all(rank == r)


def test_basis_invariance_and_bounds():
    rng = np.random.default_rng(24)
    A = rng.standard_normal((20, 9))
    G = rng.standard_normal((20, 11))
    Q = oracle.orthonormal_basis(rng.standard_normal((11, 4)))
    U, _ = np.linalg.qr(rng.standard_normal((4, 4)))
    P = rng.standard_normal((11, 3))
    h1, t1 = oracle.hutchpp_head_tail(A, G, Q, P)
    h2, t2 = oracle.hutchpp_head_tail(A, G, Q @ U, P)
    assert math.isclose(h1, h2, rel_tol=1e-12) and math.isclose(t1, t2, rel_tol=1e-12)
    n = oracle.exact_explicit(A[None], G[None])[0]
    assert 0.0 <= h1 <= n and t1 >= 0.0


def test_unbiased_over_tail_with_closed_form_variance():
    rng = np.random.default_rng(25)
    T, d, p = 16, 10, 12
    A = rng.standard_normal((T, d))
    G = rng.standard_normal((T, p)) * np.linspace(3.0, 0.2, p)
    S = rng.standard_normal((p, 3))
    m_t = 4
    Q = oracle.orthonormal_basis(oracle.hutchpp_sketch(A, G, S))
    O = G.T @ A @ A.T @ G
    Pi = np.eye(p) - Q @ Q.T
    POP = Pi @ O @ Pi
    n = float(np.trace(O))
    sd = math.sqrt(2.0 * float(np.sum(POP * POP)) / m_t)
    draws = 4000
    vals = np.empty(draws)
    r = np.random.default_rng(3)
    for j in range(draws):
        P = r.standard_normal((p, m_t)) / math.sqrt(m_t)
        vals[j] = oracle.hutchpp(A[None], G[None], S, P)[0][0]
    assert abs(vals.mean() - n) <= 4.0 * sd / math.sqrt(draws)
    assert abs(vals.var(ddof=1) / sd ** 2 - 1.0) < 0.15


def test_empty_sketch_reduces_to_hutchinson():
    rng = np.random.default_rng(26)
    A = rng.standard_normal((2, 9, 5))
    G = rng.standard_normal((2, 9, 6))
    P = rng.standard_normal((6, 4))
    n, head, tail, rank = oracle.hutchpp(A, G, np.zeros((6, 0)), P)
    np.testing.assert_allclose(n, oracle.hutch(A, G, P), rtol=1e-12)
    assert np.all(head == 0) and np.all(rank == 0)


def test_variance_below_hutchinson_on_decaying_spectrum():
    # property, not an exact pin: at equal budget the head removes the
    # dominant directions that drive Hutchinson's variance
    rng = np.random.default_rng(27)
    T, d, p, k = 24, 16, 16, 9
    A = rng.standard_normal((T, d))
    G = rng.standard_normal((T, p)) * (0.5 ** np.arange(p))
    m_s, m_t = oracle.hutchpp_split(k)
    r = np.random.default_rng(4)
    hp, hu = [], []
    for _ in range(300):
        S = r.standard_normal((p, m_s))
        P = r.standard_normal((p, m_t)) / math.sqrt(m_t)
        hp.append(oracle.hutchpp(A[None], G[None], S, P)[0][0])
        hu.append(oracle.hutch(A[None], G[None], r.standard_normal((p, k)) / math.sqrt(k))[0])
    assert np.var(hp) < 0.25 * np.var(hu)
