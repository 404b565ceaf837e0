"""Pins of the oracle's exact routes against things other than itself:
hand-worked examples, brute force in pure-Python loops, closed forms and
special cases with a known answer.

Identity used: ||A^T G||_F^2 = trace(G^T A A^T G) ('Efficient DP-SGD for LLMs
with Randomized Clipping', papernotes.org note, 切入角度; gist.science/nl
summary, Kernmechanisme).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _cases():
    with open(GOLDEN) as f:
        return {c["name"]: c for c in json.load(f)["cases"]}


def brute_force_norm(A, G):
    """Materialise W_uv = sum_t A[t][u] G[t][v] with Python loops."""
    T, d = len(A), len(A[0])
    p = len(G[0])
    total = 0.0
    for u in range(d):
        for v in range(p):
            w = 0.0
            for t in range(T):
                w += A[t][u] * G[t][v]
            total += w * w
    return total


@pytest.mark.parametrize("name", ["exact_and_hutch_nonsymmetric", "exact_rectangular"])
def test_hand_examples_exact(name):
    c = _cases()[name]
    A = np.array([c["A"]], dtype=float)
    G = np.array([c["G"]], dtype=float)
    for fn in (oracle.exact_explicit, oracle.exact_gram, oracle.exact_trace):
        assert fn(A, G)[0] == c["n_exact"], fn.__name__


@pytest.mark.parametrize("seed", range(6))
def test_three_routes_match_brute_force(seed):
    rng = np.random.default_rng(seed)
    B, T, d, p = 2, int(rng.integers(1, 7)), int(rng.integers(1, 5)), int(rng.integers(1, 5))
    A = rng.standard_normal((B, T, d))
    G = rng.standard_normal((B, T, p))
    bf = np.array([brute_force_norm(A[i].tolist(), G[i].tolist()) for i in range(B)])
    for fn in (oracle.exact_explicit, oracle.exact_gram, oracle.exact_trace):
        np.testing.assert_allclose(fn(A, G), bf, rtol=1e-12, err_msg=fn.__name__)


def test_routes_agree_medium():
    rng = np.random.default_rng(7)
    A = rng.standard_normal((3, 40, 17))
    G = rng.standard_normal((3, 40, 23))
    e1 = oracle.exact_explicit(A, G)
    np.testing.assert_allclose(oracle.exact_gram(A, G), e1, rtol=1e-12)
    np.testing.assert_allclose(oracle.exact_trace(A, G), e1, rtol=1e-12)
    # library routine, different contraction order
    ein = np.einsum("btu,btv->buv", A, G)
    np.testing.assert_allclose((ein ** 2).sum(axis=(1, 2)), e1, rtol=1e-12)


def test_single_token_closed_form():
    # T = 1: W = a g^T is rank one, so ||W||_F^2 = ||a||^2 ||g||^2
    rng = np.random.default_rng(3)
    a = rng.standard_normal(9)
    g = rng.standard_normal(5)
    want = sum(x * x for x in a) * sum(y * y for y in g)
    got = oracle.exact_explicit(a.reshape(1, 1, 9), g.reshape(1, 1, 5))[0]
    assert math.isclose(got, want, rel_tol=1e-13)


def test_scaling_and_zero():
    rng = np.random.default_rng(4)
    A = rng.standard_normal((2, 11, 6))
    G = rng.standard_normal((2, 11, 7))
    n = oracle.exact_explicit(A, G)
    np.testing.assert_allclose(oracle.exact_gram(3.0 * A, -0.5 * G), 9.0 * 0.25 * n, rtol=1e-12)
    assert np.all(oracle.exact_explicit(0 * A, G) == 0)
    assert np.all(oracle.exact_gram(A, 0 * G) == 0)


def test_orthogonal_activations():
    # A square orthogonal (A A^T = I): ||A^T G||_F^2 = ||G||_F^2
    rng = np.random.default_rng(5)
    Qm, _ = np.linalg.qr(rng.standard_normal((8, 8)))
    G = rng.standard_normal((1, 8, 5))
    want = float(np.sum(G * G))
    for fn in (oracle.exact_explicit, oracle.exact_gram, oracle.exact_trace):
        assert math.isclose(fn(Qm[None], G)[0], want, rel_tol=1e-12)


def test_orthonormal_columns_projection():
    # T > d with A^T A = I: A A^T is the orthogonal projector onto span(A), so
    # the norm is the energy of G inside that span: ||G||^2 - ||G - A A^T G||^2.
    rng = np.random.default_rng(6)
    Qm, _ = np.linalg.qr(rng.standard_normal((12, 4)))
    G = rng.standard_normal((12, 3))
    resid = G - Qm @ (Qm.T @ G)
    want = float(np.sum(G * G) - np.sum(resid * resid))
    got = oracle.exact_explicit(Qm[None], G[None])[0]
    assert math.isclose(got, want, rel_tol=1e-11)


def test_bf16_inputs_convert_exactly():
    torch = pytest.importorskip("torch")
    A = torch.randn(1, 5, 3).to(torch.bfloat16)
    G = torch.randn(1, 5, 2).to(torch.bfloat16)
    Af = [[float(x) for x in row] for row in A[0].tolist()]
    Gf = [[float(x) for x in row] for row in G[0].tolist()]
    assert math.isclose(oracle.exact_explicit(A, G)[0], brute_force_norm(Af, Gf), rel_tol=1e-13)
