"""Pins of the oracle's Hutchinson estimate with +-1 projections stored as
bits (P = S / sqrt(k), S in {-1,+1}; note 实验关键数据 › 关键发现 and
局限与展望, {-1,+1} 1-bit projections in the style of Achlioptas).

Independent of the oracle's own formula: hand-worked values; exact
unbiasedness and the exact variance 2 (||O||_F^2 - sum_u O_uu^2) over the
enumeration of all sign vectors; exactness for a diagonal O whatever the
signs; and the Rademacher statistics of random words.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sign_examples.json")
CASES = json.load(open(GOLDEN))["cases"]


def pack(S):
    """Plain-Python packing of a {-1,+1} matrix [p][k] into rows of words."""
    p, k = S.shape
    words = np.zeros((p, (k + 31) // 32), dtype=np.uint32)
    for v in range(p):
        for j in range(k):
            if S[v, j] < 0:
                words[v, j // 32] |= np.uint32(1 << (j % 32))
    return words


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_hand_examples(case):
    A = np.array(case["A"], dtype=np.float64)[None]
    G = np.array(case["G"], dtype=np.float64)[None]
    words = np.array(case["words"], dtype=np.uint32)
    got = oracle.hutch_sign(A, G, words, case["k"])
    assert got[0] == pytest.approx(case["n_hat"], rel=1e-14)


def test_enumeration_is_unbiased_with_the_rademacher_variance():
    rng = np.random.default_rng(3)
    A = rng.standard_normal((2, 6, 4))
    G = rng.standard_normal((2, 6, 5))
    n = oracle.exact_trace(A, G)
    vals = []
    for signs in itertools.product([1.0, -1.0], repeat=5):
        S = np.array(signs)[:, None]
        vals.append(oracle.hutch_sign(A, G, pack(S), 1))
    vals = np.array(vals)                        # [32][B]
    np.testing.assert_allclose(vals.mean(axis=0), n, rtol=1e-12)
    for i in range(2):
        O = G[i].T @ A[i] @ A[i].T @ G[i]
        var = 2.0 * (np.sum(O * O) - np.sum(np.diag(O) ** 2))
        assert vals[:, i].var() == pytest.approx(var, rel=1e-10)


def test_diagonal_O_is_exact_for_any_signs():
    # A with orthonormal columns (T = d) and G with orthogonal columns give
    # O = G^T G diagonal: every sign vector then returns the exact norm
    rng = np.random.default_rng(4)
    Qa, _ = np.linalg.qr(rng.standard_normal((8, 8)))
    Qg, _ = np.linalg.qr(rng.standard_normal((8, 5)))
    G = Qg * np.array([1.0, 2.0, 3.0, 0.5, 4.0])
    A, G = Qa[None], G[None]
    n = oracle.exact_trace(A, G)
    for seed in range(5):
        words = np.random.default_rng(seed).integers(0, 2 ** 32, size=(5, 2), dtype=np.uint64).astype(np.uint32)
        np.testing.assert_allclose(oracle.hutch_sign(A, G, words, 40), n, rtol=1e-12)


def test_random_words_give_an_unbiased_estimate():
    rng = np.random.default_rng(5)
    A = rng.standard_normal((1, 10, 6))
    G = rng.standard_normal((1, 10, 7))
    n = oracle.exact_trace(A, G)[0]
    O = G[0].T @ A[0] @ A[0].T @ G[0]
    k, S = 8, 3000
    sd = math.sqrt(2.0 * (np.sum(O * O) - np.sum(np.diag(O) ** 2)) / k)
    est = np.array([oracle.hutch_sign(A, G, rng.integers(0, 2 ** 32, size=(7, 1), dtype=np.uint64).astype(np.uint32),
                                      k)[0] for _ in range(S)])
    assert abs(est.mean() - n) <= 4 * sd / math.sqrt(S)
    assert est.std() == pytest.approx(sd, rel=0.1)


def test_unpack_layout():
    S = np.ones((3, 70))
    S[1, 0] = S[1, 31] = S[1, 32] = S[2, 69] = -1
    words = pack(S)
    assert words[1, 0] == (1 | (1 << 31)) and words[1, 1] == 1 and words[2, 2] == (1 << 5)
    np.testing.assert_array_equal(oracle.unpack_signs(words, 3, 70), S)
