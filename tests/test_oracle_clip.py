"""Pins of the oracle's layer sum and clip factor.

n_i = sum over linear-like layers of n_hat_i^(l) and c_i = min(C / sqrt(n_i), 1)
('Efficient DP-SGD for LLMs with Randomized Clipping', papernotes.org note,
方法详解 › 整体框架; n is a squared norm, so the clip uses its square root).
"""
import json
import math
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def test_hand_example():
    with open(GOLDEN) as f:
        c = {x["name"]: x for x in json.load(f)["cases"]}["clip"]
    assert oracle.clip_factors(c["n"], c["C"]).tolist() == c["c"]


def test_closed_forms_and_edges():
    C = 1.7
    got = oracle.clip_factors([C * C, 4 * C * C, 0.0, math.inf, 0.25 * C * C], C)
    assert got[0] == 1.0 and got[1] == 0.5 and got[2] == 1.0 and got[3] == 0.0 and got[4] == 1.0
    assert math.isnan(oracle.clip_factors([math.nan], 1.0)[0])


def test_monotone_non_increasing():
    n = np.logspace(-6, 6, 200)
    c = oracle.clip_factors(n, 1.0)
    assert np.all(np.diff(c) <= 0.0)
    assert np.all((c > 0) & (c <= 1))


def test_layer_sum_additive_and_order_free():
    rng = np.random.default_rng(31)
    rows = [rng.random(4) * 10.0 ** int(rng.integers(-3, 4)) for _ in range(9)]
    s = oracle.layer_sum(rows)
    np.testing.assert_allclose(s, np.sum(np.stack(rows), axis=0), rtol=1e-15)
    np.testing.assert_allclose(oracle.layer_sum(rows[::-1]), s, rtol=1e-14)
    # the sum of per-layer estimates equals the estimate of the concatenated
    # layer: stacking two layers side by side in p adds their norms
    A = rng.standard_normal((2, 7, 3))
    G1, G2 = rng.standard_normal((2, 7, 4)), rng.standard_normal((2, 7, 5))
    both = oracle.exact_explicit(A, np.concatenate([G1, G2], axis=2))
    np.testing.assert_allclose(oracle.layer_sum([oracle.exact_explicit(A, G1), oracle.exact_explicit(A, G2)]),
                               both, rtol=1e-12)
