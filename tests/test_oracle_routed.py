"""Pins of the oracle's route between the exact norm and the Hutchinson
estimate (LoRA factors: one side of W = A^T G is the rank r <= k).

The route rule on the workload shapes, and the routed sum against
independent pins: a routed LoRA factor equals the closed form of a
rank-one / single-token case and the brute-force sum of per-token outer
products; an estimated layer keeps the Hutchinson estimate.
"""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("d,p,k,exact", [
    (2048, 16, 32, True),     # LoRA down factor, rank 16
    (16, 2048, 32, True),     # LoRA up factor
    (2048, 32, 32, True),     # narrow side equal to k
    (2048, 40, 32, False),
    (2048, 2048, 32, False),  # base projection
    (8, 8, 1, False),
])
def test_route_rule(d, p, k, exact):
    assert oracle.routes_exact(d, p, k) is exact


def test_routed_lora_factor_is_the_brute_force_norm():
    rng = np.random.default_rng(7)
    B, T, d, r, p, k = 2, 9, 6, 2, 7, 4
    x = rng.standard_normal((B, T, d))
    g_mid = rng.standard_normal((B, T, r))
    a_mid = rng.standard_normal((B, T, r))
    g_out = rng.standard_normal((B, T, p))
    P = rng.standard_normal((p, k)) / 2.0
    layers = [(x, g_mid, None), (a_mid, g_out, None), (x, g_out, P)]
    n, routes = oracle.norms_routed(layers, k)
    assert routes == [1, 1, 0]
    # brute force: per-sample gradient as a sum of per-token outer products
    want = np.zeros(B)
    for i in range(B):
        for (A, G) in ((x, g_mid), (a_mid, g_out)):
            W = sum(np.outer(A[i, t], G[i, t]) for t in range(T))
            want[i] += np.sum(W * W)
    want += oracle.hutch(x, g_out, P)
    np.testing.assert_allclose(n, want, rtol=1e-12)


def test_single_token_factor_closed_form():
    # T = 1: ||a g^T||_F^2 = ||a||^2 ||g||^2, whatever the narrow side
    a = np.array([[[1.0, 2.0, 2.0]]])      # ||a||^2 = 9
    g = np.array([[[3.0, 4.0]]])           # ||g||^2 = 25
    n, routes = oracle.norms_routed([(a, g, None), (g, a, None)], 2)
    assert routes == [1, 1]
    assert n[0] == pytest.approx(2 * 225.0, rel=1e-15)
