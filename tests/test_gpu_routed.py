"""GPU parity of the routed call (dpnorm_norms_routed): layers whose narrow
side min(d, p) is at most k (LoRA factors) get their exact norm, the others
the Hutchinson estimate. Checked against the fp64 oracle's routed sum on the
same inputs: relative error <= 1e-3 (bf16) and 1e-5 (fp32); the routes
reported by the library must equal the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: 1e-3, torch.float32: 1e-5}


def dev():
    return torch.device("cuda:0")


def rel(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    return np.abs(got - want) / np.abs(want)


def g(shape, seed, dtype, std=1.0):
    return workloads.gaussian(shape, std, seed, dev(), dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_lora_factors_and_base_layer(dtype):
    import sample_grad_norms_amd as dp
    B, T, d, r, p, k = 2, 333, 136, 16, 264, 32
    x = g((B, T, d), 91_001, dtype)
    layers = [
        (x, g((B, T, r), 91_002, dtype), None),                                  # down factor: p = r
        (g((B, T, r), 91_003, dtype), g((B, T, p), 91_004, dtype), None),         # up factor: d = r (roles swap)
        (x, g((B, T, p), 91_005, dtype), workloads.projection(p, k, 91_006, dev(), dtype)),   # base layer
        (x, g((B, T, 32), 91_007, dtype), workloads.projection(32, k, 91_008, dev(), dtype)),  # narrow side = k
        (g((B, T, 40), 91_009, dtype), g((B, T, 40), 91_010, dtype),
         workloads.projection(40, k, 91_011, dev(), dtype)),                      # narrow side k + 8: estimated
    ]
    n, c, routes = dp.norms_routed(layers, k, C_clip=1.0, return_routes=True)
    torch.cuda.synchronize()
    want, want_routes = oracle.norms_routed(layers, k)
    assert routes == want_routes == [1, 1, 0, 1, 0]
    err = rel(n.cpu(), want)
    print(f"routed {dtype}: max rel err {err.max():.2e}", flush=True)
    assert np.all(err <= TOL[dtype])
    err = rel(c.cpu(), oracle.clip_factors(want, 1.0))
    assert np.all(err <= TOL[dtype])


def test_exact_route_matches_the_exact_call():
    # the identity projection of the narrow side is the exact norm: compare
    # with dpnorm_exact on the same tensors (both on the GPU) and the oracle
    import sample_grad_norms_amd as dp
    B, T, d, r = 3, 1000, 520, 24
    A = g((B, T, d), 92_001, torch.bfloat16)
    G = g((B, T, r), 92_002, torch.bfloat16)
    n = dp.norms_routed([(A, G, None)], 32)
    e = dp.exact(A, G)
    n_swapped = dp.norms_routed([(G, A, None)], 32)
    torch.cuda.synchronize()
    want = oracle.exact_explicit(A, G)
    for got, what in ((n, "routed"), (e, "exact call"), (n_swapped, "routed, roles swapped")):
        err = rel(got.cpu(), want)
        print(f"{what}: max rel err {err.max():.2e}", flush=True)
        assert np.all(err <= 1e-3)


def test_lora_stack_decoder_layer_full_size():
    import sample_grad_norms_amd as dp
    layers = workloads.lora_stack(device=dev(), layers=1)
    n, routes = dp.norms_routed(layers, 32, return_routes=True)
    torch.cuda.synchronize()
    want, want_routes = oracle.norms_routed(layers, 32)
    assert routes == want_routes and all(routes)
    err = rel(n.cpu(), want)
    print(f"LoRA decoder layer (14 factors): max rel err {err.max():.2e}", flush=True)
    assert np.all(err <= 1e-3)


def test_routed_needs_P_only_for_estimated_layers():
    import sample_grad_norms_amd as dp
    x = g((1, 64, 64), 93_001, torch.bfloat16)
    with pytest.raises(ValueError, match="P is needed"):
        dp.norms_routed([(x, g((1, 64, 64), 93_002, torch.bfloat16), None)], 32)
