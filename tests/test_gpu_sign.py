"""GPU parity of the Hutchinson estimate with bit-packed +-1 projections
(dpnorm_hutch_sign, dpnorm_hutch_sign_grouped) against the fp64 oracle, on
the same inputs and the same sign words: relative error <= 1e-3 (bf16
inputs) and 1e-5 (fp32). The +-1 entries are exact in either type and the
1/k scale is applied to the finished sums, so the error is that of fp32
accumulation alone.
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


def signs(p, k, seed):
    g = torch.Generator(device=dev())
    g.manual_seed(seed)
    import sample_grad_norms_amd as dp
    return dp.random_signs(p, k, device=dev(), generator=g)


SHAPES = [
    # B, T, d, p, k
    (3, 333, 1032, 520, 32),
    (2, 95, 8, 8, 1),
    (2, 300, 256, 1024, 34),     # second word per row
    (4, 200, 136, 64, 64),
    (1, 4097, 512, 128, 20),
]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("B,T,d,p,k", SHAPES)
def test_sign_single(dtype, B, T, d, p, k):
    import sample_grad_norms_amd as dp
    prob = workloads.random_problem(B, T, d, p, k, seed=81_000 + T + k, device=dev(), dtype=dtype)
    S = signs(p, k, 81_500 + p)
    n = dp.hutch_sign(prob.A, prob.G, S, k)
    torch.cuda.synchronize()
    err = rel(n.cpu(), oracle.hutch_sign(prob.A, prob.G, S, k))
    print(f"sign {dtype} {B}x{T}x{d}x{p} k={k}: max rel err {err.max():.2e}", flush=True)
    assert np.all(err <= TOL[dtype])


def test_sign_grouped_shared_inputs_clip_and_accumulate():
    import sample_grad_norms_amd as dp
    B, T, k = 2, 513, 32
    A1 = workloads.gaussian((B, T, 264), 1.0, 82_001, dev(), torch.bfloat16)
    A2 = workloads.gaussian((B, T, 128), 1.0, 82_002, dev(), torch.bfloat16)
    layers = []
    for j, (A, p) in enumerate([(A1, 264), (A1, 72), (A1, 72), (A2, 136), (A2, 512)]):
        G = workloads.gaussian((B, T, p), 0.3, 82_100 + j, dev(), torch.bfloat16)
        layers.append((A, G, signs(p, k, 82_200 + j)))
    n, c = dp.hutch_sign_grouped(layers, k, C_clip=2.0)
    n2 = dp.hutch_sign_grouped(layers[:2], k)
    dp.hutch_sign_grouped(layers[2:], k, out=n2, accumulate=True)
    torch.cuda.synchronize()
    want = oracle.layer_sum([oracle.hutch_sign(A, G, S, k) for (A, G, S) in layers])
    for got, what in ((n, "grouped"), (n2, "two calls, accumulate")):
        err = rel(got.cpu(), want)
        print(f"sign {what}: max rel err {err.max():.2e}", flush=True)
        assert np.all(err <= 1e-3)
    err = rel(c.cpu(), oracle.clip_factors(want, 2.0))
    assert np.all(err <= 1e-3)


def test_sign_full_size_gate_projection():
    # the gate projection of the Llama-3.2-1B-shaped stack (d = 2048, p = 8192)
    import sample_grad_norms_amd as dp
    prob = workloads.config3_projection(4, device=dev())
    S = signs(8192, 32, 83_000)
    n = dp.hutch_sign(prob.A, prob.G, S, 32)
    torch.cuda.synchronize()
    err = rel(n.cpu(), oracle.hutch_sign(prob.A, prob.G, S, 32))
    print(f"sign gate projection: max rel err {err.max():.2e}", flush=True)
    assert np.all(err <= 1e-3)
