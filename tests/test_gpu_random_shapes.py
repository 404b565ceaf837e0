"""Seeded random shapes within the C ABI's limits, every estimator against
the fp64 oracle: Hutchinson (single and grouped, with shared inputs,
accumulate and clip), ±1 projections, the routed call, the exact routes and
Hutch++ ('Efficient DP-SGD for LLMs with Randomized Clipping', papernotes.org
note, 关键设计 › Hutchinson and › Hutch++). Widths, T and k are drawn to hit
ragged tiles, single tokens, narrow layers and sketches of lower rank than
m_s; tolerances are 1e-3 relative for bf16 inputs and 1e-5 for fp32."""
import random

import numpy as np
import pytest
import torch

import hutchpp_parity
import oracle
import workloads

pytestmark = pytest.mark.gpu


def dev():
    return torch.device("cuda:0")


def rel(got, want):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    return float((np.abs(got - want) / np.maximum(np.abs(want), 1e-300)).max())


def draw_dtype(rng):
    dt = rng.choice([torch.bfloat16, torch.bfloat16, torch.float32])
    return dt, (8 if dt == torch.bfloat16 else 4), (1e-3 if dt == torch.bfloat16 else 1e-5)


@pytest.mark.parametrize("case", range(12))
def test_single_layer_estimators(case):
    import sample_grad_norms_amd as dp
    rng = random.Random(7000 + case)
    dt, g, tol = draw_dtype(rng)
    B = rng.randint(1, 9)
    T = rng.choice([1, 2, 31, 33, 127, 129, 300, 513, 1024])
    d, p = g * rng.randint(1, 120), g * rng.randint(1, 120)
    k = rng.choice([1, 3, 8, 16, 17, 24, 32, 33, 64])
    what = f"{dt} B{B} T{T} d{d} p{p} k{k}"
    pr = workloads.random_problem(B, T, d, p, k, seed=7100 + case, device=dev(), dtype=dt)
    n = dp.hutch(pr.A, pr.G, pr.P)
    route = rng.choice(["explicit", "gram", "auto"])
    ne = dp.exact(pr.A, pr.G, route=route)
    kk = rng.choice([3, 12, 32, 48, 96])
    ms, mt = oracle.hutchpp_split(kk)
    S = workloads.gaussian((p, ms), 1.0, 7200 + case, dev(), dt)
    Pt = workloads.projection(p, mt, 7300 + case, dev(), dt)
    nh, head, tail, rank, resid = dp.hutchpp(pr.A, pr.G, S, Pt, return_parts=True, return_residuals=True)
    torch.cuda.synchronize()
    e_h = rel(n.cpu(), oracle.hutch(pr.A, pr.G, pr.P))
    e_x = rel(ne.cpu(), oracle.exact_explicit(pr.A, pr.G))
    print(f"{what}: hutch {e_h:.1e} exact/{route} {e_x:.1e}", flush=True)
    # Hutch++ by the shared rule: the kept rank is decided on the kernel's
    # sketch; where the sketch has full rank m_s it must match the oracle's
    # and head and tail are held to their own values; where O has lower rank
    # the columns past it hold only rounding, so the rank may exceed the
    # oracle's up to m_s while the estimate is unaffected
    print(hutchpp_parity.check(pr.A, pr.G, S, (nh, head, tail, rank), oracle.hutchpp(pr.A, pr.G, S, Pt), tol,
                               f"hutch++ k{kk}", resid=resid), flush=True)
    assert e_h <= tol and e_x <= tol


@pytest.mark.parametrize("case", range(8))
def test_grouped_entry_points(case):
    import sample_grad_norms_amd as dp
    rng = random.Random(8000 + case)
    dt, g, tol = draw_dtype(rng)
    B = rng.choice([1, 2, 3, 5, 8, 17, 40])
    T = rng.choice([1, 7, 32, 65, 200, 511])
    k = rng.choice([1, 4, 16, 20, 32, 33, 64])
    layers = []
    for j in range(rng.randint(1, 6)):
        d, p = g * rng.randint(1, 80), g * rng.randint(1, 80)
        if j % 2 == 1 and rng.random() < 0.6:      # shares the previous layer's input
            A = layers[-1][0]
        else:
            A = workloads.gaussian((B, T, d), 1.0, 8100 + 10 * case + j, dev(), dt)
        G = workloads.gaussian((B, T, p), 1.0, 8200 + 10 * case + j, dev(), dt)
        layers.append((A, G, workloads.projection(p, k, 8300 + 10 * case + j, dev(), dt)))
    what = f"{dt} B{B} T{T} k{k} layers {[(A.shape[2], G.shape[2]) for A, G, _ in layers]}"
    base = torch.linspace(0.5, 1.5, B, device=dev())
    n, c = dp.hutch_grouped(layers, out=base.clone(), accumulate=True, C_clip=0.7)
    gen = torch.Generator(device="cuda").manual_seed(8400 + case)
    signs = [(A, G, dp.random_signs(G.shape[2], k, generator=gen)) for A, G, _ in layers]
    ns = dp.hutch_sign_grouped(signs, k=k)
    nr, routes = dp.norms_routed(layers, k=k, return_routes=True)
    torch.cuda.synchronize()
    e_g = rel(n.cpu(), oracle.layer_sum([oracle.hutch(*l) for l in layers]) + base.cpu().double().numpy())
    e_c = rel(c.cpu(), oracle.clip_factors(n.cpu().double().numpy(), 0.7))
    e_s = rel(ns.cpu(), oracle.layer_sum([oracle.hutch_sign(A, G, S.cpu(), k) for A, G, S in signs]))
    wr, wroutes = oracle.norms_routed(layers, k)
    e_r = rel(nr.cpu(), wr)
    print(f"{what}: grouped {e_g:.1e} clip {e_c:.1e} sign {e_s:.1e} routed {e_r:.1e} routes {list(routes)}", flush=True)
    assert e_g <= tol and e_c <= 1e-5 and e_s <= tol and e_r <= tol
    assert [int(x) for x in routes] == [int(x) for x in wroutes]


@pytest.mark.parametrize("B,T,d,p,k", [(1, 131072, 1024, 1024, 32), (256, 1, 2048, 512, 32), (64, 513, 264, 1032, 32),
                                       (2, 65536, 8, 8192, 64)])
def test_extreme_shapes(B, T, d, p, k):
    """Long sequences (T = 2^17 and 2^16 with the narrowest d), a large batch
    of single tokens and a 64-sample batch: Hutchinson and Hutch++ against
    the oracle, bf16."""
    import sample_grad_norms_amd as dp
    pr = workloads.random_problem(B, T, d, p, k, seed=B + T, device=dev(), dtype=torch.bfloat16)
    ms, mt = oracle.hutchpp_split(k)
    S = workloads.gaussian((p, ms), 1.0, 5, dev(), torch.bfloat16)
    Pt = workloads.projection(p, mt, 6, dev(), torch.bfloat16)
    n = dp.hutch(pr.A, pr.G, pr.P)
    nh = dp.hutchpp(pr.A, pr.G, S, Pt)
    torch.cuda.synchronize()
    e, eh = rel(n.cpu(), oracle.hutch(pr.A, pr.G, pr.P)), rel(nh.cpu(), oracle.hutchpp(pr.A, pr.G, S, Pt)[0])
    print(f"B{B} T{T} d{d} p{p} k{k}: hutch {e:.1e} hutch++ {eh:.1e}", flush=True)
    assert e <= 1e-3 and eh <= 1e-3
