"""GPU parity of the Hutchinson path against the fp64 CPU oracle.

Same seeded inputs and the same P on both sides; per-sample relative error
|gpu - oracle| / |oracle| must stay within 1e-3 for bf16 inputs (fp32
accumulation) and 1e-5 for fp32 inputs, for the estimates and the clip
factors. Shapes span several work items with ragged tails in T, d, p and k.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: 1e-3, torch.float32: 1e-5}


def dev():
    return torch.device("cuda:0")


def rel_err(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    out = np.empty_like(want)
    for j, (g, w) in enumerate(zip(got, want)):
        out[j] = abs(g) / 1e-30 if w == 0 else abs(g - w) / abs(w)
    return out


def check(got, want, tol, what):
    err = rel_err(got, want)
    print(f"{what}: max rel err {err.max():.3e}", flush=True)
    assert np.all(err <= tol), f"{what}: rel err {err} > {tol}"


def test_config1_fp32_hutch_and_clip():
    import sample_grad_norms_amd as dp
    prob = workloads.config1(device=dev())
    n, c = dp.hutch_grouped([(prob.A, prob.G, prob.P)], C_clip=1.0)
    n1 = dp.hutch(prob.A, prob.G, prob.P)
    torch.cuda.synchronize()
    want = oracle.hutch(prob.A, prob.G, prob.P)
    check(n.cpu(), want, 1e-5, "config1 hutch grouped")
    check(n1.cpu(), want, 1e-5, "config1 hutch")
    check(c.cpu(), oracle.clip_factors(want, 1.0), 1e-5, "config1 clip")


SHAPES_BF16 = [
    # B, T, d, p, k
    (3, 333, 1032, 520, 32),     # ragged T (not a multiple of 32 or 128), d past one column block, p % 32 != 0
    (2, 95, 8, 8, 1),            # narrowest widths, k = 1
    (1, 1, 512, 512, 32),        # a single token
    (2, 4097, 256, 1024, 20),    # T one past a tile, k padded to 32 columns
    (4, 200, 136, 64, 64),       # k = 64 (four column blocks)
    (2, 128, 2048, 512, 16),     # one 16-column block
    (1, 2500, 4096, 8192, 32),   # long rows on both sides, split T
    (32, 1000, 264, 136, 32),    # 256 stage-1 items of 128 rows (four waves), ragged T and widths
    (31, 1000, 264, 136, 32),    # 248 such items: 64-row two-wave items instead
]


@pytest.mark.parametrize("B,T,d,p,k", SHAPES_BF16)
def test_hutch_bf16_shapes(B, T, d, p, k):
    import sample_grad_norms_amd as dp
    prob = workloads.random_problem(B, T, d, p, k, seed=B * 7 + T, device=dev(), dtype=torch.bfloat16)
    n = dp.hutch(prob.A, prob.G, prob.P)
    torch.cuda.synchronize()
    check(n.cpu(), oracle.hutch(prob.A, prob.G, prob.P), 1e-3, f"bf16 B{B} T{T} d{d} p{p} k{k}")


SHAPES_F32 = [
    (2, 150, 260, 132, 8),
    (1, 33, 4, 4, 3),
    (3, 700, 1028, 36, 32),
    (2, 64, 64, 2052, 64),
]


@pytest.mark.parametrize("B,T,d,p,k", SHAPES_F32)
def test_hutch_f32_shapes(B, T, d, p, k):
    import sample_grad_norms_amd as dp
    prob = workloads.random_problem(B, T, d, p, k, seed=B * 5 + T, device=dev(), dtype=torch.float32)
    n = dp.hutch(prob.A, prob.G, prob.P)
    torch.cuda.synchronize()
    check(n.cpu(), oracle.hutch(prob.A, prob.G, prob.P), 1e-5, f"f32 B{B} T{T} d{d} p{p} k{k}")


def test_zero_inputs_give_zero_and_unit_clip():
    import sample_grad_norms_amd as dp
    prob = workloads.random_problem(2, 70, 64, 64, 8, seed=3, device=dev(), dtype=torch.bfloat16)
    prob.G[1].zero_()
    n, c = dp.hutch_grouped([(prob.A, prob.G, prob.P)], C_clip=1.0)
    torch.cuda.synchronize()
    assert n[1].item() == 0.0 and c[1].item() == 1.0
    assert n[0].item() > 0.0


def test_grouped_is_layer_sum_and_accumulates():
    import sample_grad_norms_amd as dp
    shapes = [(256, 64), (64, 512), (520, 136), (1024, 1024)]
    B, T, k = 3, 257, 32
    layers = []
    for j, (d, p) in enumerate(shapes):
        pr = workloads.random_problem(B, T, d, p, k, seed=100 + j, device=dev(), dtype=torch.bfloat16)
        layers.append((pr.A, pr.G, pr.P))
    n, c = dp.hutch_grouped(layers, C_clip=50.0)
    acc = torch.zeros(B, dtype=torch.float32, device=dev())
    for (A, G, P) in layers:
        dp.hutch(A, G, P, out=acc, accumulate=True)
    base = torch.full((B,), 5.0, dtype=torch.float32, device=dev())
    dp.hutch_grouped(layers, out=base, accumulate=True)
    torch.cuda.synchronize()
    want = oracle.layer_sum([oracle.hutch(A, G, P) for (A, G, P) in layers])
    check(n.cpu(), want, 1e-3, "grouped layer sum")
    check(acc.cpu(), want, 1e-3, "accumulated single calls")
    check(base.cpu(), want + 5.0, 1e-3, "grouped accumulate")
    check(c.cpu(), oracle.clip_factors(want, 50.0), 1e-3, "grouped clip")


def test_deterministic_bitwise():
    import sample_grad_norms_amd as dp
    prob = workloads.random_problem(2, 1500, 1024, 2048, 32, seed=9, device=dev(), dtype=torch.bfloat16)
    a = dp.hutch(prob.A, prob.G, prob.P)
    b = dp.hutch(prob.A, prob.G, prob.P)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("B,T,d,p,k", [(3, 333, 1032, 520, 32), (32, 1000, 264, 136, 32), (4, 200, 136, 64, 64),
                                       (2, 128, 2048, 512, 16), (2, 300, 40, 24, 32), (5, 64, 16, 8, 16)])
def test_projection_read_in_place_matches_packed_copy(B, T, d, p, k):
    """A single-layer bf16 call whose P is 16-byte aligned with k = 16, 32 or
    64 reads P in place; the same values 2 bytes further on take the packed
    path. Both feed the MFMAs the same operands, so the results agree bitwise
    (rows of P past the last full 64-row stage come from a zero row)."""
    import sample_grad_norms_amd as dp
    prob = workloads.random_problem(B, T, d, p, k, seed=B + T + k, device=dev(), dtype=torch.bfloat16)
    buf = torch.empty(p * k + 8, dtype=torch.bfloat16, device=dev())
    buf[1:1 + p * k].copy_(prob.P.reshape(-1))
    p_shifted = buf[1:1 + p * k].view(p, k)
    assert prob.P.data_ptr() % 16 == 0 and p_shifted.data_ptr() % 16 != 0
    a = dp.hutch(prob.A, prob.G, prob.P)
    b = dp.hutch(prob.A, prob.G, p_shifted)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    check(a.cpu(), oracle.hutch(prob.A, prob.G, prob.P), 1e-3, f"in place B{B} T{T} d{d} p{p} k{k}")


def test_grouped_projection_read_in_place_matches_packed_copy():
    """Grouped bf16 calls read every P in place when all are 16-byte aligned
    with 16, 32 or 64 columns (the prepare kernel then writes only tables);
    one P shifted by 2 bytes sends the whole call through packed copies. The
    MFMA operands are the same, so the sums agree bitwise."""
    import sample_grad_norms_amd as dp
    B, T, k = 2, 700, 32
    layers, shifted = [], []
    for j, (d, p) in enumerate(((264, 136), (128, 520), (1032, 64))):
        pr = workloads.random_problem(B, T, d, p, k, seed=50 + j, device=dev(), dtype=torch.bfloat16)
        layers.append((pr.A, pr.G, pr.P))
        shifted.append((pr.A, pr.G, pr.P))
    p0 = layers[0][2]
    buf = torch.empty(p0.numel() + 8, dtype=torch.bfloat16, device=dev())
    buf[1:1 + p0.numel()].copy_(p0.reshape(-1))
    shifted[0] = (layers[0][0], layers[0][1], buf[1:1 + p0.numel()].view(p0.shape))
    a = dp.hutch_grouped(layers)
    b = dp.hutch_grouped(shifted)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    want = sum(oracle.hutch(A, G, P) for A, G, P in layers)
    check(a.cpu(), want, 1e-3, "grouped, P in place")


def test_launch_sequence_follows_the_projection_layout():
    """The traced launches: a one-layer call whose P is read in place has no
    prepare launch; the same P 2 bytes further on is packed first (one
    prepare); a two-layer call reads both P in place but its prepare still
    writes the records and item lists."""
    import sample_grad_norms_amd as dp
    pr = workloads.random_problem(2, 1000, 264, 520, 32, seed=61, device=dev(), dtype=torch.bfloat16)
    pr2 = workloads.random_problem(2, 1000, 136, 64, 32, seed=62, device=dev(), dtype=torch.bfloat16)
    buf = torch.empty(pr.P.numel() + 8, dtype=torch.bfloat16, device=dev())
    buf[1:1 + pr.P.numel()].copy_(pr.P.reshape(-1))
    shifted = buf[1:1 + pr.P.numel()].view(pr.P.shape)
    kinds = []
    for layers in ([(pr.A, pr.G, pr.P)], [(pr.A, pr.G, shifted)], [(pr.A, pr.G, pr.P), (pr2.A, pr2.G, pr2.P)]):
        timer = dp.KernelTimer()
        dp.hutch_grouped(layers, timer=timer)
        kinds.append([name for name, _ in timer.last()])
    print(kinds, flush=True)
    assert "prepare" not in kinds[0] and kinds[0][0] == "rowproj"
    assert kinds[1].count("prepare") == 1 and kinds[1][0] == "prepare"
    assert kinds[2].count("prepare") == 1
    for ks in kinds:
        assert ks[-1] == "finish" and ks.count("rowproj") == 1


def test_clip_factor_kernel_special_values():
    import sample_grad_norms_amd as dp
    n = torch.tensor([0.0, float("inf"), float("nan"), 4.0, 16.0, 1.0, 64.0, 1e-30], device=dev())
    c = dp.clip_factors(n, 2.0)
    torch.cuda.synchronize()
    got = c.cpu().double().numpy()
    want = oracle.clip_factors(n.cpu().double().numpy(), 2.0)
    assert math.isnan(got[2]) and math.isnan(want[2])
    keep = [0, 1, 3, 4, 5, 6, 7]
    check(got[keep], want[keep], 1e-6, "clip special values")
    # in place
    m = n.clone()
    dp.clip_factors(m, 2.0, out=m)
    torch.cuda.synchronize()
    assert torch.equal(m[keep].cpu(), c[keep].cpu())


def test_config2_full_size():
    import sample_grad_norms_amd as dp
    for rescaled in (False, True):
        prob = workloads.config2(device=dev(), rescaled=rescaled)
        n, c = dp.hutch_grouped([(prob.A, prob.G, prob.P)], C_clip=1.0)
        torch.cuda.synchronize()
        want = oracle.hutch(prob.A, prob.G, prob.P)
        wc = oracle.clip_factors(want, 1.0)
        check(n.cpu(), want, 1e-3, prob.name)
        check(c.cpu(), wc, 1e-3, prob.name + " clip")
        if rescaled:
            # the rescaled sub-case puts samples on both sides of C = 1
            assert np.any(wc < 1.0) and np.any(wc == 1.0)


def test_config3_full_size_stack():
    """Llama-3.2-1B-shaped stack (16 x 7 projections, B=4, T=4096, k=32): the
    grouped call as timed by the benchmark against the oracle end to end. The
    oracle's layer sum runs over all 112 projections, one at a time; the
    clip factors are checked against the oracle's clip of that sum; every
    projection's single call against the oracle's estimate of it; and the
    grouped sum against the single calls summed."""
    import sample_grad_norms_amd as dp
    projs = [workloads.config3_projection(j, device=dev()) for j in range(112)]
    layers = [(q.A, q.G, q.P) for q in projs]
    n_all, c_all = dp.hutch_grouped(layers, C_clip=1.0)
    singles = [dp.hutch(A, G, P) for (A, G, P) in layers]
    torch.cuda.synchronize()
    parts, worst = [], (0.0, "")
    for q, (A, G, P), got in zip(projs, layers, singles):
        want = oracle.hutch(A, G, P)
        parts.append(want)
        e = float(rel_err(got.cpu(), want).max())
        assert e <= 1e-3, f"{q.name}: rel err {e:.3e}"
        worst = max(worst, (e, q.name))
    print(f"config3 single calls vs oracle, all 112 projections: worst {worst[0]:.3e} ({worst[1]})", flush=True)
    want = oracle.layer_sum(parts)
    check(n_all.cpu(), want, 1e-3, "config3 grouped vs the oracle's layer sum over 112 projections")
    wc = oracle.clip_factors(want, 1.0)
    check(c_all.cpu(), wc, 1e-3, "config3 clip vs the oracle's clip of its sum")
    tot = torch.stack(singles).double().sum(0).cpu().numpy()
    check(n_all.cpu(), tot, 1e-4, "config3 grouped vs sum of single calls")


@pytest.mark.parametrize("B,T,d,p,k", [(2, 8192, 264, 520, 32), (1, 16320, 136, 1000, 64)])
def test_stage1_two_k_slots_shapes(B, T, d, p, k):
    """Shapes with exactly 128 stage-1 items of 128 rows: they take 64-row
    items on four waves, two per 32-row group, each streaming every other
    64-column chunk of G (p ragged against the 64-column chunks; k = 32 with P
    read in place, k = 64 with four column blocks; T ragged in the second)."""
    import sample_grad_norms_amd as dp
    prob = workloads.random_problem(B, T, d, p, k, seed=73, device=dev(), dtype=torch.bfloat16)
    n = dp.hutch(prob.A, prob.G, prob.P)
    torch.cuda.synchronize()
    check(n.cpu(), oracle.hutch(prob.A, prob.G, prob.P), TOL[torch.bfloat16], f"two K slots B{B} T{T} d{d} p{p} k{k}")


@pytest.mark.parametrize("B,T,d,p,k", [(4, 8200, 2040, 264, 32), (4, 8232, 2048, 136, 16)])
def test_stage2_split_halves_shapes(B, T, d, p, k):
    """Shapes whose 512-column stage-2 items would split T: B * ceil(d/512)
    = 16 items, 257-258 chunks of 32 rows, 16 splits of at least 512 rows.
    They take 256-column items on two pairs of waves over 8 splits of 32-33
    chunks, so in some splits the second pair has one chunk fewer than the
    first and its last stage is zeroed; T and (first shape) d are ragged."""
    import sample_grad_norms_amd as dp
    prob = workloads.random_problem(B, T, d, p, k, seed=71, device=dev(), dtype=torch.bfloat16)
    n = dp.hutch(prob.A, prob.G, prob.P)
    torch.cuda.synchronize()
    check(n.cpu(), oracle.hutch(prob.A, prob.G, prob.P), TOL[torch.bfloat16], f"halves B{B} T{T} d{d} p{p} k{k}")


def test_config5_full_size_hutch():
    import sample_grad_norms_amd as dp
    prob = workloads.config5(device=dev())
    n = dp.hutch(prob.A, prob.G, prob.P)
    torch.cuda.synchronize()
    check(n.cpu(), oracle.hutch(prob.A, prob.G, prob.P), 1e-3, prob.name)
