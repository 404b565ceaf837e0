"""GPU parity of the grouped Hutchinson call when projections share their
input activations (q, k, v read one tensor, gate and up another, as in a
transformer block). Such layers share one stage-2 pass over A; the result
must still match the fp64 oracle's per-projection estimates summed over the
layers, and the same call on private copies of A (no sharing) up to
rounding order.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

INPUT_OF = (0, 0, 0, 3, 4, 4, 6)


def dev():
    return torch.device("cuda:0")


def block_layers(n_layers, B, T, dm, kv, hid, k, dtype, seed):
    """Layers of n_layers transformer blocks with shared inputs, seeded."""
    shapes = [(dm, dm), (dm, kv), (dm, kv), (dm, dm), (dm, hid), (dm, hid), (hid, dm)]
    out = []
    for layer in range(n_layers):
        inputs = {}
        for j, (d, p) in enumerate(shapes):
            idx = 7 * layer + j
            src = 7 * layer + INPUT_OF[j]
            if src not in inputs:
                inputs[src] = workloads.gaussian((B, T, d), 1.0, seed + 100 * src, dev(), dtype)
            G = workloads.gaussian((B, T, p), 0.5, seed + 100 * idx + 1, dev(), dtype)
            P = workloads.projection(p, k, seed + 100 * idx + 2, dev(), dtype)
            out.append((inputs[src], G, P))
    return out


def oracle_sum(layers):
    return oracle.layer_sum([oracle.hutch(A, G, P) for (A, G, P) in layers])


def rel(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    return np.abs(got - want) / np.abs(want)


@pytest.mark.parametrize("T", [300, 2048])
def test_shared_inputs_bf16(T):
    # T = 300: one T split (direct reduction); T = 2048: T is split and the
    # split-T reduction runs on the 96-, 64- and 32-column groups
    import sample_grad_norms_amd as dp
    layers = block_layers(2, 2, T, 136, 72, 264, 32, torch.bfloat16, 61_000)
    n = dp.hutch_grouped(layers)
    private = [(A.clone(), G, P) for (A, G, P) in layers]
    n_private = dp.hutch_grouped(private)
    torch.cuda.synchronize()
    want = oracle_sum(layers)
    err = rel(n.cpu(), want)
    print(f"shared bf16 T={T}: max rel err vs oracle {err.max():.3e}", flush=True)
    assert np.all(err <= 1e-3)
    diff = rel(n.cpu(), n_private.cpu().double().numpy())
    print(f"shared vs private inputs: max rel diff {diff.max():.3e}", flush=True)
    assert np.all(diff <= 1e-9)


def test_shared_inputs_fp32_widths():
    # k = 8: one 16-column block per projection; six projections on one input
    # form a 96-column group, five on another a 64-column and a 16-column group
    import sample_grad_norms_amd as dp
    B, T, k = 3, 200, 8
    A1 = workloads.gaussian((B, T, 64), 1.0, 62_001, dev())
    A2 = workloads.gaussian((B, T, 40), 1.0, 62_002, dev())
    layers = []
    for j, p in enumerate([64, 12, 36, 64, 8, 20]):
        layers.append((A1, workloads.gaussian((B, T, p), 1.0, 62_100 + j, dev()),
                       workloads.projection(p, k, 62_200 + j, dev())))
    for j, p in enumerate([16, 16, 44, 4, 64]):
        layers.append((A2, workloads.gaussian((B, T, p), 1.0, 62_300 + j, dev()),
                       workloads.projection(p, k, 62_400 + j, dev())))
    n = dp.hutch_grouped(layers)
    torch.cuda.synchronize()
    err = rel(n.cpu(), oracle_sum(layers))
    print(f"shared fp32: max rel err {err.max():.3e}", flush=True)
    assert np.all(err <= 1e-5)


def test_shared_inputs_bf16_k16_widths():
    # k = 16 in bf16: groups of 6, 4 and 1 column blocks
    import sample_grad_norms_amd as dp
    B, T, k = 2, 257, 16
    A1 = workloads.gaussian((B, T, 520), 1.0, 63_001, dev(), torch.bfloat16)
    A2 = workloads.gaussian((B, T, 24), 1.0, 63_002, dev(), torch.bfloat16)
    layers = [(A1, workloads.gaussian((B, T, p), 1.0, 63_100 + j, dev(), torch.bfloat16),
               workloads.projection(p, k, 63_200 + j, dev(), torch.bfloat16))
              for j, p in enumerate([8, 64, 520, 16, 136, 32])]
    layers += [(A2, workloads.gaussian((B, T, p), 1.0, 63_300 + j, dev(), torch.bfloat16),
                workloads.projection(p, k, 63_400 + j, dev(), torch.bfloat16))
               for j, p in enumerate([512, 8, 24, 1032, 40])]
    n = dp.hutch_grouped(layers)
    torch.cuda.synchronize()
    err = rel(n.cpu(), oracle_sum(layers))
    print(f"shared bf16 k=16: max rel err {err.max():.3e}", flush=True)
    assert np.all(err <= 1e-3)


def test_workspace_sized_without_sharing():
    # a workspace sized from (d, p) pairs only is smaller than the shared plan
    # here (the shared plan splits T); the call must still succeed, unshared
    import sample_grad_norms_amd as dp
    B, T = 10, 1024
    layers = block_layers(16, B, T, 128, 64, 256, 32, torch.bfloat16, 64_000)
    plain = dp.hutch_grouped_workspace([(A.shape[2], G.shape[2]) for (A, G, _) in layers], torch.bfloat16, B, T, 32)
    shared = dp.hutch_grouped_workspace(layers, torch.bfloat16, B, T, 32)
    assert shared > plain
    ws = torch.empty(plain, dtype=torch.uint8, device=dev())
    n = dp.hutch_grouped(layers, workspace=ws)
    n_shared = dp.hutch_grouped(layers)
    torch.cuda.synchronize()
    want = oracle_sum(layers)
    for got, what in ((n, "unshared fallback"), (n_shared, "shared")):
        err = rel(got.cpu(), want)
        print(f"{what}: max rel err {err.max():.3e}", flush=True)
        assert np.all(err <= 1e-3)


def test_shared_input_llama_stack_layer():
    # one decoder layer of the shared-input Llama-3.2-1B-shaped stack at full size
    import sample_grad_norms_amd as dp
    layers = workloads.shared_input_stack(device=dev(), layers=1)
    n = dp.hutch_grouped(layers)
    torch.cuda.synchronize()
    err = rel(n.cpu(), oracle_sum(layers))
    print(f"shared llama layer: max rel err {err.max():.3e}", flush=True)
    assert np.all(err <= 1e-3)
