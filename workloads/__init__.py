"""Seeded synthetic inputs for the per-sample gradient-norm path.

This module is shared by the tests, the benchmark and the smoke check. It
draws the inputs that both the HIP path and the CPU oracle consume, and it
holds none of the method's arithmetic: only shapes, seeds, distributions and
the structured low-rank construction of one workload.

Shapes follow the workloads of "Efficient DP-SGD for LLMs with Randomized
Clipping" (papernotes.org note, 实验关键数据; gist.science/nl summary,
Empirische Resultaten): Llama-3.2-1B-class linear layers, context 4096,
projection width k = 32. The datasets used there (BBC, BillSum, HotpotQA) are
not available; Gaussian tensors of the same shapes stand in for the hooked
activations A (B x T x d) and output gradients G (B x T x p).

Seed rule: seed = 1_000_000 * config + 100 * projection + role, with roles
A=0, G=1, P=2, S=3, scales=4, low-rank factors=5. Every tensor is drawn in
float32 from ``torch.randn`` on the requested device and then cast (round to
nearest even) to the workload dtype, so both sides see identical values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Tuple

import torch

ROLE_A, ROLE_G, ROLE_P, ROLE_S, ROLE_SCALE, ROLE_LOWRANK = 0, 1, 2, 3, 4, 5

# The seven linear projections of one Llama-3.2-1B decoder layer as
# (name, d = input width, p = output width).
LLAMA_1B_PROJECTIONS: Tuple[Tuple[str, int, int], ...] = (
    ("q", 2048, 2048),
    ("k", 2048, 512),
    ("v", 2048, 512),
    ("o", 2048, 2048),
    ("gate", 2048, 8192),
    ("up", 2048, 8192),
    ("down", 8192, 2048),
)
LLAMA_1B_LAYERS = 16


def seed_of(config: int, projection: int, role: int) -> int:
    return 1_000_000 * config + 100 * projection + role


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def gaussian(shape, std: float, seed: int, device="cpu", dtype=torch.float32,
             generator: Optional[torch.Generator] = None) -> torch.Tensor:
    """N(0, std^2) entries drawn in float32, then cast to ``dtype``."""
    g = generator if generator is not None else _gen(device, seed)
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def projection(p: int, k: int, seed: int, device="cpu", dtype=torch.float32) -> torch.Tensor:
    """A p x k projection with entries N(0, 1/k) (variance 1/k)."""
    return gaussian((p, k), 1.0 / math.sqrt(k), seed, device, dtype)


@dataclasses.dataclass
class Problem:
    """One layer's inputs: A [B][T][d], G [B][T][p], P [p][k] (and S for Hutch++)."""
    A: torch.Tensor
    G: torch.Tensor
    P: torch.Tensor
    S: Optional[torch.Tensor] = None
    k: int = 0
    name: str = ""

    @property
    def shape(self):
        B, T, d = self.A.shape
        return B, T, d, self.G.shape[2]


def random_problem(B: int, T: int, d: int, p: int, k: int, seed: int, device="cpu",
                   dtype=torch.float32, a_std: float = 1.0, g_std: float = 1.0) -> Problem:
    """Generic i.i.d. Gaussian layer inputs (test sizes)."""
    A = gaussian((B, T, d), a_std, seed * 16 + ROLE_A, device, dtype)
    G = gaussian((B, T, p), g_std, seed * 16 + ROLE_G, device, dtype)
    P = projection(p, k, seed * 16 + ROLE_P, device, dtype)
    return Problem(A, G, P, k=k, name=f"rand_B{B}_T{T}_d{d}_p{p}_k{k}")


# --------------------------------------------------------------------------
# The five named workloads
# --------------------------------------------------------------------------

def config1(device="cpu") -> Problem:
    """Single linear layer, fp32: B=2, T=128, d=p=64, k=8; A, G ~ N(0,1),
    P ~ N(0, 1/8); one generator seeded 0 draws A, G, P in that order."""
    g = _gen(device, 0)
    A = gaussian((2, 128, 64), 1.0, 0, device, generator=g)
    G = gaussian((2, 128, 64), 1.0, 0, device, generator=g)
    P = gaussian((64, 8), 1.0 / math.sqrt(8), 0, device, generator=g)
    return Problem(A, G, P, k=8, name="config1_fp32_B2_T128_d64_p64_k8")


def config2(device="cpu", rescaled: bool = False) -> Problem:
    """Single layer, bf16: B=8, T=1024, d=p=2048, k=32. A ~ N(0,1);
    G_i ~ s_i * N(0, 0.01) with log10 s_i ~ U[-1, 1]; P ~ N(0, 1/32).

    ``rescaled`` is an extra sub-case that divides G by sqrt(T*d*p*0.01) so
    that sqrt(n_i) is near s_i and the clip threshold C=1 splits the batch.
    """
    B, T, d, p, k = 8, 1024, 2048, 2048, 32
    A = gaussian((B, T, d), 1.0, seed_of(2, 0, ROLE_A), device, torch.float32)
    G = gaussian((B, T, p), 0.1, seed_of(2, 0, ROLE_G), device, torch.float32)
    u = torch.rand(B, generator=_gen(device, seed_of(2, 0, ROLE_SCALE)), device=device)
    s = torch.pow(10.0, 2.0 * u - 1.0)
    G.mul_(s.view(B, 1, 1))
    if rescaled:
        G.mul_(1.0 / math.sqrt(T * d * p * 0.01))
    P = projection(p, k, seed_of(2, 0, ROLE_P), device, torch.bfloat16)
    return Problem(A.to(torch.bfloat16), G.to(torch.bfloat16), P, k=k,
                   name="config2_bf16_B8_T1024_d2048_p2048_k32" + ("_rescaled" if rescaled else ""))


def config3_projection(index: int, device="cpu", B: int = 4, T: int = 4096, k: int = 32,
                       dtype=torch.bfloat16) -> Problem:
    """Projection ``index`` (0..111) of the 16-layer Llama-3.2-1B-shaped stack:
    layer = index // 7, kind = index % 7. A ~ s_A N(0,1), G ~ s_G N(0,1) with
    s_A, s_G ~ U[0.5, 2] drawn per projection; an independent P ~ N(0, 1/k)."""
    name, d, p = LLAMA_1B_PROJECTIONS[index % 7]
    sc = torch.rand(2, generator=_gen("cpu", seed_of(3, index, ROLE_SCALE)))
    s_a, s_g = (0.5 + 1.5 * sc).tolist()
    A = gaussian((B, T, d), s_a, seed_of(3, index, ROLE_A), device, dtype)
    G = gaussian((B, T, p), s_g, seed_of(3, index, ROLE_G), device, dtype)
    P = projection(p, k, seed_of(3, index, ROLE_P), device, dtype)
    return Problem(A, G, P, k=k, name=f"config3_L{index // 7}_{name}")


def config3_shapes() -> List[Tuple[int, int]]:
    return [(d, p) for _ in range(LLAMA_1B_LAYERS) for (_, d, p) in LLAMA_1B_PROJECTIONS]


# Which projection's input each projection of a decoder layer reads in the
# real model: q, k and v read the attention input; gate and up read the MLP
# input; o and down read their own.
LLAMA_1B_INPUT_OF: Tuple[int, ...] = (0, 0, 0, 3, 4, 4, 6)


def shared_input_stack(device="cpu", B: int = 4, T: int = 4096, k: int = 32, layers: int = LLAMA_1B_LAYERS,
                       dtype=torch.bfloat16) -> List[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]]:
    """The Llama-3.2-1B-shaped stack with the inputs shared as in the real
    model (workload 6 of the seed rule): per decoder layer four activation
    tensors (attention input for q, k, v; o input; MLP input for gate, up;
    down input), each s_A N(0,1) with s_A ~ U[0.5, 2]; per projection its own
    G ~ s_G N(0,1) (s_G ~ U[0.5, 2]) and P ~ N(0, 1/k). Returns (A, G, P)
    triples in the order q, k, v, o, gate, up, down per layer; projections
    that share an input hold the same A tensor object."""
    out = []
    for layer in range(layers):
        inputs = {}
        for j, (_, d, p) in enumerate(LLAMA_1B_PROJECTIONS):
            index = 7 * layer + j
            src = 7 * layer + LLAMA_1B_INPUT_OF[j]
            if src not in inputs:
                s_a = 0.5 + 1.5 * float(torch.rand(1, generator=_gen("cpu", seed_of(6, src, ROLE_SCALE)))[0])
                inputs[src] = gaussian((B, T, d), s_a, seed_of(6, src, ROLE_A), device, dtype)
            s_g = 0.5 + 1.5 * float(torch.rand(2, generator=_gen("cpu", seed_of(6, index, ROLE_SCALE)))[1])
            G = gaussian((B, T, p), s_g, seed_of(6, index, ROLE_G), device, dtype)
            P = projection(p, k, seed_of(6, index, ROLE_P), device, dtype)
            out.append((inputs[src], G, P))
    return out


def lora_stack(device="cpu", B: int = 4, T: int = 4096, k: int = 32, rank: int = 16,
               layers: int = LLAMA_1B_LAYERS, dtype=torch.bfloat16):
    """LoRA factors of every projection of the Llama-3.2-1B-shaped stack
    (workload 7 of the seed rule). For a projection d -> p with rank-r
    adapters x -> (x D) U, the per-sample gradients are those of the down
    factor D (A = x [T][d], G [T][r]) and of the up factor U (A = x D [T][r],
    G [T][p]). x is shared as in the real model (q, k, v read one input, gate
    and up another); every tensor is s N(0,1) with s ~ U[0.5, 2]. Returns
    (A, G, P) triples, down then up factor per projection, with a Gaussian
    P ~ N(0, 1/k) [G's width][k] for each (an exact route does not read it)."""
    out = []
    for layer in range(layers):
        inputs = {}
        for j, (_, d, p) in enumerate(LLAMA_1B_PROJECTIONS):
            index = 7 * layer + j
            src = 7 * layer + LLAMA_1B_INPUT_OF[j]
            sc = (0.5 + 1.5 * torch.rand(4, generator=_gen("cpu", seed_of(7, index, ROLE_SCALE)))).tolist()
            if src not in inputs:
                inputs[src] = gaussian((B, T, d), sc[0], seed_of(7, src, ROLE_A), device, dtype)
            g_mid = gaussian((B, T, rank), sc[1], seed_of(7, index, ROLE_G), device, dtype)
            a_mid = gaussian((B, T, rank), sc[2], seed_of(7, index, ROLE_S), device, dtype)
            g_out = gaussian((B, T, p), sc[3], seed_of(7, index, ROLE_LOWRANK), device, dtype)
            out.append((inputs[src], g_mid, projection(rank, k, seed_of(7, index, ROLE_P), device, dtype)))
            out.append((a_mid, g_out, projection(p, k, seed_of(7, index, ROLE_P) + 50, device, dtype)))
    return out


def hutchpp_split(k: int) -> Tuple[int, int]:
    """Budget split used by the Hutch++ workloads: ceil(k/3) sketch columns,
    the same number of head columns, and k - 2 ceil(k/3) tail columns."""
    m_s = -(-k // 3)
    return m_s, k - 2 * m_s


def config4(device="cpu", B: int = 4, T: int = 4096, d: int = 2048, p: int = 2048,
            k: int = 32, rank: int = 8, sigma1: float = 1000.0, decay: float = 0.5,
            noise_var: float = 1e-3, seed_base: int = seed_of(4, 0, 0)) -> Problem:
    """Hutch++ workload, bf16: A ~ N(0,1); G_i = U_i diag(sigma) V_i^T + E_i with
    U_i (T x rank), V_i (p x rank) orthonormal, sigma_j = sigma1 * decay^(j-1),
    E ~ N(0, noise_var). Sketch S ~ N(0,1) (p x m_s), tail P ~ N(0, 1/m_t)."""
    m_s, m_t = hutchpp_split(k)
    A = gaussian((B, T, d), 1.0, seed_base + ROLE_A, device, torch.bfloat16)
    # The orthonormal factors are drawn on the host (a seeded CPU generator, so
    # the structure does not depend on the device) and only their product is
    # moved to the device.
    g = _gen("cpu", seed_base + ROLE_LOWRANK)
    sig = sigma1 * decay ** torch.arange(rank, dtype=torch.float64)
    Gs = []
    for _ in range(B):
        U, _r = torch.linalg.qr(torch.randn(T, rank, generator=g, dtype=torch.float64))
        V, _r = torch.linalg.qr(torch.randn(p, rank, generator=g, dtype=torch.float64))
        Gs.append(((U * sig) @ V.T).to(torch.float32))
    G = torch.stack(Gs).to(device)
    G.add_(gaussian((B, T, p), math.sqrt(noise_var), seed_base + ROLE_G, device))
    S = gaussian((p, m_s), 1.0, seed_base + ROLE_S, device, torch.bfloat16)
    P = projection(p, m_t, seed_base + ROLE_P, device, torch.bfloat16)
    return Problem(A, G.to(torch.bfloat16), P, S=S, k=k,
                   name=f"config4_hutchpp_B{B}_T{T}_d{d}_p{p}_k{k}")


def config5(device="cpu") -> Problem:
    """Long-context MLP up-projection, bf16: B=1, T=32768, d=2048, p=8192,
    k=32; A, G ~ N(0,1); P ~ N(0, 1/32)."""
    B, T, d, p, k = 1, 32768, 2048, 8192, 32
    A = gaussian((B, T, d), 1.0, seed_of(5, 0, ROLE_A), device, torch.bfloat16)
    G = gaussian((B, T, p), 1.0, seed_of(5, 0, ROLE_G), device, torch.bfloat16)
    P = projection(p, k, seed_of(5, 0, ROLE_P), device, torch.bfloat16)
    return Problem(A, G, P, k=k, name="config5_bf16_B1_T32768_d2048_p8192_k32")
