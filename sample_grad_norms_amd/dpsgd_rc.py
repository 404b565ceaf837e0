"""DP-SGD with randomized clipping around the per-sample norm path.

The step follows 'Efficient DP-SGD for LLMs with Randomized Clipping'
(papernotes.org note, 方法详解 › 整体框架 and 损失函数 / 训练策略): one
forward pass in which a hook on every linear-like module records its input
activations A [B][T][d]; a first backward pass that yields each module's
output gradients G [B][T][p]; per module a norm estimate n_hat_i (Hutchinson
by default, Hutch++ or the exact norm on request) summed over the modules into
n_i; clip factors c_i = min(C / sqrt(n_i), 1); a second backward pass of the
rewritten loss sum_i c_i l_i, which gives sum_i c_i grad l_i; Gaussian noise
sigma C N(0, I) added to that sum; and the optimizer step.

Readings where the pages leave a step open:
  * The first backward pass is of sum_i l_i, so G_i is the gradient of sample
    i's own loss.
  * The noisy sum is divided by the batch size B before the optimizer, as in
    textbook DP-SGD; the pages add the noise to the aggregated gradient and
    do not state the averaging.
  * A weight applied several times in one forward pass (by one module called
    more than once, or by several linear modules that hold the same weight)
    has one per-sample gradient sum_u A_u^T G_u = [A_1; A_2; ...]^T
    [G_1; G_2; ...]: its recordings are concatenated along T.
  * A fresh projection P ~ N(0, 1/k) is drawn per weight and step.
  * The projections and the noise are internal randomness of the mechanism:
    by default each comes from its own generator seeded from the operating
    system's entropy, so neither can be replayed from the code. Fixed seeds
    exist for tests only.

Every norm estimate runs in libdpnorm on the GPU; torch runs the model and its
two backward passes. Only bias-free nn.Linear weights are clipped (Llama has
no biases). Refused, since part of a gradient would go unclipped: any other
trainable parameter, and a linear weight that a module of another kind also
holds (a tied embedding). A use of a weight that the hooks cannot see (the
weight passed to F.linear outside its module) is caught on the first step:
the clipped gradient autograd accumulates must equal sum_i c_i G_i^T A_i
from the recordings.
"""
from __future__ import annotations

import secrets
from typing import Callable, Dict, List, Optional, Tuple

import torch
from torch import nn

import sample_grad_norms_amd as dp

ProjectionFn = Callable[[int, int, torch.dtype, torch.device, torch.Generator], torch.Tensor]


def gaussian_projection(p: int, k: int, dtype: torch.dtype, device: torch.device,
                        generator: torch.Generator) -> torch.Tensor:
    """P [p][k] with i.i.d. N(0, 1/k) entries, drawn in float32 and rounded
    once to `dtype`."""
    P = torch.randn(p, k, generator=generator, device=device, dtype=torch.float32) / (k ** 0.5)
    return P.to(dtype)


class RandomizedClipping:
    """Hooks a model's bias-free linear layers and runs the DP-SGD-RC step.

    Usage::

        rc = RandomizedClipping(model, C=1.0, noise_multiplier=0.8)
        with rc.capture():
            losses = per_sample_losses(model(x), y)      # float32 [B]
        n, c = rc.clip_factors(losses)                   # backward 1 + norms
        rc.clipped_backward(losses, c)                   # backward 2
        rc.add_noise()                                   # sigma C N(0, I), / B
        optimizer.step(); optimizer.zero_grad()

    or ``rc.step(losses, optimizer)`` for the last four lines.

    estimator: "hutch" (k Gaussian columns), "hutch_sign" (k +-1 columns stored
    as bits), "hutchpp" (budget k) or "exact".
    norm_dtype: element type handed to the norm path (bfloat16 or float32;
    default: the activations' own). Widths must suit that type (multiples of
    8 for bfloat16, 4 for float32).
    keep_layers: keep the (A, G, P) triples of the last step in
    ``last_layers`` (P is the sign words for "hutch_sign", the pair (S, P)
    of sketch and tail projection for "hutchpp", None for "exact").
    timer: an optional sample_grad_norms_amd.KernelTimer given to the grouped
    Hutchinson calls (per-launch times of the norm path).
    seed, noise_seed: FOR TESTS ONLY. Fixed seeds of the projection and noise
    generators make the mechanism's randomness reproducible by anyone who
    knows them, which voids its privacy; the default (None) seeds each from
    the operating system's entropy.
    verify_coverage: on the first step, check that each clipped weight's
    gradient from the second backward pass equals sum_i c_i G_i^T A_i from
    the recordings (it does not when the weight has a use the hooks cannot
    see, such as F.linear called with it outside its module); a mismatch
    raises RuntimeError. The check assumes nothing else adds to the weights'
    .grad during that backward pass.
    """

    def __init__(self, model: nn.Module, C: float, noise_multiplier: float, k: int = 32,
                 estimator: str = "hutch", norm_dtype: Optional[torch.dtype] = None, seed: Optional[int] = None,
                 projection: ProjectionFn = gaussian_projection, keep_layers: bool = False,
                 timer: Optional["dp.KernelTimer"] = None, noise_seed: Optional[int] = None,
                 verify_coverage: bool = True):
        if estimator not in ("hutch", "hutch_sign", "hutchpp", "exact"):
            raise ValueError("estimator must be 'hutch', 'hutch_sign', 'hutchpp' or 'exact'")
        if not C > 0:
            raise ValueError("C must be positive")
        self.C, self.sigma, self.k = float(C), float(noise_multiplier), int(k)
        self.estimator, self.norm_dtype, self.projection = estimator, norm_dtype, projection
        self.seed = seed if seed is not None else secrets.randbits(63)
        self.noise_seed = noise_seed if noise_seed is not None else secrets.randbits(63)
        self.keep_layers, self.timer = keep_layers, timer
        self.last_layers: List[Tuple[torch.Tensor, torch.Tensor, Optional[torch.Tensor]]] = []
        self.modules: List[nn.Linear] = [m for m in model.modules() if isinstance(m, nn.Linear)]
        for m in self.modules:
            if m.bias is not None:
                raise ValueError("linear layers with a bias are not supported (the clipped gradient would miss it)")
        covered = {id(m.weight) for m in self.modules}
        # a linear weight that a module of another kind also holds (a tied
        # embedding) gets gradient through that module, which no hook sees
        tied = [f"{name}.{pname}" if name else pname for name, mod in model.named_modules()
                if not isinstance(mod, nn.Linear)
                for pname, p in mod.named_parameters(recurse=False) if id(p) in covered]
        if tied:
            raise ValueError(f"linear weights shared with modules that are not linear layers would go partly "
                             f"unclipped: {tied}")
        loose = [name for name, p in model.named_parameters(remove_duplicate=False)
                 if p.requires_grad and id(p) not in covered]
        if loose:
            raise ValueError(f"trainable parameters outside bias-free linear layers would go unclipped: {loose}")
        # one entry per distinct weight, in module order (modules holding the
        # same weight contribute to one per-sample gradient)
        self.params: List[nn.Parameter] = []
        self._users: Dict[int, List[nn.Linear]] = {}
        for m in self.modules:
            if id(m.weight) not in self._users:
                self._users[id(m.weight)] = []
                if m.weight.requires_grad:
                    self.params.append(m.weight)
            self._users[id(m.weight)].append(m)
        self._names = {id(p): name for name, p in model.named_parameters()}
        self._capturing = False
        self._rec: Dict[nn.Linear, List[Tuple[torch.Tensor, torch.Tensor]]] = {}
        self._gen: Optional[torch.Generator] = None
        self._noise_gen: Optional[torch.Generator] = None
        self._batch = 0
        self._verify = bool(verify_coverage)
        self._pending: Optional[List[Tuple[nn.Parameter, torch.Tensor, torch.Tensor]]] = None
        self._handles = [m.register_forward_hook(self._hook) for m in self.modules]

    # -- capture ---------------------------------------------------------
    def _hook(self, module, inputs, output):
        if self._capturing and module.weight.requires_grad:
            self._rec.setdefault(module, []).append((inputs[0], output))

    class _Capture:
        def __init__(self, rc):
            self.rc = rc

        def __enter__(self):
            self.rc._rec = {}
            self.rc._capturing = True
            return self.rc

        def __exit__(self, *exc):
            self.rc._capturing = False
            return False

    def capture(self):
        """Context in which the model's forward pass is recorded."""
        return RandomizedClipping._Capture(self)

    def remove(self):
        for h in self._handles:
            h.remove()
        self._handles = []

    # -- the step --------------------------------------------------------
    def _generator(self, device):
        if self._gen is None:
            self._gen = torch.Generator(device=device)
            self._gen.manual_seed(self.seed)
        return self._gen

    def _noise_generator(self, device):
        if self._noise_gen is None:
            self._noise_gen = torch.Generator(device=device)
            self._noise_gen.manual_seed(self.noise_seed)
        return self._noise_gen

    def _collect(self, losses: torch.Tensor) -> List[Tuple[torch.Tensor, torch.Tensor]]:
        """Backward pass 1: per recorded weight, (A [B][T'][d], G [B][T'][p])
        with every use of the weight concatenated along T."""
        if losses.dim() != 1:
            raise ValueError("losses must be the per-sample losses [B]")
        if not self._rec:
            raise RuntimeError("no forward pass was captured (run the model inside rc.capture())")
        B = losses.shape[0]
        weights = []   # (weight, [(input, output), ...]) in module order
        for m in self.modules:
            if m in self._rec:
                key = id(m.weight)
                if not weights or all(id(w) != key for w, _ in weights):
                    weights.append((m.weight, [r for u in self._users[key] for r in self._rec.get(u, [])]))
        outputs = [o for _, recs in weights for (_, o) in recs]
        grads = torch.autograd.grad(losses.sum(), outputs, retain_graph=True, allow_unused=True)
        layers, at, cast = [], 0, {}
        for w, recs in weights:
            As, Gs = [], []
            for (a, out), g in zip(recs, grads[at:at + len(recs)]):
                if g is None:  # the output did not reach the loss
                    g = torch.zeros_like(out)
                As.append(self._cast(a.detach().reshape(B, -1, a.shape[-1]), cast))
                Gs.append(self._cast(g.detach().reshape(B, -1, g.shape[-1]), cast))
            at += len(recs)
            A = As[0] if len(As) == 1 else torch.cat(As, dim=1)
            G = Gs[0] if len(Gs) == 1 else torch.cat(Gs, dim=1)
            layers.append((A, G))
        self._pending = [(w, A, G) for (w, _), (A, G) in zip(weights, layers)] if self._verify else None
        self._batch = B
        self._rec = {}
        return layers

    def clip_factors(self, losses: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
        """Backward pass 1 and the norm path: returns (n, c), float32 [B]."""
        layers = self._collect(losses)
        B = losses.shape[0]
        device = layers[0][0].device
        gen = self._generator(device)
        n = torch.zeros(B, dtype=torch.float32, device=device)
        used = []
        if self.estimator in ("hutch", "hutch_sign"):
            if self.estimator == "hutch":
                triples = [(A, G, self.projection(G.shape[2], self.k, A.dtype, device, gen)) for (A, G) in layers]
            else:
                triples = [(A, G, dp.random_signs(G.shape[2], self.k, device=device, generator=gen))
                           for (A, G) in layers]
            # one grouped call per sequence length (a module applied u times has u T rows)
            lengths = sorted({A.shape[1] for (A, _, _) in triples})
            for j, T in enumerate(lengths):
                part = [t for t in triples if t[0].shape[1] == T]
                if self.estimator == "hutch":
                    dp.hutch_grouped(part, out=n, accumulate=j > 0, timer=self.timer)
                else:
                    dp.hutch_sign_grouped(part, self.k, out=n, accumulate=j > 0)
            used = triples
        else:
            for (A, G) in layers:
                if self.estimator == "exact":
                    dp.exact(A, G, out=n, accumulate=True)
                    used.append((A, G, None))
                else:
                    m_s, m_t = dp.hutchpp_split(self.k)
                    S = torch.randn(G.shape[2], m_s, generator=gen, device=device).to(A.dtype)
                    P = self.projection(G.shape[2], m_t, A.dtype, device, gen)
                    dp.hutchpp(A, G, S, P, k=self.k, out=n, accumulate=True)
                    used.append((A, G, (S, P)))
        c = dp.clip_factors(n, self.C)
        self.last_layers = used if self.keep_layers else []
        return n, c

    def _cast(self, t: torch.Tensor, cache: dict) -> torch.Tensor:
        # layers reading one tensor keep sharing one copy (and one pass over it)
        dt = self.norm_dtype or t.dtype
        key = (t.data_ptr(), tuple(t.shape), t.dtype)
        if key not in cache:
            cache[key] = t.to(dt).contiguous()
        return cache[key]

    def clipped_backward(self, losses: torch.Tensor, c: torch.Tensor) -> None:
        """Backward pass 2: accumulates sum_i c_i grad l_i into the weights' .grad
        (on the first step, then checked against the recordings)."""
        pending, self._pending = self._pending, None
        before = None
        if pending is not None:
            before = [w.grad.detach().float().clone() if w.grad is not None else None for w, _, _ in pending]
        (c.detach().to(losses.dtype) * losses).sum().backward()
        if pending is not None:
            self._check_coverage(pending, before, c)
            self._verify = False

    def _check_coverage(self, pending, before, c: torch.Tensor) -> None:
        """Each weight's gradient from backward pass 2 must be sum_i c_i G_i^T A_i
        over its recordings (within the rounding of the recorded dtype)."""
        cw = c.detach().float()
        for (w, A, G), g0 in zip(pending, before):
            if not w.requires_grad:
                continue
            B, T, d = A.shape
            p = G.shape[2]
            want = (G.float() * cw.view(B, 1, 1)).reshape(B * T, p).t() @ A.float().reshape(B * T, d)
            got = torch.zeros_like(want) if w.grad is None else w.grad.detach().float()
            if g0 is not None:
                got = got - g0
            scale = float(torch.linalg.vector_norm(want))
            err = float(torch.linalg.vector_norm(got - want))
            if err > 5e-2 * scale + 1e-30:
                raise RuntimeError(
                    f"the gradient of linear weight {self._names.get(id(w), '')} {list(w.shape)} differs from what its "
                    f"recorded uses give (relative {err / max(scale, 1e-300):.2e}): it has a use the hooks do not "
                    f"see (e.g. F.linear called with it outside its module), which would go unclipped")

    def add_noise(self) -> None:
        """Adds sigma C N(0, I) to each clipped gradient sum and divides by B."""
        if self._batch <= 0:
            raise RuntimeError("clip_factors has not run for this step")
        for p in self.params:
            if p.grad is None:
                p.grad = torch.zeros_like(p)
            g = p.grad.float()
            if self.sigma > 0:
                g = g + self.sigma * self.C * torch.randn(p.shape, generator=self._noise_generator(p.device),
                                                          device=p.device, dtype=torch.float32)
            p.grad.copy_((g / self._batch).to(p.grad.dtype))
        self._batch = 0

    def step(self, losses: torch.Tensor, optimizer: torch.optim.Optimizer) -> Tuple[torch.Tensor, torch.Tensor]:
        """clip_factors, clipped_backward, add_noise, optimizer.step, zero_grad."""
        n, c = self.clip_factors(losses)
        self.clipped_backward(losses, c)
        self.add_noise()
        optimizer.step()
        optimizer.zero_grad(set_to_none=True)
        return n, c
