"""Host-side checks of the DP-SGD-RC step wrapper (no GPU work)."""
import pytest
import torch
import torch.nn.functional as F
from torch import nn

from workloads import llama_block as lb


def test_refuses_unclipped_parameters():
    from sample_grad_norms_amd.dpsgd_rc import RandomizedClipping
    model = lb.LlamaStack(layers=1, dim=32, heads=2, kv_heads=1, hidden=64, vocab=16)   # RMSNorm weights trainable
    with pytest.raises(ValueError, match="unclipped"):
        RandomizedClipping(model, C=1.0, noise_multiplier=1.0)
    with pytest.raises(ValueError, match="bias"):
        RandomizedClipping(nn.Linear(8, 8), C=1.0, noise_multiplier=1.0)


def test_argument_checks_and_capture_scope():
    from sample_grad_norms_amd.dpsgd_rc import RandomizedClipping
    model = lb.build(1, layers=1, dim=32, heads=2, kv_heads=1, hidden=64, vocab=16)
    with pytest.raises(ValueError, match="estimator"):
        RandomizedClipping(model, C=1.0, noise_multiplier=1.0, estimator="jl")
    with pytest.raises(ValueError, match="C must be positive"):
        RandomizedClipping(model, C=0.0, noise_multiplier=1.0)
    rc = RandomizedClipping(model, C=1.0, noise_multiplier=1.0)
    x, y = lb.batch(2, 2, 4, 32, 16)
    losses = lb.per_sample_loss(model(x), y)       # outside capture(): nothing recorded
    with pytest.raises(RuntimeError, match="captured"):
        rc.clip_factors(losses)
    with rc.capture():
        model(x)
    assert len(rc._rec) == 8 and all(len(v) == 1 for v in rc._rec.values())
    with pytest.raises(RuntimeError, match="clip_factors"):
        rc.add_noise()
    rc.remove()
    with rc.capture():
        model(x)
    assert rc._rec == {}


class _TiedLM(nn.Module):
    """Token embedding tied to the output projection, as in Llama-3.2-1B."""

    def __init__(self, vocab=16, dim=8):
        super().__init__()
        self.emb = nn.Embedding(vocab, dim)
        self.mix = nn.Linear(dim, dim, bias=False)
        self.head = nn.Linear(dim, vocab, bias=False)
        self.head.weight = self.emb.weight

    def forward(self, tok):
        return self.head(torch.tanh(self.mix(self.emb(tok))))


def test_refuses_a_linear_weight_tied_to_an_embedding():
    from sample_grad_norms_amd.dpsgd_rc import RandomizedClipping
    with pytest.raises(ValueError, match="shared with modules that are not linear"):
        RandomizedClipping(_TiedLM(), C=1.0, noise_multiplier=1.0)


class _TwoModulesOneWeight(nn.Module):
    def __init__(self):
        super().__init__()
        self.a = nn.Linear(6, 6, bias=False)
        self.b = nn.Linear(6, 6, bias=False)
        self.b.weight = self.a.weight
        self.out = nn.Linear(6, 4, bias=False)

    def forward(self, x):
        return self.out(torch.tanh(self.b(torch.tanh(self.a(x)))))


class _FunctionalReuse(nn.Module):
    """The weight of `a` is also applied through F.linear, which no hook sees."""

    def __init__(self):
        super().__init__()
        self.a = nn.Linear(6, 6, bias=False)
        self.out = nn.Linear(6, 4, bias=False)

    def forward(self, x):
        h = torch.tanh(self.a(x))
        return self.out(torch.tanh(F.linear(h, self.a.weight)))


def _losses(model, x, y):
    return lb.per_sample_loss(model(x), y)


def test_linear_modules_sharing_a_weight_form_one_gradient():
    """Two linear modules holding one weight: one entry, its recordings
    concatenated along T, and sum_i G_i^T A_i equals autograd's gradient."""
    from sample_grad_norms_amd.dpsgd_rc import RandomizedClipping
    torch.manual_seed(3)
    model = _TwoModulesOneWeight()
    rc = RandomizedClipping(model, C=1.0, noise_multiplier=0.0, seed=1, noise_seed=2)
    assert len(rc.params) == 2
    x, y = torch.randn(3, 5, 6), torch.randint(0, 4, (3, 5))
    with rc.capture():
        losses = _losses(model, x, y)
    layers = rc._collect(losses)
    assert [tuple(A.shape) for A, _ in layers] == [(3, 10, 6), (3, 5, 6)]
    # the check of backward pass 2 passes with every c_i = 1
    rc.clipped_backward(losses, torch.ones(3))


def test_a_use_outside_the_hooks_is_caught_on_the_first_step():
    from sample_grad_norms_amd.dpsgd_rc import RandomizedClipping
    torch.manual_seed(4)
    model = _FunctionalReuse()
    rc = RandomizedClipping(model, C=1.0, noise_multiplier=0.0, seed=1, noise_seed=2)
    x, y = torch.randn(3, 5, 6), torch.randint(0, 4, (3, 5))
    with rc.capture():
        losses = _losses(model, x, y)
    rc._collect(losses)
    with pytest.raises(RuntimeError, match="hooks do not see"):
        rc.clipped_backward(losses, torch.tensor([1.0, 0.5, 0.25]))


def test_clipped_backward_check_accepts_a_covered_model():
    from sample_grad_norms_amd.dpsgd_rc import RandomizedClipping
    model = lb.build(5, layers=1, dim=32, heads=2, kv_heads=1, hidden=64, vocab=16)
    rc = RandomizedClipping(model, C=1.0, noise_multiplier=0.0, seed=1, noise_seed=2)
    x, y = lb.batch(6, 3, 7, 32, 16)
    with rc.capture():
        losses = lb.per_sample_loss(model(x), y)
    rc._collect(losses)
    rc.clipped_backward(losses, torch.tensor([1.0, 0.3, 0.7]))
    assert not rc._verify           # checked once, on the first step


def _noise(noise_seed):
    from sample_grad_norms_amd.dpsgd_rc import RandomizedClipping
    model = lb.build(7, layers=1, dim=32, heads=2, kv_heads=1, hidden=64, vocab=16)
    rc = RandomizedClipping(model, C=1.0, noise_multiplier=1.0, seed=1, noise_seed=noise_seed)
    x, y = lb.batch(8, 2, 4, 32, 16)
    with rc.capture():
        losses = lb.per_sample_loss(model(x), y)
    rc._collect(losses)
    rc.clipped_backward(losses, torch.zeros(2))
    rc.add_noise()
    return torch.cat([p.grad.flatten() for p in rc.params])


def test_noise_is_seeded_from_entropy_unless_a_test_seed_is_given():
    a, b = _noise(None), _noise(None)
    assert not torch.equal(a, b)
    assert torch.equal(_noise(9), _noise(9))
