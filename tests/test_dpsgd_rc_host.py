"""Host-side checks of the DP-SGD-RC step wrapper (no GPU work)."""
import pytest
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
