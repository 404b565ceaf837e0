"""A randomly initialised Llama-shaped decoder stack for exercising the
per-sample norm path inside a training step (no trained weights).

Per decoder layer: RMSNorm, causal multi-head attention with q, k, v and o
projections (grouped key/value heads), RMSNorm, and the SiLU-gated MLP with
gate, up and down projections; a final RMSNorm and a bias-free output
projection to a small vocabulary. Every linear layer is bias-free, as in
Llama. The inputs are synthetic hidden states (no embedding table), so the
per-sample loss is the summed token cross-entropy of the output projection.
Attention scores and softmax are computed in float32. This module holds
model arithmetic only, none of the norm-estimation method.
"""
from __future__ import annotations

import math

import torch
import torch.nn.functional as F
from torch import nn


class RMSNorm(nn.Module):
    def __init__(self, dim: int, eps: float = 1e-5):
        super().__init__()
        self.weight = nn.Parameter(torch.ones(dim))
        self.eps = eps

    def forward(self, x):
        xf = x.float()
        y = xf * torch.rsqrt(xf.pow(2).mean(-1, keepdim=True) + self.eps)
        return (y * self.weight.float()).to(x.dtype)


class DecoderLayer(nn.Module):
    def __init__(self, dim: int, heads: int, kv_heads: int, hidden: int):
        super().__init__()
        self.heads, self.kv_heads, self.hd = heads, kv_heads, dim // heads
        self.attn_norm = RMSNorm(dim)
        self.q = nn.Linear(dim, heads * self.hd, bias=False)
        self.k = nn.Linear(dim, kv_heads * self.hd, bias=False)
        self.v = nn.Linear(dim, kv_heads * self.hd, bias=False)
        self.o = nn.Linear(heads * self.hd, dim, bias=False)
        self.mlp_norm = RMSNorm(dim)
        self.gate = nn.Linear(dim, hidden, bias=False)
        self.up = nn.Linear(dim, hidden, bias=False)
        self.down = nn.Linear(hidden, dim, bias=False)

    def forward(self, x):
        B, T, _ = x.shape
        h = self.attn_norm(x)
        q = self.q(h).view(B, T, self.heads, self.hd).transpose(1, 2).float()
        k = self.k(h).view(B, T, self.kv_heads, self.hd).transpose(1, 2).float()
        v = self.v(h).view(B, T, self.kv_heads, self.hd).transpose(1, 2).float()
        rep = self.heads // self.kv_heads
        k = k.repeat_interleave(rep, dim=1)
        v = v.repeat_interleave(rep, dim=1)
        scores = torch.matmul(q, k.transpose(-1, -2).contiguous()) / math.sqrt(self.hd)
        mask = torch.ones(T, T, dtype=torch.bool, device=x.device).triu(1)
        att = torch.softmax(scores.masked_fill(mask, float("-inf")), dim=-1)
        y = torch.matmul(att, v).transpose(1, 2).reshape(B, T, self.heads * self.hd).to(x.dtype)
        x = x + self.o(y)
        h = self.mlp_norm(x)
        return x + self.down(F.silu(self.gate(h)) * self.up(h))


class LlamaStack(nn.Module):
    def __init__(self, layers: int = 2, dim: int = 256, heads: int = 4, kv_heads: int = 2, hidden: int = 512,
                 vocab: int = 128):
        super().__init__()
        self.layers = nn.ModuleList(DecoderLayer(dim, heads, kv_heads, hidden) for _ in range(layers))
        self.norm = RMSNorm(dim)
        self.head = nn.Linear(dim, vocab, bias=False)

    def forward(self, x):
        for layer in self.layers:
            x = layer(x)
        return self.head(self.norm(x))


def build(seed: int, device="cpu", dtype=torch.float32, **shape) -> LlamaStack:
    """A LlamaStack with N(0, 0.02) linear weights drawn from a generator
    seeded with `seed`; RMSNorm weights stay 1 and are frozen, so only the
    linear layers train."""
    model = LlamaStack(**shape)
    g = torch.Generator().manual_seed(seed)
    for m in model.modules():
        if isinstance(m, nn.Linear):
            with torch.no_grad():
                m.weight.copy_(torch.randn(m.weight.shape, generator=g) * 0.02)
        if isinstance(m, RMSNorm):
            m.weight.requires_grad_(False)
    return model.to(device=device, dtype=dtype)


def batch(seed: int, B: int, T: int, dim: int, vocab: int, device="cpu", dtype=torch.float32):
    """Synthetic hidden states x ~ N(0, 1) [B][T][dim] and token targets."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(B, T, dim, generator=g).to(device=device, dtype=dtype)
    y = torch.randint(0, vocab, (B, T), generator=g).to(device)
    return x, y


def per_sample_loss(logits, targets):
    """Summed token cross-entropy of each sample, float32 [B]."""
    B, T, V = logits.shape
    ce = F.cross_entropy(logits.float().reshape(B * T, V), targets.reshape(B * T), reduction="none")
    return ce.view(B, T).sum(dim=1)
