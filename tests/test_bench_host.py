"""Host side of bench.py (no GPU): the one-GPU guard and the CPU baseline's
record on a tiny stand-in for the decoder stack."""
import os
import subprocess
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "--gpus 1" in r.stderr
    assert r.stdout.strip() == ""   # no JSON line for a configuration that was not run


def test_cpu_baseline_record():
    g = torch.Generator().manual_seed(3)
    B, T, k = 2, 16, 4
    layers = []
    for (d, p) in ((16, 16), (16, 8), (16, 8), (16, 16), (16, 24), (16, 24), (24, 16)):
        A = torch.randn(B, T, d, generator=g).to(torch.bfloat16)
        G = torch.randn(B, T, p, generator=g).to(torch.bfloat16)
        P = (torch.randn(p, k, generator=g) / k ** 0.5).to(torch.bfloat16)
        layers.append((A, G, P))
    rec = bench.cpu_baseline(layers, B, T, 1)
    assert rec["kind"] == "oracle" and rec["unit"] == "samples·tokens/s"
    assert rec["value"] > 0 and rec["cores"] >= 1
    assert "scaled x16" in rec["sample"] and "copies" in rec["sample"]
    assert "logical CPUs" in rec["host"]
