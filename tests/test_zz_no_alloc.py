"""dpnorm_hutch_grouped_noalloc, the entry point for callers that cannot
allocate (graph capture, tight serving loops): through the C ABI, its
estimates and clip factors against those of dpnorm_hutch_grouped with a
caller workspace on the same inputs, 1e-3 relative for bf16 and 1e-5 for
fp32 ('Efficient DP-SGD for LLMs with Randomized Clipping', 方法详解 ›
整体框架: per-sample layer sum and min(C / sqrt(n), 1)). Two calls in a row
share the library's static scratch, the second with a smaller input, so
stale contents of the first call must not reach the second."""
import ctypes as C

import numpy as np
import pytest
import torch

import workloads
from sample_grad_norms_amd import _lib

pytestmark = pytest.mark.gpu


def dev():
    return torch.device("cuda:0")


def layer_array(layers):
    arr = (_lib.Layer * len(layers))()
    for j, (A, G, P) in enumerate(layers):
        arr[j] = _lib.Layer(A.data_ptr(), G.data_ptr(), P.data_ptr(), A.shape[2], G.shape[2])
    return arr


def rel(got, want):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    return float((np.abs(got - want) / np.maximum(np.abs(want), 1e-300)).max())


def both(lib, layers, dtype, k, accumulate, C_clip):
    """(n, c) of the workspace entry point and of the static-scratch one."""
    B, T = layers[0][0].shape[:2]
    code = _lib.BF16 if dtype == torch.bfloat16 else _lib.F32
    arr = layer_array(layers)
    stream = torch.cuda.current_stream(dev()).cuda_stream
    base = torch.linspace(0.25, 2.0, B, device=dev())
    nb = C.c_size_t(0)
    assert lib.dpnorm_hutch_grouped_workspace(arr, len(layers), code, B, T, k, C.byref(nb)) == _lib.OK
    assert nb.value <= _lib.STATIC_SCRATCH_BYTES
    ws = torch.empty(max(nb.value, 1), dtype=torch.uint8, device=dev())
    out = []
    for noalloc in (False, True):
        n = base.clone() if accumulate else torch.full((B,), float("nan"), device=dev())
        c = torch.full((B,), float("nan"), device=dev())
        cp = c.data_ptr() if C_clip else None
        if noalloc:
            st = lib.dpnorm_hutch_grouped_noalloc(arr, len(layers), code, B, T, k, n.data_ptr(), int(accumulate),
                                                  cp, float(C_clip or 1.0), stream)
        else:
            st = lib.dpnorm_hutch_grouped(arr, len(layers), code, B, T, k, n.data_ptr(), int(accumulate), cp,
                                          float(C_clip or 1.0), ws.data_ptr(), nb.value, stream)
        assert st == _lib.OK, lib.dpnorm_status_string(st)
        out.append((n, c))
    torch.cuda.synchronize()
    return out, nb.value


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_the_workspace_entry_point_on_two_calls(dtype):
    lib = _lib.load()
    tol = 1e-3 if dtype == torch.bfloat16 else 1e-5
    g = 8 if dtype == torch.bfloat16 else 4
    k = 32
    # call 1: three layers (two share A), ragged T, clip factors
    A0 = workloads.gaussian((4, 1100, 64 * g), 1.0, 9101, dev(), dtype)
    big = [(A0, workloads.gaussian((4, 1100, 40 * g), 1.0, 9102, dev(), dtype),
            workloads.projection(40 * g, k, 9103, dev(), dtype)),
           (A0, workloads.gaussian((4, 1100, 16 * g), 1.0, 9104, dev(), dtype),
            workloads.projection(16 * g, k, 9105, dev(), dtype)),
           (workloads.gaussian((4, 1100, 24 * g), 1.0, 9106, dev(), dtype),
            workloads.gaussian((4, 1100, 72 * g), 1.0, 9107, dev(), dtype),
            workloads.projection(72 * g, k, 9108, dev(), dtype))]
    # call 2: one smaller layer, fewer samples and tokens, accumulating
    small = [(workloads.gaussian((2, 37, 8 * g), 1.0, 9111, dev(), dtype),
              workloads.gaussian((2, 37, 5 * g), 1.0, 9112, dev(), dtype),
              workloads.projection(5 * g, k, 9113, dev(), dtype))]
    (r1, s1), nb1 = both(lib, big, dtype, k, False, 0.5)
    (r2, s2), nb2 = both(lib, small, dtype, k, True, None)
    assert nb2 < nb1
    e1, ec1, e2 = rel(s1[0].cpu(), r1[0].cpu()), rel(s1[1].cpu(), r1[1].cpu()), rel(s2[0].cpu(), r2[0].cpu())
    same = torch.equal(s1[0], r1[0]) and torch.equal(s1[1], r1[1]) and torch.equal(s2[0], r2[0])
    print(f"{dtype}: call 1 n {e1:.1e} c {ec1:.1e}, call 2 n {e2:.1e}; bitwise equal: {same}", flush=True)
    assert e1 <= tol and ec1 <= tol and e2 <= tol
    assert torch.isfinite(s1[0]).all() and torch.isfinite(s1[1]).all() and torch.isfinite(s2[0]).all()
