"""MI355X-native randomized per-sample gradient-norm estimation (libdpnorm).

For a linear-like layer with hooked activations A_i (T x d) and output
gradients G_i (T x p) of sample i, the squared per-sample gradient norm is
||A_i^T G_i||_F^2; the Hutchinson estimate with a shared Gaussian projection
P (p x k, entries of variance 1/k) is ||A_i^T (G_i P)||_F^2. Estimates are
summed over layers per sample and turned into clip factors min(C/sqrt(n), 1)
('Efficient DP-SGD for LLMs with Randomized Clipping', papernotes.org note,
方法详解 › 整体框架 and 关键设计 › Hutchinson).

This module is a thin binding: it checks torch tensors, takes their device
pointers, allocates the workspace the library asks for and calls the C ABI
of libdpnorm.so on torch's current HIP stream. Every step of the computation
runs in the library's HIP kernels; there is no other code path, and calls
fail loudly if the library is not built or no GPU is present.
"""
from __future__ import annotations

import ctypes as C
from typing import List, Optional, Sequence, Tuple

import torch

from . import _lib

__all__ = ["DpnormError", "hutch", "hutch_grouped", "hutchpp", "exact", "clip_factors", "hutchpp_split", "KernelTimer",
           "lib", "hutch_workspace", "hutch_grouped_workspace", "hutchpp_workspace", "exact_workspace"]


class DpnormError(RuntimeError):
    """A libdpnorm call returned a non-OK status."""

    def __init__(self, status: int, what: str):
        self.status = status
        msg = lib().dpnorm_status_string(status)
        super().__init__(f"{what}: {msg.decode() if msg else status}")


def lib() -> C.CDLL:
    return _lib.load()


def _check(status: int, what: str) -> None:
    if status != _lib.OK:
        raise DpnormError(status, what)


def _code(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return _lib.BF16
    if dtype == torch.float32:
        return _lib.F32
    raise TypeError(f"libdpnorm takes bfloat16 or float32 inputs, got {dtype}")


def _need(t: torch.Tensor, name: str, ndim: int, dtype: Optional[torch.dtype] = None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (libdpnorm runs on the GPU only)")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _workspace(nbytes: int, device: torch.device) -> Tuple[Optional[torch.Tensor], int]:
    if nbytes == 0:
        return None, 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws, ws.data_ptr()


def _out(out: Optional[torch.Tensor], B: int, device: torch.device, accumulate: bool, name: str = "out"):
    if out is None:
        if accumulate:
            raise ValueError("accumulate=True needs an existing output tensor")
        return torch.empty(B, dtype=torch.float32, device=device)
    _need(out, name, 1, torch.float32)
    if out.shape[0] != B:
        raise ValueError(f"{name} must have {B} entries")
    return out


def _layer_array(layers: Sequence[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]]):
    if len(layers) == 0:
        raise ValueError("at least one layer is needed")
    A0, G0, P0 = layers[0]
    _need(A0, "A", 3)
    dtype, device = A0.dtype, A0.device
    B, T = A0.shape[0], A0.shape[1]
    k = P0.shape[1] if P0.dim() == 2 else -1
    arr = (_lib.Layer * len(layers))()
    for j, (A, G, P) in enumerate(layers):
        _need(A, f"layers[{j}].A", 3, dtype)
        _need(G, f"layers[{j}].G", 3, dtype)
        _need(P, f"layers[{j}].P", 2, dtype)
        if A.device != device or G.device != device or P.device != device:
            raise ValueError("all tensors of a call must be on one device")
        if A.shape[:2] != (B, T) or G.shape[:2] != (B, T):
            raise ValueError(f"layers[{j}]: A and G must be [B={B}][T={T}][*]")
        if P.shape[0] != G.shape[2] or P.shape[1] != k:
            raise ValueError(f"layers[{j}]: P must be [p={G.shape[2]}][k={k}]")
        arr[j] = _lib.Layer(A.data_ptr(), G.data_ptr(), P.data_ptr(), A.shape[2], G.shape[2])
    return arr, dtype, device, B, T, k


def hutch(A: torch.Tensor, G: torch.Tensor, P: torch.Tensor, out: Optional[torch.Tensor] = None,
          accumulate: bool = False, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """n_hat_i = ||A_i^T (G_i P)||_F^2 for every sample (dpnorm_hutch).

    A [B][T][d], G [B][T][p], P [p][k], all bfloat16 or all float32, on the
    GPU and contiguous. Returns float32 [B]; with accumulate=True the
    estimates are added to ``out`` (the per-sample layer sum).
    """
    arr, dtype, device, B, T, k = _layer_array([(A, G, P)])
    L = lib()
    nbytes = C.c_size_t(0)
    _check(L.dpnorm_hutch_workspace(_code(dtype), B, T, A.shape[2], G.shape[2], k, C.byref(nbytes)),
           "dpnorm_hutch_workspace")
    n = _out(out, B, device, accumulate)
    ws, wsp = _given_workspace(workspace, nbytes.value, device)
    _check(L.dpnorm_hutch(A.data_ptr(), G.data_ptr(), P.data_ptr(), _code(dtype), B, T, A.shape[2], G.shape[2], k,
                          n.data_ptr(), int(accumulate), wsp, nbytes.value, _stream(device)), "dpnorm_hutch")
    return n


def hutch_workspace(dtype: torch.dtype, B: int, T: int, d: int, p: int, k: int) -> int:
    nbytes = C.c_size_t(0)
    _check(lib().dpnorm_hutch_workspace(_code(dtype), B, T, d, p, k, C.byref(nbytes)), "dpnorm_hutch_workspace")
    return nbytes.value


def hutch_grouped_workspace(layers, dtype: torch.dtype, B: int, T: int, k: int) -> int:
    """Workspace bytes of dpnorm_hutch_grouped for layer tensors or (d, p) pairs.

    Given the (A, G, P) tensors, the size is that of the call's own plan, in
    which layers sharing one A tensor share one pass over it. Given (d, p)
    pairs, it is the size without that sharing; a call with such a workspace
    still succeeds and then streams each A separately if it must.
    """
    arr = (_lib.Layer * len(layers))()
    for j, y in enumerate(layers):
        if isinstance(y[0], torch.Tensor):
            arr[j] = _lib.Layer(y[0].data_ptr(), y[1].data_ptr(), y[2].data_ptr(), y[0].shape[2], y[1].shape[2])
        else:
            arr[j] = _lib.Layer(None, None, None, int(y[0]), int(y[1]))
    nbytes = C.c_size_t(0)
    _check(lib().dpnorm_hutch_grouped_workspace(arr, len(layers), _code(dtype), B, T, k, C.byref(nbytes)),
           "dpnorm_hutch_grouped_workspace")
    return nbytes.value


def hutch_grouped(layers: Sequence[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]],
                  out: Optional[torch.Tensor] = None, accumulate: bool = False, C_clip: Optional[float] = None,
                  clip_out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  timer: Optional["KernelTimer"] = None):
    """Per-sample sum over layers of the Hutchinson estimates (dpnorm_hutch_grouped).

    ``layers`` is a sequence of (A, G, P) triples sharing B, T, k and dtype.
    Returns n [B] float32, or (n, c) when ``C_clip`` is given, with
    c = min(C / sqrt(n), 1). ``workspace`` (uint8, GPU) may be passed to
    reuse one allocation across calls; ``timer`` records HIP events between
    the call's launches.
    """
    arr, dtype, device, B, T, k = _layer_array(layers)
    L = lib()
    nbytes = C.c_size_t(0)
    _check(L.dpnorm_hutch_grouped_workspace(arr, len(layers), _code(dtype), B, T, k, C.byref(nbytes)),
           "dpnorm_hutch_grouped_workspace")
    n = _out(out, B, device, accumulate)
    c = None
    if C_clip is not None:
        c = _out(clip_out, B, device, False, "clip_out") if clip_out is not None else torch.empty_like(n)
    if workspace is None:
        ws, wsp = _workspace(nbytes.value, device)
        ws_bytes = nbytes.value
    else:
        # the library decides whether a smaller workspace still fits a plan
        # without shared-input passes (see hutch_grouped_workspace)
        if not workspace.is_cuda:
            raise ValueError("workspace must be a GPU tensor")
        ws, wsp = workspace, workspace.data_ptr()
        ws_bytes = workspace.numel() * workspace.element_size()
    args = (arr, len(layers), _code(dtype), B, T, k, n.data_ptr(), int(accumulate),
            c.data_ptr() if c is not None else None, float(C_clip) if C_clip is not None else 1.0,
            wsp, ws_bytes, _stream(device))
    if timer is None:
        _check(L.dpnorm_hutch_grouped(*args), "dpnorm_hutch_grouped")
    else:
        tr = timer._trace()
        _check(L.dpnorm_hutch_grouped_traced(*args, C.byref(tr)), "dpnorm_hutch_grouped_traced")
        timer._record(tr)
    return (n, c) if c is not None else n


def random_signs(p: int, k: int, device="cuda", generator: Optional[torch.Generator] = None) -> torch.Tensor:
    """Uniformly random 32-bit words [p][ceil(k/32)] (int32 storage): the
    bit-packed i.i.d. Rademacher signs of a +-1 projection (see hutch_sign)."""
    return torch.randint(-2 ** 31, 2 ** 31, (p, (k + 31) // 32), dtype=torch.int32, device=device,
                         generator=generator)


def _sign_layer_array(layers, k: int):
    if len(layers) == 0:
        raise ValueError("at least one layer is needed")
    A0 = layers[0][0]
    _need(A0, "A", 3)
    dtype, device = A0.dtype, A0.device
    B, T = A0.shape[0], A0.shape[1]
    if not 1 <= k <= 64:
        raise ValueError("k must be in 1..64")
    arr = (_lib.Layer * len(layers))()
    for j, (A, G, S) in enumerate(layers):
        _need(A, f"layers[{j}].A", 3, dtype)
        _need(G, f"layers[{j}].G", 3, dtype)
        _need(S, f"layers[{j}].S_bits", 2, torch.int32)
        if A.device != device or G.device != device or S.device != device:
            raise ValueError("all tensors of a call must be on one device")
        if A.shape[:2] != (B, T) or G.shape[:2] != (B, T):
            raise ValueError(f"layers[{j}]: A and G must be [B={B}][T={T}][*]")
        if tuple(S.shape) != (G.shape[2], (k + 31) // 32):
            raise ValueError(f"layers[{j}]: S_bits must be [p={G.shape[2]}][{(k + 31) // 32}] int32 words")
        arr[j] = _lib.Layer(A.data_ptr(), G.data_ptr(), S.data_ptr(), A.shape[2], G.shape[2])
    return arr, dtype, device, B, T


def hutch_sign(A: torch.Tensor, G: torch.Tensor, S_bits: torch.Tensor, k: int, out: Optional[torch.Tensor] = None,
               accumulate: bool = False, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """n_hat_i = ||A_i^T (G_i S)||_F^2 / k with S in {-1,+1}^{p x k} stored as
    bits (dpnorm_hutch_sign): S_bits is int32 [p][ceil(k/32)], bit j % 32 of
    word j // 32 of row v set for S[v][j] = -1."""
    _sign_layer_array([(A, G, S_bits)], k)
    B, T = A.shape[0], A.shape[1]
    L = lib()
    nbytes = C.c_size_t(0)
    _check(L.dpnorm_hutch_workspace(_code(A.dtype), B, T, A.shape[2], G.shape[2], k, C.byref(nbytes)),
           "dpnorm_hutch_workspace")
    n = _out(out, B, A.device, accumulate)
    ws, wsp = _given_workspace(workspace, nbytes.value, A.device)
    _check(L.dpnorm_hutch_sign(A.data_ptr(), G.data_ptr(), S_bits.data_ptr(), _code(A.dtype), B, T, A.shape[2],
                               G.shape[2], k, n.data_ptr(), int(accumulate), wsp, nbytes.value, _stream(A.device)),
           "dpnorm_hutch_sign")
    return n


def hutch_sign_grouped(layers, k: int, out: Optional[torch.Tensor] = None, accumulate: bool = False,
                       C_clip: Optional[float] = None, clip_out: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None):
    """hutch_grouped with +-1 projections (dpnorm_hutch_sign_grouped): layers
    are (A, G, S_bits) triples. Returns n, or (n, c) when C_clip is given."""
    arr, dtype, device, B, T = _sign_layer_array(layers, k)
    L = lib()
    nbytes = C.c_size_t(0)
    _check(L.dpnorm_hutch_grouped_workspace(arr, len(layers), _code(dtype), B, T, k, C.byref(nbytes)),
           "dpnorm_hutch_grouped_workspace")
    n = _out(out, B, device, accumulate)
    c = None
    if C_clip is not None:
        c = _out(clip_out, B, device, False, "clip_out") if clip_out is not None else torch.empty_like(n)
    if workspace is None:
        ws, wsp = _workspace(nbytes.value, device)
        ws_bytes = nbytes.value
    else:
        if not workspace.is_cuda:
            raise ValueError("workspace must be a GPU tensor")
        ws, wsp = workspace, workspace.data_ptr()
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(L.dpnorm_hutch_sign_grouped(arr, len(layers), _code(dtype), B, T, k, n.data_ptr(), int(accumulate),
                                       c.data_ptr() if c is not None else None,
                                       float(C_clip) if C_clip is not None else 1.0, wsp, ws_bytes,
                                       _stream(device)), "dpnorm_hutch_sign_grouped")
    return (n, c) if c is not None else n


def routes_exact(d: int, p: int, k: int) -> bool:
    """True when norms_routed computes a layer's exact norm (min(d, p) <= k)."""
    return min(d, p) <= k


def norms_routed(layers, k: int, out: Optional[torch.Tensor] = None, accumulate: bool = False,
                 C_clip: Optional[float] = None, clip_out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, return_routes: bool = False):
    """Per-sample sum over layers of the exact norm (layers with min(d, p) <= k)
    or the Hutchinson estimate (the others), dpnorm_norms_routed. ``layers``
    are (A, G, P) triples; P may be None for exactly routed layers, else it
    is [p][k] of the inputs' type. Returns n, (n, c) with C_clip, and the
    per-layer routes (1 exact, 0 estimated) last when return_routes."""
    if len(layers) == 0:
        raise ValueError("at least one layer is needed")
    A0 = layers[0][0]
    _need(A0, "A", 3)
    dtype, device = A0.dtype, A0.device
    B, T = A0.shape[0], A0.shape[1]
    arr = (_lib.Layer * len(layers))()
    for j, (A, G, P) in enumerate(layers):
        _need(A, f"layers[{j}].A", 3, dtype)
        _need(G, f"layers[{j}].G", 3, dtype)
        if A.shape[:2] != (B, T) or G.shape[:2] != (B, T):
            raise ValueError(f"layers[{j}]: A and G must be [B={B}][T={T}][*]")
        if P is None:
            if not routes_exact(A.shape[2], G.shape[2], k):
                raise ValueError(f"layers[{j}]: P is needed (min(d, p) > k)")
        else:
            _need(P, f"layers[{j}].P", 2, dtype)
            if tuple(P.shape) != (G.shape[2], k):
                raise ValueError(f"layers[{j}]: P must be [p={G.shape[2]}][k={k}]")
        arr[j] = _lib.Layer(A.data_ptr(), G.data_ptr(), P.data_ptr() if P is not None else None, A.shape[2],
                            G.shape[2])
    L = lib()
    nbytes = C.c_size_t(0)
    _check(L.dpnorm_norms_routed_workspace(arr, len(layers), _code(dtype), B, T, k, C.byref(nbytes)),
           "dpnorm_norms_routed_workspace")
    n = _out(out, B, device, accumulate)
    c = None
    if C_clip is not None:
        c = _out(clip_out, B, device, False, "clip_out") if clip_out is not None else torch.empty_like(n)
    ws, wsp = _given_workspace(workspace, nbytes.value, device)
    routes = (C.c_int32 * len(layers))()
    _check(L.dpnorm_norms_routed(arr, len(layers), _code(dtype), B, T, k, n.data_ptr(), int(accumulate),
                                 c.data_ptr() if c is not None else None,
                                 float(C_clip) if C_clip is not None else 1.0, routes, wsp, nbytes.value,
                                 _stream(device)), "dpnorm_norms_routed")
    res = (n, c) if c is not None else (n,)
    if return_routes:
        res = res + (list(routes),)
    return res if len(res) > 1 else res[0]


def read_probe(buf: torch.Tensor) -> None:
    """Calibration: stream the whole of ``buf`` (a contiguous GPU tensor whose
    size is a multiple of 16384 bytes) once with the stage kernels' direct
    global-to-LDS loads (dpnorm_read_probe); time it to get that path's read
    rate."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    _check(lib().dpnorm_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(), _stream(buf.device)),
           "dpnorm_read_probe")


_ROUTES = {"auto": _lib.EXACT_AUTO, "explicit": _lib.EXACT_EXPLICIT, "gram": _lib.EXACT_GRAM}


def _given_workspace(workspace: Optional[torch.Tensor], nbytes: int, device: torch.device):
    if workspace is None:
        return _workspace(nbytes, device)
    if not workspace.is_cuda or workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace must be a GPU tensor of at least {nbytes} bytes")
    return workspace, workspace.data_ptr()


def hutchpp_workspace(dtype: torch.dtype, B: int, T: int, d: int, p: int, k: int) -> int:
    nbytes = C.c_size_t(0)
    _check(lib().dpnorm_hutchpp_workspace(_code(dtype), B, T, d, p, k, C.byref(nbytes)), "dpnorm_hutchpp_workspace")
    return nbytes.value


def exact_workspace(dtype: torch.dtype, B: int, T: int, d: int, p: int, route: str = "auto") -> int:
    nbytes = C.c_size_t(0)
    _check(lib().dpnorm_exact_workspace(_code(dtype), B, T, d, p, _ROUTES[route], C.byref(nbytes)),
           "dpnorm_exact_workspace")
    return nbytes.value


def hutchpp(A: torch.Tensor, G: torch.Tensor, S: torch.Tensor, P: torch.Tensor, k: Optional[int] = None,
            out: Optional[torch.Tensor] = None, accumulate: bool = False, return_parts: bool = False,
            workspace: Optional[torch.Tensor] = None, return_residuals: bool = False):
    """Hutch++ estimate with total budget k (dpnorm_hutchpp).

    S [p][m_s] is the sketch and P [p][m_t] the tail projection, with
    (m_s, m_t) = hutchpp_split(k); by default k = 2 m_s + m_t from the
    shapes. Returns n [B], or (n, head, tail, rank) with return_parts;
    return_residuals appends resid [B][m_s], the relative residual of each
    sketch column that the rank rule compared with its threshold.
    ``workspace`` (uint8, GPU) may be passed to reuse one allocation.
    """
    _need(A, "A", 3)
    dtype, device = A.dtype, A.device
    _need(G, "G", 3, dtype)
    _need(S, "S", 2, dtype)
    _need(P, "P", 2, dtype)
    B, T, d = A.shape
    p = G.shape[2]
    if G.shape[:2] != (B, T) or S.shape[0] != p or P.shape[0] != p:
        raise ValueError("shapes must be A [B][T][d], G [B][T][p], S [p][m_s], P [p][m_t]")
    if k is None:
        k = 2 * S.shape[1] + P.shape[1]
    ms, mt = hutchpp_split(k)
    if S.shape[1] != ms or P.shape[1] != mt:
        raise ValueError(f"budget {k} needs S with {ms} and P with {mt} columns")
    L = lib()
    nbytes = C.c_size_t(0)
    _check(L.dpnorm_hutchpp_workspace(_code(dtype), B, T, d, p, k, C.byref(nbytes)), "dpnorm_hutchpp_workspace")
    n = _out(out, B, device, accumulate)
    head = torch.empty(B, dtype=torch.float32, device=device) if return_parts else None
    tail = torch.empty(B, dtype=torch.float32, device=device) if return_parts else None
    rank = torch.empty(B, dtype=torch.int32, device=device) if return_parts else None
    resid = torch.empty(B, ms, dtype=torch.float32, device=device) if return_residuals else None
    ws, wsp = _given_workspace(workspace, nbytes.value, device)
    ptr = lambda t: t.data_ptr() if t is not None else None
    _check(L.dpnorm_hutchpp(A.data_ptr(), G.data_ptr(), S.data_ptr(), P.data_ptr(), _code(dtype), B, T, d, p, k,
                            n.data_ptr(), int(accumulate), ptr(head), ptr(tail), ptr(rank), ptr(resid), wsp,
                            nbytes.value, _stream(device)), "dpnorm_hutchpp")
    out_ = (n, head, tail, rank) if return_parts else (n,)
    if return_residuals:
        out_ = out_ + (resid,)
    return out_ if len(out_) > 1 else n


def exact(A: torch.Tensor, G: torch.Tensor, route: str = "auto", out: Optional[torch.Tensor] = None,
          accumulate: bool = False, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Exact n_i = ||A_i^T G_i||_F^2 (dpnorm_exact); route 'auto', 'explicit' or 'gram'."""
    _need(A, "A", 3)
    dtype, device = A.dtype, A.device
    _need(G, "G", 3, dtype)
    B, T, d = A.shape
    p = G.shape[2]
    if G.shape[:2] != (B, T):
        raise ValueError("A and G must be [B][T][*]")
    r = _ROUTES[route]
    L = lib()
    nbytes = C.c_size_t(0)
    _check(L.dpnorm_exact_workspace(_code(dtype), B, T, d, p, r, C.byref(nbytes)), "dpnorm_exact_workspace")
    n = _out(out, B, device, accumulate)
    ws, wsp = _given_workspace(workspace, nbytes.value, device)
    _check(L.dpnorm_exact(A.data_ptr(), G.data_ptr(), _code(dtype), B, T, d, p, r, n.data_ptr(), int(accumulate), wsp,
                          nbytes.value, _stream(device)), "dpnorm_exact")
    return n


def clip_factors(n: torch.Tensor, C_clip: float, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """c_i = min(C / sqrt(n_i), 1) (dpnorm_clip_factors); ``out`` may be ``n``."""
    _need(n, "n", 1, torch.float32)
    c = torch.empty_like(n) if out is None else out
    _need(c, "out", 1, torch.float32)
    _check(lib().dpnorm_clip_factors(n.data_ptr(), n.shape[0], float(C_clip), c.data_ptr(), _stream(n.device)),
           "dpnorm_clip_factors")
    return c


def hutchpp_split(k: int) -> Tuple[int, int]:
    """Hutch++ budget split (m_s, m_t) used by the library."""
    ms, mt = C.c_int64(0), C.c_int64(0)
    _check(lib().dpnorm_hutchpp_split(k, C.byref(ms), C.byref(mt)), "dpnorm_hutchpp_split")
    return ms.value, mt.value


class KernelTimer:
    """HIP events recorded by the library between the launches of one call.

    After each traced call, ``last`` lists (kernel kind, milliseconds) for the
    call's launches once the stream has reached the last event.
    """

    def __init__(self, capacity: int = 64):
        self.capacity = capacity
        self._events = (C.c_void_p * capacity)()
        self._kinds = (C.c_int32 * capacity)()
        L = lib()
        for j in range(capacity):
            ev = C.c_void_p()
            _check(L.dpnorm_event_create(C.byref(ev)), "dpnorm_event_create")
            self._events[j] = ev
        self._count = 0

    def _trace(self) -> _lib.Trace:
        return _lib.Trace(C.cast(self._events, C.POINTER(C.c_void_p)), C.cast(self._kinds, C.POINTER(C.c_int32)),
                          self.capacity, 0)

    def _record(self, tr: _lib.Trace) -> None:
        self._count = int(tr.count)

    def last(self) -> List[Tuple[str, float]]:
        L = lib()
        if self._count == 0:
            return []
        _check(L.dpnorm_event_synchronize(self._events[self._count - 1]), "dpnorm_event_synchronize")
        res = []
        for j in range(1, self._count):
            ms = C.c_float(0.0)
            _check(L.dpnorm_event_elapsed_ms(self._events[j - 1], self._events[j], C.byref(ms)),
                   "dpnorm_event_elapsed_ms")
            res.append((_lib.KERNEL_NAMES.get(self._kinds[j - 1], "?"), ms.value))
        return res

    def close(self) -> None:
        L = lib()
        for j in range(self.capacity):
            if self._events[j]:
                L.dpnorm_event_destroy(self._events[j])
                self._events[j] = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
