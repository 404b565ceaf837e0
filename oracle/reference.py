"""CPU oracle for the per-sample gradient-norm path: TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 definitions of what the path computes. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this module; the product path never does, and it shares no code with
the HIP kernels (the seeded input generators in ``workloads`` are the only
common code, and they hold none of the arithmetic below).

Sources (the pages' titles and sections; formulas restated, not quoted):

* [RC-note] "Efficient DP-SGD for LLMs with Randomized Clipping",
  papernotes.org ICML 2026 note: 方法详解 › 整体框架 (overall framework) and
  关键设计 (key design: Hutchinson projection; Hutch++ head-tail split).
* [RC-nl] "Technische Samenvatting: Efficiënte DP-SGD voor LLM's met
  Geoptimaliseerde Randomized Clipping", gist.science/nl: Kernmechanisme,
  Algorithmische Flow.

Conventions. A is [B][T][d] (hooked activations), G is [B][T][p] (output
gradients), P is [p][k]. Every array is converted exactly to float64 before
any arithmetic. Matrix products use numpy's ``@`` (a library primitive) and
nothing is blocked, fused or reordered beyond the definitions.

Readings taken where the pages are silent or garbled (each is listed with its
reason in the design notes of the repository):

* P carries the 1/k: its entries have variance 1/k and the estimate is the
  plain sum ||A^T G P||_F^2, with no further division.
* Hutch++ works on the p x p matrix O = G^T A A^T G; the head is the exact
  trace of Q^T O Q and the tail is a Hutchinson estimate on (I - QQ^T).
* The sketch is O S = G^T (A (A^T (G S))), formed with two passes.
* Q is an orthonormal basis of the sketch's columns with a numerical rank
  rule: a column is kept when its residual after projecting out the kept
  basis exceeds ``tau`` times the largest column norm of the sketch.
* Clip factor min(C / sqrt(n), 1) (n is a squared norm).
"""
from __future__ import annotations

import math
from typing import Iterable, Sequence, Tuple

import numpy as np

RANK_TAU = 1e-4   # well above the rounding an fp32 sketch of bf16 data carries (about 1e-5 of its norm)


def to_f64(x) -> np.ndarray:
    """Exact conversion of a torch tensor (any float dtype) or array to float64."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch  # plain CPU op for the dtype conversion only
        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# Exact per-sample squared norm, three independent routes
# [RC-note 研究背景与动机: the exact per-sample norm ||A_i^T G_i||_F^2 is the
#  bottleneck; FGC materialises the gradient, GC forms T x T Gram matrices]
# [RC-note 切入角度 / RC-nl Kernmechanisme: ||A^T G||_F^2 = trace(G^T A A^T G)]
# --------------------------------------------------------------------------

def exact_explicit(A, G) -> np.ndarray:
    """n_i = ||W_i||_F^2 with the per-sample gradient W_i = A_i^T G_i (d x p)
    materialised (the explicit, FGC-style route)."""
    A, G = to_f64(A), to_f64(G)
    out = np.empty(A.shape[0])
    for i in range(A.shape[0]):
        W = A[i].T @ G[i]
        out[i] = np.sum(W * W)
    return out


def exact_gram(A, G) -> np.ndarray:
    """n_i = <A_i A_i^T, G_i G_i^T>_F: the ghost-norm route over T x T Gram
    matrices."""
    A, G = to_f64(A), to_f64(G)
    out = np.empty(A.shape[0])
    for i in range(A.shape[0]):
        KA = A[i] @ A[i].T
        KG = G[i] @ G[i].T
        out[i] = np.sum(KA * KG)
    return out


def exact_trace(A, G) -> np.ndarray:
    """n_i = trace(O_i) with O_i = G_i^T A_i A_i^T G_i formed explicitly (p x p).
    Tiny inputs only."""
    A, G = to_f64(A), to_f64(G)
    out = np.empty(A.shape[0])
    for i in range(A.shape[0]):
        O = G[i].T @ A[i] @ A[i].T @ G[i]
        out[i] = np.trace(O)
    return out


# --------------------------------------------------------------------------
# Hutchinson estimate [RC-note 关键设计 › Hutchinson 随机投影估范数]
# --------------------------------------------------------------------------

def hutch(A, G, P) -> np.ndarray:
    """n_hat_i = ||Y_i||_F^2 with Y_i = A_i^T (G_i P): G P is formed first, then
    A^T times it, then the squared Frobenius norm; neither the d x p gradient
    nor any T x T matrix is formed. P is shared by the B samples."""
    A, G, P = to_f64(A), to_f64(G), to_f64(P)
    out = np.empty(A.shape[0])
    for i in range(A.shape[0]):
        GP = G[i] @ P
        Y = A[i].T @ GP
        out[i] = np.sum(Y * Y)
    return out


def hutch_trace_form(A, G, P) -> np.ndarray:
    """The same estimate written as trace(P^T O_i P) with O_i explicit (p x p).
    Tiny inputs only."""
    A, G, P = to_f64(A), to_f64(G), to_f64(P)
    out = np.empty(A.shape[0])
    for i in range(A.shape[0]):
        O = G[i].T @ A[i] @ A[i].T @ G[i]
        out[i] = np.trace(P.T @ O @ P)
    return out


# --------------------------------------------------------------------------
# Hutchinson with a +-1 projection [RC-note 实验关键数据 › 关键发现 and
#  局限与展望: {-1,+1} 1-bit projection matrices in the style of Achlioptas
#  shrink P; RC-nl Betekenis en Claims: +-1-valued sketches]
# Reading: P = S / sqrt(k) with S in {-1,+1}^{p x k}, so that E[P P^T] = I as
# for the N(0, 1/k) matrix and the estimate stays unbiased.
# --------------------------------------------------------------------------

def unpack_signs(S_bits, p: int, k: int) -> np.ndarray:
    """S [p][k] in {-1,+1} from bit-packed rows of 32-bit words: entry (v, j)
    is bit j % 32 of word j // 32 of row v, 0 meaning +1 and 1 meaning -1."""
    if hasattr(S_bits, "detach"):
        S_bits = S_bits.detach().to("cpu").numpy()
    words = np.asarray(S_bits).view(np.uint32).reshape(p, -1)
    S = np.empty((p, k))
    for v in range(p):
        for j in range(k):
            bit = (int(words[v, j // 32]) >> (j % 32)) & 1
            S[v, j] = -1.0 if bit else 1.0
    return S


def hutch_sign(A, G, S_bits, k: int) -> np.ndarray:
    """n_hat_i = ||A_i^T (G_i P)||_F^2 with P = S / sqrt(k) and S the unpacked
    signs (the same estimate as hutch with that P)."""
    p = G.shape[-1]
    return hutch(A, G, unpack_signs(S_bits, p, k) / math.sqrt(k))


# --------------------------------------------------------------------------
# Route between the exact norm and the estimate [RC-note 实验关键数据: full
#  fine-tuning and LoRA; 研究背景与动机: the exact norm is what the estimate
#  replaces]. Reading: a layer whose narrow side min(d, p) is at most k gets
#  its exact norm (a k-column estimate would cost as much); the others get the
#  Hutchinson estimate with their P.
# --------------------------------------------------------------------------

def routes_exact(d: int, p: int, k: int) -> bool:
    return min(int(d), int(p)) <= int(k)


def norms_routed(layers, k: int):
    """Per-sample sum over (A, G, P) layers of exact_explicit (routed layers)
    or hutch (the others); returns (n, routes) with routes 1 for exact."""
    parts, routes = [], []
    for (A, G, P) in layers:
        exact = routes_exact(A.shape[-1], G.shape[-1], k)
        parts.append(exact_explicit(A, G) if exact else hutch(A, G, P))
        routes.append(1 if exact else 0)
    return layer_sum(parts), routes


# --------------------------------------------------------------------------
# Hutch++ [RC-note 关键设计 › Hutch++ 头-尾分解的低误差变体;
#          RC-nl Kernmechanisme item 2]
# --------------------------------------------------------------------------

def hutchpp_split(k: int) -> Tuple[int, int]:
    """Budget k -> (m_s, m_t): ceil(k/3) sketch columns (and as many head
    columns), k - 2 ceil(k/3) tail columns."""
    m_s = -(-int(k) // 3)
    return m_s, int(k) - 2 * m_s


def _gram_schmidt(X, tau: float):
    """Sequential Gram-Schmidt over the columns of X (p x m), each column
    projected against the kept basis twice; column j is kept iff its residual
    norm exceeds tau * max_a ||x_a||. Returns the kept unit vectors and, per
    column, that residual norm over max_a ||x_a|| (0 for a zero X)."""
    X = to_f64(X)
    p, m = X.shape
    scale = max((np.linalg.norm(X[:, j]) for j in range(m)), default=0.0)
    basis, resid = [], []
    for j in range(m):
        v = X[:, j].copy()
        for _ in range(2):
            for q in basis:
                v -= q * np.dot(q, v)
        nv = np.linalg.norm(v)
        resid.append(nv / scale if scale > 0.0 else 0.0)
        if nv > tau * scale and nv > 0.0:
            basis.append(v / nv)
    return basis, np.array(resid)


def orthonormal_basis(X, tau: float = RANK_TAU) -> np.ndarray:
    """Orthonormal basis of the column span of X (p x m) by sequential
    Gram-Schmidt, each column projected against the kept basis twice.
    A column is kept iff its residual norm exceeds tau * max_j ||x_j||.
    Returns Q (p x r), r <= m."""
    basis, _ = _gram_schmidt(X, tau)
    if not basis:
        return np.zeros((to_f64(X).shape[0], 0))
    return np.stack(basis, axis=1)


def basis_residuals(X, tau: float = RANK_TAU) -> np.ndarray:
    """Per column of X, the residual norm that the rank rule of
    orthonormal_basis compares with tau (relative to the largest column
    norm): column j is kept iff this value exceeds tau."""
    return _gram_schmidt(X, tau)[1]


def hutchpp_sample(A_i, G_i, S, P, tau: float = RANK_TAU):
    """One sample of Hutch++ on O = G^T A A^T G (p x p).

    1. sketch: X = O S = G^T (A (A^T (G S)))
    2. Q = orthonormal basis of Col(X)
    3. head = trace(Q^T O Q) = ||A^T (G Q)||_F^2 (exact on span Q)
    4. tail = ||A^T (G P')||_F^2 with P' = (I - Q Q^T) P (Hutchinson on the
       complement; P has entries of variance 1/m_t)
    Returns (n_hat, head, tail, rank).
    """
    A_i, G_i, S, P = to_f64(A_i), to_f64(G_i), to_f64(S), to_f64(P)
    X = hutchpp_sketch(A_i, G_i, S)
    Q = orthonormal_basis(X, tau)
    head, tail = hutchpp_head_tail(A_i, G_i, Q, P)
    return head + tail, head, tail, Q.shape[1]


def hutchpp_sketch(A_i, G_i, S) -> np.ndarray:
    """X = O S = G^T (A (A^T (G S))) for one sample (p x m_s), two passes."""
    A_i, G_i, S = to_f64(A_i), to_f64(G_i), to_f64(S)
    YS = A_i.T @ (G_i @ S)
    return G_i.T @ (A_i @ YS)


def hutchpp_head_tail(A_i, G_i, Q, P):
    """Given an orthonormal Q (p x r) and tail projection P (p x m_t):
    head = ||A^T (G Q)||_F^2 = trace(Q^T O Q),
    tail = ||A^T (G P')||_F^2 with P' = P - Q (Q^T P)."""
    A_i, G_i, Q, P = to_f64(A_i), to_f64(G_i), to_f64(Q), to_f64(P)
    H = A_i.T @ (G_i @ Q)
    head = float(np.sum(H * H))
    Pt = P - Q @ (Q.T @ P)
    R = A_i.T @ (G_i @ Pt)
    tail = float(np.sum(R * R))
    return head, tail


def hutchpp(A, G, S, P, tau: float = RANK_TAU):
    """Per-sample Hutch++ estimates; returns (n_hat, head, tail, rank) arrays."""
    A, G = to_f64(A), to_f64(G)
    B = A.shape[0]
    res = [hutchpp_sample(A[i], G[i], S, P, tau) for i in range(B)]
    n = np.array([r[0] for r in res])
    head = np.array([r[1] for r in res])
    tail = np.array([r[2] for r in res])
    rank = np.array([r[3] for r in res], dtype=np.int64)
    return n, head, tail, rank


# --------------------------------------------------------------------------
# Layer sum and clip factors [RC-note 方法详解 › 整体框架]
# --------------------------------------------------------------------------

def layer_sum(per_layer: Iterable[Sequence[float]]) -> np.ndarray:
    """n_i = sum over linear-like layers l of n_hat_i^(l)."""
    total = None
    for n in per_layer:
        n = np.asarray(n, dtype=np.float64)
        total = n.copy() if total is None else total + n
    return total


def clip_factors(n, C: float) -> np.ndarray:
    """c_i = min(C / sqrt(n_i), 1); n_i = 0 gives 1, n_i = inf gives 0."""
    n = np.asarray(n, dtype=np.float64)
    out = np.empty_like(n)
    for i, v in enumerate(n):
        if math.isnan(v):
            out[i] = math.nan
        elif v <= 0.0:
            out[i] = 1.0
        else:
            out[i] = min(C / math.sqrt(v), 1.0)
    return out
