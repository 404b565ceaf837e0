"""Parity rule for Hutch++ results against the fp64 oracle (shared by the GPU
tests).

Hutch++ ('Efficient DP-SGD for LLMs with Randomized Clipping', papernotes.org
note, 关键设计 › Hutch++): an exact head trace(Q^T O Q) on an orthonormal
basis Q of Col(O S) and a Hutchinson tail on (I - Q Q^T).

* The estimate n_hat is held to ``tol`` relative, always.
* Where the oracle keeps all m_s sketch columns and the complement of Q is
  not empty (m_s < p), head and tail are each a well-defined quantity of the
  inputs; each is held to ``tol`` of its own value, unless the tail is below
  TAIL_FLOOR of n_hat (then it is the rounding of a sketch that spans almost
  all of O, on both sides, and is held to ``tol`` of n_hat like the head).
* Where the oracle's sketch has lower rank than m_s, the columns past that
  rank hold only rounding on either side and their keep decision is not a
  property of the inputs: head and tail are held to ``tol`` of n_hat, and the
  kernel's rank may lie between the oracle's and m_s.
* The residuals that decided the rank (column residual over the largest
  column norm) agree with the oracle's to RESID_ATOL + RESID_RTOL of their
  value wherever the oracle's residual is above RESID_ROUNDING; on sketches of
  full rank that agreement and the oracle's distance from the threshold make
  the decision the same on both sides.
"""
import numpy as np

import oracle

TAIL_FLOOR = 1e-4
RESID_ROUNDING = 1e-3 * oracle.RANK_TAU   # a column this close to dependent holds rounding only
RESID_ATOL = 0.25 * oracle.RANK_TAU
RESID_RTOL = 1e-2


def oracle_residuals(A, G, S):
    """Per sample, the oracle's residuals of the sketch X_i = O_i S."""
    A, G, S = oracle.to_f64(A), oracle.to_f64(G), oracle.to_f64(S)
    return np.stack([oracle.basis_residuals(oracle.hutchpp_sketch(A[i], G[i], S)) for i in range(A.shape[0])])


def check(A, G, S, got, want, tol, what, resid=None):
    """got = (n, head, tail, rank) from the kernel, want = oracle.hutchpp(...).
    Returns a one-line summary; raises AssertionError on a violation."""
    n, head, tail, rank = [np.asarray(x.cpu().double().numpy() if hasattr(x, "cpu") else x, np.float64)
                           for x in got]
    wn, wh, wt, wr = [np.asarray(x, np.float64) for x in want]
    ms = S.shape[1]
    p = G.shape[2]
    full = (wr == ms) & (ms < p)
    own = full & (wt >= TAIL_FLOOR * np.abs(wn))
    scale_n = np.maximum(np.abs(wn), 1e-300)
    en = np.abs(n - wn) / scale_n
    eh = np.abs(head - wh) / np.where(own, np.maximum(np.abs(wh), 1e-300), scale_n)
    et = np.abs(tail - wt) / np.where(own, np.maximum(np.abs(wt), 1e-300), scale_n)
    line = (f"{what}: n {en.max():.2e} head {eh.max():.2e} tail {et.max():.2e} "
            f"(own value for {int(own.sum())}/{len(own)} samples) rank {rank.astype(int).tolist()} "
            f"oracle {wr.astype(int).tolist()}")
    bad = []
    if not np.all(en <= tol):
        bad.append("estimate")
    if not np.all(eh <= tol):
        bad.append("head")
    if not np.all(et <= tol):
        bad.append("tail")
    whole = wr == np.minimum(ms, p)
    if not np.array_equal(rank[whole], wr[whole]):
        bad.append("rank where the oracle keeps every column")
    if not (np.all(rank[~whole] >= wr[~whole]) and np.all(rank <= ms)):
        bad.append("rank bounds")
    if resid is not None:
        r = np.asarray(resid.cpu().double().numpy() if hasattr(resid, "cpu") else resid, np.float64)
        wres = oracle_residuals(A, G, S)
        meaningful = wres > RESID_ROUNDING
        d = np.abs(r - wres)[meaningful]
        lim = (RESID_ATOL + RESID_RTOL * wres)[meaningful]
        line += f" resid max diff {d.max() if d.size else 0.0:.1e}"
        if not np.all(d <= lim):
            bad.append("residuals")
        # the kernel compares in fp64 and reports a float residual: a band of
        # 1e-5 around the threshold absorbs that rounding
        lo = (r > oracle.RANK_TAU * (1 + 1e-5)).sum(axis=1)
        hi = (r > oracle.RANK_TAU * (1 - 1e-5)).sum(axis=1)
        if not (np.all(lo <= rank) and np.all(rank <= hi)):
            bad.append("rank is not the count of residuals above the threshold")
    assert not bad, line + " -- failed: " + ", ".join(bad)
    return line


def margins(resid, tau=oracle.RANK_TAU):
    """(smallest kept residual / tau, largest dropped residual / tau or 0)."""
    r = np.asarray(resid.cpu().double().numpy() if hasattr(resid, "cpu") else resid, np.float64)
    kept = r[r > tau]
    dropped = r[r <= tau]
    return (kept.min() / tau if kept.size else np.inf), (dropped.max() / tau if dropped.size else 0.0)
