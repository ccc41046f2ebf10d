"""Float64 CPU oracle for MaxSim scoring, forward and backward.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests, the
smoke check and the benchmark's CPU-baseline leg, never by the library.

What is computed (README "Late Interaction Kernels", *What does it compute?*):

    MaxSim(Q, D) = sum over valid query tokens i of
                   max over valid document tokens j of  Q_i . D_j

with the *Scoring interface* rules: a query mask removes tokens from the sum,
a document mask removes tokens from the max, a document with no valid token
scores exactly -1e9, dot products are raw (no normalisation), and scores are
reported in float32 by the library (kept in float64 here).

The social thread (post (2/N)) and the colpali pull request (*What this PR
adds*: "einsum + amax + sum") describe the naive path: materialise the
similarity grid, take the max over document tokens, sum over query tokens.
This module is that naive path, evaluated in float64 one document at a time
(the grid of a single document against its queries; never the full 4-D
grid).  Post (5/N) states the fused method is mathematically identical to
it, so the definition itself is the oracle.

Backward (post (5/N): the backward is fused too; colpali PR *Results*: only
the input gradients are produced).  The score is piecewise linear in Q and D;
at the chosen argmax a(q,d,i) its gradient is

    dL/dQ[q,i,:] = sum over non-empty d of g[q,d] * D[d, a(q,d,i), :]
    dL/dD[d,j,:] = sum over (q, valid i) with a(q,d,i) = j of g[q,d] * Q[q,i,:]

Readings where the pages are silent (all listed in the design notes):

* ties: the lowest valid document index wins; all gradient goes to it;
* a query with no valid token against a non-empty doc scores 0 (empty sum);
* an empty document scores -1e9 for every query, including empty queries,
  and passes no gradient;
* masked query tokens and empty documents report argmax -1;
* kd masks are q_mask [B, Lq] and d_mask [B, N, Ld];
* inputs are assumed finite.
"""

from __future__ import annotations

from dataclasses import dataclass
import numpy as np

#: Score of a document with no valid token (README, *Scoring interface*).
EMPTY_DOC_SCORE = -1e9
#: Gap between the top two similarities below which several argmax indices
#: are equally admissible.
TIE_GAP = 1e-5


@dataclass
class ForwardResult:
    """Oracle forward output for one layout.

    scores : float64, [Nq, Nd] / [B] / [B, N]
    argmax : int64, scores.shape + [Lq]; lowest valid j reaching the max, or -1
             for masked query tokens and empty documents
    gap    : float64, same shape as argmax; max minus the largest similarity
             over the other valid doc tokens (inf when the doc has one valid
             token, or where argmax is -1)
    """

    scores: np.ndarray
    argmax: np.ndarray
    gap: np.ndarray

    @property
    def tie(self) -> np.ndarray:
        """True where the top two similarities lie within TIE_GAP."""
        return self.gap <= TIE_GAP


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------

def _f64(x) -> np.ndarray:
    a = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(a)):
        raise ValueError("oracle inputs must be finite")
    return a


def _mask(m, shape) -> np.ndarray:
    if m is None:
        return np.ones(shape, dtype=bool)
    a = np.asarray(m).astype(bool)
    if a.shape != tuple(shape):
        raise ValueError(f"mask shape {a.shape} != expected {tuple(shape)}")
    return a


def maxsim_block(Qb: np.ndarray, qmask_b: np.ndarray, Dd: np.ndarray,
                 dmask_d: np.ndarray):
    """MaxSim of n queries against ONE document.

    Qb [n, Lq, dim] float64, qmask_b [n, Lq] bool, Dd [Ld, dim] float64,
    dmask_d [Ld] bool.  Returns (scores [n], argmax [n, Lq], gap [n, Lq]).

    This is the naive grid for one document: S[(q,i), j] = Q[q,i] . D[j] over
    the valid j, then max (and argmax) over j, then the sum over valid i.
    """
    n, Lq, dim = Qb.shape
    valid_j = np.flatnonzero(dmask_d)
    argmax = np.full((n, Lq), -1, dtype=np.int64)
    gap = np.full((n, Lq), np.inf)
    if valid_j.size == 0:
        # README *Scoring interface*: no valid document token -> -1e9.
        return np.full(n, EMPTY_DOC_SCORE), argmax, gap
    S = Qb.reshape(n * Lq, dim) @ Dd[valid_j].T            # [(n*Lq), |V|]
    k = np.argmax(S, axis=1)                               # first = lowest j
    rows = np.arange(n * Lq)
    m = S[rows, k]
    if valid_j.size > 1:
        S[rows, k] = -np.inf
        second = S.max(axis=1)
        g = m - second
    else:
        g = np.full(n * Lq, np.inf)
    m = m.reshape(n, Lq)
    qv = qmask_b
    # Query mask: masked tokens leave the sum (contribute exactly 0).
    scores = np.where(qv, m, 0.0).sum(axis=1)
    argmax[qv] = valid_j[k.reshape(n, Lq)][qv]
    gap[qv] = g.reshape(n, Lq)[qv]
    return scores, argmax, gap


def _bwd_block(Qb, qmask_b, Dd, dmask_d, g_b, argmax_b, gQ_b, gD_d):
    """Accumulate the gradients of n (query, doc) pairs sharing ONE doc.

    gQ_b [n, Lq, dim] and gD_d [Ld, dim] are float64 accumulators updated in
    place.  argmax_b [n, Lq] must name a valid doc token wherever the query
    token is valid and the doc is non-empty; elsewhere it is ignored.
    """
    if not dmask_d.any():
        return                      # empty doc: constant score, zero gradient
    sel = qmask_b
    rows = argmax_b[sel]
    if rows.size == 0:
        return
    if rows.min() < 0 or rows.max() >= Dd.shape[0] or not dmask_d[rows].all():
        raise ValueError("argmax names an invalid document token")
    w = np.broadcast_to(g_b[:, None], qmask_b.shape)[sel]          # g[q,d]
    gQ_b[sel] += w[:, None] * Dd[rows]
    np.add.at(gD_d, rows, w[:, None] * Qb[sel])


def token_similarity(Q, D, qidx, didx, i: int, j: int) -> float:
    """float64 Q[qidx][i] . D[didx][j] (used to admit tie-broken indices)."""
    return float(np.dot(_f64(Q[qidx][i]), _f64(D[didx][j])))


def admissible_argmax(fwd: ForwardResult, other: np.ndarray, Q, D,
                      d_mask, layout: str) -> np.ndarray:
    """Merge another implementation's argmax with the oracle's.

    Outside ties (gap > TIE_GAP) the indices must be identical, -1 sentinels
    included.  At a tie the other index is adopted if it names a valid doc
    token whose similarity is within TIE_GAP of the maximum.  Raises
    AssertionError on any other difference.  Returns the merged argmax,
    which then drives the oracle backward.
    """
    other = np.asarray(other).astype(np.int64)
    if other.shape != fwd.argmax.shape:
        raise AssertionError(f"argmax shape {other.shape} != {fwd.argmax.shape}")
    diff = np.argwhere(other != fwd.argmax)
    merged = fwd.argmax.copy()
    for pos in diff:
        pos = tuple(int(p) for p in pos)
        mine, theirs = int(fwd.argmax[pos]), int(other[pos])
        if not fwd.tie[pos] or mine < 0:
            raise AssertionError(
                f"argmax mismatch at {pos}: oracle {mine}, other {theirs}, "
                f"gap {fwd.gap[pos]:.3e}")
        if layout == "allpairs":
            q, d, i = pos
            qidx, didx = q, d
            dm = None if d_mask is None else np.asarray(d_mask)[d]
        elif layout == "pairwise":
            b, i = pos
            qidx, didx = b, b
            dm = None if d_mask is None else np.asarray(d_mask)[b]
        elif layout == "kd":
            b, n, i = pos
            qidx, didx = b, (b, n)
            dm = None if d_mask is None else np.asarray(d_mask)[b, n]
        else:
            raise ValueError(layout)
        Ld = np.asarray(D[didx]).shape[0]
        if not (0 <= theirs < Ld) or (dm is not None and not dm[theirs]):
            raise AssertionError(f"argmax at {pos} names invalid doc token {theirs}")
        s_max = token_similarity(Q, D, qidx, didx, i, mine)
        s_their = token_similarity(Q, D, qidx, didx, i, theirs)
        if s_their < s_max - TIE_GAP:
            raise AssertionError(
                f"argmax at {pos}: token {theirs} similarity {s_their} is not "
                f"within {TIE_GAP} of the max {s_max}")
        merged[pos] = theirs
    return merged


# --------------------------------------------------------------------------
# all-pairs:  Q [Nq, Lq, dim] x D [Nd, Ld, dim] -> [Nq, Nd]
# --------------------------------------------------------------------------

def maxsim_allpairs(Q, D, q_mask=None, d_mask=None) -> ForwardResult:
    """Every query against every document (README *Scoring interface*,
    layer MaxSim: [Nq, Lq, dim] x [Nd, Ld, dim] -> [Nq, Nd])."""
    Q, D = _f64(Q), _f64(D)
    Nq, Lq, dim = Q.shape
    Nd, Ld, dim2 = D.shape
    if dim != dim2:
        raise ValueError("query and document embedding dims differ")
    qm = _mask(q_mask, (Nq, Lq))
    dm = _mask(d_mask, (Nd, Ld))
    scores = np.empty((Nq, Nd))
    argmax = np.empty((Nq, Nd, Lq), dtype=np.int64)
    gap = np.empty((Nq, Nd, Lq))
    for d in range(Nd):
        s, a, g = maxsim_block(Q, qm, D[d], dm[d])
        scores[:, d], argmax[:, d], gap[:, d] = s, a, g
    return ForwardResult(scores, argmax, gap)


def maxsim_allpairs_bwd(Q, D, grad_scores, argmax, q_mask=None, d_mask=None):
    """Gradients of sum(grad_scores * scores) w.r.t. Q and D (float64)."""
    Q, D = _f64(Q), _f64(D)
    g = _f64(grad_scores)
    Nq, Lq, dim = Q.shape
    Nd, Ld, _ = D.shape
    qm = _mask(q_mask, (Nq, Lq))
    dm = _mask(d_mask, (Nd, Ld))
    argmax = np.asarray(argmax)
    gQ = np.zeros_like(Q)
    gD = np.zeros_like(D)
    for d in range(Nd):
        _bwd_block(Q, qm, D[d], dm[d], g[:, d], argmax[:, d], gQ, gD[d])
    return gQ, gD


# --------------------------------------------------------------------------
# pairwise:  Q [B, Lq, dim] x D [B, Ld, dim] -> [B]
# --------------------------------------------------------------------------

def maxsim_pairwise(Q, D, q_mask=None, d_mask=None) -> ForwardResult:
    """Query b against document b only (README *Scoring interface*, layer
    MaxSimPairwise: [B, Lq, dim] x [B, Ld, dim] -> [B])."""
    Q, D = _f64(Q), _f64(D)
    B, Lq, dim = Q.shape
    B2, Ld, dim2 = D.shape
    if B != B2 or dim != dim2:
        raise ValueError("pairwise inputs disagree in batch or dim")
    qm = _mask(q_mask, (B, Lq))
    dm = _mask(d_mask, (B, Ld))
    scores = np.empty(B)
    argmax = np.empty((B, Lq), dtype=np.int64)
    gap = np.empty((B, Lq))
    for b in range(B):
        s, a, g = maxsim_block(Q[b:b + 1], qm[b:b + 1], D[b], dm[b])
        scores[b], argmax[b], gap[b] = s[0], a[0], g[0]
    return ForwardResult(scores, argmax, gap)


def maxsim_pairwise_bwd(Q, D, grad_scores, argmax, q_mask=None, d_mask=None):
    Q, D = _f64(Q), _f64(D)
    g = _f64(grad_scores)
    B, Lq, _ = Q.shape
    Ld = D.shape[1]
    qm = _mask(q_mask, (B, Lq))
    dm = _mask(d_mask, (B, Ld))
    argmax = np.asarray(argmax)
    gQ = np.zeros_like(Q)
    gD = np.zeros_like(D)
    for b in range(B):
        _bwd_block(Q[b:b + 1], qm[b:b + 1], D[b], dm[b], g[b:b + 1],
                   argmax[b:b + 1], gQ[b:b + 1], gD[b])
    return gQ, gD


# --------------------------------------------------------------------------
# kd (per-query candidates):  Q [B, Lq, dim] x D [B, N, Ld, dim] -> [B, N]
# --------------------------------------------------------------------------

def maxsim_kd(Q, D, q_mask=None, d_mask=None) -> ForwardResult:
    """Query b against each of its own N candidate documents (colpali PR,
    *Design*: the per-query candidate layout [B, N, Ld, d])."""
    Q, D = _f64(Q), _f64(D)
    B, Lq, dim = Q.shape
    B2, N, Ld, dim2 = D.shape
    if B != B2 or dim != dim2:
        raise ValueError("kd inputs disagree in batch or dim")
    qm = _mask(q_mask, (B, Lq))
    dm = _mask(d_mask, (B, N, Ld))
    scores = np.empty((B, N))
    argmax = np.empty((B, N, Lq), dtype=np.int64)
    gap = np.empty((B, N, Lq))
    for b in range(B):
        for n in range(N):
            s, a, g = maxsim_block(Q[b:b + 1], qm[b:b + 1], D[b, n], dm[b, n])
            scores[b, n], argmax[b, n], gap[b, n] = s[0], a[0], g[0]
    return ForwardResult(scores, argmax, gap)


def maxsim_kd_bwd(Q, D, grad_scores, argmax, q_mask=None, d_mask=None):
    Q, D = _f64(Q), _f64(D)
    g = _f64(grad_scores)
    B, Lq, _ = Q.shape
    _, N, Ld, _ = D.shape
    qm = _mask(q_mask, (B, Lq))
    dm = _mask(d_mask, (B, N, Ld))
    argmax = np.asarray(argmax)
    gQ = np.zeros_like(Q)
    gD = np.zeros_like(D)
    for b in range(B):
        for n in range(N):
            _bwd_block(Q[b:b + 1], qm[b:b + 1], D[b, n], dm[b, n],
                       g[b, n:n + 1], argmax[b, n][None], gQ[b:b + 1], gD[b, n])
    return gQ, gD


def scores_as_float32(scores: np.ndarray) -> np.ndarray:
    """The library reports float32 scores (README *Scoring interface*)."""
    return np.asarray(scores, dtype=np.float32)


__all__ = [
    "EMPTY_DOC_SCORE", "TIE_GAP", "ForwardResult", "maxsim_block",
    "maxsim_allpairs", "maxsim_allpairs_bwd", "maxsim_pairwise",
    "maxsim_pairwise_bwd", "maxsim_kd", "maxsim_kd_bwd", "token_similarity",
    "admissible_argmax", "scores_as_float32",
]

