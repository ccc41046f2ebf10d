"""Pure-Python brute force MaxSim, for tiny inputs only.

TEST INFRASTRUCTURE ONLY.  It pins the numpy oracle (``oracle.maxsim``)
independently of BLAS: every dot product is an exactly rounded ``math.fsum``
of elementwise products, every max/argmax an explicit loop in increasing j,
every gradient an explicit loop.  Inputs are nested Python lists (or anything
with ``.tolist()``); masks are nested lists of bools or None.

Definition followed: README "Late Interaction Kernels", *What does it
compute?* and *Scoring interface* (valid-token max, valid-token sum, -1e9 for
an empty document).
"""

from __future__ import annotations

import math

EMPTY_DOC_SCORE = -1e9


def _lst(x):
    return x.tolist() if hasattr(x, "tolist") else x


def dot(u, v) -> float:
    """Exactly rounded dot product of two float vectors."""
    return math.fsum(a * b for a, b in zip(u, v))


def pair(q_tokens, q_valid, d_tokens, d_valid):
    """One query against one document.

    Returns (score, argmax list, second-best gap list).  argmax is -1 for
    masked query tokens and for an empty document.
    """
    Lq = len(q_tokens)
    valid_js = [j for j, ok in enumerate(d_valid) if ok]
    if not valid_js:
        return EMPTY_DOC_SCORE, [-1] * Lq, [math.inf] * Lq
    maxima, arg, gaps = [], [], []
    for i in range(Lq):
        if not q_valid[i]:
            arg.append(-1)
            gaps.append(math.inf)
            continue
        best, best_j, second = -math.inf, -1, -math.inf
        for j in valid_js:
            s = dot(q_tokens[i], d_tokens[j])
            if s > best:                     # strict: the lowest j keeps ties
                second = best
                best, best_j = s, j
            elif s > second:
                second = s
        maxima.append(best)
        arg.append(best_j)
        gaps.append(best - second if len(valid_js) > 1 else math.inf)
    return math.fsum(maxima), arg, gaps


def _masks(m, n, L):
    if m is None:
        return [[True] * L for _ in range(n)]
    return [[bool(x) for x in row] for row in _lst(m)]


def allpairs(Q, D, q_mask=None, d_mask=None):
    """scores[q][d], argmax[q][d][i] for every (query, doc)."""
    Q, D = _lst(Q), _lst(D)
    qm = _masks(q_mask, len(Q), len(Q[0]))
    dm = _masks(d_mask, len(D), len(D[0]))
    scores = [[0.0] * len(D) for _ in Q]
    argmax = [[None] * len(D) for _ in Q]
    for q in range(len(Q)):
        for d in range(len(D)):
            s, a, _ = pair(Q[q], qm[q], D[d], dm[d])
            scores[q][d] = s
            argmax[q][d] = a
    return scores, argmax


def allpairs_bwd(Q, D, g, argmax, q_mask=None, d_mask=None):
    """Explicit-loop gradients at the given argmax (lists of lists)."""
    Q, D, g = _lst(Q), _lst(D), _lst(g)
    Nq, Lq, dim = len(Q), len(Q[0]), len(Q[0][0])
    Nd, Ld = len(D), len(D[0])
    qm = _masks(q_mask, Nq, Lq)
    dm = _masks(d_mask, Nd, Ld)
    gQ_terms = [[[[] for _ in range(dim)] for _ in range(Lq)] for _ in range(Nq)]
    gD_terms = [[[[] for _ in range(dim)] for _ in range(Ld)] for _ in range(Nd)]
    for q in range(Nq):
        for d in range(Nd):
            if not any(dm[d]):
                continue
            for i in range(Lq):
                if not qm[q][i]:
                    continue
                j = argmax[q][d][i]
                w = g[q][d]
                for k in range(dim):
                    gQ_terms[q][i][k].append(w * D[d][j][k])
                    gD_terms[d][j][k].append(w * Q[q][i][k])
    gQ = [[[math.fsum(t) for t in row] for row in qq] for qq in gQ_terms]
    gD = [[[math.fsum(t) for t in row] for row in dd] for dd in gD_terms]
    return gQ, gD


def pairwise(Q, D, q_mask=None, d_mask=None):
    Q, D = _lst(Q), _lst(D)
    qm = _masks(q_mask, len(Q), len(Q[0]))
    dm = _masks(d_mask, len(D), len(D[0]))
    out = [pair(Q[b], qm[b], D[b], dm[b]) for b in range(len(Q))]
    return [o[0] for o in out], [o[1] for o in out]


def kd(Q, D, q_mask=None, d_mask=None):
    Q, D = _lst(Q), _lst(D)
    B, N, Ld = len(D), len(D[0]), len(D[0][0])
    qm = _masks(q_mask, B, len(Q[0]))
    dm = ([[[True] * Ld for _ in range(N)] for _ in range(B)] if d_mask is None
          else [[[bool(x) for x in r] for r in m] for m in _lst(d_mask)])
    scores = [[0.0] * N for _ in range(B)]
    argmax = [[None] * N for _ in range(B)]
    for b in range(B):
        for n in range(N):
            s, a, _ = pair(Q[b], qm[b], D[b][n], dm[b][n])
            scores[b][n], argmax[b][n] = s, a
    return scores, argmax
