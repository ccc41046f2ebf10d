"""Float64 CPU oracle for the cross-entropy loss head over MaxSim scores.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests, the
smoke check and the benchmark's CPU-baseline leg, never by the library.

The colpali pull request routes its in-batch ColBERT loss and its
negative-doc losses (over the per-query candidate, kd, layout) through the
MaxSim operator (*What this PR adds*), and its *Results* benchmark the loss
head on top of the scores.  The pages name these losses but do not define
them.  The reading taken here, the plainest one the rest supports: softmax
cross-entropy over each score row with one target column per row -- the
diagonal for the in-batch loss (query b against its own document b), column
0 for the negative-doc loss over kd scores [B, N] (candidate 0 is the
positive) -- averaged over the rows, with a logit scale s (1 unless given):

    l_r  = logsumexp_c(s * S[r, c]) - s * S[r, t_r]
    L    = (1 / R) * sum_r l_r
    dL/dS[r, c] = (s / R) * (softmax_c(s * S[r, :]) - [c == t_r])

Every step is float64; the log-sum-exp subtracts the row maximum first.
"""

from __future__ import annotations

import numpy as np


def ce_rows(scores, labels=None, scale: float = 1.0):
    """(mean loss, per-row losses [R], grad [R, C]) of the row cross-entropy.

    ``labels`` is an int array [R] of target columns, or None for the
    diagonal (target r for row r, which needs C >= R)."""
    S = np.asarray(scores, dtype=np.float64)
    assert S.ndim == 2 and np.all(np.isfinite(S))
    R, C = S.shape
    t = np.arange(R) if labels is None else np.asarray(labels, dtype=np.int64)
    assert t.shape == (R,) and np.all((t >= 0) & (t < C))
    z = float(scale) * S
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    tot = e.sum(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(tot[:, 0])
    rows = np.arange(R)
    row_loss = lse - z[rows, t]
    p = e / tot
    p[rows, t] -= 1.0
    grad = (float(scale) / R) * p
    return float(row_loss.mean()), row_loss, grad
