"""Seeded synthetic inputs for the MaxSim workloads.

This module only draws and rounds inputs; it holds none of the scoring
arithmetic, and both the GPU path's tests/benchmark and the CPU oracle's tests
take their inputs from it.

Recipe (identical bits go to the GPU and to the oracle):

1. ``numpy.random.default_rng(seed)``; fixed draw order: query normals, doc
   normals, query lengths, doc lengths, candidate-0 noise (kd), upstream grad.
2. Tokens are drawn in float32 and L2-normalised per token in float32, then
   rounded once to the workload dtype (round-to-nearest-even via torch CPU).
3. Lengths are integers uniform in [lo, hi] inclusive; token rows at or past
   the length are set to exactly zero after rounding and masked False.
4. Very large document tensors are drawn per document from
   ``default_rng([seed, doc_index])`` in a thread pool, so no multi-GiB
   float32 temporary is needed.

The shapes and value distributions are those of the pages' workloads
(ColBERT-style text at Lq=32, ColPali-scale pages at Ld=1030, negative-doc
candidates B x N, long documents); the real datasets named there are not
available, and these synthetic tensors stand in for them.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


@dataclass
class Workload:
    """One scoring call: inputs on the CPU in the workload dtype."""

    name: str
    layout: str                      # "allpairs" | "pairwise" | "kd"
    dtype: str                       # "f16" | "bf16" | "f32"
    Q: torch.Tensor                  # [Nq|B, Lq, dim]
    D: torch.Tensor                  # [Nd, Ld, dim] | [B, Ld, dim] | [B, N, Ld, dim]
    q_mask: Optional[torch.Tensor]   # bool [Nq|B, Lq] or None (all valid)
    d_mask: Optional[torch.Tensor]   # bool, D.shape[:-1] or None
    grad: Optional[torch.Tensor]     # float32, scores shape, or None (fwd only)
    meta: dict = field(default_factory=dict)

    @property
    def dim(self) -> int:
        return int(self.Q.shape[-1])

    @property
    def scores_shape(self):
        if self.layout == "allpairs":
            return (self.Q.shape[0], self.D.shape[0])
        if self.layout == "pairwise":
            return (self.Q.shape[0],)
        return (self.D.shape[0], self.D.shape[1])

    def numpy_inputs(self):
        """float32 numpy copies (exact for every supported dtype) for the oracle."""
        m = lambda x: None if x is None else x.numpy()
        return (self.Q.float().numpy(), self.D.float().numpy(),
                m(self.q_mask), m(self.d_mask))


def _normalize_round(x: np.ndarray, dtype: str) -> torch.Tensor:
    """L2-normalise each token (last axis) in float32, round once to dtype."""
    x = np.asarray(x, dtype=np.float32)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    x = x / n
    return torch.from_numpy(np.ascontiguousarray(x)).to(DTYPES[dtype])


def _lengths(rng, n, lo, hi) -> np.ndarray:
    return rng.integers(lo, hi + 1, size=n)


def _length_mask(lengths: np.ndarray, L: int) -> torch.Tensor:
    return torch.from_numpy(np.arange(L)[None, :] < lengths[:, None])


def _zero_padding(x: torch.Tensor, mask: torch.Tensor) -> torch.Tensor:
    x = x.clone()
    x[~mask] = 0
    return x


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _docs_per_seed(seed: int, n_docs: int, Ld: int, dim: int, dtype: str,
                   first_index: int = 0) -> torch.Tensor:
    """Doc d drawn from default_rng([seed, first_index + d]) and normalised."""
    out = torch.empty((n_docs, Ld, dim), dtype=DTYPES[dtype])

    def one(d):
        r = np.random.default_rng([seed, first_index + d])
        x = r.standard_normal((Ld, dim), dtype=np.float32)
        out[d] = _normalize_round(x, dtype)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(n_docs)))
    return out


# --------------------------------------------------------------------------
# the five workloads (sizes are parameters so tests can shrink them while
# keeping the recipe: lengths, masks, dtype and value distribution)
# --------------------------------------------------------------------------

def tiny_allpairs(seed: int = 1001, Nq: int = 2, Lq: int = 32, Nd: int = 4,
                  Ld: int = 180, dim: int = 128, dtype: str = "f16",
                  masked_from: int = 150):
    """Quickstart of the README (*Quickstart*): 2 queries x 4 documents,
    fp16, normalised Gaussian tokens, document positions 150.. masked.

    Returns (allpairs workload, pairwise workload on the first 2 documents).
    The document rows past position 150 stay random (only masked), as in the
    README example.
    """
    rng = np.random.default_rng(seed)
    Q = _normalize_round(rng.standard_normal((Nq, Lq, dim), dtype=np.float32), dtype)
    D = _normalize_round(rng.standard_normal((Nd, Ld, dim), dtype=np.float32), dtype)
    q_mask = torch.ones((Nq, Lq), dtype=torch.bool)
    d_mask = torch.ones((Nd, Ld), dtype=torch.bool)
    d_mask[:, masked_from:] = False
    g = torch.from_numpy(rng.standard_normal((Nq, Nd), dtype=np.float32))
    g_pair = torch.from_numpy(rng.standard_normal((Nq,), dtype=np.float32))
    ap = Workload("tiny-allpairs", "allpairs", dtype, Q, D, q_mask, d_mask, g)
    npair = min(Nq, Nd)
    pw = Workload("tiny-pairwise", "pairwise", dtype, Q[:npair].contiguous(),
                  D[:npair].contiguous(), q_mask[:npair].clone(),
                  d_mask[:npair].clone(), g_pair[:npair].clone())
    return ap, pw


def inbatch_text(seed: int = 1002, B: int = 256, Lq: int = 32, Ld: int = 300,
                 dim: int = 128, dtype: str = "bf16", d_lo: int = 64,
                 d_hi: int = 300, Nd: Optional[int] = None) -> Workload:
    """ColBERT-text in-batch contrastive: B queries x B docs padded to Ld,
    doc lengths uniform in [d_lo, d_hi], padded rows zero and masked,
    Gaussian upstream grad on the [B, B] scores."""
    Nd = B if Nd is None else Nd
    rng = np.random.default_rng(seed)
    Q = _normalize_round(rng.standard_normal((B, Lq, dim), dtype=np.float32), dtype)
    D = _normalize_round(rng.standard_normal((Nd, Ld, dim), dtype=np.float32), dtype)
    d_len = _lengths(rng, Nd, d_lo, min(d_hi, Ld))
    d_mask = _length_mask(d_len, Ld)
    D = _zero_padding(D, d_mask)
    g = torch.from_numpy(rng.standard_normal((B, Nd), dtype=np.float32))
    return Workload("inbatch-text", "allpairs", dtype, Q, D, None, d_mask, g,
                    meta={"d_len": d_len})


def inbatch_pages(seed: int = 1003, B: int = 128, Lq: int = 32, Ld: int = 1030,
                  dim: int = 128, dtype: str = "bf16", q_lo: int = 8,
                  q_hi: int = 32) -> Workload:
    """ColPali-scale in-batch contrastive: query lengths uniform in
    [q_lo, q_hi] (zero, masked tail), docs all valid.  The upstream grad is
    the gradient of a cross-entropy over the diagonal of the scores, so it is
    left None here: the loss head forms it from the scores."""
    rng = np.random.default_rng(seed)
    Q = _normalize_round(rng.standard_normal((B, Lq, dim), dtype=np.float32), dtype)
    D = _normalize_round(rng.standard_normal((B, Ld, dim), dtype=np.float32), dtype)
    q_len = _lengths(rng, B, q_lo, min(q_hi, Lq))
    q_mask = _length_mask(q_len, Lq)
    Q = _zero_padding(Q, q_mask)
    return Workload("inbatch-pages", "allpairs", dtype, Q, D, q_mask, None, None,
                    meta={"q_len": q_len, "grad": "ce_diag"})


def kd_candidates(seed: int = 1004, B: int = 256, Lq: int = 32, N: int = 16,
                  Ld: int = 1030, dim: int = 128, dtype: str = "bf16",
                  noise: float = 0.3) -> Workload:
    """Negative-doc kd layout: B queries, N candidates each of Ld tokens, all
    valid.  Candidate 0 of query b holds the query's tokens plus N(0, noise^2)
    noise, renormalised, at positions j < Lq; its remaining tokens and the
    other candidates are normalised Gaussians."""
    rng = np.random.default_rng(seed)
    q32 = rng.standard_normal((B, Lq, dim), dtype=np.float32)
    q32 /= np.sqrt(np.sum(q32 * q32, axis=-1, keepdims=True, dtype=np.float32))
    Q = torch.from_numpy(q32).to(DTYPES[dtype])
    D = torch.empty((B, N, Ld, dim), dtype=DTYPES[dtype])

    def one(b):
        r = np.random.default_rng([seed, b])
        x = r.standard_normal((N, Ld, dim), dtype=np.float32)
        D[b] = _normalize_round(x, dtype)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(B)))
    k = min(Lq, Ld)
    z = rng.standard_normal((B, k, dim), dtype=np.float32)
    base = Q[:, :k].float().numpy()          # the rounded query tokens
    D[:, 0, :k] = _normalize_round(base + noise * z, dtype)
    g = torch.from_numpy(rng.standard_normal((B, N), dtype=np.float32))
    return Workload("kd-candidates", "kd", dtype, Q, D, None, None, g)


def long_docs(seed: int = 1005, Nq: int = 16, Lq: int = 32, Nd: int = 1000,
              Ld: int = 8192, dim: int = 128, dtype: str = "f16",
              d_lo: int = 4096, d_hi: int = 8192) -> Workload:
    """Long-document all-pairs scoring, forward only: doc lengths uniform in
    [d_lo, d_hi] with a zero, masked tail; doc d drawn from
    default_rng([seed, d])."""
    rng = np.random.default_rng(seed)
    Q = _normalize_round(rng.standard_normal((Nq, Lq, dim), dtype=np.float32), dtype)
    d_len = _lengths(rng, Nd, d_lo, min(d_hi, Ld))
    D = _docs_per_seed(seed, Nd, Ld, dim, dtype)
    d_mask = _length_mask(d_len, Ld)
    D[~d_mask] = 0
    return Workload("long-docs", "allpairs", dtype, Q, D, None, d_mask, None,
                    meta={"d_len": d_len})


def long_rerank(seed: int = 10052, B: int = 64, Lq: int = 32, Ld: int = 32768,
                dim: int = 128, dtype: str = "f16") -> Workload:
    """Long-document pairwise rerank, forward only, all tokens valid."""
    rng = np.random.default_rng(seed)
    Q = _normalize_round(rng.standard_normal((B, Lq, dim), dtype=np.float32), dtype)
    D = _docs_per_seed(seed, B, Ld, dim, dtype, first_index=1)
    return Workload("long-rerank", "pairwise", dtype, Q, D, None, None, None)


def gaussian_grad(seed: int, shape) -> torch.Tensor:
    """A separate seeded N(0,1) float32 upstream grad."""
    return torch.from_numpy(
        np.random.default_rng(seed).standard_normal(shape, dtype=np.float32))
