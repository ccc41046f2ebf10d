"""GPU parity of LIK_F32_BF16X3: float32 inputs whose all-pairs scoring runs
on the bfloat16 matrix cores with every value split into a bfloat16 high
part and a bfloat16 low part (three products per element pair, float32
accumulation), against the float64 oracle.

Besides the operator's usual bar (scores within 1e-4, admissible argmax,
gradients), every small case checks each score against the error bound
stated in include/lik.h, computed here from the inputs alone: a
similarity's dropped terms are within 3 * 2^-16 * sum_k |q_k d_k| (with a
little slack for the parts' rounding), float32 accumulation of the 3 * dim
products within 3 * dim * 2^-24 of the same sum, and a score moves by at most
the sum over valid query tokens of the largest such bound over valid
document tokens (plus the float32 sum of Lq maxima).  Integer inputs split
exactly (lo = 0), so their scores and argmaxes are bit-exact; calls the
split does not serve (pairwise, kd, dim 256) must equal LIK_F32 bitwise.
"""

import numpy as np
import pytest
import torch

import oracle
from maxsim_scoring_02_amd import _lib
from maxsim_scoring_02_amd import workloads as wl
from maxsim_scoring_02_amd.workloads import Workload
from parity import (ORACLE_FWD, check_scores, full_check, gpu_backward, gpu_forward, say)

pytestmark = pytest.mark.gpu

X3 = _lib.LIK_F32_BF16X3


def _tokens(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _w(name, layout, Q, D, qm=None, dm=None, g=None):
    t = lambda x, dt: None if x is None else torch.as_tensor(x, dtype=dt).contiguous()
    return Workload(name, layout, "f32", t(Q, torch.float32), t(D, torch.float32),
                    t(qm, torch.bool), t(dm, torch.bool), t(g, torch.float32))


def _score_bound(Qn, Dn, qm, dm):
    """Per-score bound [Nq, Nd] of the split's error (all-pairs)."""
    Nq, Lq, dim = Qn.shape
    aq, ad = np.abs(Qn).astype(np.float64), np.abs(Dn).astype(np.float64)
    S = np.einsum("qik,djk->qdij", aq, ad)            # sum_k |q_k d_k|
    if dm is not None:
        S = np.where(dm[None, :, None, :], S, 0.0)
    c = 3.1 * 2.0 ** -16 + 3 * dim * 2.0 ** -24 + Lq * 2.0 ** -24
    per_tok = S.max(axis=3)                           # [Nq, Nd, Lq]
    if qm is not None:
        per_tok = np.where(qm[:, None, :], per_tok, 0.0)
    return c * per_tok.sum(axis=2)


def _check_bound(w):
    Qn, Dn, qm, dm = w.numpy_inputs()
    ref = ORACLE_FWD["allpairs"](Qn, Dn, qm, dm)
    s, _ = gpu_forward(w, fp32_split=True)
    bound = _score_bound(Qn, Dn, qm, dm)
    live = ref.scores != oracle.EMPTY_DOC_SCORE
    err = np.abs(s.astype(np.float64) - ref.scores)
    assert np.all(err[live] <= bound[live]), (
        f"{w.name}: score error {float(err[live].max()):.3e} above its bound")
    return float(err[live].max()) if live.any() else 0.0, float(bound[live].max())


CASES = [
    # name, Nq, Lq, Nd, Ld, query mask, document mask
    ("packed-masked", 9, 32, 7, 77, True, True),
    ("short-queries", 11, 7, 5, 70, False, True),
    ("flattened", 4, 100, 5, 90, False, False),
    ("split-docs", 3, 32, 4, 2049, False, True),
    ("single-row-docs", 5, 32, 6, 1, False, False),
]


@pytest.mark.parametrize("dim", [64, 128])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_split_against_the_oracle_and_its_error_bound(case, dim):
    name, Nq, Lq, Nd, Ld, qmask, dmask = case
    rng = np.random.default_rng(2000 + dim + Ld + Lq)
    Q = _tokens(rng, (Nq, Lq, dim))
    D = _tokens(rng, (Nd, Ld, dim))
    qm = (rng.random((Nq, Lq)) < 0.8) if qmask else None
    dm = None
    if dmask:
        dm = np.arange(Ld)[None] < rng.integers(1, Ld + 1, Nd)[:, None]
        dm[Nd // 2] = False                      # an empty document
    g = rng.standard_normal((Nq, Nd))
    w = _w(f"x3-{name}-d{dim}", "allpairs", Q, D, qm, dm, g)
    dims = (Nq, Lq, Nd, Ld, dim)
    flags = 1 | (2 if dmask else 0) | (4 if qmask else 0)
    assert _lib.lik_plan_value(_lib.LIK_OP_FWD, dims, X3, flags, "split") == 1
    out = full_check(w, fp32_split=True)
    err, bound = _check_bound(w)
    say(f"[split] {w.name}: {out} max err {err:.2e} (largest bound {bound:.2e})")
    # the backward that recomputes the argmax runs the split forward again
    a = gpu_forward(w, fp32_split=True)[1]
    q1, d1 = gpu_backward(w, g, a, fp32_split=True)
    q2, d2 = gpu_backward(w, g, None, fp32_split=True)
    assert np.array_equal(q1, q2) and np.array_equal(d1, d2)


def test_split_integer_inputs_are_bit_exact():
    """Entries in {-3..3} are their own high part (low part 0): every score
    is an exact integer and the argmax follows the lowest-index rule."""
    rng = np.random.default_rng(2100)
    for dim in (64, 128):
        Q = rng.integers(-3, 4, (7, 32, dim)).astype(np.float32)
        D = rng.integers(-3, 4, (9, 200, dim)).astype(np.float32)
        dm = rng.random((9, 200)) < 0.7
        w = _w(f"x3-int-d{dim}", "allpairs", Q, D, None, dm)
        ref = oracle.maxsim_allpairs(*w.numpy_inputs())
        s, a = gpu_forward(w, fp32_split=True)
        assert np.array_equal(s.astype(np.float64), ref.scores)
        assert np.array_equal(a, ref.argmax)


def test_split_scores_without_argmax_and_determinism():
    """The max-only variant gives the argmax variant's scores bitwise, and
    repeated calls give the same bits."""
    rng = np.random.default_rng(2200)
    Q = _tokens(rng, (9, 32, 128))
    D = _tokens(rng, (11, 300, 128))
    dm = np.arange(300)[None] < rng.integers(1, 301, 11)[:, None]
    w = _w("x3-noarg", "allpairs", Q, D, None, dm)
    s0, a0 = gpu_forward(w, keep_argmax=False, fp32_split=True)
    s1, a1 = gpu_forward(w, keep_argmax=True, fp32_split=True)
    s2, a2 = gpu_forward(w, keep_argmax=True, fp32_split=True)
    assert a0 is None
    assert np.array_equal(s0, s1) and np.array_equal(s1, s2) and np.array_equal(a1, a2)
    check_scores(s0, ORACLE_FWD["allpairs"](*w.numpy_inputs()))


def test_calls_the_split_does_not_serve_equal_exact_float32():
    """Pairwise, kd and dim 256 compute exactly as LIK_F32 (bitwise)."""
    rng = np.random.default_rng(2300)
    Q = _tokens(rng, (6, 32, 128))
    g6 = rng.standard_normal(6)
    cases = [
        _w("x3-pair", "pairwise", Q, _tokens(rng, (6, 300, 128)), g=g6),
        _w("x3-kd", "kd", Q, _tokens(rng, (6, 3, 200, 128)), g=rng.standard_normal((6, 3))),
        _w("x3-dim256", "allpairs", _tokens(rng, (6, 32, 256)), _tokens(rng, (5, 90, 256)),
           g=rng.standard_normal((6, 5))),
    ]
    for w in cases:
        s0, a0 = gpu_forward(w)
        s1, a1 = gpu_forward(w, fp32_split=True)
        assert np.array_equal(s0, s1) and np.array_equal(a0, a1), w.name
        q0, d0 = gpu_backward(w, w.grad.numpy(), None)
        q1, d1 = gpu_backward(w, w.grad.numpy(), None, fp32_split=True)
        assert np.array_equal(q0, q1) and np.array_equal(d0, d1), w.name


def test_inbatch_text_f32_split_full_size():
    """The in-batch text step with float32 inputs through the split (256
    queries x 256 documents, the benchmark's shapes), every element against
    the oracle."""
    w = wl.inbatch_text(dtype="f32")
    w.name = "inbatch-text-f32x3"
    dims = (256, 32, 256, 300, 128)
    assert _lib.lik_plan_value(_lib.LIK_OP_FWD, dims, X3, 3, "split") == 1
    assert _lib.lik_plan_value(_lib.LIK_OP_FWD, dims, X3, 3, "upw") > 1
    out = full_check(w, fp32_split=True)
    say(f"[fullsize] inbatch-text-f32x3: {out}")


def test_split_through_the_allocation_free_forward():
    """lik_maxsim_fwd_noalloc with LIK_F32_BF16X3 keeps the split copies in
    its fixed scratch: bitwise equal to the workspace forward, twice in a
    row with a smaller call between."""
    rng = np.random.default_rng(2400)
    dev = torch.device("cuda:0")
    cases = []
    for Nq, Nd, Ld in ((12, 40, 300), (5, 7, 70)):
        Q = torch.from_numpy(_tokens(rng, (Nq, 32, 128))).to(dev)
        D = torch.from_numpy(_tokens(rng, (Nd, Ld, 128))).to(dev)
        dm = torch.from_numpy(np.arange(Ld)[None] < rng.integers(1, Ld + 1, Nd)[:, None]).to(dev)
        cases.append((Q, D, dm))
    for Q, D, dm in (cases[0], cases[1], cases[0]):
        s0, a0 = _lib.lik_maxsim_fwd(Q, D, None, dm, fp32_split=True)
        s1, a1 = _lib.lik_maxsim_fwd_noalloc(Q, D, None, dm, fp32_split=True)
        torch.cuda.synchronize()
        assert torch.equal(s0, s1) and torch.equal(a0, a1)


def test_split_degenerate_shapes_equal_exact_float32():
    """Shapes where the split has nothing to multiply follow the same rules
    as LIK_F32, bitwise: queries with no tokens (Lq = 0), every document
    empty, fully masked queries, single documents and single queries."""
    rng = np.random.default_rng(2500)
    cases = [
        _w("x3-lq0", "allpairs", np.zeros((3, 0, 128), np.float32), _tokens(rng, (4, 50, 128))),
        _w("x3-all-empty", "allpairs", _tokens(rng, (3, 32, 128)), _tokens(rng, (4, 50, 128)),
           dm=np.zeros((4, 50), bool)),
        _w("x3-masked-queries", "allpairs", _tokens(rng, (3, 32, 64)), _tokens(rng, (4, 70, 64)),
           qm=np.array([[False] * 32, [True] * 32, [False] * 31 + [True]])),
        _w("x3-one-doc", "allpairs", _tokens(rng, (5, 33, 128)), _tokens(rng, (1, 97, 128))),
        _w("x3-one-query", "allpairs", _tokens(rng, (1, 7, 64)), _tokens(rng, (9, 31, 64))),
    ]
    for w in cases:
        s0, a0 = gpu_forward(w)
        s1, a1 = gpu_forward(w, fp32_split=True)
        ref = ORACLE_FWD["allpairs"](*w.numpy_inputs())
        check_scores(s1, ref)
        empty = ref.scores == oracle.EMPTY_DOC_SCORE
        assert np.array_equal(s0[empty], s1[empty]), w.name
        if w.Q.shape[1] == 0 or not (~empty).any():
            assert np.array_equal(s0, s1) and np.array_equal(a0, a1), w.name
