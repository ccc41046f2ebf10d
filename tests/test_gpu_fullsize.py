"""GPU parity at the benchmark's full workload sizes, in the launch plans the
benchmark times.

Each test builds the workload exactly as `bench.py` does (same generator,
seed, dtype, masks and argmax flags), so the library picks the same launch
plan; the plan values are read back through lik_plan_value, printed and
asserted where they select a code path (several document units per
all-pairs workgroup, split documents, compacted query tokens, the grad_Q
slices and the grad_D kernel).  Where the oracle can take the whole batch in
seconds it does (in-batch text in bf16 and fp32, in-batch pages with the
loss head's gradient); for the larger shapes the GPU runs the whole batch
and a sample of documents is compared element by element, chosen to include
the shortest, the longest and lengths at the 1024-row piece boundaries, with
the upstream gradient zeroed outside the sample so that the oracle's grad_Q
needs only the sampled documents while the GPU still runs every document.
"""

import numpy as np
import pytest
import torch

import oracle
from maxsim_scoring_02_amd import _lib
from maxsim_scoring_02_amd import workloads as wl
from maxsim_scoring_02_amd.workloads import Workload
from parity import (ORACLE_BWD, ORACLE_FWD, check_argmax, check_grads, check_scores, full_check,
                    say)

pytestmark = pytest.mark.gpu

OPS = {"allpairs": (_lib.LIK_OP_FWD, _lib.LIK_OP_BWD),
       "pairwise": (_lib.LIK_OP_PAIRWISE_FWD, _lib.LIK_OP_PAIRWISE_BWD),
       "kd": (_lib.LIK_OP_KD_FWD, _lib.LIK_OP_KD_BWD)}
FWD_KEYS = ("nb", "upw", "n_groups", "n_sb", "nchunks", "tpc", "compact", "partial", "qpw",
            "n_units")
BWD_KEYS = ("gd_mode", "gd_parts", "gs_split", "gs_sw", "gs_lds", "gq_ap", "gq_slices",
            "recompute")


def plan(w, backward: bool, keep_argmax: bool = True) -> dict:
    """The plan values of the calls the benchmark makes for workload `w`."""
    Lq, dim = w.Q.shape[1], w.dim
    if w.layout == "allpairs":
        dims = (w.Q.shape[0], Lq, w.D.shape[0], w.D.shape[1], dim)
    elif w.layout == "pairwise":
        dims = (w.Q.shape[0], Lq, 1, w.D.shape[1], dim)
    else:
        dims = (w.Q.shape[0], Lq, w.D.shape[1], w.D.shape[2], dim)
    masks = (2 if w.d_mask is not None else 0) | (4 if w.q_mask is not None else 0)
    dt = _lib.DTYPE_CODE[w.Q.dtype]
    opf, opb = OPS[w.layout]
    out = {k: _lib.lik_plan_value(opf, dims, dt, (1 if keep_argmax else 0) | masks, k)
           for k in FWD_KEYS}
    if backward:
        out.update({"bwd_" + k: _lib.lik_plan_value(opb, dims, dt, 1 | masks, k)
                    for k in BWD_KEYS})
    say(f"[plan] {w.name}: {out}")
    return out


def _dev(t):
    return None if t is None else t.to("cuda:0").contiguous()


def _sub_allpairs_docs(w, docs, Q=None):
    """The all-pairs workload restricted to documents `docs` (CPU copies)."""
    return Workload(f"{w.name}-docs", "allpairs", w.dtype, (w.Q if Q is None else Q),
                    w.D[docs].contiguous(),
                    None if w.q_mask is None else w.q_mask,
                    None if w.d_mask is None else w.d_mask[docs].contiguous(), None)


def _sample_long_docs(d_len, piece=1024, extra=(0, 1, 2)):
    """Documents at the extremes of the length range and at piece boundaries
    (length = k * piece, k * piece + 1, k * piece - 1), plus a few fixed ones."""
    idx = {int(np.argmin(d_len)), int(np.argmax(d_len))}
    for r in (0, 1, piece - 1):
        hit = np.flatnonzero(d_len % piece == r)
        if hit.size:
            idx.add(int(hit[0]))
    idx.update(extra)
    return sorted(idx)


# ------------------------------------------------------------ in-batch text

def test_inbatch_text_full_size_bench_plan():
    """256 queries x 256 documents (lengths U{64..300}), bf16, forward with
    argmax then backward, every element against the oracle."""
    w = wl.inbatch_text()
    p = plan(w, backward=True)
    assert p["upw"] > 1 and p["partial"] == 0 and p["nchunks"] == 1 and p["nb"] == 2
    out = full_check(w)
    say(f"[fullsize] inbatch-text: {out}")


def test_inbatch_text_f32_full_size_bench_plan():
    """The in-batch text step with float32 inputs (the exact fp32 path)."""
    w = wl.inbatch_text(dtype="f32")
    w.name = "inbatch-text-f32"
    p = plan(w, backward=True)
    assert p["upw"] > 1 and p["nb"] == 1
    out = full_check(w)
    say(f"[fullsize] inbatch-text-f32: {out}")


# ------------------------------------------------------------ in-batch pages

def test_inbatch_pages_full_size_with_loss_head():
    """128 queries (lengths U{8..32}, masked tails) x 128 documents of 1030
    tokens, bf16: the GPU forward, the GPU loss head (cross-entropy over the
    diagonal) and the GPU backward fed with the loss head's gradient, as in
    the benchmark's step.  The oracle's backward takes the same float32
    gradient; the loss head's own output is checked against the oracle's
    cross-entropy of the GPU scores."""
    w = wl.inbatch_pages()
    p = plan(w, backward=True)
    assert p["compact"] == 1 and p["partial"] == 1
    Q, D, qm = _dev(w.Q), _dev(w.D), _dev(w.q_mask)
    s, a = _lib.lik_maxsim_fwd(Q, D, qm, None)
    loss, _, g = _lib.lik_ce_rows(s)
    gQ, gD = _lib.lik_maxsim_bwd(Q, D, g, a, qm, None)
    torch.cuda.synchronize()
    s_h, a_h, g_h = s.cpu().numpy(), a.cpu().numpy(), g.cpu().numpy()
    Qn, Dn, qmn, _ = w.numpy_inputs()
    ref = oracle.maxsim_allpairs(Qn, Dn, qmn, None)
    err = check_scores(s_h, ref)
    merged = check_argmax(a_h, ref, w)
    rl, _, rg = oracle.ce_rows(s_h.astype(np.float64))
    assert abs(float(loss.cpu()[0]) - rl) <= 4e-6 * (1 + np.abs(s_h).max())
    assert np.max(np.abs(g_h - rg)) <= 1e-6
    rQ, rD = oracle.maxsim_allpairs_bwd(Qn, Dn, g_h.astype(np.float64), merged, qmn, None)
    gq = check_grads(gQ.cpu().numpy(), rQ, "grad_Q")
    gd = check_grads(gD.cpu().numpy(), rD, "grad_D")
    say(f"[fullsize] inbatch-pages: score err {err:.2e}, grad_Q rel {gq:.2e}, grad_D rel {gd:.2e}")


# ------------------------------------------------------------ kd candidates

def test_kd_candidates_full_size_sampled():
    """256 queries x 16 candidates x 1030 tokens, bf16: the GPU runs the whole
    batch (forward with argmax, backward); queries at both ends and inside
    the batch are compared with all 16 of their candidates."""
    w = wl.kd_candidates()
    p = plan(w, backward=True)
    assert p["nchunks"] >= 2 and p["partial"] == 1 and p["bwd_gd_mode"] == 2
    Q, D = _dev(w.Q), _dev(w.D)
    g = w.grad.to("cuda:0")
    s, a = _lib.lik_maxsim_kd_fwd(Q, D)
    gQ, gD = _lib.lik_maxsim_kd_bwd(Q, D, g, a)
    torch.cuda.synchronize()
    idx = [0, 1, 77, 128, 255]
    sub = Workload("kd-sample", "kd", w.dtype, w.Q[idx].contiguous(), w.D[idx].contiguous(),
                   None, None, None)
    Qn, Dn, _, _ = sub.numpy_inputs()
    ref = oracle.maxsim_kd(Qn, Dn)
    err = check_scores(s[idx].cpu().numpy(), ref)
    merged = check_argmax(a[idx].cpu().numpy(), ref, sub)
    gs = w.grad.numpy()[idx].astype(np.float64)
    rQ, rD = oracle.maxsim_kd_bwd(Qn, Dn, gs, merged)
    check_grads(gQ[idx].cpu().numpy(), rQ, "grad_Q")
    check_grads(gD[idx].cpu().numpy(), rD, "grad_D")
    say(f"[fullsize] kd-candidates: sampled {idx}, score err {err:.2e}")


# ------------------------------------------------------------ long documents

def test_long_docs_forward_full_size_sampled():
    """16 queries x 1000 documents of up to 8192 tokens (lengths
    U{4096..8192}, masked tails), fp16, scores only (no argmax), as the
    benchmark scores them; sampled documents against the oracle."""
    w = wl.long_docs()
    p = plan(w, backward=False, keep_argmax=False)
    assert p["nchunks"] == 8 and p["upw"] > 1 and p["partial"] == 1
    Q, D, dm = _dev(w.Q), _dev(w.D), _dev(w.d_mask)
    s, a = _lib.lik_maxsim_fwd(Q, D, None, dm, keep_argmax=False)
    torch.cuda.synchronize()
    assert a is None
    docs = _sample_long_docs(w.meta["d_len"])
    sub = _sub_allpairs_docs(w, docs)
    ref = oracle.maxsim_allpairs(*sub.numpy_inputs())
    err = check_scores(s[:, docs].cpu().numpy(), ref)
    assert torch.isfinite(s).all() and (s > -1e9).all()
    say(f"[fullsize] long-docs: sampled docs {docs} (lengths "
        f"{[int(x) for x in w.meta['d_len'][docs]]}), score err {err:.2e}")


def test_long_docs_backward_full_size_sampled():
    """The long-context backward at the long-document shape: the forward keeps
    the argmax, the backward runs over all 1000 documents (4.2 GB of float32
    grad_D).  The upstream gradient is the benchmark's, zeroed outside the
    sampled documents: grad_Q then sums the sampled documents only (compared
    with the oracle), the sampled documents' grad_D is compared element by
    element, and every other document's grad_D must be exactly zero."""
    w = wl.long_docs()
    p = plan(w, backward=True)
    say(f"[plan] long-docs-bwd grad_Q slices {p['bwd_gq_slices']}, grad_D mode "
        f"{p['bwd_gd_mode']}, sorted split {p['bwd_gs_split']}")
    docs = _sample_long_docs(w.meta["d_len"])
    g = wl.gaussian_grad(2005, (w.Q.shape[0], w.D.shape[0])).numpy()
    keep = np.zeros(w.D.shape[0], bool)
    keep[docs] = True
    g[:, ~keep] = 0.0
    Q, D, dm = _dev(w.Q), _dev(w.D), _dev(w.d_mask)
    gd = torch.from_numpy(g).to("cuda:0")
    s, a = _lib.lik_maxsim_fwd(Q, D, None, dm)
    gQ, gD = _lib.lik_maxsim_bwd(Q, D, gd, a, None, dm)
    torch.cuda.synchronize()
    # every non-zero of grad_D lies in the sampled documents
    assert int(torch.count_nonzero(gD)) == int(torch.count_nonzero(gD[docs]))
    sub = _sub_allpairs_docs(w, docs)
    Qn, Dn, _, dmn = sub.numpy_inputs()
    ref = oracle.maxsim_allpairs(Qn, Dn, None, dmn)
    err = check_scores(s[:, docs].cpu().numpy(), ref)
    merged = check_argmax(a[:, docs].cpu().numpy(), ref, sub)
    rQ, rD = oracle.maxsim_allpairs_bwd(Qn, Dn, g[:, docs].astype(np.float64), merged, None, dmn)
    gq = check_grads(gQ.cpu().numpy(), rQ, "grad_Q")
    gdr = check_grads(gD[docs].cpu().numpy(), rD, "grad_D")
    say(f"[fullsize] long-docs-bwd: sampled docs {docs}, score err {err:.2e}, "
        f"grad_Q rel {gq:.2e}, grad_D rel {gdr:.2e}")
