"""GPU parity of the loss head (row cross-entropy over scores) against the
float64 oracle ``oracle.ce_rows``, through the C ABI.

Tolerance, from the float32 arithmetic of the kernel: the logits z = s*S are
rounded once (|dz| <= 2^-24 |z|), exp and log are within a few ulp, and a
row sum of C positive terms in float32 is within about C * 2^-24 relative
(far less in practice).  So the row log-sum-exp, and with it the row loss, is
within 4e-6 * (1 + max|z|) absolute; a softmax probability p within that
relative error, so a gradient entry (s/R)(p - [c == t]) within
(|s|/R) * (4e-6 * (1 + max|z|) * p + 1e-7).  The mean adds no error beyond
its terms (float64 sum).
"""

import numpy as np
import pytest
import torch

import oracle
from maxsim_scoring_02_amd import _lib
from maxsim_scoring_02_amd import workloads as wl
from parity import gpu_backward, gpu_forward, say, to_gpu

pytestmark = pytest.mark.gpu


def _check(S, labels=None, scale=1.0):
    S = np.asarray(S, dtype=np.float32)
    R, C = S.shape
    say(f"[loss] R={R} C={C} scale={scale} labels={'diag' if labels is None else 'given'}")
    lab = None if labels is None else torch.as_tensor(labels, dtype=torch.int32).cuda()
    loss, rows, grad = _lib.lik_ce_rows(torch.from_numpy(S).cuda(), lab, scale)
    torch.cuda.synchronize()
    loss, rows, grad = float(loss.cpu()[0]), rows.cpu().numpy(), grad.cpu().numpy()
    rl, rrows, rgrad = oracle.ce_rows(S.astype(np.float64), labels, scale)
    zmax = float(np.max(np.abs(scale * S.astype(np.float64)), axis=1).max())
    tol = 4e-6 * (1.0 + zmax)
    assert np.all(np.abs(rows - rrows) <= tol), np.max(np.abs(rows - rrows))
    assert abs(loss - rl) <= tol
    t = np.arange(R) if labels is None else np.asarray(labels)
    p = rgrad * R / scale
    p[np.arange(R), t] += 1.0
    gtol = abs(scale) / R * (tol * p + 1e-7)
    assert np.all(np.abs(grad - rgrad) <= gtol), np.max(np.abs(grad - rgrad) - gtol)
    return loss, rows, grad


def test_inbatch_loss_on_forward_scores():
    w = wl.inbatch_pages(B=24)
    s, _ = gpu_forward(w)
    _check(s)


def test_negative_doc_loss_on_kd_scores():
    w = wl.kd_candidates(B=6, N=5, Ld=300)
    s, _ = gpu_forward(w)
    _check(s, labels=np.zeros(6, dtype=np.int32))


@pytest.mark.parametrize("scale", [1.0, 0.05, 20.0, -3.0])
def test_random_scores_labels_and_scales(scale):
    rng = np.random.default_rng(80)
    S = (rng.standard_normal((37, 300)) * 8).astype(np.float32)
    _check(S, rng.integers(0, 300, size=37), scale)


@pytest.mark.parametrize("R,C", [(1, 1), (1, 65), (64, 64), (300, 1000), (5, 4097)])
def test_shapes(R, C):
    rng = np.random.default_rng(81 + R + C)
    S = (rng.standard_normal((R, C)) * 30).astype(np.float32)
    labels = None if C >= R and R % 2 == 0 else rng.integers(0, C, size=R)
    _check(S, labels)


def test_out_of_range_label_gives_nan_row_and_mean():
    S = torch.zeros((3, 4), dtype=torch.float32, device="cuda")
    loss, rows, grad = _lib.lik_ce_rows(S, torch.tensor([0, 7, 1], dtype=torch.int32), 1.0)
    rows = rows.cpu().numpy()
    assert np.isnan(rows[1]) and np.isfinite(rows[[0, 2]]).all()
    assert np.isnan(float(loss.cpu()[0]))
    g = grad.cpu().numpy()
    assert np.allclose(g[1], 0.25 / 3)              # softmax row without the -1 term


def test_loss_is_bitwise_reproducible():
    rng = np.random.default_rng(82)
    S = torch.from_numpy((rng.standard_normal((256, 256)) * 20).astype(np.float32)).cuda()
    a = _lib.lik_ce_rows(S)
    b = _lib.lik_ce_rows(S)
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_training_step_forward_loss_backward():
    """The in-batch pages step on the GPU (forward, loss head, backward)
    against the oracle chain (forward, ce_rows, backward) on the same inputs."""
    w = wl.inbatch_pages(B=20)
    Q, D, qm, dm = to_gpu(w)
    s, a = _lib.lik_maxsim_fwd(Q, D, qm, dm)
    loss, _, g = _lib.lik_ce_rows(s)
    gQ, gD = _lib.lik_maxsim_bwd(Q, D, g, a, qm, dm)
    torch.cuda.synchronize()
    Qn, Dn, qmn, dmn = w.numpy_inputs()
    ref = oracle.maxsim_allpairs(Qn, Dn, qmn, dmn)
    rl, _, rg = oracle.ce_rows(ref.scores)
    assert abs(float(loss.cpu()[0]) - rl) <= 1e-4
    merged = oracle.admissible_argmax(ref, a.cpu().numpy(), Qn, Dn, dmn, "allpairs")
    rQ, rD = oracle.maxsim_allpairs_bwd(Qn, Dn, rg, merged, qmn, dmn)
    for x, y in ((gQ.cpu().numpy(), rQ), (gD.cpu().numpy(), rD)):
        assert np.all(np.abs(x - y) <= 1e-3 * np.abs(y) + 1e-5 * np.abs(y).max())


def test_loss_without_gradient_output():
    rng = np.random.default_rng(83)
    S = torch.from_numpy((rng.standard_normal((70, 33)) * 5).astype(np.float32)).cuda()
    lab = torch.from_numpy(rng.integers(0, 33, size=70).astype(np.int32)).cuda()
    l1, r1, g1 = _lib.lik_ce_rows(S, lab, 2.5)
    l2, r2, g2 = _lib.lik_ce_rows(S, lab, 2.5, want_grad=False)
    assert g2 is None and g1 is not None
    assert torch.equal(l1, l2) and torch.equal(r1, r2)


def test_empty_documents_in_a_row():
    # scores of empty documents are -1e9: a row of them has loss log C
    S = torch.full((3, 5), -1e9, dtype=torch.float32, device="cuda")
    S[1, 2] = 4.0
    _check(S.cpu().numpy())
