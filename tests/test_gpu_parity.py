"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Sizes are cut so the oracle finishes in seconds while every case still spans
several tiles and a ragged tail, and together the cases reach every kernel
mode: all-pairs with packed and flattened query slots, single-chunk and
split documents, pairwise/kd direct and split, fp16/bf16/fp32, dims 64/128/256,
masks of every kind and the degenerate shapes.
"""

import numpy as np
import pytest
import torch

import oracle
from maxsim_scoring_02_amd import workloads as wl
from maxsim_scoring_02_amd.workloads import Workload
from parity import (ORACLE_BWD, ORACLE_FWD, check_argmax, check_grads, check_scores, full_check,
                    gpu_backward, gpu_forward, say)

pytestmark = pytest.mark.gpu


def _custom(name, layout, dtype, Q, D, q_mask=None, d_mask=None, grad=None):
    t = lambda x, dt=None: None if x is None else torch.as_tensor(x, dtype=dt)
    torch_dt = wl.DTYPES[dtype]
    return Workload(name, layout, dtype, t(Q).to(torch_dt).contiguous(),
                    t(D).to(torch_dt).contiguous(), t(q_mask, torch.bool),
                    t(d_mask, torch.bool), t(grad, torch.float32))


def _rand_tokens(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


# ------------------------------------------------------------ the workloads

def test_tiny_quickstart_allpairs_and_pairwise():
    ap, pw = wl.tiny_allpairs()
    full_check(ap)
    full_check(pw)


def test_inbatch_text_reduced():
    w = wl.inbatch_text(B=40, Nd=37)
    full_check(w)


def test_inbatch_pages_reduced_with_ce_grad():
    w = wl.inbatch_pages(B=24)
    Qn, Dn, qm, dm = w.numpy_inputs()
    ref = oracle.maxsim_allpairs(Qn, Dn, qm, dm)
    g = oracle.ce_rows(ref.scores)[2].astype(np.float32)   # from the oracle's scores only
    full_check(w, grad=g)


def test_kd_candidates_reduced_split():
    w = wl.kd_candidates(B=6, N=5, Ld=1030)
    full_check(w)


def test_long_docs_reduced_split_chunks():
    w = wl.long_docs(Nq=5, Nd=6, Ld=8192)
    full_check(w, backward=False, keep_argmax=True)


def test_long_rerank_reduced_split():
    w = wl.long_rerank(B=3, Ld=32768)
    full_check(w, backward=False)


# ------------------------------------------------- long-context backward

def test_long_docs_backward_masked_tails():
    """All-pairs backward at Ld = 8192 with masked tails of every length."""
    w = wl.long_docs(Nq=5, Nd=6, Ld=8192)
    g = wl.gaussian_grad(7005, (5, 6)).numpy()
    full_check(w, grad=g)


def test_long_rerank_backward_reduced():
    """Pairwise backward at Ld = 32768 (streamed grad_D, no row tables)."""
    w = wl.long_rerank(B=3, Ld=32768)
    g = wl.gaussian_grad(7006, (3,)).numpy()
    full_check(w, grad=g)


def test_kd_backward_past_the_sort_limit():
    """kd backward with Ld = 20000, above the workspace sort's row limit."""
    rng = np.random.default_rng(7007)
    Q = _rand_tokens(rng, (2, 32, 128))
    D = _rand_tokens(rng, (2, 3, 20000, 128))
    dm = np.ones((2, 3, 20000), dtype=bool)
    dm[0, 1, 12345:] = False
    dm[1, 2, :19000] = False
    g = rng.standard_normal((2, 3))
    full_check(_custom("kd-ld20000", "kd", "f16", Q, D, None, dm, g))


def test_allpairs_backward_long_documents_workspace_sort_in_windows():
    """All-pairs backward with Ld = 30000: the document's row table does not
    fit in LDS, so grad_D is sorted through the workspace, in row windows of
    16000.  Query tokens are copied into rows on both sides of the window edge
    (15999, 16000) and near the end, so hits land in every window."""
    from maxsim_scoring_02_amd import _lib

    rng = np.random.default_rng(7009)
    Nq, Lq, Nd, Ld, dim = 2, 32, 3, 30000, 128
    assert _lib.lik_plan_value(_lib.LIK_OP_BWD, (Nq, Lq, Nd, Ld, dim), _lib.LIK_BF16, 1 | 2,
                               "gd_mode") == 0
    Q = _rand_tokens(rng, (Nq, Lq, dim))
    D = _rand_tokens(rng, (Nd, Ld, dim))
    for d in range(Nd):
        D[d, 15999] = Q[0, 3]
        D[d, 16000] = Q[1, 5]
        D[d, 29990] = Q[0, 7]
        D[d, 100] = Q[1, 9]
    dm = np.ones((Nd, Ld), dtype=bool)
    dm[1, 20000:] = False                             # a masked tail
    dm[2, :16001] = False                             # only the second window
    g = rng.standard_normal((Nq, Nd))
    full_check(_custom("ap-ld30000", "allpairs", "bf16", Q, D, None, dm, g))


def _sub_pairwise(w, idx):
    return Workload(f"{w.name}-sample", "pairwise", w.dtype, w.Q[idx].contiguous(),
                    w.D[idx].contiguous(), None, None, None)


def test_long_rerank_backward_full_size_sampled():
    """The full long-rerank shape (64 pairs x 32768 tokens) in the launch
    configuration of the full batch: sampled pairs against the oracle, the
    Euler identity over the whole batch, and the recomputed-argmax backward
    bitwise equal to the one given the forward's argmax."""
    w = wl.long_rerank()
    B = w.Q.shape[0]
    g = wl.gaussian_grad(7008, (B,)).numpy()
    s, a = gpu_forward(w)
    gQ, gD = gpu_backward(w, g, a)
    idx = [0, 17, B - 1]
    sub = _sub_pairwise(w, idx)
    Qn, Dn, _, _ = sub.numpy_inputs()
    ref = ORACLE_FWD["pairwise"](Qn, Dn, None, None)
    check_scores(s[idx], ref)
    merged = check_argmax(a[idx], ref, sub)
    rQ, rD = ORACLE_BWD["pairwise"](Qn, Dn, g[idx].astype(np.float64), merged, None, None)
    check_grads(gQ[idx], rQ, "grad_Q")
    check_grads(gD[idx], rD, "grad_D")
    # Euler identity (the score is 1-homogeneous in Q and in D)
    rhs = float(np.sum(g.astype(np.float64) * s))
    lq = float(np.sum(w.Q.double().numpy() * gQ))
    ld = float(torch.sum(w.D.double() * torch.from_numpy(gD).double()))
    assert abs(lq - rhs) <= 1e-4 * max(1.0, abs(rhs))
    assert abs(ld - rhs) <= 1e-4 * max(1.0, abs(rhs))
    gQ2, gD2 = gpu_backward(w, g, None)
    assert np.array_equal(gQ, gQ2) and np.array_equal(gD, gD2)


# ------------------------------------------------------------- shape sweep

@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("layout", ["allpairs", "pairwise", "kd"])
def test_dtypes_and_layouts(dtype, layout):
    seed = 1200 + 10 * ["f16", "bf16", "f32"].index(dtype) + ["allpairs", "pairwise", "kd"].index(layout)
    rng = np.random.default_rng(seed)
    B, N, Lq, Ld, dim = 5, 3, 32, 77, 128
    Q = _rand_tokens(rng, (B, Lq, dim))
    qm = rng.random((B, Lq)) < 0.85
    if layout == "allpairs":
        D = _rand_tokens(rng, (7, Ld, dim))
        dm = rng.random((7, Ld)) < 0.8
        g = rng.standard_normal((B, 7))
    elif layout == "pairwise":
        D = _rand_tokens(rng, (B, Ld, dim))
        dm = rng.random((B, Ld)) < 0.8
        g = rng.standard_normal(B)
    else:
        D = _rand_tokens(rng, (B, N, Ld, dim))
        dm = rng.random((B, N, Ld)) < 0.8
        g = rng.standard_normal((B, N))
    full_check(_custom(f"sweep-{layout}-{dtype}", layout, dtype, Q, D, qm, dm, g))


@pytest.mark.parametrize("Lq", [1, 7, 20, 32, 33, 64, 100])
def test_query_lengths(Lq):
    """Packed slots (Lq <= 64, several queries per wave, uneven segments) and
    flattened slots (Lq > 64, queries spanning waves)."""
    rng = np.random.default_rng(300 + Lq)
    Nq, Nd, Ld, dim = 9, 5, 70, 128
    Q = _rand_tokens(rng, (Nq, Lq, dim))
    D = _rand_tokens(rng, (Nd, Ld, dim))
    qm = rng.random((Nq, Lq)) < 0.9
    g = rng.standard_normal((Nq, Nd))
    full_check(_custom(f"lq{Lq}", "allpairs", "bf16", Q, D, qm, None, g))
    Dp = _rand_tokens(rng, (Nq, Ld, dim))
    full_check(_custom(f"lq{Lq}-pair", "pairwise", "bf16", Q, Dp, qm, None, g[:, 0]))


@pytest.mark.parametrize("dim", [64, 256])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_other_dims(dim, dtype):
    rng = np.random.default_rng(400 + dim)
    Q = _rand_tokens(rng, (6, 32, dim))
    D = _rand_tokens(rng, (5, 90, dim))
    dm = np.arange(90)[None] < rng.integers(1, 91, 5)[:, None]
    g = rng.standard_normal((6, 5))
    full_check(_custom(f"dim{dim}", "allpairs", dtype, Q, D, None, dm, g))
    Dk = _rand_tokens(rng, (6, 2, 90, dim))
    full_check(_custom(f"dim{dim}-kd", "kd", dtype, Q, Dk, None, None,
                       rng.standard_normal((6, 2))))


@pytest.mark.parametrize("Ld", [1, 31, 32, 33, 2049, 2111])
def test_doc_lengths_and_tails(Ld):
    """Single-token docs, tiles cut at every boundary, and Ld > 2048 so the
    all-pairs kernel splits documents into chunks."""
    rng = np.random.default_rng(500 + Ld)
    Q = _rand_tokens(rng, (3, 32, 128))
    D = _rand_tokens(rng, (4, Ld, 128))
    g = rng.standard_normal((3, 4))
    full_check(_custom(f"ld{Ld}", "allpairs", "f16", Q, D, None, None, g))
    full_check(_custom(f"ld{Ld}-pair", "pairwise", "f16", Q, D[:3], None, None, g[:, 0]))


@pytest.mark.parametrize("Lq,Ld", [(20, 2100), (100, 300)])
def test_partials_without_a_query_mask(Lq, Ld):
    """Per-token partials of uncompacted slots: three queries of 20 tokens
    per wave (4 slots unused) with documents cut into chunks, and queries of
    100 tokens spanning waves; only slots that hold a token write partials,
    and the combine reads each token's at its (q, i) position."""
    from maxsim_scoring_02_amd import _lib
    rng = np.random.default_rng(700 + Lq)
    Nq, Nd, dim = 5, 4, 128
    dims = (Nq, Lq, Nd, Ld, dim)
    pv = lambda key: _lib.lik_plan_value(_lib.LIK_OP_FWD, dims, _lib.LIK_BF16, 1 | 2, key)
    assert pv("partial") == 1 and pv("compact") == 0
    assert (pv("qpw"), pv("nchunks") > 1) == ((3, True) if Lq == 20 else (0, False))
    Q = _rand_tokens(rng, (Nq, Lq, dim))
    D = _rand_tokens(rng, (Nd, Ld, dim))
    dm = np.arange(Ld)[None] < rng.integers(1, Ld + 1, Nd)[:, None]
    g = rng.standard_normal((Nq, Nd))
    full_check(_custom(f"partials-lq{Lq}-ld{Ld}", "allpairs", "bf16", Q, D, None, dm, g))


def test_many_documents_grad_q_per_xcd_slice():
    """Nd >= 64: grad_Q is gathered per document slice (one slice per XCD)
    and the slice partials are added in order."""
    rng = np.random.default_rng(1300)
    Nq, Nd, Lq, Ld, dim = 10, 75, 32, 60, 128
    Q = _rand_tokens(rng, (Nq, Lq, dim))
    D = _rand_tokens(rng, (Nd, Ld, dim))
    qm = rng.random((Nq, Lq)) < 0.9
    dm = np.arange(Ld)[None] < rng.integers(1, Ld + 1, Nd)[:, None]
    dm[17] = False                                   # an empty document
    g = rng.standard_normal((Nq, Nd))
    full_check(_custom("many-docs", "allpairs", "bf16", Q, D, qm, dm, g))


def test_grad_q_alone_and_grad_d_alone_match_the_joint_call():
    """With both gradients the grad_D kernel also adds the grad_Q slice
    partials; asked for one gradient only, the partials go through their own
    kernel.  Both routes add the same partials in the same order: grad_Q and
    grad_D are bitwise equal either way (and the joint call is checked
    against the oracle)."""
    from maxsim_scoring_02_amd import _lib

    rng = np.random.default_rng(1301)
    Nq, Nd, Lq, Ld, dim = 12, 80, 32, 70, 128
    pv = lambda k: _lib.lik_plan_value(_lib.LIK_OP_BWD, (Nq, Lq, Nd, Ld, dim), _lib.LIK_BF16,
                                       1 | 2, k)
    assert pv("gq_ap") == 1 and pv("gq_slices") > 1 and pv("gd_mode") == 1
    Q = _rand_tokens(rng, (Nq, Lq, dim))
    D = _rand_tokens(rng, (Nd, Ld, dim))
    dm = np.arange(Ld)[None] < rng.integers(1, Ld + 1, Nd)[:, None]
    g = rng.standard_normal((Nq, Nd))
    w = _custom("grad-routes", "allpairs", "bf16", Q, D, None, dm, g)
    full_check(w)
    dev = torch.device("cuda:0")
    Qd, Dd, dmd = w.Q.to(dev), w.D.to(dev), w.d_mask.to(dev)
    gd = w.grad.to(dev)
    _, a = _lib.lik_maxsim_fwd(Qd, Dd, None, dmd)
    gQ, gD = _lib.lik_maxsim_bwd(Qd, Dd, gd, a, None, dmd)
    gQ1, none_d = _lib.lik_maxsim_bwd(Qd, Dd, gd, a, None, dmd, need_grad_d=False)
    none_q, gD1 = _lib.lik_maxsim_bwd(Qd, Dd, gd, a, None, dmd, need_grad_q=False)
    torch.cuda.synchronize()
    assert none_d is None and none_q is None
    assert torch.equal(gQ, gQ1) and torch.equal(gD, gD1)


def test_mask_bytes_of_any_nonzero_value_on_both_mask_paths():
    """Mask bytes of any nonzero value count as valid.  Mask rows of whole
    dwords at a 4-byte aligned address are turned into tile words four bytes
    per lane; the same mask at an odd address one byte per lane: scores and
    argmax must be bitwise equal, and both match the oracle."""
    from maxsim_scoring_02_amd import _lib

    rng = np.random.default_rng(1302)
    Nq, Lq, Nd, Ld, dim = 6, 32, 9, 100, 128
    Q = _rand_tokens(rng, (Nq, Lq, dim))
    D = _rand_tokens(rng, (Nd, Ld, dim))
    vals = np.array([1, 2, 0x7F, 0x80, 0xFF], dtype=np.uint8)
    u = np.where(rng.random((Nd, Ld)) < 0.7, rng.choice(vals, (Nd, Ld)), 0).astype(np.uint8)
    u[1, 32:64] = 0                                   # a masked middle tile
    u[2] = 0                                          # an empty document
    u[3] = 0
    u[3, Ld - 1] = 0x80                               # only the last row
    u[4, :] = 0xFF                                    # every row
    dev = torch.device("cuda:0")
    w = _custom("byte-mask", "allpairs", "bf16", Q, D, None, u != 0, None)
    Qd, Dd = w.Q.to(dev), w.D.to(dev)
    aligned = torch.from_numpy(u).to(dev).view(torch.bool)
    assert aligned.data_ptr() % 4 == 0 and Ld % 4 == 0
    buf = torch.zeros(Nd * Ld + 1, dtype=torch.uint8, device=dev)
    buf[1:] = torch.from_numpy(u.reshape(-1)).to(dev)
    odd = buf[1:].view(Nd, Ld).view(torch.bool)
    assert odd.data_ptr() % 4 != 0
    s1, a1 = _lib.lik_maxsim_fwd(Qd, Dd, None, aligned)
    s2, a2 = _lib.lik_maxsim_fwd(Qd, Dd, None, odd)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2) and torch.equal(a1, a2)
    Qn, Dn, _, dmn = w.numpy_inputs()
    ref = oracle.maxsim_allpairs(Qn, Dn, None, dmn)
    check_scores(s1.cpu().numpy(), ref)
    check_argmax(a1.cpu().numpy(), ref, w)
    assert float(s1[0, 2]) == -1e9


@pytest.mark.parametrize("layout", ["pairwise", "kd"])
def test_pairs_one_gradient_calls_match_the_joint_call(layout):
    """Pairwise / kd with both gradients run grad_Q and grad_D in one launch;
    asked for one gradient they run separately.  The same terms are added
    in the same order, so either way the results are bitwise equal."""
    from maxsim_scoring_02_amd import _lib

    rng = np.random.default_rng(1303 if layout == "kd" else 1304)
    B, N, Lq, Ld, dim = 6, 5, 32, 300, 128
    Q = _rand_tokens(rng, (B, Lq, dim))
    D = _rand_tokens(rng, (B, N, Ld, dim) if layout == "kd" else (B, Ld, dim))
    g = rng.standard_normal((B, N) if layout == "kd" else (B,))
    w = _custom(f"one-grad-{layout}", layout, "bf16", Q, D, None, None, g)
    full_check(w)
    dev = torch.device("cuda:0")
    Qd, Dd, gd = w.Q.to(dev), w.D.to(dev), w.grad.to(dev)
    fwd = _lib.lik_maxsim_kd_fwd if layout == "kd" else _lib.lik_maxsim_pairwise_fwd
    bwd = _lib.lik_maxsim_kd_bwd if layout == "kd" else _lib.lik_maxsim_pairwise_bwd
    _, a = fwd(Qd, Dd)
    gQ, gD = bwd(Qd, Dd, gd, a)
    gQ1, none_d = bwd(Qd, Dd, gd, a, need_grad_d=False)
    none_q, gD1 = bwd(Qd, Dd, gd, a, need_grad_q=False)
    torch.cuda.synchronize()
    assert none_d is None and none_q is None
    assert torch.equal(gQ, gQ1) and torch.equal(gD, gD1)


def test_workspace_sort_in_document_batches():
    """More than 65535 hits per document (2100 queries x 32 tokens) puts
    grad_D on the workspace sort, whose workspace holds a bounded batch of
    documents: 600 documents run as two batches.  The GPU runs the whole
    problem; sampled documents at the batch edges are compared with the
    oracle, with the upstream grad zeroed outside them (so grad_Q sums the
    sampled documents only) and every other document's grad_D exactly zero."""
    from maxsim_scoring_02_amd import _lib

    rng = np.random.default_rng(1600)
    Nq, Lq, Nd, Ld, dim = 2100, 32, 600, 64, 128
    pv = lambda k: _lib.lik_plan_value(_lib.LIK_OP_BWD, (Nq, Lq, Nd, Ld, dim), _lib.LIK_BF16, 1 | 2,
                                       k)
    nb = pv("sort_batch")
    assert pv("gd_mode") == 0 and 1 <= nb < Nd, (pv("gd_mode"), nb)
    say(f"[plan] workspace sort: {nb} documents per batch, "
        f"workspace {pv('workspace') / 2**20:.1f} MiB")
    Q = _rand_tokens(rng, (Nq, Lq, dim))
    D = _rand_tokens(rng, (Nd, Ld, dim))
    dm = np.arange(Ld)[None] < rng.integers(1, Ld + 1, Nd)[:, None]
    dm[5] = False                                    # an empty document
    docs = sorted({0, 5, nb - 1, nb, Nd - 1})
    g = rng.standard_normal((Nq, Nd)).astype(np.float32)
    keep = np.zeros(Nd, bool)
    keep[docs] = True
    g[:, ~keep] = 0.0
    w = _custom("sort-batches", "allpairs", "bf16", Q, D, None, dm, g)
    dev = torch.device("cuda:0")
    Qd, Dd, dmd = w.Q.to(dev), w.D.to(dev), w.d_mask.to(dev)
    s, a = _lib.lik_maxsim_fwd(Qd, Dd, None, dmd)
    gQ, gD = _lib.lik_maxsim_bwd(Qd, Dd, torch.from_numpy(g).to(dev), a, None, dmd)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(gD)) == int(torch.count_nonzero(gD[docs]))
    sub = Workload("sort-batches-docs", "allpairs", "bf16", w.Q, w.D[docs].contiguous(), None,
                   w.d_mask[docs].contiguous(), None)
    Qn, Dn, _, dmn = sub.numpy_inputs()
    ref = oracle.maxsim_allpairs(Qn, Dn, None, dmn)
    check_scores(s[:, docs].cpu().numpy(), ref)
    merged = check_argmax(a[:, docs].cpu().numpy(), ref, sub)
    rQ, rD = oracle.maxsim_allpairs_bwd(Qn, Dn, g[:, docs].astype(np.float64), merged, None, dmn)
    check_grads(gQ.cpu().numpy(), rQ, "grad_Q")
    check_grads(gD[docs].cpu().numpy(), rD, "grad_D")


def test_hub_rows_collect_most_hits():
    """A few document rows are the argmax of almost every query token, so a
    row's sorted hits span many lane groups and its gradient row is put
    together from their partials; duplicated hub tokens tie exactly and the
    lower index takes the hits.  Rows with no hit stay exactly zero."""
    rng = np.random.default_rng(1400)
    Nq, Nd, Lq, Ld, dim = 48, 3, 32, 90, 128
    Q = _rand_tokens(rng, (Nq, Lq, dim))
    Q[..., 0] = np.abs(Q[..., 0]) + 1.0
    Q /= np.linalg.norm(Q, axis=-1, keepdims=True)
    D = 0.3 * _rand_tokens(rng, (Nd, Ld, dim))
    hub = np.zeros(dim, np.float32)
    hub[0] = 1.0
    D[0, 7] = hub
    D[1, 3] = hub
    D[1, 50] = hub                                   # exact duplicate: ties go to row 3
    D[2, 80] = hub
    D[2, 81] = 0.5 * hub
    g = rng.standard_normal((Nq, Nd))
    w = _custom("hubs", "allpairs", "bf16", Q, D, None, None, g)
    full_check(w)
    s, a = gpu_forward(w)
    assert np.mean(a[:, 0] == 7) > 0.9 and np.all(a[:, 1] != 50)


def test_scores_without_argmax_output():
    """With no argmax buffer the forward keeps running maxima only (all-pairs)
    or drops the indices of split partials; the scores must be bitwise those
    of the argmax-keeping forward, in direct, split and masked modes."""
    rng = np.random.default_rng(1500)
    Q = _rand_tokens(rng, (9, 32, 128))
    D = _rand_tokens(rng, (11, 2200, 128))
    dm = np.arange(2200)[None] < rng.integers(1, 2201, 11)[:, None]
    dm[4] = False
    cases = [wl.inbatch_text(B=20, Nd=30),
             _custom("noarg-split", "allpairs", "f16", Q, D, None, dm),
             _custom("noarg-full", "allpairs", "bf16", Q, D[:, :300], None, None),
             _custom("noarg-pair", "pairwise", "bf16", Q, D[:9], None, dm[:9])]
    for w in cases:
        s0, a0 = gpu_forward(w, keep_argmax=False)
        s1, _ = gpu_forward(w, keep_argmax=True)
        assert a0 is None
        assert np.array_equal(s0, s1), w.name
        check_scores(s0, ORACLE_FWD[w.layout](*w.numpy_inputs()))


def test_arbitrary_masks_and_degenerate_rows():
    """Scattered (not suffix) masks, fully masked tiles inside a document, an
    empty document, an empty query, and a document whose valid similarities
    are all negative while its masked rows are zero (they must not win)."""
    rng = np.random.default_rng(600)
    Nq, Nd, Lq, Ld, dim = 6, 6, 32, 150, 128
    Q = _rand_tokens(rng, (Nq, Lq, dim))
    Q[0, :, 0] = np.abs(Q[0, :, 0]) + 0.5          # query 0: positive first coordinate
    Q[0] /= np.linalg.norm(Q[0], axis=-1, keepdims=True)
    D = _rand_tokens(rng, (Nd, Ld, dim))
    qm = rng.random((Nq, Lq)) < 0.5
    qm[0] = True
    qm[2] = False                                    # empty query
    dm = rng.random((Nd, Ld)) < 0.3
    dm[1] = False                                    # empty document
    dm[3, 32:96] = False                             # two whole masked tiles
    D[4] = 0.0                                       # doc 4: zero rows, masked ...
    D[4, 40:45, 0] = -1.0                            # ... except five -e0 tokens
    dm[4] = False
    dm[4, 40:45] = True
    g = rng.standard_normal((Nq, Nd))
    w = _custom("masks", "allpairs", "bf16", Q, D, qm, dm, g)
    full_check(w)
    s, a = gpu_forward(w)
    assert s[0, 4] < 0                               # masked zero rows never win
    assert np.all(a[0, 4] == 40)                     # equal similarities: lowest index
    Dk = D.reshape(3, 2, Ld, dim)
    dk = dm.reshape(3, 2, Ld)
    full_check(_custom("masks-kd", "kd", "bf16", Q[:3], Dk, qm[:3], dk,
                       rng.standard_normal((3, 2))))


def test_all_documents_empty_and_no_query_tokens():
    rng = np.random.default_rng(700)
    Q = _rand_tokens(rng, (3, 8, 64))
    D = _rand_tokens(rng, (4, 40, 64))
    dm = np.zeros((4, 40), bool)
    w = _custom("all-empty", "allpairs", "bf16", Q, D, None, dm, rng.standard_normal((3, 4)))
    s, a = gpu_forward(w)
    assert np.all(s == np.float32(-1e9)) and np.all(a == -1)
    gQ, gD = gpu_backward(w, w.grad.numpy(), a)
    assert np.all(gQ == 0) and np.all(gD == 0)
    qm = np.zeros((3, 8), bool)
    dm2 = np.ones((4, 40), bool)
    dm2[2] = False
    w2 = _custom("no-query-tokens", "allpairs", "bf16", Q, D, qm, dm2, rng.standard_normal((3, 4)))
    s2, a2 = gpu_forward(w2)
    expect = np.zeros((3, 4), np.float32)
    expect[:, 2] = -1e9
    assert np.array_equal(s2, expect) and np.all(a2 == -1)


def test_zero_sized_batches_are_noops():
    dev = torch.device("cuda:0")
    Q = torch.zeros((0, 32, 128), dtype=torch.bfloat16, device=dev)
    D = torch.zeros((3, 40, 128), dtype=torch.bfloat16, device=dev)
    s, a = _lib_fwd(Q, D)
    assert s.shape == (0, 3)


def _lib_fwd(Q, D):
    from maxsim_scoring_02_amd import _lib
    return _lib.lik_maxsim_fwd(Q, D)


# ------------------------------------------------- exactness and invariants

@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_integer_inputs_are_bit_exact(dtype):
    """Entries in {-3..3}: every dot and every score is an integer below
    2^24, so the GPU scores must equal the oracle's exactly and the argmax
    must follow the lowest-index rule through the many exact ties."""
    rng = np.random.default_rng(800)
    Nq, Nd, Lq, Ld, dim = 7, 9, 32, 200, 128
    Q = rng.integers(-3, 4, (Nq, Lq, dim)).astype(np.float32)
    D = rng.integers(-3, 4, (Nd, Ld, dim)).astype(np.float32)
    dm = rng.random((Nd, Ld)) < 0.7
    w = _custom(f"int-{dtype}", "allpairs", dtype, Q, D, None, dm,
                rng.integers(-2, 3, (Nq, Nd)).astype(np.float32))
    Qn, Dn, qm, dmn = w.numpy_inputs()
    ref = oracle.maxsim_allpairs(Qn, Dn, qm, dmn)
    s, a = gpu_forward(w)
    assert np.array_equal(s.astype(np.float64), ref.scores)
    assert np.array_equal(a, ref.argmax)
    gQ, gD = gpu_backward(w, w.grad.numpy(), a)
    rQ, rD = oracle.maxsim_allpairs_bwd(Qn, Dn, w.grad.numpy(), ref.argmax, qm, dmn)
    assert np.array_equal(gQ.astype(np.float64), rQ) and np.array_equal(gD.astype(np.float64), rD)
    Dk = D[:7].reshape(7, 1, Ld, dim)
    wk = _custom(f"int-kd-{dtype}", "kd", dtype, Q, Dk)
    rk = oracle.maxsim_kd(*wk.numpy_inputs())
    sk, ak = gpu_forward(wk)
    assert np.array_equal(sk.astype(np.float64), rk.scores) and np.array_equal(ak, rk.argmax)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_doc_holding_the_query_scores_exactly_Lq(dtype):
    rng = np.random.default_rng(900)
    Lq, Ld, dim = 32, 300, 128
    toks, seen = [], set()
    while len(toks) < Lq:
        idx = tuple(sorted(rng.choice(dim, 4, replace=False)))
        sg = tuple(rng.choice([-0.5, 0.5], 4))
        if (idx, sg) in seen:
            continue
        seen.add((idx, sg))
        t = np.zeros(dim, np.float32)
        t[list(idx)] = sg
        toks.append(t)
    q = np.stack(toks)
    doc = 0.5 * _rand_tokens(rng, (Ld, dim))
    pos = rng.choice(Ld, Lq, replace=False)
    doc[pos] = q
    w = _custom(f"unit-{dtype}", "allpairs", dtype, q[None], doc[None])
    s, a = gpu_forward(w)
    assert s[0, 0] == np.float32(Lq)
    assert list(a[0, 0]) == list(pos)


def test_determinism_bitwise():
    w = wl.inbatch_text(B=24, Nd=20)
    s1, a1 = gpu_forward(w)
    s2, a2 = gpu_forward(w)
    assert np.array_equal(s1, s2) and np.array_equal(a1, a2)
    g = w.grad.numpy()
    q1, d1 = gpu_backward(w, g, a1)
    q2, d2 = gpu_backward(w, g, a2)
    assert np.array_equal(q1, q2) and np.array_equal(d1, d2)
    # the backward that recomputes the argmax gives the same bits
    q3, d3 = gpu_backward(w, g, None)
    assert np.array_equal(q1, q3) and np.array_equal(d1, d3)


def test_pairwise_matches_allpairs_diagonal_and_kd_shared_docs():
    rng = np.random.default_rng(1000)
    B, Lq, Ld, dim = 6, 32, 250, 128
    Q = _rand_tokens(rng, (B, Lq, dim))
    D = _rand_tokens(rng, (B, Ld, dim))
    dm = rng.random((B, Ld)) < 0.9
    ap = _custom("diag-ap", "allpairs", "bf16", Q, D, None, dm)
    pw = _custom("diag-pw", "pairwise", "bf16", Q, D, None, dm)
    sa, aa = gpu_forward(ap)
    sp, ap_ = gpu_forward(pw)
    assert np.max(np.abs(np.diag(sa) - sp)) <= 2e-5
    kd = _custom("shared-kd", "kd", "bf16", Q, np.broadcast_to(D[None], (B,) + D.shape).copy(),
                 None, np.broadcast_to(dm[None], (B,) + dm.shape).copy())
    sk, ak = gpu_forward(kd)
    assert np.max(np.abs(sk - sa)) <= 2e-5


def test_power_of_two_scaling_is_bitwise():
    rng = np.random.default_rng(1100)
    Q = _rand_tokens(rng, (5, 32, 128))
    D = _rand_tokens(rng, (6, 130, 128))
    g = rng.standard_normal((5, 6)).astype(np.float32)
    w1 = _custom("pow2-a", "allpairs", "bf16", Q, D, grad=g)
    w2 = _custom("pow2-b", "allpairs", "bf16", 2 * Q, D, grad=g)
    s1, a1 = gpu_forward(w1)
    s2, a2 = gpu_forward(w2)
    assert np.array_equal(2 * s1, s2) and np.array_equal(a1, a2)
    q1, d1 = gpu_backward(w1, g, a1)
    q2, d2 = gpu_backward(w2, g, a2)
    assert np.array_equal(q1, q2) and np.array_equal(2 * d1, d2)


def test_euler_identity_on_gpu_outputs():
    w = wl.inbatch_text(B=32, Nd=32)
    s, a = gpu_forward(w)
    g = w.grad.numpy()
    gQ, gD = gpu_backward(w, g, a)
    Qn, Dn, _, _ = w.numpy_inputs()
    rhs = float(np.sum(g.astype(np.float64) * s))
    lq = float(np.sum(Qn.astype(np.float64) * gQ))
    ld = float(np.sum(Dn.astype(np.float64) * gD))
    assert abs(lq - rhs) <= 1e-4 * max(1.0, abs(rhs))
    assert abs(ld - rhs) <= 1e-4 * max(1.0, abs(rhs))


# ------------------------------------------------------------- op memory

def test_op_memory_is_linear_in_batch():
    """Peak device memory of forward + backward on in-batch text shapes at
    B = 32..256: exactly what the operator's outputs, argmax, gradients and
    workspaces take (the library allocates nothing itself), with no term of
    the [B, B, Lq, Ld] similarity grid the naive path holds."""
    from maxsim_scoring_02_amd import _lib

    rows = []
    for B in (32, 64, 128, 256):
        w = wl.inbatch_text(B=B, Nd=B)
        Q, D = w.Q.cuda(), w.D.cuda()
        dm = w.d_mask.cuda()
        g = w.grad.cuda()
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        s, a = _lib.lik_maxsim_fwd(Q, D, None, dm)
        gQ, gD = _lib.lik_maxsim_bwd(Q, D, g, a, None, dm)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        Lq, Ld, dim = 32, 300, 128
        L = _lib.lib()
        wsf = L.lik_workspace_bytes(_lib.LIK_OP_FWD, B, Lq, B, Ld, dim, _lib.LIK_BF16, 1 | 2)
        wsb = L.lik_workspace_bytes(_lib.LIK_OP_BWD, B, Lq, B, Ld, dim, _lib.LIK_BF16, 1 | 2)
        outs = B * B * 4 + B * B * Lq * 4 + B * Lq * dim * 4 + B * Ld * dim * 4
        rnd = lambda n: (n + 511) // 512 * 512            # the allocator's block size
        # outputs and workspaces, plus 1 MiB for the binding's small
        # argument copies (mask bytes, upstream grad)
        bound = rnd(B * B * 4) + rnd(B * B * Lq * 4) + rnd(B * Lq * dim * 4) + \
            rnd(B * Ld * dim * 4) + rnd(max(wsf, 256)) + rnd(max(wsb, 256)) + (1 << 20)
        grid = B * B * Lq * Ld * 4
        rows.append((B, peak, outs, grid))
        say(f"[memory] B={B}: peak {peak / 2**20:.1f} MiB, outputs {outs / 2**20:.1f} MiB, "
            f"workspaces {(wsf + wsb) / 2**20:.1f} MiB, naive grid {grid / 2**30:.2f} GiB")
        assert outs <= peak <= bound
        assert peak < grid / 4
        del s, a, gQ, gD
    for B, p, o, _ in rows:
        # beyond the outputs, memory is linear in B: per query at most two
        # grad_Q partial rows (Lq x dim x 4 bytes each) and the tile words
        assert p - o <= B * (2 * 32 * 128 * 4 + 2 * 4 * 10 + 64) + (1 << 20)
    for (B1, p1, o1, g1), (B2, p2, o2, g2) in zip(rows, rows[1:]):
        # the naive grid outgrows the operator's memory as B doubles
        assert g2 / p2 > 1.5 * (g1 / p1)
