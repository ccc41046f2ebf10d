"""Benchmark of the fused MaxSim operator on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch of synthetic input
that is already resident in HBM: the forward (scores + int32 argmax) and, for
training workloads, the backward (grad_Q and grad_D in float32).  W untimed
steps, then exactly K timed steps between two device synchronisations, with
one HIP event at each end of them and none in between; rank 0 prints one JSON
line.  Two untimed passes follow: K steps with events between forward and
backward (`config.fwd_ms`, `config.bwd_ms`) and K forwards with the
library's events attached to its main kernel's launch
(`roofline.kernel_ms`).

Default workload: ColBERT-text in-batch contrastive fwd+bwd -- 256 queries x
32 tokens against 256 documents padded to 300 tokens (true lengths uniform in
[64, 300], masked, zero padding), dim 128, bf16, Gaussian upstream grad.

Throughput counts algorithmic work on valid tokens only:
  forward   2 * dim * sum over (q, d) of Lq_valid(q) * Ld_valid(d)
  backward  4 * dim * (valid (q, i, d) triples with d non-empty)
(one gathered row-FMA for grad_Q and one scattered row-FMA for grad_D).

Memory-bound workloads count bytes of compulsory traffic over the step:
every valid input row read once, masks, scores and the kept argmax written,
and for the backward the upstream grad and argmax read and the float32
gradients written.

Other workloads (--workload): inbatch-pages, kd-candidates, long-docs,
long-rerank, or `all` (one line each); `next` runs the long-context backward
(long-docs-bwd, long-rerank-bwd: the long-document inputs with a Gaussian
upstream grad, forward + backward), kd-loss-head (the kd-candidates
inputs with the negative-doc cross-entropy as the loss head) and
inbatch-text-f32 (the in-batch text step with float32 inputs, computed
exactly on the fp32 MFMA and reported against its 157.3 TFLOP/s peak) and
inbatch-text-f32x3 (the same float32 inputs through LIK_F32_BF16X3: the
forward splits every value into bfloat16 high and low parts and takes three
bfloat16 MFMA products per element pair; `value` counts the float32 MaxSim
flops, the kernel roofline the three bfloat16 products per pair against the
2.5 PFLOP/s bfloat16 peak);
`loss-sweep` runs the loss head over batch x negatives, one line per point
kd-loss-head-b{64,128,256}-n{2,4,8,16}: kd forward with Lq 32 and Ld 1030 in
bf16, the negative-doc cross-entropy, and the backward, with the step's
device memory in `config.op_bytes`.

In-batch pages and kd-loss-head steps run the loss head on the GPU between
forward and backward (cross-entropy over the score rows, library entry
lik_ce_rows); its time is part of the step and of `config.bwd_ms`.

`cpu_baseline` is the CPU oracle timed on this machine's cores on a bounded
sample of the same workload (the sample is named in the JSON).

`roofline.frac` is the dominant kernel alone against its peak;
`roofline.step_frac` is the whole step (`value`) against the same peak.  The
default line also carries `secondary`: the metric's memory-bound half, the
long-document pairwise rerank (64 query-document pairs, 32 query tokens
against 32768 document tokens,
fp16, forward only) in GB/s and as a fraction of HBM peak, timed in the same
run with the same step counts (`--no-secondary` leaves it out).
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MaxSim fwd+bwd TFLOP/s (% MFMA peak); pairwise rerank GB/s (% HBM peak)"
PEAK_MFMA_16BIT = 2500.0        # TFLOP/s, MI355X dense bf16/fp16
PEAK_MFMA_F32 = 157.3           # TFLOP/s, MI355X dense fp32 (matrix)
PEAK_HBM = 8000.0               # GB/s, MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")


def _threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


# --------------------------------------------------------------------------
# algorithmic work
# --------------------------------------------------------------------------

def _valid_lengths(w):
    qv = (np.full(w.Q.shape[0], w.Q.shape[1]) if w.q_mask is None
          else w.q_mask.numpy().sum(axis=1))
    dshape = tuple(w.D.shape[:-1])
    dv = (np.full(dshape[:-1], dshape[-1]) if w.d_mask is None
          else w.d_mask.numpy().sum(axis=-1))
    return qv.astype(np.int64), dv.astype(np.int64)


def work(w, keep_argmax=True):
    """(forward flops, backward flops, forward bytes, backward bytes).  The
    forward writes the int32 argmax only when it is kept (training)."""
    dim = w.dim
    eb = w.Q.element_size()
    qv, dv = _valid_lengths(w)
    if w.layout == "allpairs":
        pairs_q = np.repeat(qv, len(dv))
        pairs_d = np.tile(dv, len(qv))
    elif w.layout == "pairwise":
        pairs_q, pairs_d = qv, dv
    else:
        B, N = dv.shape
        pairs_q = np.repeat(qv, N)
        pairs_d = dv.reshape(-1)
    f_fwd = float(2 * dim * np.sum(pairs_q * pairs_d))
    f_bwd = float(4 * dim * np.sum(pairs_q * (pairs_d > 0)))
    n_scores = pairs_q.size
    Lq = w.Q.shape[1]
    q_bytes = float(qv.sum() * dim * eb)
    d_bytes = float(dv.sum() * dim * eb)
    mask_bytes = (0 if w.q_mask is None else w.q_mask.numel()) + \
                 (0 if w.d_mask is None else w.d_mask.numel())
    b_fwd = q_bytes + d_bytes + mask_bytes + n_scores * 4 + (n_scores * Lq * 4 if keep_argmax else 0)
    # over a step every input row counts once (in the forward's bytes): the
    # backward adds the upstream grad and argmax it reads and the float32
    # gradients it writes
    d_rows = float(np.prod(w.D.shape[:-1]))
    b_bwd = (n_scores * 4 + n_scores * Lq * 4
             + w.Q.shape[0] * Lq * dim * 4 + d_rows * dim * 4)
    return f_fwd, f_bwd, b_fwd, b_bwd


# --------------------------------------------------------------------------
# GPU operator with preallocated buffers (direct C-ABI calls)
# --------------------------------------------------------------------------

class Op:
    def __init__(self, w, backward: bool):
        import torch
        from maxsim_scoring_02_amd import _lib

        self.torch = torch
        self.L = _lib.lib()
        self.w = w
        dev = torch.device("cuda:0")
        self.dev = dev
        self.Q = w.Q.to(dev).contiguous()
        self.D = w.D.to(dev).contiguous()
        self.qm = None if w.q_mask is None else w.q_mask.to(dev).contiguous().view(torch.uint8)
        self.dm = None if w.d_mask is None else w.d_mask.to(dev).contiguous().view(torch.uint8)
        self.dt = (_lib.LIK_F32_BF16X3 if w.meta.get("fp32_split")
                   else _lib.DTYPE_CODE[self.Q.dtype])
        self.backward = backward
        Lq, dim = w.Q.shape[1], w.dim
        shape = w.scores_shape
        self.scores = torch.empty(shape, dtype=torch.float32, device=dev)
        # scoring-only workloads (no backward) do not keep the argmax
        self.argmax = (torch.empty(tuple(shape) + (Lq,), dtype=torch.int32, device=dev)
                       if backward else None)
        lay = w.layout
        if lay == "allpairs":
            self.dims = (w.Q.shape[0], Lq, w.D.shape[0], w.D.shape[1], dim)
            ops = (_lib.LIK_OP_FWD, _lib.LIK_OP_BWD)
        elif lay == "pairwise":
            self.dims = (w.Q.shape[0], Lq, 1, w.D.shape[1], dim)
            ops = (_lib.LIK_OP_PAIRWISE_FWD, _lib.LIK_OP_PAIRWISE_BWD)
        else:
            self.dims = (w.Q.shape[0], Lq, w.D.shape[1], w.D.shape[2], dim)
            ops = (_lib.LIK_OP_KD_FWD, _lib.LIK_OP_KD_BWD)
        masks = (2 if self.dm is not None else 0) | (4 if self.qm is not None else 0)
        flags_f = (1 if self.argmax is not None else 0) | masks
        flags_b = 1 | masks
        self.wsf_n = self.L.lik_workspace_bytes(ops[0], *self.dims, self.dt, flags_f)
        self.wsb_n = self.L.lik_workspace_bytes(ops[1], *self.dims, self.dt, flags_b)
        mk = lambda n: torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
        self.wsf = mk(self.wsf_n)
        self.wsb = mk(self.wsb_n)
        # loss head (cross-entropy over the score rows) run by bwd() first:
        # "diag" targets the diagonal, "label0" candidate 0
        self.loss_head = w.meta.get("loss_head") if backward else None
        if self.loss_head:
            R, C = shape
            self.row_loss = torch.empty((R,), dtype=torch.float32, device=dev)
            self.loss = torch.empty((1,), dtype=torch.float32, device=dev)
            self.labels = (torch.zeros((R,), dtype=torch.int32, device=dev)
                           if self.loss_head == "label0" else None)
        if backward:
            g = w.grad if w.grad is not None else None
            self.g = (g.to(dev).contiguous() if g is not None
                      else torch.zeros(shape, dtype=torch.float32, device=dev))
            self.gQ = torch.empty(tuple(w.Q.shape), dtype=torch.float32, device=dev)
            self.gD = torch.empty(tuple(w.D.shape), dtype=torch.float32, device=dev)
        p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
        self.p = p
        self.lay = lay

    def stream(self):
        return ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream)

    def op_bytes(self) -> int:
        ts = [self.scores, self.argmax, self.wsf, self.wsb]
        if self.backward:
            ts += [self.gQ, self.gD, self.g]
        if self.loss_head:
            ts += [self.row_loss, self.loss, self.labels]
        return int(sum(t.numel() * t.element_size() for t in ts if t is not None))

    def fwd(self):
        p, L = self.p, self.L
        Nq, Lq, Nx, Ld, dim = self.dims
        if self.lay == "allpairs":
            st = L.lik_maxsim_fwd(p(self.Q), p(self.D), self.dt, Nq, Lq, Nx, Ld, dim, p(self.qm),
                                  p(self.dm), p(self.scores), p(self.argmax), p(self.wsf),
                                  self.wsf_n, self.stream())
        elif self.lay == "pairwise":
            st = L.lik_maxsim_pairwise_fwd(p(self.Q), p(self.D), self.dt, Nq, Lq, Ld, dim,
                                           p(self.qm), p(self.dm), p(self.scores), p(self.argmax),
                                           p(self.wsf), self.wsf_n, self.stream())
        else:
            st = L.lik_maxsim_kd_fwd(p(self.Q), p(self.D), self.dt, Nq, Lq, Nx, Ld, dim,
                                     p(self.qm), p(self.dm), p(self.scores), p(self.argmax),
                                     p(self.wsf), self.wsf_n, self.stream())
        if st != 0:
            raise RuntimeError(f"forward failed: {L.lik_last_error().decode()}")

    def bwd(self):
        p, L = self.p, self.L
        Nq, Lq, Nx, Ld, dim = self.dims
        if self.loss_head:
            R, C = self.scores.shape
            st = L.lik_ce_rows(p(self.scores), R, C, p(self.labels), 1.0, p(self.row_loss),
                               p(self.loss), p(self.g), self.stream())
            if st != 0:
                raise RuntimeError(f"loss head failed: {L.lik_last_error().decode()}")
        args = (p(self.qm), p(self.dm), p(self.g), p(self.argmax), p(self.gQ), p(self.gD),
                p(self.wsb), self.wsb_n, self.stream())
        if self.lay == "allpairs":
            st = L.lik_maxsim_bwd(p(self.Q), p(self.D), self.dt, Nq, Lq, Nx, Ld, dim, *args)
        elif self.lay == "pairwise":
            st = L.lik_maxsim_pairwise_bwd(p(self.Q), p(self.D), self.dt, Nq, Lq, Ld, dim, *args)
        else:
            st = L.lik_maxsim_kd_bwd(p(self.Q), p(self.D), self.dt, Nq, Lq, Nx, Ld, dim, *args)
        if st != 0:
            raise RuntimeError(f"backward failed: {L.lik_last_error().decode()}")


# --------------------------------------------------------------------------
# measured HBM traffic recorded from rocprofv3 counters
# --------------------------------------------------------------------------

# the sources the forward kernels (the ones whose traffic is recorded) and
# their launch plans are built from
FORWARD_SOURCES = ("lik_device.h", "lik_fwd.hip", "lik_kernels.h", "lik_plan.h")


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "maxsim_scoring_02_amd", "csrc")
    for f in FORWARD_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, kernel: str):
    """Bytes per launch of `kernel` from profiles/traffic_<kernel>_<workload>.md,
    or None when absent or taken from different kernel sources."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"bytes_per_launch:\s*([0-9.eE+]+)", text)
    d = re.search(r"kernel_sources_sha256_16:\s*([0-9a-f]+)", text)
    if not m or not d or d.group(1) != kernel_source_digest():
        return None
    return float(m.group(1))


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

def make_workload(name: str):
    from maxsim_scoring_02_amd import workloads as wl

    if name == "inbatch-text":
        return wl.inbatch_text(), True
    if name == "inbatch-pages":
        w = wl.inbatch_pages()
        # the upstream grad is the loss head's: cross-entropy over the
        # diagonal of the step's own scores, on the GPU inside every step
        w.meta["loss_head"] = "diag"
        return w, True
    if name == "inbatch-text-f32":
        # float32 inputs, computed exactly on the fp32 MFMA (no downcast)
        w = wl.inbatch_text(dtype="f32")
        w.name = name
        return w, True
    if name == "inbatch-text-f32x3":
        # the same float32 inputs scored through split bfloat16 parts
        w = wl.inbatch_text(dtype="f32")
        w.name = name
        w.meta["fp32_split"] = True
        return w, True
    if name == "kd-loss-head":
        # the pages' loss-head benchmark shape (B 256 x 16 candidates, Lq 32,
        # Ld 1030): kd forward, negative-doc cross-entropy with candidate 0
        # as the target, backward
        w = wl.kd_candidates()
        w.name = name
        w.grad = None
        w.meta["loss_head"] = "label0"
        return w, True
    m = re.fullmatch(r"kd-loss-head-b(\d+)-n(\d+)", name)
    if m:
        # one point of the loss-head sweep over batch x negatives (Lq 32,
        # Ld 1030, bf16): kd forward, negative-doc cross-entropy, backward
        B, N = int(m.group(1)), int(m.group(2))
        w = wl.kd_candidates(B=B, N=N)
        w.name = name
        w.grad = None
        w.meta["loss_head"] = "label0"
        return w, True
    if name == "kd-candidates":
        return wl.kd_candidates(), True
    if name == "long-docs":
        return wl.long_docs(), False
    if name == "long-rerank":
        return wl.long_rerank(), False
    # the long-context backward (the step after the long-document forward):
    # the same inputs with a Gaussian upstream grad, forward + backward
    if name == "long-docs-bwd":
        w = wl.long_docs()
        w.grad = wl.gaussian_grad(2005, (w.Q.shape[0], w.D.shape[0]))
        w.name = name
        return w, True
    if name == "long-rerank-bwd":
        w = wl.long_rerank()
        w.grad = wl.gaussian_grad(2006, (w.Q.shape[0],))
        w.name = name
        return w, True
    raise SystemExit(f"unknown workload {name}")


# workloads whose line also carries the metric's memory-bound half
SECONDARY = {"inbatch-text": "long-rerank"}

LOSS_SWEEP = [f"kd-loss-head-b{b}-n{n}" for b in (64, 128, 256) for n in (2, 4, 8, 16)]

DOMINANT = {  # kernel whose roofline is reported, and its bound
    "inbatch-text": ("allpairs_fwd", "mfma"),
    "inbatch-pages": ("allpairs_fwd", "mfma"),
    "long-docs": ("allpairs_fwd", "mfma"),
    "kd-candidates": ("pairs_fwd", "hbm"),
    "long-rerank": ("pairs_fwd", "hbm"),
    "long-docs-bwd": ("allpairs_fwd", "mfma"),
    "long-rerank-bwd": ("pairs_fwd", "hbm"),
    "kd-loss-head": ("pairs_fwd", "hbm"),
    "inbatch-text-f32": ("allpairs_fwd", "mfma"),
    "inbatch-text-f32x3": ("allpairs_fwd", "mfma"),
}


# --------------------------------------------------------------------------
# CPU oracle baseline on a bounded sample
# --------------------------------------------------------------------------

def cpu_baseline(w, backward: bool, budget_s: float = 12.0):
    import oracle
    from maxsim_scoring_02_amd.workloads import Workload

    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    cores = _threads()
    Qn, Dn, qm, dm = w.numpy_inputs()
    g = None if w.grad is None else w.grad.numpy()
    lay = w.layout
    # sample: the first n queries (all-pairs: against every document; pairs:
    # their own documents), growing n until the budget is used
    n_total = Qn.shape[0]
    n = 1
    spent, flops = 0.0, 0.0

    def run(k):
        sub_q = slice(0, k)
        Qs = Qn[sub_q]
        qms = None if qm is None else qm[sub_q]
        if lay == "allpairs":
            Ds, dms = Dn, dm
            gs = None if g is None else g[sub_q]
            fw, bw = oracle.maxsim_allpairs, oracle.maxsim_allpairs_bwd
        else:
            Ds = Dn[sub_q]
            dms = None if dm is None else dm[sub_q]
            gs = None if g is None else g[sub_q]
            fw = oracle.maxsim_pairwise if lay == "pairwise" else oracle.maxsim_kd
            bw = oracle.maxsim_pairwise_bwd if lay == "pairwise" else oracle.maxsim_kd_bwd
        t0 = time.perf_counter()
        r = fw(Qs, Ds, qms, dms)
        if backward:
            head = w.meta.get("loss_head")
            if head:
                labels = None if head == "diag" else np.zeros(k, dtype=np.int64)
                gs = oracle.ce_rows(r.scores, labels)[2]
            bw(Qs, Ds, gs, r.argmax, qms, dms)
        dt = time.perf_counter() - t0
        import torch
        sub = Workload(w.name, lay, w.dtype, torch.from_numpy(Qs), torch.from_numpy(Ds),
                       None if qms is None else torch.from_numpy(qms),
                       None if dms is None else torch.from_numpy(dms), None)
        f = work(sub)
        return dt, (f[0] + (f[1] if backward else 0.0)), (f[2] + (f[3] if backward else 0.0))

    ctx = threadpool_limits(cores) if threadpool_limits else None
    try:
        if ctx:
            ctx.__enter__()
        while True:
            dt, fl, by = run(n)
            if dt >= 0.6 * budget_s or n >= n_total:
                break
            n = min(n_total, max(n + 1, int(n * min(8.0, budget_s / max(dt, 1e-3)))))
        spent, flops, nbytes = dt, fl, by
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    what = ("fwd+bwd" if backward else "fwd")
    sample = (f"{what} of the first {n} of {n_total} queries"
              + (" against all documents" if lay == "allpairs" else " with their documents"))
    return spent, flops, nbytes, cores, sample


# --------------------------------------------------------------------------
# main
# --------------------------------------------------------------------------

class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime liblik.so is linked to, for
    lik_set_profile_events (which records them around the main kernel)."""

    def __init__(self, L, n):
        self.L = L
        L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                          ctypes.c_void_p]
        L.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            if L.hipEventCreate(ctypes.byref(a)) != 0 or L.hipEventCreate(ctypes.byref(b)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append((a, b))

    def elapsed_ms(self, k):
        ms = ctypes.c_float()
        a, b = self.ev[k]
        if self.L.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self):
        for a, b in self.ev:
            self.L.hipEventDestroy(a)
            self.L.hipEventDestroy(b)


def bench_one(name: str, steps: int, warmup: int, with_cpu: bool, dump_dir=None):
    import torch

    w, backward = make_workload(name)
    op = Op(w, backward)
    f_fwd, f_bwd, b_fwd, b_bwd = work(w, keep_argmax=backward)
    for _ in range(warmup):
        op.fwd()
        if backward:
            op.bwd()
    E = lambda: torch.cuda.Event(enable_timing=True)
    # Timed region: K whole steps with one event at each end and nothing
    # between them (every event between kernels adds a marker packet and
    # idles the GPU for a few microseconds).
    s0, s1 = E(), E()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    s0.record()
    for _ in range(steps):
        op.fwd()
        if backward:
            op.bwd()
    s1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = s0.elapsed_time(s1) / steps
    # Breakdown pass, outside the timed region: forward and backward apart.
    ev = [(E(), E(), E()) for _ in range(steps)]
    for e0, e1, e2 in ev:
        e0.record()
        op.fwd()
        e1.record()
        if backward:
            op.bwd()
        e2.record()
    torch.cuda.synchronize()
    fwd_ms = [a.elapsed_time(b) for a, b, _ in ev]
    bwd_ms = [b.elapsed_time(c) for _, b, c in ev]
    # Kernel pass: HIP events the library attaches to the main forward
    # kernel's launch (they carry the kernel's own start and end: the
    # roofline's duration).
    kev = HipEvents(op.L, steps)
    for k in range(steps):
        op.L.lik_set_profile_events(*kev.ev[k])
        op.fwd()
    op.L.lik_set_profile_events(None, None)
    torch.cuda.synchronize()
    kern_ms = [kev.elapsed_ms(k) for k in range(steps)]
    kev.close()
    t_fwd = float(np.mean(fwd_ms))
    t_bwd = float(np.mean(bwd_ms)) if backward else 0.0
    t_kern = float(np.mean(kern_ms))
    kern, bound = DOMINANT.get(name, ("pairs_fwd", "hbm") if name.startswith("kd-loss-head-b")
                               else (None, None))
    split = bool(w.meta.get("fp32_split"))
    if bound == "mfma":
        flops = f_fwd + (f_bwd if backward else 0.0)
        value = flops / (ms_step * 1e-3) / 1e12
        unit = "TFLOP/s"
        # the split forward's own work: three bfloat16 products per pair
        achieved = (3.0 if split else 1.0) * f_fwd / (t_kern * 1e-3) / 1e12
        peak = PEAK_MFMA_F32 if (w.dtype == "f32" and not split) else PEAK_MFMA_16BIT
        rl_unit = "TFLOP/s"
    else:
        nbytes = b_fwd + (b_bwd if backward else 0.0)
        value = nbytes / (ms_step * 1e-3) / 1e9
        unit = "GB/s"
        achieved = b_fwd / (t_kern * 1e-3) / 1e9
        peak = PEAK_HBM
        rl_unit = "GB/s"
    traffic = recorded_traffic(name, kern)
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32-bf16x3" if split else w.dtype,
        "data": "synthetic (seeded; shapes of the pages' workloads)",
        "config": {
            "workload": name,
            "layout": w.layout,
            "Q": list(w.Q.shape),
            "D": list(w.D.shape),
            "backward": backward,
            "fwd_ms": round(t_fwd, 5),
            "bwd_ms": round(t_bwd, 5),
            "fwd_flops_valid": f_fwd,
            "bwd_flops_valid": f_bwd,
            "fwd_bytes": b_fwd,
            "bwd_bytes": b_bwd,
            "wall_s_timed": round(wall, 4),
            # device memory the operator holds for one step: outputs, argmax,
            # float32 gradients, loss-head buffers and workspaces (the
            # library allocates nothing itself)
            "op_bytes": op.op_bytes(),
        },
        "roofline": {
            "bound": bound,
            "kernel": kern,
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": rl_unit,
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "kernel_ms": round(t_kern, 5),
            "timed_as": "main forward kernel alone, HIP events attached to its launch by the library",
            # the whole step (every kernel of forward and backward) against
            # the same peak: `value` / `peak`
            "step_frac": round(value / peak, 4),
        },
        "cpu_baseline": None,
    }
    if dump_dir:
        np.save(os.path.join(dump_dir, f"{name}_scores.npy"), op.scores.cpu().numpy())
    if with_cpu:
        spent, fl, nb, cores, sample = cpu_baseline(w, backward)
        if bound == "mfma":
            cv, cu = fl / spent / 1e12, "TFLOP/s"
        else:
            cv, cu = nb / spent / 1e9, "GB/s"
        line["cpu_baseline"] = {"value": round(cv, 6), "unit": cu, "cores": cores,
                                "kind": "oracle", "sample": sample,
                                "seconds": round(spent, 3)}
    return line


def copy_calibration(mib: int, reps: int):
    """Plain device-to-device copies of `mib` MiB: under rocprofv3 the copy
    kernel's FETCH_SIZE / WRITE_SIZE per dispatch, divided by the known byte
    count, is the scale factor applied to the MaxSim kernels' counters."""
    import torch

    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps first (the GPU clock needs tens of ms of load to settle)")
    ap.add_argument("--workload", default="inbatch-text")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="do not time the long-document rerank alongside the in-batch step")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of a workload, run plain device copies of MIB MiB "
                         "(reference kernel for scaling HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this operator build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration, max(args.steps, 1))
        return
    groups = {"all": ["inbatch-text", "inbatch-pages", "kd-candidates", "long-docs", "long-rerank"],
              "next": ["long-docs-bwd", "long-rerank-bwd", "kd-loss-head", "inbatch-text-f32",
                       "inbatch-text-f32x3"],
              "loss-sweep": LOSS_SWEEP}
    names = groups.get(args.workload, [args.workload])
    for i, name in enumerate(names):
        line = bench_one(name, args.steps, args.warmup,
                         with_cpu=(not args.no_cpu_baseline))
        if name in SECONDARY and not args.no_secondary:
            # the metric's second half, timed in the same run: the
            # memory-bound long-document rerank (pairwise, forward only)
            torch.cuda.empty_cache()
            sec = bench_one(SECONDARY[name], args.steps, args.warmup, with_cpu=False)
            line["secondary"] = {
                "metric": "pairwise rerank GB/s (% HBM peak)",
                "workload": sec["config"]["workload"],
                "value": sec["value"],
                "unit": sec["unit"],
                "frac": sec["roofline"]["step_frac"],
                "ms_per_step": sec["ms_per_step"],
                "dtype": sec["dtype"],
                "Q": sec["config"]["Q"],
                "D": sec["config"]["D"],
                "kernel": sec["roofline"]["kernel"],
                "kernel_ms": sec["roofline"]["kernel_ms"],
                "kernel_frac": sec["roofline"]["frac"],
            }
        print(json.dumps(line), flush=True)
        if i + 1 < len(names):
            torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
