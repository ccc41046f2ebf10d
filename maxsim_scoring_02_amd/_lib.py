"""ctypes binding of liblik.so: argument marshalling only.

Every function here has the name of the C entry point it calls.  Tensors are
torch tensors on the GPU (PyTorch supplies device memory and the current
stream); outputs and the workspace are allocated with torch and handed to the
library as plain pointers.  All computation happens in the library's HIP
kernels.  There is no fallback: if liblik.so is missing or the call fails, an
exception is raised.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liblik.so")
HEADER_PATH = os.path.join(os.path.dirname(PKG), "include", "lik.h")

LIK_OK, LIK_ERR_INVALID_ARG, LIK_ERR_UNSUPPORTED, LIK_ERR_HIP = 0, 1, 2, 3
LIK_F16, LIK_BF16, LIK_F32, LIK_F32_BF16X3 = 0, 1, 2, 3
(LIK_OP_FWD, LIK_OP_BWD, LIK_OP_PAIRWISE_FWD, LIK_OP_PAIRWISE_BWD,
 LIK_OP_KD_FWD, LIK_OP_KD_BWD) = range(6)

DTYPE_CODE = {torch.float16: LIK_F16, torch.bfloat16: LIK_BF16, torch.float32: LIK_F32}

_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_I = ctypes.c_int

_FWD_ALLPAIRS = [_P, _P, _I, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P, _SZ, _P]
_BWD_ALLPAIRS = [_P, _P, _I, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
_FWD_PAIRWISE = [_P, _P, _I, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P, _SZ, _P]
_BWD_PAIRWISE = [_P, _P, _I, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]

SIGNATURES = {
    "lik_abi_version": ([], _I),
    "lik_status_string": ([_I], ctypes.c_char_p),
    "lik_last_error": ([], ctypes.c_char_p),
    "lik_supported_dim": ([_I64], _I),
    "lik_set_profile_events": ([_P, _P], _I),
    "lik_workspace_bytes": ([_I, _I64, _I64, _I64, _I64, _I64, _I, _I], _SZ),
    "lik_plan_value": ([_I, _I64, _I64, _I64, _I64, _I64, _I, _I, ctypes.c_char_p], _I64),
    "lik_maxsim_fwd": (_FWD_ALLPAIRS, _I),
    "lik_maxsim_fwd_noalloc": ([_P, _P, _I, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P], _I),
    "lik_maxsim_bwd": (_BWD_ALLPAIRS, _I),
    "lik_maxsim_pairwise_fwd": (_FWD_PAIRWISE, _I),
    "lik_maxsim_pairwise_bwd": (_BWD_PAIRWISE, _I),
    "lik_maxsim_kd_fwd": (_FWD_ALLPAIRS, _I),
    "lik_maxsim_kd_bwd": (_BWD_ALLPAIRS, _I),
    "lik_ce_rows": ([_P, _I64, _I64, _P, ctypes.c_float, _P, _P, _P, _P], _I),
}


class LikError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"liblik status {status}: {detail}")
        self.status = status


def header_functions() -> list:
    """Names of the functions declared in include/lik.h."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"^[a-z0-9_ ]+?\**\s*\b(lik_[a-z_]+)\s*\(", text, re.M)))


def lib() -> ctypes.CDLL:
    """Load liblik.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m maxsim_scoring_02_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.argtypes = args
            fn.restype = res
        _lib = l
    return _lib


def _check(status: int):
    if status != LIK_OK:
        raise LikError(status, lib().lik_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _embeddings(Q: torch.Tensor, D: torch.Tensor, fp32_split: bool = False) -> int:
    """dtype code of the inputs; fp32_split asks for LIK_F32_BF16X3 (float32
    inputs scored through bfloat16 high/low parts, see include/lik.h)."""
    if not (Q.is_cuda and D.is_cuda):
        raise ValueError("Q and D must be GPU tensors")
    if Q.device != D.device:
        raise ValueError("Q and D must be on the same device")
    if Q.dtype != D.dtype or Q.dtype not in DTYPE_CODE:
        raise ValueError("Q and D must share a dtype among float16, bfloat16, float32")
    if Q.shape[-1] != D.shape[-1]:
        raise ValueError("Q and D must share the embedding dim")
    if not (Q.is_contiguous() and D.is_contiguous()):
        raise ValueError("Q and D must be contiguous")
    if fp32_split:
        if Q.dtype != torch.float32:
            raise ValueError("fp32_split applies to float32 inputs only")
        return LIK_F32_BF16X3
    return DTYPE_CODE[Q.dtype]


def _same_batch(Q: torch.Tensor, D: torch.Tensor, layout: str) -> None:
    """Pairwise and kd pair query b with document (row) b of D.  The C ABI
    receives B only, so a D with fewer rows would be read past its end on the
    device: the shapes are checked here, before anything is launched."""
    want = 3 if layout == "pairwise" else 4
    if Q.dim() != 3 or D.dim() != want:
        raise ValueError(f"{layout}: Q must be [B, Lq, dim] and D "
                         f"{'[B, Ld, dim]' if want == 3 else '[B, N, Ld, dim]'}")
    if D.shape[0] != Q.shape[0]:
        raise ValueError(f"{layout} Q and D must share the batch size "
                         f"(Q has {Q.shape[0]}, D has {D.shape[0]})")


def _flags(argmax_given: bool, dm, qm) -> int:
    """lik_workspace_bytes flags: bit 0 argmax, bit 1 document mask, bit 2 query mask."""
    return (1 if argmax_given else 0) | (2 if dm is not None else 0) | (4 if qm is not None else 0)


def _mask(m: Optional[torch.Tensor], shape, device) -> Optional[torch.Tensor]:
    if m is None:
        return None
    if tuple(m.shape) != tuple(shape):
        raise ValueError(f"mask shape {tuple(m.shape)} != {tuple(shape)}")
    if m.device != device or m.dtype != torch.bool or not m.is_contiguous():
        raise ValueError("masks must be contiguous bool tensors on the embeddings' device")
    return m.view(torch.uint8)


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------

def lik_plan_value(op: int, dims, dtype: int, flags: int, key: str) -> int:
    """One value of the launch plan for a call (see include/lik.h); dims =
    (nq_or_b, lq, nd_or_n, ld, dim) as for lik_workspace_bytes."""
    return int(lib().lik_plan_value(op, *dims, dtype, flags, key.encode()))


def lik_maxsim_fwd(Q, D, q_mask=None, d_mask=None, keep_argmax=True, fp32_split=False):
    """All-pairs: Q [Nq, Lq, dim] x D [Nd, Ld, dim] -> scores [Nq, Nd] float32,
    argmax [Nq, Nd, Lq] int32 (or None)."""
    dt = _embeddings(Q, D, fp32_split)
    Nq, Lq, dim = Q.shape
    Nd, Ld, _ = D.shape
    qm = _mask(q_mask, (Nq, Lq), Q.device)
    dm = _mask(d_mask, (Nd, Ld), Q.device)
    scores = torch.empty((Nq, Nd), dtype=torch.float32, device=Q.device)
    am = (torch.empty((Nq, Nd, Lq), dtype=torch.int32, device=Q.device)
          if keep_argmax else None)
    flags = _flags(keep_argmax, dm, qm)
    wsb = lib().lik_workspace_bytes(LIK_OP_FWD, Nq, Lq, Nd, Ld, dim, dt, flags)
    ws = _workspace(wsb, Q.device)
    _check(lib().lik_maxsim_fwd(_ptr(Q), _ptr(D), dt, Nq, Lq, Nd, Ld, dim, _ptr(qm), _ptr(dm),
                                _ptr(scores), _ptr(am), _ptr(ws), wsb, _stream()))
    return scores, am


def lik_maxsim_fwd_noalloc(Q, D, q_mask=None, d_mask=None, keep_argmax=True, fp32_split=False):
    """All-pairs forward through the allocation-free entry point: the library
    takes its scratch from a fixed per-device array (the outputs are still
    the caller's, allocated here)."""
    dt = _embeddings(Q, D, fp32_split)
    Nq, Lq, dim = Q.shape
    Nd, Ld, _ = D.shape
    qm = _mask(q_mask, (Nq, Lq), Q.device)
    dm = _mask(d_mask, (Nd, Ld), Q.device)
    scores = torch.empty((Nq, Nd), dtype=torch.float32, device=Q.device)
    am = (torch.empty((Nq, Nd, Lq), dtype=torch.int32, device=Q.device)
          if keep_argmax else None)
    _check(lib().lik_maxsim_fwd_noalloc(_ptr(Q), _ptr(D), dt, Nq, Lq, Nd, Ld, dim, _ptr(qm),
                                        _ptr(dm), _ptr(scores), _ptr(am), _stream()))
    return scores, am


def lik_maxsim_pairwise_fwd(Q, D, q_mask=None, d_mask=None, keep_argmax=True, fp32_split=False):
    """Pairwise: Q [B, Lq, dim] x D [B, Ld, dim] -> scores [B], argmax [B, Lq]."""
    _same_batch(Q, D, "pairwise")
    dt = _embeddings(Q, D, fp32_split)
    B, Lq, dim = Q.shape
    _, Ld, _ = D.shape
    qm = _mask(q_mask, (B, Lq), Q.device)
    dm = _mask(d_mask, (B, Ld), Q.device)
    scores = torch.empty((B,), dtype=torch.float32, device=Q.device)
    am = torch.empty((B, Lq), dtype=torch.int32, device=Q.device) if keep_argmax else None
    flags = _flags(keep_argmax, dm, qm)
    wsb = lib().lik_workspace_bytes(LIK_OP_PAIRWISE_FWD, B, Lq, 1, Ld, dim, dt, flags)
    ws = _workspace(wsb, Q.device)
    _check(lib().lik_maxsim_pairwise_fwd(_ptr(Q), _ptr(D), dt, B, Lq, Ld, dim, _ptr(qm),
                                         _ptr(dm), _ptr(scores), _ptr(am), _ptr(ws), wsb,
                                         _stream()))
    return scores, am


def lik_maxsim_kd_fwd(Q, D, q_mask=None, d_mask=None, keep_argmax=True, fp32_split=False):
    """kd: Q [B, Lq, dim] x D [B, N, Ld, dim] -> scores [B, N], argmax [B, N, Lq]."""
    _same_batch(Q, D, "kd")
    dt = _embeddings(Q, D, fp32_split)
    B, Lq, dim = Q.shape
    _, N, Ld, _ = D.shape
    qm = _mask(q_mask, (B, Lq), Q.device)
    dm = _mask(d_mask, (B, N, Ld), Q.device)
    scores = torch.empty((B, N), dtype=torch.float32, device=Q.device)
    am = torch.empty((B, N, Lq), dtype=torch.int32, device=Q.device) if keep_argmax else None
    flags = _flags(keep_argmax, dm, qm)
    wsb = lib().lik_workspace_bytes(LIK_OP_KD_FWD, B, Lq, N, Ld, dim, dt, flags)
    ws = _workspace(wsb, Q.device)
    _check(lib().lik_maxsim_kd_fwd(_ptr(Q), _ptr(D), dt, B, Lq, N, Ld, dim, _ptr(qm), _ptr(dm),
                                   _ptr(scores), _ptr(am), _ptr(ws), wsb, _stream()))
    return scores, am


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

def _grad_scores(g: torch.Tensor, shape, device) -> torch.Tensor:
    if tuple(g.shape) != tuple(shape) or g.dtype != torch.float32 or g.device != device:
        raise ValueError(f"grad_scores must be float32 {tuple(shape)} on the embeddings' device")
    return g.contiguous()


def _argmax_in(am: Optional[torch.Tensor], shape, device) -> Optional[torch.Tensor]:
    if am is None:
        return None
    if tuple(am.shape) != tuple(shape) or am.dtype != torch.int32 or am.device != device:
        raise ValueError(f"argmax must be int32 {tuple(shape)} from the forward")
    return am.contiguous()


def lik_maxsim_bwd(Q, D, grad_scores, argmax=None, q_mask=None, d_mask=None,
                   need_grad_q=True, need_grad_d=True, fp32_split=False) -> Tuple:
    dt = _embeddings(Q, D, fp32_split)
    Nq, Lq, dim = Q.shape
    Nd, Ld, _ = D.shape
    qm = _mask(q_mask, (Nq, Lq), Q.device)
    dm = _mask(d_mask, (Nd, Ld), Q.device)
    g = _grad_scores(grad_scores, (Nq, Nd), Q.device)
    am = _argmax_in(argmax, (Nq, Nd, Lq), Q.device)
    gQ = torch.empty((Nq, Lq, dim), dtype=torch.float32, device=Q.device) if need_grad_q else None
    gD = torch.empty((Nd, Ld, dim), dtype=torch.float32, device=Q.device) if need_grad_d else None
    flags = _flags(am is not None, dm, qm)
    wsb = lib().lik_workspace_bytes(LIK_OP_BWD, Nq, Lq, Nd, Ld, dim, dt, flags)
    ws = _workspace(wsb, Q.device)
    _check(lib().lik_maxsim_bwd(_ptr(Q), _ptr(D), dt, Nq, Lq, Nd, Ld, dim, _ptr(qm), _ptr(dm),
                                _ptr(g), _ptr(am), _ptr(gQ), _ptr(gD), _ptr(ws), wsb, _stream()))
    return gQ, gD


def lik_maxsim_pairwise_bwd(Q, D, grad_scores, argmax=None, q_mask=None, d_mask=None,
                            need_grad_q=True, need_grad_d=True, fp32_split=False) -> Tuple:
    _same_batch(Q, D, "pairwise")
    dt = _embeddings(Q, D, fp32_split)
    B, Lq, dim = Q.shape
    _, Ld, _ = D.shape
    qm = _mask(q_mask, (B, Lq), Q.device)
    dm = _mask(d_mask, (B, Ld), Q.device)
    g = _grad_scores(grad_scores, (B,), Q.device)
    am = _argmax_in(argmax, (B, Lq), Q.device)
    gQ = torch.empty((B, Lq, dim), dtype=torch.float32, device=Q.device) if need_grad_q else None
    gD = torch.empty((B, Ld, dim), dtype=torch.float32, device=Q.device) if need_grad_d else None
    flags = _flags(am is not None, dm, qm)
    wsb = lib().lik_workspace_bytes(LIK_OP_PAIRWISE_BWD, B, Lq, 1, Ld, dim, dt, flags)
    ws = _workspace(wsb, Q.device)
    _check(lib().lik_maxsim_pairwise_bwd(_ptr(Q), _ptr(D), dt, B, Lq, Ld, dim, _ptr(qm),
                                         _ptr(dm), _ptr(g), _ptr(am), _ptr(gQ), _ptr(gD),
                                         _ptr(ws), wsb, _stream()))
    return gQ, gD


def lik_maxsim_kd_bwd(Q, D, grad_scores, argmax=None, q_mask=None, d_mask=None,
                      need_grad_q=True, need_grad_d=True, fp32_split=False) -> Tuple:
    _same_batch(Q, D, "kd")
    dt = _embeddings(Q, D, fp32_split)
    B, Lq, dim = Q.shape
    _, N, Ld, _ = D.shape
    qm = _mask(q_mask, (B, Lq), Q.device)
    dm = _mask(d_mask, (B, N, Ld), Q.device)
    g = _grad_scores(grad_scores, (B, N), Q.device)
    am = _argmax_in(argmax, (B, N, Lq), Q.device)
    gQ = torch.empty((B, Lq, dim), dtype=torch.float32, device=Q.device) if need_grad_q else None
    gD = torch.empty((B, N, Ld, dim), dtype=torch.float32, device=Q.device) if need_grad_d else None
    flags = _flags(am is not None, dm, qm)
    wsb = lib().lik_workspace_bytes(LIK_OP_KD_BWD, B, Lq, N, Ld, dim, dt, flags)
    ws = _workspace(wsb, Q.device)
    _check(lib().lik_maxsim_kd_bwd(_ptr(Q), _ptr(D), dt, B, Lq, N, Ld, dim, _ptr(qm), _ptr(dm),
                                   _ptr(g), _ptr(am), _ptr(gQ), _ptr(gD), _ptr(ws), wsb,
                                   _stream()))
    return gQ, gD


def lik_ce_rows(scores, labels=None, scale=1.0, want_grad=True) -> Tuple:
    """Loss head: row cross-entropy of float32 scores [R, C] with targets
    `labels` [R] (int32) or the diagonal (None).  Returns (loss [1],
    row_loss [R], grad [R, C] or None), all float32 on the scores' device."""
    if scores.dtype != torch.float32 or scores.dim() != 2 or not scores.is_cuda:
        raise ValueError("scores must be a 2-D float32 CUDA tensor")
    S = scores.contiguous()
    R, C = S.shape
    lab = None
    if labels is not None:
        lab = labels.to(device=S.device, dtype=torch.int32).contiguous()
        if tuple(lab.shape) != (R,):
            raise ValueError(f"labels must have shape ({R},)")
    row_loss = torch.empty((R,), dtype=torch.float32, device=S.device)
    loss = torch.empty((1,), dtype=torch.float32, device=S.device)
    grad = torch.empty((R, C), dtype=torch.float32, device=S.device) if want_grad else None
    _check(lib().lik_ce_rows(_ptr(S), R, C, _ptr(lab), float(scale), _ptr(row_loss), _ptr(loss),
                             _ptr(grad), _stream()))
    return loss, row_loss, grad


FORWARD = {"allpairs": lik_maxsim_fwd, "pairwise": lik_maxsim_pairwise_fwd,
           "kd": lik_maxsim_kd_fwd}
BACKWARD = {"allpairs": lik_maxsim_bwd, "pairwise": lik_maxsim_pairwise_bwd,
            "kd": lik_maxsim_kd_bwd}
