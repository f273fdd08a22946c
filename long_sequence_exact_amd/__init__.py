"""seqattn for MI355X: segmented exact softmax attention in HIP for gfx950.

Python face of libseqattn.so (C ABI in include/seqattn.h).  Functions take
torch tensors on the GPU, [B,H,N,d] or [H,N,d] with d contiguous, and run on
torch's current stream.  All computation happens in the library's kernels.

    attn_segment_fwd(q, k, v, causal_offset=None, ...) -> (o, lse)
    lse_merge(o_acc, lse_acc, o_b, lse_b)               (in place)
    dilated_attn_fwd(q, k, v, segment_lengths, dilations, causal=False) -> (o, lse)
    attn_segment_bwd(q, k, v, o, lse, d_o, causal_offset=None, ...) -> (dq, dk, dv)
    dilated_attn_bwd(q, k, v, o, lse, d_o, segment_lengths, dilations, ...) -> (dq, dk, dv)
    head_relayout(src, dst)                             (dst[f][n] = src[f][n])
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import ACCUMULATE, CAUSAL, HEAD_SHIFT, NONCAUSAL, SeqattnError

__all__ = ["attn_segment_fwd", "lse_merge", "dilated_attn_fwd", "attn_segment_bwd",
           "attn_segment_bwd_noalloc", "dilated_attn_bwd", "head_relayout", "workspace_size",
           "NONCAUSAL", "SeqattnError", "version"]


def version() -> int:
    return int(_lib.lib().seqattn_version())


def _lse_shape(q):
    return q.shape[:-1]


def attn_segment_fwd(q, k, v, causal_offset=None, scale=None, out=None, lse=None,
                     accumulate=False, out_dtype=None, workspace=None, split=True):
    """Partial attention of q against one KV segment.

    causal_offset: None (non-causal) or delta = q_start - k_start; key j is
    visible to query i iff j <= i + delta.  With accumulate=True, ``out``
    (fp32) and ``lse`` hold a running partial that receives the merge.
    A call too short to fill the GPU splits its key range over more
    workgroups (seqattn_attn_segment_fwd_ws); its workspace is allocated
    here unless given.  split=False runs seqattn_attn_segment_fwd instead.
    """
    L = _lib.lib()
    if out is None:
        if accumulate:
            raise ValueError("accumulate=True needs out= and lse=")
        dt = out_dtype or (torch.float32 if q.dtype == torch.float32 else q.dtype)
        out = torch.empty(q.shape, dtype=dt, device=q.device)
    if lse is None:
        lse = torch.empty(_lse_shape(q), dtype=torch.float32, device=q.device)
    delta = NONCAUSAL if causal_offset is None else int(causal_offset)
    dq, dk, dv = _lib.desc(q), _lib.desc(k), _lib.desc(v)
    do_, dl = _lib.desc(out), _lib.desc(lse, lse=True)
    if not split:
        _lib.check(L.seqattn_attn_segment_fwd(
            ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), delta,
            float(scale or 0.0), ACCUMULATE if accumulate else 0,
            ctypes.byref(do_), ctypes.byref(dl), ctypes.c_void_p(_lib.stream_handle())))
        return out, lse
    need = 0 if accumulate else int(L.seqattn_workspace_size(
        _lib.OP_SEGMENT_FWD, ctypes.byref(dq), ctypes.byref(dk), 0))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None and not workspace.is_cuda:
        raise ValueError("workspace must be on the GPU")
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _lib.check(L.seqattn_attn_segment_fwd_ws(
        ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), delta,
        float(scale or 0.0), ACCUMULATE if accumulate else 0,
        ctypes.byref(do_), ctypes.byref(dl), ctypes.c_void_p(wptr), wbytes,
        ctypes.c_void_p(_lib.stream_handle())))
    return out, lse


def lse_merge(o_acc, lse_acc, o_b, lse_b):
    """In place: (o_acc, lse_acc) <- LSE merge of itself with (o_b, lse_b)."""
    L = _lib.lib()
    a, la = _lib.desc(o_acc), _lib.desc(lse_acc, lse=True)
    b, lb = _lib.desc(o_b), _lib.desc(lse_b, lse=True)
    _lib.check(L.seqattn_lse_merge(ctypes.byref(a), ctypes.byref(la), ctypes.byref(b),
                                   ctypes.byref(lb), ctypes.c_void_p(_lib.stream_handle())))
    return o_acc, lse_acc


def workspace_size(op: int, q, other) -> int:
    L = _lib.lib()
    a = _lib.desc(q, on_device=False)
    b = _lib.desc(other, on_device=False)
    return int(L.seqattn_workspace_size(op, ctypes.byref(a), ctypes.byref(b), 0))


def _dilated_flags(causal, head_shift):
    return (CAUSAL if causal else 0) | (HEAD_SHIFT if head_shift else 0)


def dilated_attn_fwd(q, k, v, segment_lengths, dilations, causal=False, scale=None,
                     out=None, lse=None, out_dtype=torch.float32, workspace=None,
                     head_shift=False):
    """LongNet dilated attention: branch partials merged by log-sum-exp.

    head_shift=True: query head h selects offset h mod r_i inside each
    segment (offset 0 for every head otherwise).
    """
    L = _lib.lib()
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty(_lse_shape(q), dtype=torch.float32, device=q.device)
    n = len(segment_lengths)
    if len(dilations) != n:
        raise ValueError("segment_lengths and dilations differ in length")
    w = (ctypes.c_int64 * n)(*[int(x) for x in segment_lengths])
    r = (ctypes.c_int64 * n)(*[int(x) for x in dilations])
    dqd, dkd, dvd = _lib.desc(q), _lib.desc(k), _lib.desc(v)
    dod, dld = _lib.desc(out), _lib.desc(lse, lse=True)
    need = int(L.seqattn_workspace_size(_lib.OP_DILATED_FWD, ctypes.byref(dqd),
                                        ctypes.byref(dod), n))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None and not workspace.is_cuda:
        raise ValueError("workspace must be on the GPU")
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _lib.check(L.seqattn_dilated_attn_fwd(
        ctypes.byref(dqd), ctypes.byref(dkd), ctypes.byref(dvd), w, r, n,
        float(scale or 0.0), _dilated_flags(causal, head_shift), ctypes.byref(dod),
        ctypes.byref(dld),
        ctypes.c_void_p(wptr), wbytes, ctypes.c_void_p(_lib.stream_handle())))
    return out, lse


def attn_segment_bwd(q, k, v, o, lse, d_o, causal_offset=None, scale=None, dq=None,
                     dk=None, dv=None, grad_dtype=torch.float32, workspace=None,
                     accumulate_kv=False):
    """Gradients of one (query block, KV segment) pair from the global O/LSE.

    dq (fp32) is accumulated into (zeros if not given); dk, dv are written,
    or, with accumulate_kv=True, accumulated (fp32).
    """
    L = _lib.lib()
    if dq is None:
        dq = torch.zeros(q.shape, dtype=torch.float32, device=q.device)
    if dk is None:
        dk = torch.empty(k.shape, dtype=grad_dtype, device=k.device)
    if dv is None:
        dv = torch.empty(v.shape, dtype=grad_dtype, device=v.device)
    delta = NONCAUSAL if causal_offset is None else int(causal_offset)
    ds = [_lib.desc(t) for t in (q, k, v, o)]
    dl = _lib.desc(lse, lse=True)
    ddo = _lib.desc(d_o)
    gq, gk, gv = _lib.desc(dq), _lib.desc(dk), _lib.desc(dv)
    need = int(L.seqattn_workspace_size(_lib.OP_SEGMENT_BWD, ctypes.byref(ds[0]),
                                        ctypes.byref(ds[1]), 0))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None and not workspace.is_cuda:
        raise ValueError("workspace must be on the GPU")
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _lib.check(L.seqattn_attn_segment_bwd(
        *[ctypes.byref(x) for x in ds], ctypes.byref(dl), ctypes.byref(ddo), delta,
        float(scale or 0.0), ACCUMULATE if accumulate_kv else 0, ctypes.byref(gq),
        ctypes.byref(gk), ctypes.byref(gv), ctypes.c_void_p(wptr), wbytes,
        ctypes.c_void_p(_lib.stream_handle())))
    return dq, dk, dv


def attn_segment_bwd_noalloc(q, k, v, o, lse, d_o, dq, dk, dv, causal_offset=None,
                             scale=None, accumulate_kv=False):
    """attn_segment_bwd through the entry point that allocates nothing: the
    caller passes every output (dq accumulated, dk/dv written or, with
    accumulate_kv, accumulated) and no workspace is used.  Calls on one GPU
    share the library's fixed scratch, so they must not overlap."""
    L = _lib.lib()
    delta = NONCAUSAL if causal_offset is None else int(causal_offset)
    ds = [_lib.desc(t) for t in (q, k, v, o)]
    dl = _lib.desc(lse, lse=True)
    ddo = _lib.desc(d_o)
    gq, gk, gv = _lib.desc(dq), _lib.desc(dk), _lib.desc(dv)
    _lib.check(L.seqattn_attn_segment_bwd_noalloc(
        *[ctypes.byref(x) for x in ds], ctypes.byref(dl), ctypes.byref(ddo), delta,
        float(scale or 0.0), ACCUMULATE if accumulate_kv else 0, ctypes.byref(gq),
        ctypes.byref(gk), ctypes.byref(gv), ctypes.c_void_p(_lib.stream_handle())))
    return dq, dk, dv


def dilated_attn_bwd(q, k, v, o, lse, d_o, segment_lengths, dilations, causal=False,
                     scale=None, dq=None, dk=None, dv=None, workspace=None,
                     head_shift=False):
    """Gradients of dilated_attn_fwd from its merged (o, lse).

    dq (fp32) is accumulated into (zeros if not given); dk, dv (fp32) are written.
    """
    L = _lib.lib()
    if dq is None:
        dq = torch.zeros(q.shape, dtype=torch.float32, device=q.device)
    if dk is None:
        dk = torch.empty(k.shape, dtype=torch.float32, device=k.device)
    if dv is None:
        dv = torch.empty(v.shape, dtype=torch.float32, device=v.device)
    n = len(segment_lengths)
    if len(dilations) != n:
        raise ValueError("segment_lengths and dilations differ in length")
    w = (ctypes.c_int64 * n)(*[int(x) for x in segment_lengths])
    r = (ctypes.c_int64 * n)(*[int(x) for x in dilations])
    ds = [_lib.desc(t) for t in (q, k, v, o)]
    dl = _lib.desc(lse, lse=True)
    ddo = _lib.desc(d_o)
    gq, gk, gv = _lib.desc(dq), _lib.desc(dk), _lib.desc(dv)
    need = int(L.seqattn_workspace_size(_lib.OP_DILATED_BWD, ctypes.byref(ds[0]),
                                        ctypes.byref(ds[1]), n))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None and not workspace.is_cuda:
        raise ValueError("workspace must be on the GPU")
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _lib.check(L.seqattn_dilated_attn_bwd(
        *[ctypes.byref(x) for x in ds], ctypes.byref(dl), ctypes.byref(ddo), w, r, n,
        float(scale or 0.0), _dilated_flags(causal, head_shift), ctypes.byref(gq),
        ctypes.byref(gk),
        ctypes.byref(gv), ctypes.c_void_p(wptr), wbytes,
        ctypes.c_void_p(_lib.stream_handle())))
    return dq, dk, dv


def head_relayout(src, dst):
    """Copy each (flat head, row) vector of src into dst: two [B,H,N,d] views
    of the same B*H heads in different layouts (the re-layouts around the
    Ulysses all-to-all)."""
    L = _lib.lib()
    a, b = _lib.desc(src), _lib.desc(dst)
    _lib.check(L.seqattn_head_relayout(ctypes.byref(a), ctypes.byref(b),
                                       ctypes.c_void_p(_lib.stream_handle())))
    return dst
