"""ctypes binding of libseqattn.so (argument marshalling only).

Each function turns torch CUDA tensors into ``seqattn_tensor`` descriptors,
passes torch's current HIP stream, and raises on a non-OK status.  Every step
of the computation runs in the library's HIP kernels; there is no host or CPU
fallback -- if the library is missing, the first call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libseqattn.so")

BF16, F32 = 1, 2
NONCAUSAL = (1 << 63) - 1
ACCUMULATE = 1
CAUSAL = 2
HEAD_SHIFT = 4
OP_SEGMENT_FWD, OP_LSE_MERGE, OP_DILATED_FWD, OP_SEGMENT_BWD, OP_DILATED_BWD = 0, 1, 2, 3, 4

EXPORTS = ("seqattn_attn_segment_fwd", "seqattn_attn_segment_fwd_ws", "seqattn_lse_merge",
           "seqattn_dilated_attn_fwd",
           "seqattn_attn_segment_bwd", "seqattn_attn_segment_bwd_noalloc",
           "seqattn_dilated_attn_bwd", "seqattn_head_relayout",
           "seqattn_workspace_size", "seqattn_status_string", "seqattn_last_error",
           "seqattn_version")


class Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("b", ctypes.c_int64), ("h", ctypes.c_int64), ("n", ctypes.c_int64),
                ("d", ctypes.c_int64), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("stride_n", ctypes.c_int64)]


class SeqattnError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"seqattn status {status}: {detail}")
        self.status = status


_lib = None


def lib():
    """Load libseqattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m long_sequence_exact_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(Tensor)
    I64, F, U32, VP = ctypes.c_int64, ctypes.c_float, ctypes.c_uint32, ctypes.c_void_p
    L.seqattn_attn_segment_fwd.argtypes = [P, P, P, I64, F, U32, P, P, VP]
    L.seqattn_attn_segment_fwd_ws.argtypes = [P, P, P, I64, F, U32, P, P, VP, ctypes.c_size_t,
                                              VP]
    L.seqattn_lse_merge.argtypes = [P, P, P, P, VP]
    L.seqattn_dilated_attn_fwd.argtypes = [P, P, P, ctypes.POINTER(I64), ctypes.POINTER(I64),
                                           ctypes.c_int32, F, U32, P, P, VP, ctypes.c_size_t,
                                           VP]
    L.seqattn_attn_segment_bwd.argtypes = [P, P, P, P, P, P, I64, F, U32, P, P, P, VP,
                                           ctypes.c_size_t, VP]
    L.seqattn_attn_segment_bwd_noalloc.argtypes = [P, P, P, P, P, P, I64, F, U32, P, P, P, VP]
    L.seqattn_dilated_attn_bwd.argtypes = [P, P, P, P, P, P, ctypes.POINTER(I64),
                                           ctypes.POINTER(I64), ctypes.c_int32, F, U32, P, P,
                                           P, VP, ctypes.c_size_t, VP]
    L.seqattn_head_relayout.argtypes = [P, P, VP]
    L.seqattn_workspace_size.argtypes = [ctypes.c_int, P, P, ctypes.c_int32]
    L.seqattn_workspace_size.restype = ctypes.c_size_t
    L.seqattn_status_string.restype = ctypes.c_char_p
    L.seqattn_status_string.argtypes = [ctypes.c_int]
    L.seqattn_last_error.restype = ctypes.c_char_p
    for f in ("seqattn_attn_segment_fwd", "seqattn_attn_segment_fwd_ws", "seqattn_lse_merge",
              "seqattn_dilated_attn_fwd", "seqattn_attn_segment_bwd",
              "seqattn_attn_segment_bwd_noalloc", "seqattn_dilated_attn_bwd",
              "seqattn_head_relayout", "seqattn_version"):
        getattr(L, f).restype = ctypes.c_int
    _lib = L
    return L


def check(status: int):
    if status != 0:
        L = lib()
        raise SeqattnError(status, f"{L.seqattn_status_string(status).decode()}: "
                                   f"{L.seqattn_last_error().decode()}")


def desc(t: torch.Tensor, lse: bool = False, on_device: bool = True) -> Tensor:
    """Descriptor of a [B,H,N,d] / [H,N,d] tensor, or of an LSE [B,H,N] / [H,N].
    The kernels read and write these addresses, so they must be GPU memory
    (on_device=False only for size queries)."""
    if on_device and not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if t.dtype == torch.bfloat16:
        dt = BF16
    elif t.dtype == torch.float32:
        dt = F32
    else:
        raise TypeError(f"unsupported dtype {t.dtype}")
    if lse:
        if t.dim() == 2:
            t = t.unsqueeze(0)
        if t.dim() != 3:
            raise ValueError("LSE tensors are [B,H,N] or [H,N]")
        b, h, n = t.shape
        sb, sh, sn = t.stride()
        return Tensor(t.data_ptr(), dt, b, h, n, 1, sb, sh, sn)
    if t.dim() == 3:
        t = t.unsqueeze(0)
    if t.dim() != 4:
        raise ValueError("tensors are [B,H,N,d] or [H,N,d]")
    if t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError("the last dimension must be contiguous")
    b, h, n, d = t.shape
    sb, sh, sn, _ = t.stride()
    return Tensor(t.data_ptr(), dt, b, h, n, d, sb, sh, sn)


def stream_handle() -> int:
    return torch.cuda.current_stream().cuda_stream
