"""fp64 CPU oracle for segmented exact softmax attention (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does.  It
shares no code with the HIP library (it loads ``liboracle.so`` built from
``oracle.c`` with gcc, and nothing else).

Every function takes numpy arrays holding the exact values the GPU receives
(bf16 and fp32 values are exact in float32) and returns float64 results.
See ``oracle.c`` for the definitions and the passages of the pages they
follow.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

NONCAUSAL = np.iinfo(np.int64).max

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc -O2 -fopenmp (no fast-math)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-std=c99", "-Wall", "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB):
        build()
    lib = ctypes.CDLL(LIB)
    P = ctypes.c_void_p
    I = ctypes.c_int64
    D = ctypes.c_double
    lib.oracle_attn_fwd.argtypes = [P, P, P, I, I, I, I, I, I, I, D, P, I, P, P]
    lib.oracle_lse_merge.argtypes = [P, P, P, P, I, I, P, P]
    lib.oracle_dilated_fwd.argtypes = [P, P, P, I, I, I, I, I, P, P, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int32, D, P, I, P, P]
    lib.oracle_attn_bwd_dq_rows.argtypes = [P, P, P, P, I, I, I, I, I, I, I, D,
                                            P, I, P, P, P]
    lib.oracle_attn_bwd.argtypes = [P, P, P, P, I, I, I, I, I, I, I, D, P, P, P]
    lib.oracle_dilated_bwd.argtypes = [P, P, P, P, I, I, I, I, I, P, P, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int32, D, P, P, P]
    lib.oracle_num_threads.restype = ctypes.c_int
    for f in ("oracle_attn_fwd", "oracle_lse_merge", "oracle_dilated_fwd",
              "oracle_attn_bwd_dq_rows", "oracle_attn_bwd", "oracle_dilated_bwd"):
        getattr(lib, f).restype = None
    _lib = lib
    return lib


def _f32(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    return a


def _ptr(a):
    return a.ctypes.data if a is not None else None


def _as4(a):
    """[H,N,d] -> [1,H,N,d]; [B,H,N,d] unchanged."""
    a = _f32(a)
    if a.ndim == 3:
        a = a[None]
    assert a.ndim == 4
    return a


def _rows_arg(rows):
    if rows is None:
        return None
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    return r


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def attn_fwd(q, k, v, delta=NONCAUSAL, scale=0.0, rows=None):
    """(O, LSE) of q [B,Hq,Nq,d] (or [Hq,Nq,d]) against k, v [B,Hkv,Nk,d].

    Key j is visible to query i iff j <= i + delta.  ``rows`` is an optional
    list of flat row ids (b*Hq + h)*Nq + i; then O is [len(rows), d] and LSE
    [len(rows)], else O is [B,Hq,Nq,d] and LSE [B,Hq,Nq].
    """
    lib = _load()
    q4, k4, v4 = _as4(q), _as4(k), _as4(v)
    B, Hq, Nq, d = q4.shape
    _, Hkv, Nk, _ = k4.shape
    r = _rows_arg(rows)
    n = len(r) if r is not None else B * Hq * Nq
    o = np.empty((n, d), np.float64)
    lse = np.empty((n,), np.float64)
    lib.oracle_attn_fwd(_ptr(q4), _ptr(k4), _ptr(v4), B, Hq, Hkv, Nq, Nk, d,
                        int(delta), float(scale), _ptr(r), n, _ptr(o), _ptr(lse))
    if r is None:
        o = o.reshape(B, Hq, Nq, d)
        lse = lse.reshape(B, Hq, Nq)
        if np.asarray(q).ndim == 3:
            o, lse = o[0], lse[0]
    return o, lse


def lse_merge(o_a, lse_a, o_b, lse_b):
    """Row-wise log-sum-exp merge of two partials (any leading shape)."""
    lib = _load()
    oa = np.ascontiguousarray(o_a, np.float64)
    ob = np.ascontiguousarray(o_b, np.float64)
    la = np.ascontiguousarray(lse_a, np.float64)
    lb = np.ascontiguousarray(lse_b, np.float64)
    d = oa.shape[-1]
    nrows = la.size
    o = np.empty_like(oa)
    lse = np.empty_like(la)
    lib.oracle_lse_merge(_ptr(oa), _ptr(la), _ptr(ob), _ptr(lb), nrows, d,
                         _ptr(o), _ptr(lse))
    return o, lse


def dilated_fwd(q, k, v, segment_lengths, dilations, causal=False, scale=0.0,
                rows=None, head_shift=False):
    """LongNet dilated attention, branch partials folded by the LSE merge.
    head_shift: query head h selects offset h mod r_i inside each segment
    (offset 0 for every head otherwise)."""
    lib = _load()
    q4, k4, v4 = _as4(q), _as4(k), _as4(v)
    B, Hq, N, d = q4.shape
    Hkv = k4.shape[1]
    w = np.ascontiguousarray(segment_lengths, np.int64)
    rr = np.ascontiguousarray(dilations, np.int64)
    assert w.shape == rr.shape
    r = _rows_arg(rows)
    n = len(r) if r is not None else B * Hq * N
    o = np.empty((n, d), np.float64)
    lse = np.empty((n,), np.float64)
    lib.oracle_dilated_fwd(_ptr(q4), _ptr(k4), _ptr(v4), B, Hq, Hkv, N, d,
                           _ptr(w), _ptr(rr), len(w), int(bool(causal)),
                           int(bool(head_shift)), float(scale), _ptr(r), n, _ptr(o),
                           _ptr(lse))
    if r is None:
        o = o.reshape(B, Hq, N, d)
        lse = lse.reshape(B, Hq, N)
        if np.asarray(q).ndim == 3:
            o, lse = o[0], lse[0]
    return o, lse


def attn_bwd_dq_rows(q, k, v, dout, delta=NONCAUSAL, scale=0.0, rows=None):
    """dQ (and O, LSE) for selected query rows, from the full key set."""
    lib = _load()
    q4, k4, v4, do4 = _as4(q), _as4(k), _as4(v), _as4(dout)
    B, Hq, Nq, d = q4.shape
    _, Hkv, Nk, _ = k4.shape
    r = _rows_arg(rows)
    n = len(r) if r is not None else B * Hq * Nq
    dq = np.empty((n, d), np.float64)
    o = np.empty((n, d), np.float64)
    lse = np.empty((n,), np.float64)
    lib.oracle_attn_bwd_dq_rows(_ptr(q4), _ptr(k4), _ptr(v4), _ptr(do4), B, Hq,
                                Hkv, Nq, Nk, d, int(delta), float(scale),
                                _ptr(r), n, _ptr(dq), _ptr(o), _ptr(lse))
    return dq, o, lse


def attn_bwd(q, k, v, dout, delta=NONCAUSAL, scale=0.0):
    """Full (dQ, dK, dV) of L = sum(dO * O) for the attention defined above."""
    lib = _load()
    q4, k4, v4, do4 = _as4(q), _as4(k), _as4(v), _as4(dout)
    B, Hq, Nq, d = q4.shape
    _, Hkv, Nk, _ = k4.shape
    dq = np.empty((B, Hq, Nq, d), np.float64)
    dk = np.empty((B, Hkv, Nk, d), np.float64)
    dv = np.empty((B, Hkv, Nk, d), np.float64)
    lib.oracle_attn_bwd(_ptr(q4), _ptr(k4), _ptr(v4), _ptr(do4), B, Hq, Hkv, Nq,
                        Nk, d, int(delta), float(scale), _ptr(dq), _ptr(dk),
                        _ptr(dv))
    if np.asarray(q).ndim == 3:
        return dq[0], dk[0], dv[0]
    return dq, dk, dv


def dilated_bwd(q, k, v, dout, segment_lengths, dilations, causal=False, scale=0.0,
                head_shift=False):
    """(dQ, dK, dV) of L = sum(dO * O) for dilated_fwd's attention."""
    lib = _load()
    q4, k4, v4, do4 = _as4(q), _as4(k), _as4(v), _as4(dout)
    B, Hq, N, d = q4.shape
    Hkv = k4.shape[1]
    w = np.ascontiguousarray(segment_lengths, np.int64)
    rr = np.ascontiguousarray(dilations, np.int64)
    dq = np.empty((B, Hq, N, d), np.float64)
    dk = np.empty((B, Hkv, N, d), np.float64)
    dv = np.empty((B, Hkv, N, d), np.float64)
    lib.oracle_dilated_bwd(_ptr(q4), _ptr(k4), _ptr(v4), _ptr(do4), B, Hq, Hkv, N, d,
                           _ptr(w), _ptr(rr), len(w), int(bool(causal)),
                           int(bool(head_shift)), float(scale), _ptr(dq), _ptr(dk), _ptr(dv))
    if np.asarray(q).ndim == 3:
        return dq[0], dk[0], dv[0]
    return dq, dk, dv
