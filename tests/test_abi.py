"""The C ABI on the CPU: the library loads, exports what include/seqattn.h
declares, and every validation error is returned before any HIP call (fake,
never dereferenced device addresses are used)."""
import ctypes
import os
import re
import subprocess

import pytest

from long_sequence_exact_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "seqattn.h")

OK, ENULL, EDTYPE, ESHAPE, ESTRIDE, EALIAS, EUNSUP, EWS, EHIP = 0, -1, -2, -3, -4, -5, -6, -7, -8


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        from long_sequence_exact_amd import build
        build.build()
    return _lib.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(seqattn_[a-z_]+)\s*\(", src)))


def test_header_declares_the_four_ops_and_helpers():
    names = declared_functions()
    for f in ("seqattn_attn_segment_fwd", "seqattn_lse_merge", "seqattn_dilated_attn_fwd",
              "seqattn_attn_segment_bwd"):
        assert f in names
    assert set(names) == set(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (seqattn_\w+)", out))
    assert set(declared_functions()) <= exported
    assert L.seqattn_version() == 110


BASE = 0x7f0000000000  # fake, 256-byte aligned device addresses (never touched)


def T(addr, dtype, b, h, n, d, contiguous=True, **kw):
    t = _lib.Tensor(addr, dtype, b, h, n, d, h * n * d, n * d, d)
    for key, val in kw.items():
        setattr(t, key, val)
    return t


def LSE(addr, b, h, n):
    return _lib.Tensor(addr, _lib.F32, b, h, n, 1, h * n, n, 1)


def qkvo(dtype=_lib.BF16, hq=4, hkv=2, nq=256, nk=512, d=128, odtype=None):
    step = 1 << 30
    q = T(BASE, dtype, 1, hq, nq, d)
    k = T(BASE + step, dtype, 1, hkv, nk, d)
    v = T(BASE + 2 * step, dtype, 1, hkv, nk, d)
    o = T(BASE + 3 * step, odtype or dtype, 1, hq, nq, d)
    lse = LSE(BASE + 4 * step, 1, hq, nq)
    return q, k, v, o, lse


def fwd(L, q, k, v, o, lse, delta=0, flags=0):
    r = ctypes.byref
    return L.seqattn_attn_segment_fwd(r(q) if q is not None else None, r(k), r(v), delta, 0.0,
                                      flags, r(o), r(lse), None)


def test_fwd_validation_errors(L):
    q, k, v, o, lse = qkvo()
    assert fwd(L, None, k, v, o, lse) == ENULL
    q2 = T(BASE, _lib.F32, 1, 4, 256, 128)
    assert fwd(L, q2, k, v, o, lse) == EDTYPE
    qbad = T(BASE, 7, 1, 4, 256, 128)
    assert fwd(L, qbad, k, v, o, lse) == EDTYPE
    q96, k96, v96, o96, l96 = qkvo(d=96)
    assert fwd(L, q96, k96, v96, o96, l96) == ESHAPE
    q3, k3, v3, o3, l3 = qkvo(hq=6, hkv=4)
    assert fwd(L, q3, k3, v3, o3, l3) == ESHAPE
    qm = T(BASE + 8, _lib.BF16, 1, 4, 256, 128)
    assert fwd(L, qm, k, v, o, lse) == ESTRIDE
    qs = T(BASE, _lib.BF16, 1, 4, 256, 128, stride_n=132)
    assert fwd(L, qs, k, v, o, lse) == ESTRIDE
    neg = T(BASE, _lib.BF16, 1, 4, -1, 128)
    assert fwd(L, neg, k, v, o, lse) == ESHAPE
    oal = T(BASE + 64, _lib.BF16, 1, 4, 256, 128)  # overlaps q
    assert fwd(L, q, k, v, oal, lse) == EALIAS
    assert fwd(L, q, k, v, o, lse, flags=1) == EDTYPE  # accumulate needs fp32 o
    assert fwd(L, q, k, v, o, lse, flags=8) == EUNSUP
    lbad = _lib.Tensor(lse.data, _lib.BF16, 1, 4, 256, 1, 1024, 256, 1)
    assert fwd(L, q, k, v, o, lbad) == EDTYPE
    lshape = LSE(lse.data, 1, 4, 255)
    assert fwd(L, q, k, v, o, lshape) == ESHAPE
    kv_mis = T(BASE + (1 << 30), _lib.BF16, 1, 2, 500, 128)
    assert fwd(L, q, kv_mis, v, o, lse) == ESHAPE
    # fp32 inputs need an fp32 output
    qf, kf, vf, of, lf = qkvo(dtype=_lib.F32, odtype=_lib.BF16)
    assert fwd(L, qf, kf, vf, of, lf) == EDTYPE
    msg = L.seqattn_last_error().decode()
    assert "fp32" in msg
    assert L.seqattn_status_string(EALIAS).decode() == "output aliases an input"


def test_oversized_dimensions_and_strides_are_rejected(L):
    q, k, v, o, lse = qkvo()
    # b * h would overflow int64 if multiplied first
    huge = T(BASE, _lib.BF16, 1 << 40, 1 << 40, 256, 128)
    assert fwd(L, huge, k, v, o, lse) == ESHAPE
    # a stride beyond 2^40 elements
    far = T(BASE, _lib.BF16, 2, 4, 256, 128, stride_b=1 << 50)
    assert fwd(L, far, k, v, o, lse) == ESTRIDE
    # rows x row stride beyond 2^64 bytes: rejected, not wrapped around
    wide = T(BASE, _lib.BF16, 1, 4, (1 << 30) - 1, 128, stride_n=(1 << 39))
    assert fwd(L, wide, k, v, o, lse) == ESTRIDE
    assert "2^56" in L.seqattn_last_error().decode()
    # a head spanning 16 GiB through its row stride: the 2 GiB per-head limit
    q1, k1, v1, o1, l1 = qkvo(hq=1, hkv=1, nq=1 << 20)
    tall = T(BASE, _lib.BF16, 1, 1, 1 << 20, 128, stride_n=8192, stride_h=8192 << 20)
    o1 = T(BASE + (1 << 40), _lib.BF16, 1, 1, 1 << 20, 128)
    l1 = LSE(BASE + (2 << 40), 1, 1, 1 << 20)
    assert fwd(L, tall, k1, v1, o1, l1) == EUNSUP
    assert "2 GiB" in L.seqattn_last_error().decode()


def test_fwd_empty_query_block_returns_ok_without_launch(L):
    q, k, v, o, lse = qkvo(nq=0)
    assert fwd(L, q, k, v, o, lse) == OK


def test_lse_merge_validation_errors(L):
    r = ctypes.byref
    step = 1 << 28
    oa = T(BASE, _lib.F32, 1, 2, 64, 128)
    la = LSE(BASE + step, 1, 2, 64)
    ob = T(BASE + 2 * step, _lib.BF16, 1, 2, 64, 128)
    lb = LSE(BASE + 3 * step, 1, 2, 64)
    oa16 = T(BASE, _lib.BF16, 1, 2, 64, 128)
    assert L.seqattn_lse_merge(r(oa16), r(la), r(ob), r(lb), None) == EDTYPE
    ob_bad = T(BASE + 2 * step, _lib.BF16, 1, 2, 63, 128)
    assert L.seqattn_lse_merge(r(oa), r(la), r(ob_bad), r(lb), None) == ESHAPE
    assert L.seqattn_lse_merge(r(oa), r(la), r(oa), r(lb), None) == EALIAS
    assert L.seqattn_lse_merge(None, r(la), r(ob), r(lb), None) == ENULL


def test_dilated_validation_errors(L):
    r = ctypes.byref
    q, k, v, o, lse = qkvo(hq=2, hkv=2, nq=512, nk=512, d=64, odtype=_lib.BF16)
    w = (ctypes.c_int64 * 2)(128, 512)
    rr = (ctypes.c_int64 * 2)(1, 2)
    call = lambda w_, r_, nb, flags=0, ws=None, wsb=0, oo=o: L.seqattn_dilated_attn_fwd(
        r(q), r(k), r(v), w_, r_, nb, 0.0, flags, r(oo), r(lse), ws, wsb, None)
    assert call(w, rr, 0) == ESHAPE
    assert call(None, rr, 2) == ENULL
    w0 = (ctypes.c_int64 * 2)(0, 512)
    assert call(w0, rr, 2) == ESHAPE
    assert call(w, rr, 2, flags=1) == EUNSUP
    assert call(w, rr, 2, flags=8) == EUNSUP
    assert call(w, rr, 2) == EWS  # bf16 o needs the fp32 workspace
    need = L.seqattn_workspace_size(_lib.OP_DILATED_FWD, r(q), r(o), 2)
    assert need == 2 * 512 * 64 * 4
    assert call(w, rr, 2, ws=BASE + (5 << 30), wsb=need - 1) == EWS
    qn = T(BASE, _lib.BF16, 1, 2, 500, 64)
    assert L.seqattn_dilated_attn_fwd(r(qn), r(k), r(v), w, rr, 2, 0.0, 0, r(o), r(lse),
                                      None, 0, None) == ESHAPE


def test_bwd_validation_errors(L):
    r = ctypes.byref
    step = 1 << 30
    q, k, v, o, lse = qkvo()
    do = T(BASE + 5 * step, _lib.BF16, 1, 4, 256, 128)
    dq = T(BASE + 6 * step, _lib.F32, 1, 4, 256, 128)
    dk = T(BASE + 7 * step, _lib.F32, 1, 2, 512, 128)
    dv = T(BASE + 8 * step, _lib.F32, 1, 2, 512, 128)
    need = L.seqattn_workspace_size(_lib.OP_SEGMENT_BWD, r(q), r(k), 0)
    assert need == 4 * 256 * 4
    ws = BASE + 9 * step

    def call(q_=q, dq_=dq, dk_=dk, dv_=dv, ws_=ws, wsb=need, flags=0):
        return L.seqattn_attn_segment_bwd(r(q_), r(k), r(v), r(o), r(lse), r(do), 0, 0.0,
                                          flags, r(dq_), r(dk_), r(dv_), ws_, wsb, None)
    assert call(wsb=need - 4) == EWS
    assert call(ws_=None, wsb=0) == EWS
    dq16 = T(dq.data, _lib.BF16, 1, 4, 256, 128)
    assert call(dq_=dq16) == EDTYPE
    dv_al = T(dk.data + 256, _lib.F32, 1, 2, 512, 128)
    assert call(dv_=dv_al) == EALIAS
    dk_bad = T(dk.data, _lib.F32, 1, 2, 511, 128)
    assert call(dk_=dk_bad) == ESHAPE
    assert call(flags=4) == EUNSUP
    dk16 = T(dk.data, _lib.BF16, 1, 2, 512, 128)
    assert call(dk_=dk16, flags=1) == EDTYPE  # accumulated dK/dV must be fp32
    qf, kf, vf, _, _ = qkvo(dtype=_lib.F32)
    assert L.seqattn_attn_segment_bwd(r(qf), r(kf), r(vf), r(o), r(lse), r(do), 0, 0.0, 0,
                                      r(dq), r(dk), r(dv), ws, need, None) == EUNSUP
    # K / V heads spanning 2 GiB: the dQ kernel addresses them with 32-bit offsets
    nbig = (1 << 31) // 256
    kb = T(BASE + step, _lib.BF16, 1, 2, nbig, 128)
    vb = T(BASE + 40 * step, _lib.BF16, 1, 2, nbig, 128)
    dkb = T(BASE + 80 * step, _lib.F32, 1, 2, nbig, 128)
    dvb = T(BASE + 120 * step, _lib.F32, 1, 2, nbig, 128)
    assert L.seqattn_attn_segment_bwd(r(q), r(kb), r(vb), r(o), r(lse), r(do), 0, 0.0, 0,
                                      r(dq), r(dkb), r(dvb), ws, need, None) == EUNSUP
    assert "2 GiB" in L.seqattn_last_error().decode()


def test_dilated_bwd_validation_errors(L):
    r = ctypes.byref
    step = 1 << 30
    q, k, v, o, lse = qkvo(hq=4, hkv=2, nq=512, nk=512, d=64, odtype=_lib.F32)
    do = T(BASE + 5 * step, _lib.BF16, 1, 4, 512, 64)
    dq = T(BASE + 6 * step, _lib.F32, 1, 4, 512, 64)
    dk = T(BASE + 7 * step, _lib.F32, 1, 2, 512, 64)
    dv = T(BASE + 8 * step, _lib.F32, 1, 2, 512, 64)
    ws = BASE + 9 * step
    w = (ctypes.c_int64 * 2)(128, 512)
    rr = (ctypes.c_int64 * 2)(1, 2)
    need = L.seqattn_workspace_size(_lib.OP_DILATED_BWD, r(q), r(k), 2)
    assert need == 4 * 512 * 4

    def call(w_=w, r_=rr, nb=2, flags=0, dq_=dq, dk_=dk, dv_=dv, do_=do, ws_=ws, wsb=need):
        return L.seqattn_dilated_attn_bwd(r(q), r(k), r(v), r(o), r(lse), r(do_), w_, r_, nb,
                                          0.0, flags, r(dq_), r(dk_), r(dv_), ws_, wsb, None)
    assert call(nb=0) == ESHAPE
    assert call(nb=65) == ESHAPE
    assert call(w_=None) == ENULL
    assert call(w_=(ctypes.c_int64 * 2)(128, 0)) == ESHAPE
    assert call(r_=(ctypes.c_int64 * 2)(0, 2)) == ESHAPE
    assert call(flags=1) == EUNSUP  # only SEQATTN_CAUSAL | SEQATTN_HEAD_SHIFT
    assert call(flags=8) == EUNSUP
    assert call(wsb=need - 4) == EWS
    assert call(ws_=None, wsb=0) == EWS
    assert call(ws_=ws + 4) == EWS  # misaligned
    assert call(dk_=T(dk.data, _lib.BF16, 1, 2, 512, 64)) == EDTYPE
    assert call(do_=T(do.data, _lib.F32, 1, 4, 512, 64)) == EDTYPE
    assert call(dv_=T(dv.data, _lib.F32, 1, 2, 256, 64)) == ESHAPE
    assert call(dq_=T(dk.data + 512, _lib.F32, 1, 4, 512, 64)) == EALIAS
    assert call(dv_=T(q.data, _lib.F32, 1, 2, 512, 64)) == EALIAS


def test_head_relayout_validation_errors(L):
    r = ctypes.byref
    src = T(BASE, _lib.BF16, 1, 8, 256, 128)
    dst = T(BASE + (1 << 30), _lib.BF16, 4, 2, 256, 128)
    call = lambda s=src, d_=dst: L.seqattn_head_relayout(r(s), r(d_), None)
    assert call(d_=T(dst.data, _lib.F32, 4, 2, 256, 128)) == EDTYPE
    assert call(d_=T(dst.data, _lib.BF16, 3, 2, 256, 128)) == ESHAPE  # b*h differs
    assert call(d_=T(dst.data, _lib.BF16, 4, 2, 255, 128)) == ESHAPE
    # 8-byte vectors (rows padded to 16 bytes)
    odd = T(BASE, _lib.BF16, 1, 8, 256, 4, stride_n=8, stride_h=256 * 8)
    odd_d = T(dst.data, _lib.BF16, 4, 2, 256, 4, stride_n=8, stride_h=256 * 8,
              stride_b=2 * 256 * 8)
    assert call(s=odd, d_=odd_d) == ESHAPE
    assert call(d_=T(BASE + 4096, _lib.BF16, 4, 2, 256, 128)) == EALIAS
    same_rows = T(dst.data, _lib.BF16, 4, 2, 256, 128, stride_h=0)
    assert call(d_=same_rows) == ESTRIDE
    big_s = T(BASE, _lib.BF16, 1, 1 << 10, 1 << 18, 128)
    big_d = T(BASE + (1 << 40), _lib.BF16, 1, 1 << 10, 1 << 18, 128)
    assert call(s=big_s, d_=big_d) == EUNSUP
    assert call(s=T(BASE, _lib.BF16, 1, 8, 0, 128), d_=T(dst.data, _lib.BF16, 4, 2, 0, 128)) == OK


def test_outputs_with_overlapping_rows_are_rejected(L):
    r = ctypes.byref
    q, k, v, o, lse = qkvo()
    o_bad = T(o.data, o.dtype, 1, 4, 256, 128, stride_h=0)
    assert fwd(L, q, k, v, o_bad, lse) == ESTRIDE
    lse_bad = _lib.Tensor(lse.data, _lib.F32, 1, 4, 256, 1, 4 * 256, 128, 1)
    assert fwd(L, q, k, v, o, lse_bad) == ESTRIDE


def test_bwd_noalloc_validation_errors(L):
    """The no-allocation backward validates like the workspace one, and
    rejects more query rows than its fixed scratch holds, before any HIP call."""
    r = ctypes.byref
    step = 1 << 30
    q, k, v, o, lse = qkvo()
    do = T(BASE + 5 * step, _lib.BF16, 1, 4, 256, 128)
    dq = T(BASE + 6 * step, _lib.F32, 1, 4, 256, 128)
    dk = T(BASE + 7 * step, _lib.F32, 1, 2, 512, 128)
    dv = T(BASE + 8 * step, _lib.F32, 1, 2, 512, 128)

    def call(q_=q, o_=o, lse_=lse, do_=do, dq_=dq, dk_=dk, dv_=dv, flags=0):
        return L.seqattn_attn_segment_bwd_noalloc(r(q_), r(k), r(v), r(o_), r(lse_), r(do_), 0,
                                                  0.0, flags, r(dq_), r(dk_), r(dv_), None)
    dq16 = T(dq.data, _lib.BF16, 1, 4, 256, 128)
    assert call(dq_=dq16) == EDTYPE
    dv_al = T(dk.data + 256, _lib.F32, 1, 2, 512, 128)
    assert call(dv_=dv_al) == EALIAS
    assert call(flags=4) == EUNSUP
    assert L.seqattn_attn_segment_bwd_noalloc(None, r(k), r(v), r(o), r(lse), r(do), 0, 0.0, 0,
                                              r(dq), r(dk), r(dv), None) == ENULL
    # 4,194,305 query rows: one more than the 16 MiB scratch holds
    rows = (16 << 20) // 4
    for hq, nq in ((4, rows // 4 + 1), (1, rows + 1)):
        qb = T(BASE, _lib.BF16, 1, hq, nq, 128)
        ob = T(BASE + 3 * step, _lib.BF16, 1, hq, nq, 128)
        lb = LSE(BASE + 12 * step, 1, hq, nq)
        dob = T(BASE + 5 * step, _lib.BF16, 1, hq, nq, 128)
        dqb = T(BASE + 16 * step, _lib.F32, 1, hq, nq, 128)
        kb = T(BASE + step, _lib.BF16, 1, 1 if hq == 1 else 2, 512, 128)
        assert L.seqattn_attn_segment_bwd_noalloc(
            r(qb), r(kb), r(T(BASE + 2 * step, _lib.BF16, 1, kb.h, 512, 128)), r(ob), r(lb),
            r(dob), 0, 0.0, 0, r(dqb), r(T(dk.data, _lib.F32, 1, kb.h, 512, 128)),
            r(T(dv.data, _lib.F32, 1, kb.h, 512, 128)), None) == EWS
        assert "scratch" in L.seqattn_last_error().decode()


C_PROGRAM = r"""
#include <stddef.h>
#include <stdio.h>
#include <string.h>
#include "seqattn.h"

/* A plain C caller: the descriptor layout it sees, and calls whose arguments
   are rejected before any HIP call (fake device addresses, never touched). */
int main(void)
{
    printf("size %zu data %zu dtype %zu b %zu d %zu stride_n %zu\n", sizeof(seqattn_tensor),
           offsetof(seqattn_tensor, data), offsetof(seqattn_tensor, dtype),
           offsetof(seqattn_tensor, b), offsetof(seqattn_tensor, d),
           offsetof(seqattn_tensor, stride_n));
    printf("version %d\n", seqattn_version());
    seqattn_tensor q = {(void *)0x7f0000000000ull, SEQATTN_BF16, 1, 4, 256, 128,
                        4 * 256 * 128, 256 * 128, 128};
    seqattn_tensor k = q, v = q, o = q, lse = q;
    k.data = (void *)0x7f0040000000ull;
    v.data = (void *)0x7f0080000000ull;
    o.data = (void *)0x7f00c0000000ull;
    lse.data = (void *)0x7f0100000000ull;
    lse.dtype = SEQATTN_F32;
    lse.d = 1;
    lse.stride_b = 4 * 256;
    lse.stride_h = 256;
    lse.stride_n = 1;
    int st = seqattn_attn_segment_fwd(NULL, &k, &v, 0, 0.f, 0, &o, &lse, NULL);
    printf("null %d %s | %s\n", st, seqattn_status_string(st), seqattn_last_error());
    k.d = 64;
    st = seqattn_attn_segment_fwd(&q, &k, &v, 0, 0.f, 0, &o, &lse, NULL);
    printf("shape %d %s\n", st, seqattn_status_string(st));
    k.d = 128;
    o.data = q.data;
    st = seqattn_attn_segment_fwd(&q, &k, &v, 0, 0.f, 0, &o, &lse, NULL);
    printf("alias %d %s\n", st, seqattn_status_string(st));
    return 0;
}
"""


def test_plain_c_caller(L, tmp_path):
    """The header compiles as C99 with warnings as errors, a C program links
    against the library, sees the same descriptor layout as the binding, and
    gets the documented error codes back."""
    src = tmp_path / "caller.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "caller"
    libdir = os.path.dirname(_lib.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I",
                    os.path.join(ROOT, "include"), str(src), "-o", str(exe), "-L", libdir,
                    "-lseqattn", f"-Wl,-rpath,{libdir}"], check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    lines = dict(line.split(" ", 1) for line in out.strip().splitlines())
    f = _lib.Tensor
    assert lines["size"] == (f"{ctypes.sizeof(f)} data {f.data.offset} dtype {f.dtype.offset} "
                             f"b {f.b.offset} d {f.d.offset} stride_n {f.stride_n.offset}")
    assert lines["version"] == "110"
    assert lines["null"].startswith(f"{ENULL} ")
    assert lines["null"].split(" | ")[1]          # the detail message is set
    assert lines["shape"].startswith(f"{ESHAPE} ")
    assert lines["alias"].startswith(f"{EALIAS} ")


def test_split_forward_workspace(L):
    """seqattn_attn_segment_fwd_ws: the workspace size follows the split rule
    for a causal call, which never takes fewer chunks than a non-causal one
    (bf16, d = 128, at least 1024 keys, fewer 256-row tiles than two per
    compute unit, about two items per CU, at most eight chunks, the longest
    tile's at least 1024 keys from 4096 keys on, else 512), and a split call without enough aligned, non-overlapping
    workspace is refused before any HIP call."""
    r = ctypes.byref
    step = 1 << 30

    def size(hq, nq, nk, d=128, dt=_lib.BF16):
        qq = T(BASE, dt, 1, hq, nq, d)
        kk = T(BASE + step, dt, 1, 1, nk, d)
        return L.seqattn_workspace_size(_lib.OP_SEGMENT_FWD, r(qq), r(kk), 0)

    def chunks(hq, nq, nk):
        per = hq * nq * (128 + 1) * 4  # fp32 O and LSE of every row
        assert size(hq, nq, nk) % per == 0
        return size(hq, nq, nk) // per

    assert chunks(4, 16384, 16384) == 2    # 256 tiles: two items per CU
    assert chunks(2, 16384, 16384) == 4    # 128 tiles
    assert chunks(4, 4096, 4096) == 4      # 64 tiles: parts of 1024 from 4096 keys on
    assert chunks(4, 2048, 2048) == 4      # 32 tiles: at most 2048 / 512 chunks
    assert chunks(1, 1000, 9000) == 8      # 4 tiles: at most eight
    assert chunks(3, 5000, 9000) == 8      # 60 tiles, ragged
    assert size(8, 16384, 16384) == 0      # 512 tiles fill the chip twice
    assert size(2, 16384, 1023) == 0       # too few keys
    assert size(2, 16384, 16384, dt=_lib.F32) == 0
    assert size(2, 16384, 16384, d=64) == 0
    # 2 heads x 16384 rows, split in four
    q = T(BASE, _lib.BF16, 1, 2, 16384, 128)
    k = T(BASE + step, _lib.BF16, 1, 2, 16384, 128)
    v = T(BASE + 2 * step, _lib.BF16, 1, 2, 16384, 128)
    o = T(BASE + 3 * step, _lib.BF16, 1, 2, 16384, 128)
    lse = LSE(BASE + 4 * step, 1, 2, 16384)
    need = L.seqattn_workspace_size(_lib.OP_SEGMENT_FWD, r(q), r(k), 0)
    assert need == 4 * (2 * 16384) * (128 + 1) * 4
    ws = BASE + 5 * step

    def call(ws_=ws, wsb=need, flags=0, o_=o):
        return L.seqattn_attn_segment_fwd_ws(r(q), r(k), r(v), 0, 0.0, flags, r(o_), r(lse),
                                             ws_, wsb, None)

    assert call(ws_=None, wsb=0) == EWS
    assert call(wsb=need - 4) == EWS
    assert call(ws_=ws + 4) == EWS                     # misaligned
    assert call(ws_=BASE + 2 * step + 4096) == EALIAS  # inside v
    # an accumulating call is not split (and checks its output dtype first)
    assert call(ws_=None, wsb=0, flags=1) == EDTYPE
