"""GPU parity of LongNet dilated attention against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import long_sequence_exact_amd as sa
from long_sequence_exact_amd import emulate
from long_sequence_exact_amd.synth import (WORKLOADS, draw, sample_rows, sample_rows_per_tile,
                                           workload_inputs)
from tests.parity import TOL, assert_parity, check_close, dilated_key_list, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _np32(t):
    return t.float().numpy()


BTOL = TOL[torch.bfloat16]

DILATED_CASES = [
    (512, 64, 2, 2, (64, 128, 256, 512), (1, 2, 4, 8), False),
    (512, 128, 4, 2, (64, 128, 256, 512), (1, 2, 4, 8), True),
    (600, 64, 2, 1, (64, 128, 256), (1, 2, 4), False),          # segment tails
    (640, 64, 1, 1, (8 * 10, 16 * 10, 32 * 10, 64 * 10), (1, 2, 6, 12), False),  # r not 2^k
    (384, 64, 2, 2, (96, 384), (2, 4), False),                  # first branch r > 1
    (300, 128, 2, 2, (1000,), (3,), True),                      # w > N
]


def _grads_parity(grads, ref, what):
    for name, x, r in zip(("dq", "dk", "dv"), grads, ref):
        assert not torch.isnan(x).any(), f"{what}: NaN in {name}"
        check_close(x, r, BTOL, what=what, name=name)


@pytest.mark.parametrize("n,d,hq,hkv,ws,rs,causal", DILATED_CASES)
def test_dilated_small(n, d, hq, hkv, ws, rs, causal):
    q, k, v = draw([(1, hq, n, d), (1, hkv, n, d), (1, hkv, n, d)], 500 + n + d)
    o_ref, l_ref = oracle.dilated_fwd(_np32(q), _np32(k), _np32(v), ws, rs, causal=causal)
    o, lse = sa.dilated_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), ws, rs, causal=causal)
    torch.cuda.synchronize()
    assert_parity(to_np(o), to_np(lse), o_ref, l_ref, torch.bfloat16, what="dilated f32 out")
    ob, lb = sa.dilated_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), ws, rs, causal=causal,
                                 out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert_parity(to_np(ob), to_np(lb), o_ref, l_ref, torch.bfloat16, what="dilated bf16 out")


def test_dilated_long_dense_first_branch_d128():
    """A first branch with r = 1 over a segment of at least 16384 rows writes
    the accumulator directly and runs with 384-row workgroups; the second
    branch merges into it.  O and LSE must be fully written; one seeded row
    in every 32-row slice of both heads against the oracle."""
    n, d, hq, hkv = 16384 + 96, 128, 2, 1
    ws, rs = (n, 4096), (1, 2)
    q, k, v = draw([(1, hq, n, d), (1, hkv, n, d), (1, hkv, n, d)], 560)
    o, lse = sa.dilated_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), ws, rs, causal=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    rows = []
    for h in range(hq):
        rows += [h * n + i for i in sample_rows_per_tile(n, 32, 1, 570 + h, must=(0, n - 1))]
    rows = np.array(rows, np.int64)
    o_ref, l_ref = oracle.dilated_fwd(_np32(q), _np32(k), _np32(v), ws, rs, causal=True,
                                      rows=rows)
    assert_parity(to_np(o).reshape(-1, d)[rows], to_np(lse).reshape(-1)[rows], o_ref, l_ref,
                  torch.bfloat16, rows_heads=rows // n, what="dilated long dense first branch")


HEAD_SHIFT_CASES = [
    # query head h selects offset h mod r inside each segment
    (512, 64, 8, 8, (64, 128, 256, 512), (1, 2, 4, 8), False),   # heads > r
    (515, 128, 8, 8, (64, 256, 512), (1, 4, 8), True),           # 3-row tails: offsets past them
    (640, 64, 6, 6, (80, 160, 320, 640), (1, 2, 6, 12), True),   # r not 2^k, r > heads
    (384, 64, 4, 2, (96, 384), (2, 4), False),                   # grouped KV heads, first r > 1
]


@pytest.mark.parametrize("n,d,hq,hkv,ws,rs,causal", HEAD_SHIFT_CASES)
def test_dilated_head_shift_small(n, d, hq, hkv, ws, rs, causal):
    q, k, v, do = draw([(1, hq, n, d), (1, hkv, n, d), (1, hkv, n, d), (1, hq, n, d)],
                       560 + n + d)
    q32, k32, v32, do32 = (_np32(t) for t in (q, k, v, do))
    o_ref, l_ref = oracle.dilated_fwd(q32, k32, v32, ws, rs, causal=causal, head_shift=True)
    ref = oracle.dilated_bwd(q32, k32, v32, do32, ws, rs, causal=causal, head_shift=True)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = sa.dilated_attn_fwd(qd, kd, vd, ws, rs, causal=causal, head_shift=True)
    ob, lb = sa.dilated_attn_fwd(qd, kd, vd, ws, rs, causal=causal, head_shift=True,
                                 out_dtype=torch.bfloat16)
    grads = sa.dilated_attn_bwd(qd, kd, vd, o, lse, dod, ws, rs, causal=causal,
                                head_shift=True)
    torch.cuda.synchronize()
    assert_parity(to_np(o), to_np(lse), o_ref, l_ref, torch.bfloat16, what="head shift f32 out")
    assert_parity(to_np(ob), to_np(lb), o_ref, l_ref, torch.bfloat16, what="head shift bf16 out")
    _grads_parity(grads, ref, "head shift bwd")


def test_longnet_32k_full_size_full_oracle():
    """16 heads, d=64, 32768 tokens, w = 2048..32768, r = 1..16, non-causal,
    in bf16 and fp32 output: every row of every head against the full
    forward oracle (0.53 TFLOP fp64: about 14 s on 16 host cores).  Outputs
    start as NaN, so a row no branch writes fails."""
    w = WORKLOADS["longnet_32k_bf16"]
    q, k, v = workload_inputs(w)
    o_ref, l_ref = oracle.dilated_fwd(_np32(q), _np32(k), _np32(v), w.segment_lengths,
                                      w.dilations)
    for dt in (torch.bfloat16, torch.float32):
        out = torch.full(q.shape, float("nan"), dtype=dt, device=DEV)
        lse = torch.full(q.shape[:-1], float("nan"), dtype=torch.float32, device=DEV)
        sa.dilated_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), w.segment_lengths,
                            w.dilations, out=out, lse=lse)
        torch.cuda.synchronize()
        assert_parity(to_np(out), to_np(lse), o_ref, l_ref, torch.bfloat16,
                      what=f"longnet 32k ({dt} out)")


@pytest.mark.parametrize("n,d,hq,hkv,ws,rs,causal", DILATED_CASES)
def test_dilated_bwd_small(n, d, hq, hkv, ws, rs, causal):
    q, k, v, do = draw([(1, hq, n, d), (1, hkv, n, d), (1, hkv, n, d), (1, hq, n, d)],
                       700 + n + d)
    ref = oracle.dilated_bwd(_np32(q), _np32(k), _np32(v), _np32(do), ws, rs, causal=causal)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = sa.dilated_attn_fwd(qd, kd, vd, ws, rs, causal=causal)
    grads = sa.dilated_attn_bwd(qd, kd, vd, o, lse, dod, ws, rs, causal=causal)
    torch.cuda.synchronize()
    _grads_parity(grads, ref, "dilated bwd")
    # bf16 O from the forward, dq accumulated onto a non-zero start
    ob, lb = sa.dilated_attn_fwd(qd, kd, vd, ws, rs, causal=causal, out_dtype=torch.bfloat16)
    dq0 = torch.randn(q.shape, generator=torch.Generator().manual_seed(9), dtype=torch.float32)
    dq = dq0.to(DEV)
    dk = torch.full(k.shape, 7.0, dtype=torch.float32, device=DEV)  # overwritten
    dv = torch.full(v.shape, 7.0, dtype=torch.float32, device=DEV)
    sa.dilated_attn_bwd(qd, kd, vd, ob, lb, dod, ws, rs, causal=causal, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    _grads_parity((dq.cpu() - dq0, dk, dv), ref, "dilated bwd (bf16 O, dq accumulated)")


def test_dilated_bwd_is_deterministic():
    n, d, hq, hkv, ws, rs = 1024, 128, 4, 2, (256, 1024), (1, 4)
    q, k, v, do = (t.to(DEV) for t in draw([(1, hq, n, d), (1, hkv, n, d), (1, hkv, n, d),
                                             (1, hq, n, d)], 780))
    o, lse = sa.dilated_attn_fwd(q, k, v, ws, rs)
    a = sa.dilated_attn_bwd(q, k, v, o, lse, do, ws, rs)
    b = sa.dilated_attn_bwd(q, k, v, o, lse, do, ws, rs)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_longnet_32k_bwd_full_size_sampled_and_invariants():
    """Full LongNet workload (16 heads, d=64, 32768 tokens, 5 branches): dQ on
    seeded rows against the oracle's backward over each row's listed keys
    (a key listed by m branches counts m times in the merged softmax); dK
    and dV over all keys through sum_j dV_j = sum_i dO_i and sum_j dK_j = 0
    per head."""
    w = WORKLOADS["longnet_32k_bf16"]
    q, k, v, do = workload_inputs(w, with_dout=True)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = sa.dilated_attn_fwd(qd, kd, vd, w.segment_lengths, w.dilations)
    dq, dk, dv = sa.dilated_attn_bwd(qd, kd, vd, o, lse, dod, w.segment_lengths, w.dilations)
    torch.cuda.synchronize()
    q32, k32, v32, do32 = (_np32(t)[0] for t in (q, k, v, do))
    dq_np = to_np(dq)[0]
    errs = []
    for h in (0, 5, 15):
        must = (0, 16, 2048, 4096 + 8, w.nq - 1, w.nq - 16)
        for i in sample_rows(w.nq, 6, 5000 + h, must=must):
            keys = dilated_key_list(i, w.nq, w.segment_lengths, w.dilations, False)
            g = h * w.hkv // w.hq
            ref, _, _ = oracle.attn_bwd_dq_rows(q32[h:h + 1, i:i + 1], k32[g:g + 1, keys],
                                                v32[g:g + 1, keys], do32[h:h + 1, i:i + 1])
            errs.append(np.linalg.norm(dq_np[h, i] - ref[0]) /
                        max(np.linalg.norm(ref[0]), 1e-30))
    assert max(errs) <= BTOL, f"dq sampled rows: max rowwise error {max(errs):.3e}"
    do64 = do.double()[0]
    group = w.hq // w.hkv
    for g in range(w.hkv):
        sdv = dv[0, g].double().sum(0).cpu()
        sdo = do64[g * group:(g + 1) * group].sum(dim=(0, 1))
        assert (sdv - sdo).abs().max() <= BTOL * sdo.abs().max()
        sdk = dk[0, g].double().sum(0).cpu()
        mag = dk[0, g].double().abs().sum(0).cpu().max()
        assert sdk.abs().max() <= 1e-3 * mag


SPLIT_CASES = [
    # (n, P, hq, hkv, d, ws, rs, causal)
    (768, 4, 2, 2, 64, (48, 96, 384, 768), (1, 2, 6, 12), True),
    (768, 4, 4, 2, 128, (48, 96, 384, 768), (1, 2, 6, 12), False),
    (1152, 3, 2, 1, 64, (128, 384, 768), (1, 4, 6), True),     # tail segment
]


@pytest.mark.parametrize("n,P,hq,hkv,d,ws,rs,causal", SPLIT_CASES)
def test_longnet_split_matches_oracle_small(n, P, hq, hkv, d, ws, rs, causal):
    q, k, v, do = draw([(1, hq, n, d), (1, hkv, n, d), (1, hkv, n, d), (1, hq, n, d)],
                       900 + n + d)
    o_ref, l_ref = oracle.dilated_fwd(_np32(q), _np32(k), _np32(v), ws, rs, causal=causal)
    ref = oracle.dilated_bwd(_np32(q), _np32(k), _np32(v), _np32(do), ws, rs, causal=causal)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = emulate.longnet_split_fwd(qd, kd, vd, ws, rs, P, causal=causal)
    grads = emulate.longnet_split_bwd(qd, kd, vd, o, lse, dod, ws, rs, P, causal=causal)
    torch.cuda.synchronize()
    assert_parity(to_np(o), to_np(lse), o_ref, l_ref, torch.bfloat16, what="longnet split fwd")
    _grads_parity(grads, ref, "longnet split bwd")


def test_longnet_page_config_full_size():
    """LongNet's own mixture (w = 2048..32768, r = 1,2,4,6,12), causal, 16
    heads, d=64, 32768 tokens: the single-GPU path and the 4-device split.
    Forward: every row against the full oracle (about 8 s on 16 host
    cores).  Backward: dQ on seeded rows against the oracle (the full
    dilated backward oracle takes many minutes), dK/dV through the sum
    identities."""
    w = WORKLOADS["longnet_page_32k_bf16"]
    ws, rs, P = w.segment_lengths, w.dilations, w.segments
    q, k, v, do = workload_inputs(w, with_dout=True)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o1, l1 = sa.dilated_attn_fwd(qd, kd, vd, ws, rs, causal=True)
    g1 = sa.dilated_attn_bwd(qd, kd, vd, o1, l1, dod, ws, rs, causal=True)
    o2, l2 = emulate.longnet_split_fwd(qd, kd, vd, ws, rs, P, causal=True)
    g2 = emulate.longnet_split_bwd(qd, kd, vd, o2, l2, dod, ws, rs, P, causal=True)
    torch.cuda.synchronize()
    rows = []
    for h in (0, 7, 15):
        must = (0, 11, 12, 8191, 8196, 16392, 24576, w.nq - 1)
        for i in sample_rows(w.nq, 16, 6000 + h, must=must):
            rows.append(h * w.nq + i)
    rows = np.array(rows, np.int64)
    o_ref, l_ref = oracle.dilated_fwd(_np32(q), _np32(k), _np32(v), ws, rs, causal=True)
    q32, k32, v32, do32 = (_np32(t)[0] for t in (q, k, v, do))
    dq_ref = []
    for row in rows:
        h, i = divmod(int(row), w.nq)
        keys = dilated_key_list(i, w.nq, ws, rs, True)
        r_, _, _ = oracle.attn_bwd_dq_rows(q32[h:h + 1, i:i + 1], k32[h:h + 1, keys],
                                           v32[h:h + 1, keys], do32[h:h + 1, i:i + 1])
        dq_ref.append(r_[0])
    dq_ref = np.array(dq_ref)
    do64 = do.double()[0]
    for what, o, lse, (dq, dk, dv) in (("single GPU", o1, l1, g1), ("split", o2, l2, g2)):
        assert_parity(to_np(o), to_np(lse), o_ref, l_ref, torch.bfloat16,
                      what=f"longnet page {what}")
        check_close(to_np(dq).reshape(-1, w.d)[rows], dq_ref, BTOL, rows // w.nq, what, "dq")
        for g in range(w.hkv):
            sdv = dv[0, g].double().sum(0).cpu()
            sdo = do64[g].sum(0)
            assert (sdv - sdo).abs().max() <= BTOL * sdo.abs().max(), what
            sdk = dk[0, g].double().sum(0).cpu()
            assert sdk.abs().max() <= 1e-3 * dk[0, g].double().abs().sum(0).cpu().max(), what


def test_longnet_page_config_head_shift_full_size():
    """LongNet's mixture (w = 2048..32768, r = 1,2,4,6,12), causal, 16 heads,
    d=64, 32768 tokens, with head h at offset h mod r_i: every forward row
    against the full oracle (output NaN-filled first), dQ rows against the
    oracle, dK/dV through the sum identities (the r = 1 branch selects every
    query)."""
    w = WORKLOADS["longnet_page_32k_bf16"]
    ws, rs = w.segment_lengths, w.dilations
    q, k, v, do = workload_inputs(w, with_dout=True)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full(q.shape[:-1], float("nan"), dtype=torch.float32, device=DEV)
    sa.dilated_attn_fwd(qd, kd, vd, ws, rs, causal=True, head_shift=True, out=o, lse=lse)
    dq, dk, dv = sa.dilated_attn_bwd(qd, kd, vd, o, lse, dod, ws, rs, causal=True,
                                     head_shift=True)
    torch.cuda.synchronize()
    rows = []
    for h in (0, 5, 11, 15):
        must = (0, 5, 11, 12, 2048 + h % 12, 8191, 16392 + h % 4, w.nq - 1)
        for i in sample_rows(w.nq, 12, 6100 + h, must=must):
            rows.append(h * w.nq + i)
    rows = np.array(rows, np.int64)
    o_ref, l_ref = oracle.dilated_fwd(_np32(q), _np32(k), _np32(v), ws, rs, causal=True,
                                      head_shift=True)
    assert_parity(to_np(o), to_np(lse), o_ref, l_ref, torch.bfloat16,
                  what="longnet page head shift")
    q32, k32, v32, do32 = (_np32(t)[0] for t in (q, k, v, do))
    dq_ref = []
    for row in rows:
        h, i = divmod(int(row), w.nq)
        keys = dilated_key_list(i, w.nq, ws, rs, True, shift=h)
        r_, _, _ = oracle.attn_bwd_dq_rows(q32[h:h + 1, i:i + 1], k32[h:h + 1, keys],
                                           v32[h:h + 1, keys], do32[h:h + 1, i:i + 1])
        dq_ref.append(r_[0])
    check_close(to_np(dq).reshape(-1, w.d)[rows], np.array(dq_ref), BTOL, rows // w.nq,
                "head shift", "dq")
    do64 = do.double()[0]
    for g in range(w.hkv):
        sdv = dv[0, g].double().sum(0).cpu()
        sdo = do64[g].sum(0)
        assert (sdv - sdo).abs().max() <= BTOL * sdo.abs().max()
        sdk = dk[0, g].double().sum(0).cpu()
        assert sdk.abs().max() <= 1e-3 * dk[0, g].double().abs().sum(0).cpu().max()
