"""GPU parity of the segment backward (dQ, dK, dV) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import long_sequence_exact_amd as sa
from long_sequence_exact_amd import emulate
from long_sequence_exact_amd.synth import WORKLOADS, draw, sample_rows, workload_inputs
from tests.parity import LSE_TOL, TOL, check_close, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
BTOL = TOL[torch.bfloat16]


def _np32(t):
    return t.float().numpy()


def _grads_parity(dq, dk, dv, ref, what):
    for name, x, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        check_close(x, r, BTOL, what=what, name=name)


BWD_CASES = [
    # (Hq, Hkv, Nq, Nk, d, delta)
    (2, 2, 200, 333, 128, None),
    (4, 1, 257, 513, 128, 100),
    (8, 2, 130, 300, 128, 200),
    (2, 2, 256, 256, 128, -50),      # leading rows see no key
    (2, 2, 300, 300, 64, 0),
    (4, 2, 100, 1000, 64, 700),
    (2, 1, 1, 1, 128, 0),
]


@pytest.mark.parametrize("hq,hkv,nq,nk,d,delta", BWD_CASES)
@pytest.mark.parametrize("grad_dtype", [torch.float32, torch.bfloat16])
def test_segment_bwd_small(hq, hkv, nq, nk, d, delta, grad_dtype):
    q, k, v, do = draw([(1, hq, nq, d), (1, hkv, nk, d), (1, hkv, nk, d), (1, hq, nq, d)],
                       2000 + nq + nk)
    dl = oracle.NONCAUSAL if delta is None else delta
    ref = oracle.attn_bwd(_np32(q), _np32(k), _np32(v), _np32(do), delta=dl)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = sa.attn_segment_fwd(qd, kd, vd, causal_offset=delta, out_dtype=torch.float32)
    dq, dk, dv = sa.attn_segment_bwd(qd, kd, vd, o, lse, dod, causal_offset=delta,
                                     grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    assert dk.dtype == grad_dtype and dq.dtype == torch.float32
    _grads_parity(dq, dk, dv, ref, f"bwd {grad_dtype}")


def test_bwd_bf16_output_o():
    hq, hkv, nq, nk, d = 4, 2, 192, 256, 128
    q, k, v, do = draw([(1, hq, nq, d), (1, hkv, nk, d), (1, hkv, nk, d), (1, hq, nq, d)], 2100)
    ref = oracle.attn_bwd(_np32(q), _np32(k), _np32(v), _np32(do), delta=64)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = sa.attn_segment_fwd(qd, kd, vd, causal_offset=64)  # bf16 O
    dq, dk, dv = sa.attn_segment_bwd(qd, kd, vd, o, lse, dod, causal_offset=64)
    torch.cuda.synchronize()
    _grads_parity(dq, dk, dv, ref, "bwd with bf16 O")


def test_bwd_sweep_accumulates_dq_over_segments():
    """Two KV segments with the merged O/LSE: dQ sums over both calls, each
    call writes its own segment's dK/dV; together they equal the full
    backward."""
    hq, hkv, nq, nk, d, delta = 4, 2, 160, 384, 128, 224
    q, k, v, do = draw([(2, hq, nq, d), (2, hkv, nk, d), (2, hkv, nk, d), (2, hq, nq, d)], 2200)
    ref = oracle.attn_bwd(_np32(q), _np32(k), _np32(v), _np32(do), delta=delta)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = sa.attn_segment_fwd(qd, kd, vd, causal_offset=delta, out_dtype=torch.float32)
    dq = torch.zeros(q.shape, dtype=torch.float32, device=DEV)
    dk = torch.empty(k.shape, dtype=torch.float32, device=DEV)
    dv = torch.empty(v.shape, dtype=torch.float32, device=DEV)
    cut = 128
    sa.attn_segment_bwd(qd, kd[..., :cut, :], vd[..., :cut, :], o, lse, dod,
                        causal_offset=delta, dq=dq, dk=dk[..., :cut, :], dv=dv[..., :cut, :])
    sa.attn_segment_bwd(qd, kd[..., cut:, :], vd[..., cut:, :], o, lse, dod,
                        causal_offset=delta - cut, dq=dq, dk=dk[..., cut:, :],
                        dv=dv[..., cut:, :])
    torch.cuda.synchronize()
    _grads_parity(dq, dk, dv, ref, "bwd sweep")


def test_usp_scaled_replica_full_oracle():
    """The USP share at 1/64 scale (GQA 8/2, d=128, query block 7 of 8 KV
    blocks of 512): forward + backward sweeps against the full oracle."""
    hq, hkv, blk, nb, d, qb = 8, 2, 512, 8, 128, 7
    q, k, v, do = draw([(1, hq, blk, d), (1, hkv, nb * blk, d), (1, hkv, nb * blk, d),
                        (1, hq, blk, d)], 2300)
    delta = qb * blk
    o_ref, l_ref = oracle.attn_fwd(_np32(q), _np32(k), _np32(v), delta=delta)
    ref = oracle.attn_bwd(_np32(q), _np32(k), _np32(v), _np32(do), delta=delta)
    o, lse, dq, dk, dv = emulate.usp_fwd_bwd(*(t.to(DEV) for t in (q, k, v, do)), nb, qb)
    torch.cuda.synchronize()
    check_close(o, o_ref, BTOL, what="usp replica", name="o")
    _grads_parity(dq, dk, dv, ref, "usp replica")


def test_usp_full_size_sampled_and_invariants():
    """Full USP share: Q block 7 (32768 rows), GQA 8/2, 8 KV blocks of 32768.
    dQ (and O, LSE) on 2 heads x 512 seeded rows against the oracle; dK and
    dV over all 262144 keys through the identities sum_j dV_j = sum_i dO_i
    and sum_j dK_j = 0 per KV head."""
    w = WORKLOADS["usp_gqa_256k_bf16"]
    q, k, v, do = workload_inputs(w, with_dout=True)
    o, lse, dq, dk, dv = emulate.usp_fwd_bwd(*(t.to(DEV) for t in (q, k, v, do)),
                                             w.segments, w.q_block)
    torch.cuda.synchronize()
    blk = w.nk // w.segments
    rows = []
    for h in (1, 6):
        for i in sample_rows(w.nq, 512, 4000 + h, must=(0, w.nq - 1)):
            rows.append(h * w.nq + i)
    rows = np.array(rows, np.int64)
    dq_ref, o_ref, l_ref = oracle.attn_bwd_dq_rows(_np32(q), _np32(k), _np32(v), _np32(do),
                                                   delta=w.q_block * blk, rows=rows)
    heads = rows // w.nq
    dq_g = to_np(dq).reshape(-1, w.d)[rows]
    check_close(dq_g, dq_ref, BTOL, heads, "usp full size", "dq")
    check_close(to_np(o).reshape(-1, w.d)[rows], o_ref, BTOL, heads, "usp full size", "o")
    assert np.abs(to_np(lse).reshape(-1)[rows] - l_ref).max() <= LSE_TOL
    group = w.hq // w.hkv
    do64 = do.double()[0]
    for g in range(w.hkv):
        sdv = dv[0, g].double().sum(0).cpu()
        sdo = do64[g * group:(g + 1) * group].sum(dim=(0, 1))
        assert (sdv - sdo).abs().max() <= BTOL * sdo.abs().max()
        sdk = dk[0, g].double().sum(0).cpu()
        mag = dk[0, g].double().abs().sum(0).cpu().max()
        assert sdk.abs().max() <= 1e-3 * mag


def test_bwd_accumulate_kv_over_query_blocks():
    """Two query blocks against one KV segment (the ring backward, where a KV
    block's gradient collects every query block's share): the second call
    adds to dK/dV (SEQATTN_ACCUMULATE); together they equal the full backward."""
    hq, hkv, nq, nk, d = 4, 2, 320, 256, 128
    q, k, v, do = draw([(1, hq, nq, d), (1, hkv, nk, d), (1, hkv, nk, d), (1, hq, nq, d)], 2300)
    ref = oracle.attn_bwd(_np32(q), _np32(k), _np32(v), _np32(do), delta=0)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = sa.attn_segment_fwd(qd, kd, vd, causal_offset=0, out_dtype=torch.float32)
    dq = torch.zeros(q.shape, dtype=torch.float32, device=DEV)
    dk = torch.full(k.shape, 5.0, dtype=torch.float32, device=DEV)
    dv = torch.full(v.shape, 5.0, dtype=torch.float32, device=DEV)
    cut = 96
    sa.attn_segment_bwd(qd[..., :cut, :], kd, vd, o[..., :cut, :], lse[..., :cut],
                        dod[..., :cut, :], causal_offset=0, dq=dq[..., :cut, :], dk=dk, dv=dv)
    sa.attn_segment_bwd(qd[..., cut:, :], kd, vd, o[..., cut:, :], lse[..., cut:],
                        dod[..., cut:, :], causal_offset=cut, dq=dq[..., cut:, :], dk=dk, dv=dv,
                        accumulate_kv=True)
    torch.cuda.synchronize()
    _grads_parity(dq, dk, dv, ref, "bwd accumulate_kv")


def test_bwd_sequence_major_layout_views():
    """Backward on [B, N, H, d]-stored tensors passed as permuted views."""
    B, N, H, Hkv, d, delta = 1, 300, 4, 2, 128, 0
    qs, ks, vs, dos = draw([(B, N, H, d), (B, N, Hkv, d), (B, N, Hkv, d), (B, N, H, d)], 2400)
    q, k, v, do = (t.permute(0, 2, 1, 3) for t in (qs, ks, vs, dos))
    ref = oracle.attn_bwd(*(t.contiguous().float().numpy() for t in (q, k, v, do)), delta=delta)
    qd, kd, vd, dod = (t.to(DEV).permute(0, 2, 1, 3) for t in (qs, ks, vs, dos))
    o, lse = sa.attn_segment_fwd(qd, kd, vd, causal_offset=delta, out_dtype=torch.float32)
    dq = torch.zeros((B, N, H, d), dtype=torch.float32, device=DEV).permute(0, 2, 1, 3)
    dk = torch.empty((B, N, Hkv, d), dtype=torch.float32, device=DEV).permute(0, 2, 1, 3)
    dv = torch.empty((B, N, Hkv, d), dtype=torch.float32, device=DEV).permute(0, 2, 1, 3)
    sa.attn_segment_bwd(qd, kd, vd, o, lse, dod, causal_offset=delta, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    _grads_parity(dq, dk, dv, ref, "bwd seq-major")


def test_bwd_empty_and_fully_masked_segments():
    """A KV segment entirely in the queries' causal future contributes nothing:
    dq unchanged, dk = dv = 0; an empty query block gives dk = dv = 0."""
    q, k, v, do = (t.to(DEV) for t in draw([(1, 2, 128, 128), (1, 1, 256, 128),
                                             (1, 1, 256, 128), (1, 2, 128, 128)], 2500))
    o, lse = sa.attn_segment_fwd(q, k, v, causal_offset=0, out_dtype=torch.float32)
    dq0 = torch.randn(q.shape, device=DEV)
    dq = dq0.clone()
    _, dk, dv = sa.attn_segment_bwd(q, k, v, o, lse, do, causal_offset=-1000, dq=dq)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq0)
    assert torch.all(dk == 0) and torch.all(dv == 0)
    qz = q[..., :0, :]
    _, dk2, dv2 = sa.attn_segment_bwd(qz, k, v, o[..., :0, :], lse[..., :0], do[..., :0, :])
    torch.cuda.synchronize()
    assert torch.all(dk2 == 0) and torch.all(dv2 == 0)


def test_largest_query_extent():
    """One query head whose Q, dO (and fp32 O, dQ rows) span the largest extent
    the library accepts (8,388,088 rows of d = 128, just under 2 GiB of bf16
    per head, addressed with 32-bit byte offsets) against 200 keys,
    non-causal: dQ on sampled rows, including the last, against the oracle;
    dK and dV through sum_j dV_j = sum_i dO_i and sum_j dK_j = 0."""
    d = 128
    nq = (1 << 31) // (2 * d) - 512 - 8
    nk = 200
    q, k, v, do = draw([(1, 1, nq, d), (1, 1, nk, d), (1, 1, nk, d), (1, 1, nq, d)], 2600)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = sa.attn_segment_fwd(qd, kd, vd, out_dtype=torch.float32)
    dq, dk, dv = sa.attn_segment_bwd(qd, kd, vd, o, lse, dod)
    torch.cuda.synchronize()
    rows = np.array(sample_rows(nq, 4, 2601, must=(0, nq - 1)), np.int64)
    ref, _, _ = oracle.attn_bwd_dq_rows(_np32(q), _np32(k), _np32(v), _np32(do), rows=rows)
    check_close(to_np(dq[0, 0, torch.from_numpy(rows).to(DEV)]), ref, BTOL,
                np.zeros(len(rows), np.int64), "largest query extent", "dq")
    sdo = do[0, 0].double().sum(0)
    assert (dv[0, 0].double().sum(0).cpu() - sdo).abs().max() <= BTOL * sdo.abs().max()
    mag = dk[0, 0].double().abs().sum(0).cpu().max()
    assert dk[0, 0].double().sum(0).abs().max().cpu() <= 1e-3 * mag
