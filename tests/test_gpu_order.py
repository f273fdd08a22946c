"""Launches with many (batch, head) groups of few query or key tiles take the
XCD-grouped work order, including group counts that are not a multiple of 8
(the launch then holds empty padding items).  Outputs start as NaN, so a row
that no workgroup writes fails; every row must match the fp64 oracle."""
import pytest
import torch

import oracle
import long_sequence_exact_amd as sa
from long_sequence_exact_amd.synth import draw
from tests.parity import TOL, assert_parity, check_close, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"

ORDER_CASES = [
    # (B, Hq, Hkv, Nq, Nk, d, delta)
    (1, 8, 8, 300, 300, 128, 0),        # 8 groups of 2 query tiles
    (3, 3, 3, 257, 400, 64, None),      # 9 groups
    (1, 13, 13, 520, 520, 64, 20),      # 13 groups, 3 query tiles
    (2, 10, 5, 200, 700, 128, 500),     # 20 query / 10 KV groups, GQA
    (1, 33, 11, 100, 300, 64, -40),     # 33 query / 11 KV groups
    (1, 8, 8, 9216, 100, 64, None),     # 36 query tiles: grouped only at d = 64 (bands of 64)
    (1, 8, 4, 9216, 100, 64, 9000),     # the same, causal, GQA
]


def _np32(t):
    return t.float().numpy()


@pytest.mark.parametrize("b,hq,hkv,nq,nk,d,delta", ORDER_CASES)
def test_grouped_order_fwd_bwd(b, hq, hkv, nq, nk, d, delta):
    q, k, v, do = draw([(b, hq, nq, d), (b, hkv, nk, d), (b, hkv, nk, d), (b, hq, nq, d)],
                       9100 + b * hq + nq)
    dl = oracle.NONCAUSAL if delta is None else delta
    o_ref, l_ref = oracle.attn_fwd(_np32(q), _np32(k), _np32(v), delta=dl)
    g_ref = oracle.attn_bwd(_np32(q), _np32(k), _np32(v), _np32(do), delta=dl)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full(q.shape[:-1], float("nan"), dtype=torch.float32, device=DEV)
    sa.attn_segment_fwd(qd, kd, vd, causal_offset=delta, out=o, lse=lse)
    dk = torch.full(k.shape, float("nan"), dtype=torch.float32, device=DEV)
    dv = torch.full(v.shape, float("nan"), dtype=torch.float32, device=DEV)
    dq, dk, dv = sa.attn_segment_bwd(qd, kd, vd, o, lse, dod, causal_offset=delta, dk=dk, dv=dv)
    torch.cuda.synchronize()
    what = f"B={b} Hq={hq} Hkv={hkv} {nq}x{nk} d={d} delta={delta}"
    assert not torch.isnan(o).any() and not torch.isnan(lse).any(), f"{what}: unwritten rows"
    assert_parity(to_np(o), to_np(lse), o_ref, l_ref, torch.bfloat16, what=what)
    for name, x, r in zip(("dq", "dk", "dv"), (dq, dk, dv), g_ref):
        assert not torch.isnan(x).any(), f"{what}: unwritten rows in {name}"
        check_close(x, r, TOL[torch.bfloat16], what=f"{what}", name=name)
