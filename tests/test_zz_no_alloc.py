"""The backward entry point that allocates nothing, through the C ABI, against
the workspace entry point on the same inputs (and both against the oracle):
two calls in a row, the second with a smaller input, so the scratch array
holding the first call's D values must not leak into the second."""
import pytest
import torch

import oracle
import long_sequence_exact_amd as sa
from long_sequence_exact_amd.synth import draw
from tests.parity import TOL, check_close

pytestmark = pytest.mark.gpu
DEV = "cuda"
BTOL = TOL[torch.bfloat16]

CALLS = [
    # (B, Hq, Hkv, Nq, Nk, d, delta, accumulate_kv)
    (2, 8, 2, 700, 900, 128, 300, False),
    (1, 4, 2, 190, 333, 64, None, True),
]


def _np32(t):
    return t.float().cpu().numpy()


def test_noalloc_backward_matches_workspace_backward():
    for i, (B, hq, hkv, nq, nk, d, delta, acc) in enumerate(CALLS):
        print(f"noalloc call {i}: B={B} hq={hq} hkv={hkv} nq={nq} nk={nk} d={d} "
              f"delta={delta} accumulate_kv={acc}", flush=True)
        q, k, v, do = draw([(B, hq, nq, d), (B, hkv, nk, d), (B, hkv, nk, d), (B, hq, nq, d)],
                           4700 + i)
        qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
        o, lse = sa.attn_segment_fwd(qd, kd, vd, causal_offset=delta, out_dtype=torch.float32)
        dq0 = torch.randn(q.shape, generator=torch.Generator().manual_seed(i),
                          dtype=torch.float32).to(DEV)
        kv0 = torch.randn(k.shape, generator=torch.Generator().manual_seed(10 + i),
                          dtype=torch.float32).to(DEV)
        outs = []
        for noalloc in (False, True):
            dq = dq0.clone()
            dk = kv0.clone()
            dv = kv0.clone()
            if noalloc:
                sa.attn_segment_bwd_noalloc(qd, kd, vd, o, lse, dod, dq, dk, dv,
                                            causal_offset=delta, accumulate_kv=acc)
            else:
                sa.attn_segment_bwd(qd, kd, vd, o, lse, dod, causal_offset=delta, dq=dq, dk=dk,
                                    dv=dv, accumulate_kv=acc)
            torch.cuda.synchronize()
            outs.append((dq, dk, dv))
        for a, b, name in zip(outs[0], outs[1], ("dq", "dk", "dv")):
            assert torch.equal(a, b), f"call {i}: {name} differs from the workspace entry point"
        dl = oracle.NONCAUSAL if delta is None else delta
        ref = oracle.attn_bwd(_np32(q), _np32(k), _np32(v), _np32(do), delta=dl)
        dq, dk, dv = outs[1]
        got = (dq - dq0, dk - kv0 if acc else dk, dv - kv0 if acc else dv)
        for name, x, r in zip(("dq", "dk", "dv"), got, ref):
            check_close(x, r, BTOL, what=f"noalloc call {i}", name=name)
