"""GPU parity of LongNet dilated attention against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import long_sequence_exact_amd as sa
from long_sequence_exact_amd.synth import WORKLOADS, draw, sample_rows, workload_inputs
from tests.parity import assert_parity, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _np32(t):
    return t.float().numpy()


@pytest.mark.parametrize("n,d,hq,hkv,ws,rs,causal", [
    (512, 64, 2, 2, (64, 128, 256, 512), (1, 2, 4, 8), False),
    (512, 128, 4, 2, (64, 128, 256, 512), (1, 2, 4, 8), True),
    (600, 64, 2, 1, (64, 128, 256), (1, 2, 4), False),          # segment tails
    (640, 64, 1, 1, (8 * 10, 16 * 10, 32 * 10, 64 * 10), (1, 2, 6, 12), False),  # r not 2^k
    (384, 64, 2, 2, (96, 384), (2, 4), False),                  # first branch r > 1
    (300, 128, 2, 2, (1000,), (3,), True),                      # w > N
])
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


def test_longnet_32k_full_size_sampled():
    """16 heads, d=64, 32768 tokens, w = 2048..32768, r = 1..16, non-causal."""
    w = WORKLOADS["longnet_32k_bf16"]
    q, k, v = workload_inputs(w)
    o, lse = sa.dilated_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), w.segment_lengths,
                                 w.dilations)
    torch.cuda.synchronize()
    rows = []
    for h in range(w.hq):
        # positions selected by 1..5 branches, plus random ones
        must = (0, 16, 2048, 4096 + 8, w.nq - 1, w.nq - 16)
        for i in sample_rows(w.nq, 40, 3000 + h, must=must):
            rows.append(h * w.nq + i)
    rows = np.array(rows, np.int64)
    o_ref, l_ref = oracle.dilated_fwd(_np32(q), _np32(k), _np32(v), w.segment_lengths,
                                      w.dilations, rows=rows)
    og = to_np(o).reshape(-1, w.d)[rows]
    lg = to_np(lse).reshape(-1)[rows]
    assert_parity(og, lg, o_ref, l_ref, torch.bfloat16, rows_heads=rows // w.nq,
                  what="longnet 32k")
