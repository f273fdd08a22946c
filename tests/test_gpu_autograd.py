"""GPU parity of the autograd functions (forward and backward through the
library's kernels) against the fp64 oracle, and against direct calls."""
import pytest
import torch

import oracle
import long_sequence_exact_amd as sa
from long_sequence_exact_amd.autograd import dilated_attention, segment_attention
from long_sequence_exact_amd.synth import draw
from tests.parity import TOL, check_close

pytestmark = pytest.mark.gpu
DEV = "cuda"
BTOL = TOL[torch.bfloat16]


def _np32(t):
    return t.float().numpy()


@pytest.mark.parametrize("hq,hkv,nq,nk,d,delta", [
    (4, 2, 300, 520, 128, 250),
    (2, 2, 200, 333, 64, None),
])
def test_segment_attention_backward(hq, hkv, nq, nk, d, delta):
    """loss = sum(o * w): the gradients autograd returns match the oracle's
    (with dO = w rounded to bf16, as the bf16 output passes it back) and are
    bit-identical to attn_segment_fwd followed by attn_segment_bwd."""
    q, k, v, w = draw([(1, hq, nq, d), (1, hkv, nk, d), (1, hkv, nk, d), (1, hq, nq, d)], 31 + d)
    qd, kd, vd = (t.to(DEV).requires_grad_() for t in (q, k, v))
    wd = w.to(DEV)
    o = segment_attention(qd, kd, vd, causal_offset=delta)
    assert o.dtype == torch.bfloat16
    (o.float() * wd.float()).sum().backward()
    torch.cuda.synchronize()
    ref = oracle.attn_bwd(_np32(q), _np32(k), _np32(v), _np32(w),
                          delta=oracle.NONCAUSAL if delta is None else delta)
    for name, x, r in zip(("dq", "dk", "dv"), (qd.grad, kd.grad, vd.grad), ref):
        assert x.dtype == torch.bfloat16
        check_close(x, r, BTOL, what=f"autograd segment {hq}/{hkv} {nq}x{nk}", name=name)
    # the same kernels called directly
    q2, k2, v2 = q.to(DEV), k.to(DEV), v.to(DEV)
    o2, lse2 = sa.attn_segment_fwd(q2, k2, v2, causal_offset=delta)
    g2 = sa.attn_segment_bwd(q2, k2, v2, o2, lse2, wd, causal_offset=delta)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2)
    for x, y in zip((qd.grad, kd.grad, vd.grad), g2):
        assert torch.equal(x, y.to(torch.bfloat16))


@pytest.mark.parametrize("head_shift", [False, True])
def test_dilated_attention_backward(head_shift):
    """The same for dilated attention (causal, three branches, grouped KV
    heads, with and without head-dependent offsets); its output is the fp32
    merge accumulator, so dO = w in fp32 is rounded to bf16 on the way into
    the backward."""
    hq, hkv, n, d = 4, 2, 700, 64
    ws, rs = (128, 256, 512), (1, 2, 4)
    q, k, v, w = draw([(1, hq, n, d), (1, hkv, n, d), (1, hkv, n, d), (1, hq, n, d)], 41)
    qd, kd, vd = (t.to(DEV).requires_grad_() for t in (q, k, v))
    wd = w.to(DEV)
    o = dilated_attention(qd, kd, vd, ws, rs, causal=True, head_shift=head_shift)
    assert o.dtype == torch.float32
    (o * wd.float()).sum().backward()
    torch.cuda.synchronize()
    o_ref, _ = oracle.dilated_fwd(_np32(q), _np32(k), _np32(v), ws, rs, causal=True,
                                  head_shift=head_shift)
    check_close(o.detach(), o_ref, BTOL, what="autograd dilated", name="o")
    ref = oracle.dilated_bwd(_np32(q), _np32(k), _np32(v), _np32(w), ws, rs, causal=True,
                             head_shift=head_shift)
    for name, x, r in zip(("dq", "dk", "dv"), (qd.grad, kd.grad, vd.grad), ref):
        check_close(x, r, BTOL, what="autograd dilated", name=name)
