"""GPU tests of the head re-layout copy and of the Ulysses pipeline built on it."""
import numpy as np
import pytest
import torch

import oracle
import long_sequence_exact_amd as sa
from long_sequence_exact_amd import emulate
from long_sequence_exact_amd.synth import draw, sample_rows
from tests.parity import assert_parity, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _views(buf, shape, strides):
    return buf.as_strided(shape, strides, buf.storage_offset())


# (src buffer shape, src view shape, src strides, dst buffer shape, dst view shape,
#  dst strides) with the view shapes' b*h equal
def _cases():
    P, ns, H, d = 4, 48, 8, 128
    hp = H // P
    yield ("ulysses pack", (P * ns, H, d), (1, H, ns, d), (0, d, H * d, 1),
           (P, ns, hp, d), (P, hp, ns, d), (ns * hp * d, d, hp * d, 1))
    yield ("ulysses unpack", (P, ns, hp, d), (P, hp, ns, d), (ns * hp * d, d, hp * d, 1),
           (P * ns, H, d), (1, H, ns, d), (0, d, H * d, 1))
    B, N = 2, 100
    yield ("[B,H,N,d] -> [B,N,H,d]", (B, H, N, 64), (B, H, N, 64), (H * N * 64, N * 64, 64, 1),
           (B, N, H, 64), (B, H, N, 64), (N * H * 64, 64, H * 64, 1))
    yield ("padded rows", (3, 5, 80), (1, 3, 5, 64), (0, 5 * 80, 80, 1),
           (5, 3, 96), (3, 1, 5, 64), (96, 0, 3 * 96, 1))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("case", list(_cases()), ids=lambda c: c[0])
def test_head_relayout_copies_every_vector_and_nothing_else(case, dtype):
    _, sbuf, sshape, sstr, dbuf, dshape, dstr = case
    src_buf = draw([sbuf], 60, torch.float32)[0].to(dtype)
    s = _views(src_buf.to(DEV), sshape, sstr)
    dst_buf = torch.full(dbuf, -7.0, dtype=dtype, device=DEV)
    dv = _views(dst_buf, dshape, dstr)
    sa.head_relayout(s, dv)
    torch.cuda.synchronize()
    F = sshape[0] * sshape[1]
    want = _views(src_buf, sshape, sstr).reshape(F, sshape[2], sshape[3])
    got = dv.cpu().reshape(F, dshape[2], dshape[3])
    assert torch.equal(got, want)
    # bytes of dst not covered by the view keep their value
    mask = torch.ones(dbuf, dtype=torch.bool)
    _views(mask, dshape, dstr).fill_(False)
    assert (dst_buf.cpu()[mask] == -7.0).all()


def test_head_relayout_large_grid_stride():
    # more 16-byte units than one pass of the grid covers
    n, H, d, P = 65536, 16, 128, 8
    x = torch.randn((n, H, d), dtype=torch.float32, device=DEV).to(torch.bfloat16)
    ns, hp = n // P, H // P
    send = torch.empty((P, P, ns, hp, d), dtype=torch.bfloat16, device=DEV)
    sa.head_relayout(_views(x, (P, H, ns, d), (ns * H * d, d, H * d, 1)),
                     _views(send, (P * P, hp, ns, d), (ns * hp * d, d, hp * d, 1)))
    torch.cuda.synchronize()
    want = x.view(P, ns, P, hp, d).permute(0, 2, 1, 3, 4)
    assert torch.equal(send, want)


@pytest.mark.parametrize("n,H,Hkv,P,d,causal", [
    (1024, 8, 4, 4, 128, True),
    (768, 6, 6, 3, 64, False),
    (512, 4, 2, 2, 128, True),
])
def test_ulysses_pipeline_matches_full_attention_small(n, H, Hkv, P, d, causal):
    q, k, v = draw([(n, H, d), (n, Hkv, d), (n, Hkv, d)], 70 + n)
    to_hn = lambda t: t.permute(1, 0, 2).contiguous().float().numpy()
    o_ref, l_ref = oracle.attn_fwd(to_hn(q), to_hn(k), to_hn(v),
                                   delta=0 if causal else oracle.NONCAUSAL)
    out, lse = emulate.ulysses_pipeline_fwd(q.to(DEV), k.to(DEV), v.to(DEV), P, causal=causal)
    torch.cuda.synchronize()
    assert out.shape == (n, H, d)
    assert_parity(to_np(out.permute(1, 0, 2)), to_np(lse), o_ref, l_ref, torch.bfloat16,
                  what="ulysses pipeline")


def test_ulysses_pipeline_16k_sampled():
    """8 ranks, 16 heads, d=128, 16384 tokens, causal; seeded rows of every
    head against the oracle."""
    n, H, P, d = 16384, 16, 8, 128
    q, k, v = draw([(n, H, d)] * 3, 77)
    out, lse = emulate.ulysses_pipeline_fwd(q.to(DEV), k.to(DEV), v.to(DEV), P)
    torch.cuda.synchronize()
    to_hn = lambda t: t.permute(1, 0, 2).contiguous().float().numpy()
    rows = np.array([h * n + i for h in range(H)
                     for i in sample_rows(n, 8, 780 + h, must=(0, 2047, 2048, n - 1))], np.int64)
    o_ref, l_ref = oracle.attn_fwd(to_hn(q), to_hn(k), to_hn(v), delta=0, rows=rows)
    og = to_np(out.permute(1, 0, 2)).reshape(-1, d)[rows]
    lg = to_np(lse).reshape(-1)[rows]
    assert_parity(og, lg, o_ref, l_ref, torch.bfloat16, rows_heads=rows // n,
                  what="ulysses pipeline 16k")
