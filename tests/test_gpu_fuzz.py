"""Seeded random sweep against the fp64 oracle: shapes, causal offsets, head
groupings, layouts and flags drawn by one generator, for the segment forward
(bf16 and fp32, with and without the fused merge; short d = 128 calls with
and without the key-range split), its backward and dilated
attention (forward and backward, with and without head-dependent offsets),
batch 1 or 2.

Each case prints its parameters in the assertion message, so a failure names
the case; the draw is deterministic (numpy generator, fixed seed).  The
environment variable SEQATTN_FUZZ_SCALE multiplies the number of cases (the
first cases of a longer draw are the default ones).
"""
import os

import numpy as np
import pytest
import torch

import oracle
import long_sequence_exact_amd as sa
from long_sequence_exact_amd.synth import draw
from tests.parity import LSE_TOL, TOL, assert_parity, check_close, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
SCALE = max(1, int(os.environ.get("SEQATTN_FUZZ_SCALE", "1")))


def _np32(t):
    return t.float().numpy()


def _dev(t, seq_major):
    """Device copy of a [B, H, N, d] host tensor, optionally stored [B, N, H, d]
    and passed as a permuted (strided) view."""
    if not seq_major:
        return t.to(DEV)
    return t.permute(0, 2, 1, 3).contiguous().to(DEV).permute(0, 2, 1, 3)


def _fwd_cases(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        d = int(rng.choice([64, 128]))
        hkv = int(rng.integers(1, 3))
        group = int(rng.choice([1, 2, 4]))
        nq = int(rng.integers(1, 600))
        nk = int(rng.integers(1, 700))
        delta = None if rng.random() < 0.25 else int(rng.integers(-nq - 50, nk + 50))
        dtype = torch.float32 if rng.random() < 0.15 else torch.bfloat16
        split = int(rng.integers(1, nk)) if (nk > 1 and rng.random() < 0.35) else 0
        out_bf16 = dtype == torch.bfloat16 and split == 0 and rng.random() < 0.5
        seq_major = bool(rng.random() < 0.3)
        bsz = 2 if rng.random() < 0.25 else 1
        out.append((i, d, hkv, group, nq, nk, delta, dtype, split, out_bf16, seq_major, bsz))
    return out


@pytest.mark.parametrize("case", _fwd_cases(40 * SCALE, 20261203), ids=lambda c: f"fwd{c[0]}")
def test_fuzz_segment_fwd(case):
    i, d, hkv, group, nq, nk, delta, dtype, split, out_bf16, seq_major, bsz = case
    hq = hkv * group
    q, k, v = draw([(bsz, hq, nq, d), (bsz, hkv, nk, d), (bsz, hkv, nk, d)], 7000 + i, dtype)
    o_ref, l_ref = oracle.attn_fwd(_np32(q), _np32(k), _np32(v),
                                   delta=oracle.NONCAUSAL if delta is None else delta)
    qd, kd, vd = (_dev(t, seq_major) for t in (q, k, v))
    what = f"case {case}"
    if split:
        # two KV segments, the second merged into the first by the epilogue
        out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=DEV)
        d2 = None if delta is None else delta - split
        sa.attn_segment_fwd(qd, kd[:, :, :split], vd[:, :, :split], causal_offset=delta,
                            out=out, lse=lse)
        sa.attn_segment_fwd(qd, kd[:, :, split:], vd[:, :, split:], causal_offset=d2,
                            out=out, lse=lse, accumulate=True)
        o, l = out, lse
    else:
        o, l = sa.attn_segment_fwd(qd, kd, vd, causal_offset=delta,
                                   out_dtype=torch.bfloat16 if out_bf16 else torch.float32)
    torch.cuda.synchronize()
    assert_parity(to_np(o), to_np(l), o_ref, l_ref, dtype, what=what)


def _split_cases(count, seed):
    """d = 128 bf16 calls short enough for the key-range split (fewer 256-row
    query tiles than compute units, at least 1024 keys)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        hkv = int(rng.integers(1, 3))
        group = int(rng.choice([1, 2, 4]))
        nq = int(rng.integers(1, 1200))
        nk = int(rng.integers(1024, 4097))
        delta = None if rng.random() < 0.25 else int(rng.integers(-nq - 50, nk + 50))
        out_bf16 = bool(rng.random() < 0.5)
        seq_major = bool(rng.random() < 0.3)
        bsz = 2 if rng.random() < 0.25 else 1
        out.append((i, hkv, group, nq, nk, delta, out_bf16, seq_major, bsz))
    return out


@pytest.mark.parametrize("case", _split_cases(12 * SCALE, 20261204), ids=lambda c: f"split{c[0]}")
def test_fuzz_split_fwd(case):
    """The split call against the oracle on every row, and against the
    unsplit call (same -inf rows, LSE within its tolerance, O by the per-row
    measure)."""
    i, hkv, group, nq, nk, delta, out_bf16, seq_major, bsz = case
    hq, d = hkv * group, 128
    q, k, v = draw([(bsz, hq, nq, d), (bsz, hkv, nk, d), (bsz, hkv, nk, d)], 7500 + i)
    o_ref, l_ref = oracle.attn_fwd(_np32(q), _np32(k), _np32(v),
                                   delta=oracle.NONCAUSAL if delta is None else delta)
    qd, kd, vd = (_dev(t, seq_major) for t in (q, k, v))
    odt = torch.bfloat16 if out_bf16 else torch.float32
    res = [sa.attn_segment_fwd(qd, kd, vd, causal_offset=delta, out_dtype=odt, split=sp)
           for sp in (True, False)]
    torch.cuda.synchronize()
    (o, l), (o1, l1) = res
    what = f"case {case}"
    assert_parity(to_np(o), to_np(l), o_ref, l_ref, torch.bfloat16, what=what)
    assert torch.equal(torch.isneginf(l), torch.isneginf(l1)), what
    fin = torch.isfinite(l1)
    if fin.any():
        assert (l[fin] - l1[fin]).abs().max().item() <= LSE_TOL, what
    check_close(o, to_np(o1), TOL[torch.bfloat16], what=what + " split vs unsplit", name="o")


def _bwd_cases(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        d = int(rng.choice([64, 128]))
        hkv = int(rng.integers(1, 3))
        group = int(rng.choice([1, 2, 4]))
        nq = int(rng.integers(1, 400))
        nk = int(rng.integers(1, 500))
        delta = None if rng.random() < 0.25 else int(rng.integers(-nq - 20, nk + 20))
        grads_bf16 = bool(rng.random() < 0.3)
        seq_major = bool(rng.random() < 0.3)
        bsz = 2 if rng.random() < 0.25 else 1
        out.append((i, d, hkv, group, nq, nk, delta, grads_bf16, seq_major, bsz))
    return out


@pytest.mark.parametrize("case", _bwd_cases(20 * SCALE, 20261204), ids=lambda c: f"bwd{c[0]}")
def test_fuzz_segment_bwd(case):
    i, d, hkv, group, nq, nk, delta, grads_bf16, seq_major, bsz = case
    hq = hkv * group
    q, k, v, do = draw([(bsz, hq, nq, d), (bsz, hkv, nk, d), (bsz, hkv, nk, d),
                        (bsz, hq, nq, d)], 7500 + i)
    dl = oracle.NONCAUSAL if delta is None else delta
    ref = oracle.attn_bwd(_np32(q), _np32(k), _np32(v), _np32(do), delta=dl)
    qd, kd, vd, dod = (_dev(t, seq_major) for t in (q, k, v, do))
    o, lse = sa.attn_segment_fwd(qd, kd, vd, causal_offset=delta, out_dtype=torch.float32)
    grads = sa.attn_segment_bwd(qd, kd, vd, o, lse, dod, causal_offset=delta,
                                grad_dtype=torch.bfloat16 if grads_bf16 else torch.float32)
    torch.cuda.synchronize()
    for name, x, r in zip(("dq", "dk", "dv"), grads, ref):
        assert not torch.isnan(x).any(), f"case {case}: NaN in {name}"
        check_close(x, r, TOL[torch.bfloat16], what=f"case {case}", name=name)


def _dilated_cases(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        d = int(rng.choice([64, 128]))
        hkv = int(rng.integers(1, 4))
        group = int(rng.choice([1, 2]))
        n = int(rng.integers(64, 700))
        nb = int(rng.integers(1, 5))
        ws = [int(rng.integers(8, int(1.5 * n))) for _ in range(nb)]
        rs = [int(rng.integers(1, 13)) for _ in range(nb)]
        causal = bool(rng.random() < 0.5)
        head_shift = bool(rng.random() < 0.4)
        bsz = 2 if rng.random() < 0.25 else 1
        out.append((i, d, hkv, group, n, tuple(ws), tuple(rs), causal, head_shift, bsz))
    return out


@pytest.mark.parametrize("case", _dilated_cases(16 * SCALE, 20261205), ids=lambda c: f"dil{c[0]}")
def test_fuzz_dilated(case):
    i, d, hkv, group, n, ws, rs, causal, head_shift, bsz = case
    hq = hkv * group
    q, k, v, do = draw([(bsz, hq, n, d), (bsz, hkv, n, d), (bsz, hkv, n, d), (bsz, hq, n, d)],
                       7800 + i)
    q32, k32, v32, do32 = (_np32(t) for t in (q, k, v, do))
    o_ref, l_ref = oracle.dilated_fwd(q32, k32, v32, ws, rs, causal=causal, head_shift=head_shift)
    ref = oracle.dilated_bwd(q32, k32, v32, do32, ws, rs, causal=causal, head_shift=head_shift)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = sa.dilated_attn_fwd(qd, kd, vd, ws, rs, causal=causal, head_shift=head_shift)
    grads = sa.dilated_attn_bwd(qd, kd, vd, o, lse, dod, ws, rs, causal=causal,
                                head_shift=head_shift)
    torch.cuda.synchronize()
    assert_parity(to_np(o), to_np(lse), o_ref, l_ref, torch.bfloat16, what=f"case {case}")
    for name, x, r in zip(("dq", "dk", "dv"), grads, ref):
        assert not torch.isnan(x).any(), f"case {case}: NaN in {name}"
        check_close(x, r, TOL[torch.bfloat16], what=f"case {case}", name=name)
