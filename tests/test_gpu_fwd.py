"""GPU parity of the segment forward, the LSE merge and the sweep drivers.

Every case draws seeded host tensors, runs the HIP path through the C ABI
(Python binding) and compares with the fp64 oracle on the same values.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import long_sequence_exact_amd as sa
from long_sequence_exact_amd import emulate
from long_sequence_exact_amd.synth import (WORKLOADS, draw, sample_rows, sample_rows_per_tile,
                                           workload_inputs)
from tests.parity import LSE_TOL, TOL, assert_parity, check_close, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _np32(t):
    return t.float().numpy()


def _delta_arg(delta):
    return oracle.NONCAUSAL if delta is None else delta


# ---------------------------------------------------------------- tiny fp32

def test_tiny_fp32_segments_then_merge():
    """1 head, d=64, 1024 tokens as 4 KV segments of 256, non-causal, seed 0:
    per-segment (O, LSE), then lse_merge, equals full attention."""
    w = WORKLOADS["tiny_fp32_segments"]
    q, k, v = workload_inputs(w)
    o_ref, l_ref = oracle.attn_fwd(_np32(q), _np32(k), _np32(v))
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    seg = w.nk // w.segments
    parts = [sa.attn_segment_fwd(qd, kd[..., s * seg:(s + 1) * seg, :],
                                 vd[..., s * seg:(s + 1) * seg, :])
             for s in range(w.segments)]
    acc_o, acc_l = parts[0][0].clone(), parts[0][1].clone()
    for o_s, l_s in parts[1:]:
        sa.lse_merge(acc_o, acc_l, o_s, l_s)
    torch.cuda.synchronize()
    assert_parity(to_np(acc_o), to_np(acc_l), o_ref, l_ref, torch.float32, what="merge")
    # the same sweep with the fused merge epilogue
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=DEV)
    for s in range(w.segments):
        sa.attn_segment_fwd(qd, kd[..., s * seg:(s + 1) * seg, :],
                            vd[..., s * seg:(s + 1) * seg, :], out=out, lse=lse,
                            accumulate=s > 0)
    torch.cuda.synchronize()
    assert_parity(to_np(out), to_np(lse), o_ref, l_ref, torch.float32, what="fused")


# ---------------------------------------------------------- small shapes

CASES = [
    # (dtype, Hq, Hkv, Nq, Nk, d, delta)
    (torch.bfloat16, 2, 2, 200, 333, 128, None),
    (torch.bfloat16, 2, 2, 300, 300, 128, 0),
    (torch.bfloat16, 4, 1, 257, 513, 128, 100),
    (torch.bfloat16, 8, 2, 130, 700, 128, 400),
    (torch.bfloat16, 2, 2, 256, 256, 128, -50),
    (torch.bfloat16, 3, 3, 129, 64, 128, -200),     # every row masked
    (torch.bfloat16, 2, 1, 1, 1, 128, 0),
    (torch.bfloat16, 2, 2, 333, 271, 64, None),
    (torch.bfloat16, 4, 2, 385, 385, 64, 0),
    (torch.bfloat16, 2, 2, 100, 1000, 64, 700),
    (torch.float32, 2, 1, 150, 333, 64, 20),
    (torch.float32, 2, 2, 65, 97, 128, None),
    (torch.float32, 1, 1, 70, 70, 128, 0),
]


@pytest.mark.parametrize("dtype,hq,hkv,nq,nk,d,delta", CASES)
def test_segment_fwd_small(dtype, hq, hkv, nq, nk, d, delta):
    q, k, v = draw([(1, hq, nq, d), (1, hkv, nk, d), (1, hkv, nk, d)], 1000 + nq + nk, dtype)
    o_ref, l_ref = oracle.attn_fwd(_np32(q), _np32(k), _np32(v), delta=_delta_arg(delta))
    o, lse = sa.attn_segment_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal_offset=delta,
                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_parity(to_np(o), to_np(lse), o_ref, l_ref, dtype, what="fp32 out")
    if dtype == torch.bfloat16:
        ob, lb = sa.attn_segment_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal_offset=delta)
        torch.cuda.synchronize()
        assert ob.dtype == torch.bfloat16
        assert_parity(to_np(ob), to_np(lb), o_ref, l_ref, dtype, what="bf16 out")


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.bfloat16, 64),
                                     (torch.float32, 64)])
def test_fused_accumulate_two_segments(dtype, d):
    nq, nk = 300, 520
    q, k, v = draw([(2, 4, nq, d), (2, 2, nk, d), (2, 2, nk, d)], 77, dtype)
    delta = 250  # causal: q_start - k_start for the whole key range
    o_ref, l_ref = oracle.attn_fwd(_np32(q), _np32(k), _np32(v), delta=delta)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=DEV)
    cut = 190  # segments [0, 190) and [190, 520): second one seen from delta-190
    sa.attn_segment_fwd(qd, kd[..., cut:, :], vd[..., cut:, :], causal_offset=delta - cut,
                        out=out, lse=lse)
    sa.attn_segment_fwd(qd, kd[..., :cut, :], vd[..., :cut, :], causal_offset=delta,
                        out=out, lse=lse, accumulate=True)
    torch.cuda.synchronize()
    assert_parity(to_np(out), to_np(lse), o_ref, l_ref, dtype, what="accumulate")


def test_empty_inputs():
    q, k, v = draw([(1, 2, 64, 128), (1, 2, 64, 128), (1, 2, 64, 128)], 5)
    qd = q.to(DEV)
    kz = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device=DEV)
    o, lse = sa.attn_segment_fwd(qd, kz, kz, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    # accumulating an empty segment leaves the accumulator as it was
    o2, l2 = sa.attn_segment_fwd(qd, k.to(DEV), v.to(DEV))
    o3 = o2.float().clone()
    l3 = l2.clone()
    sa.attn_segment_fwd(qd, kz, kz, out=o3, lse=l3, accumulate=True)
    sa.attn_segment_fwd(qd, k.to(DEV), v.to(DEV), causal_offset=-10**12, out=o3, lse=l3,
                        accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(o3, o2.float()) and torch.equal(l3, l2)
    # empty query block: nothing to do
    qz = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device=DEV)
    o4, l4 = sa.attn_segment_fwd(qz, k.to(DEV), v.to(DEV))
    assert o4.shape == (1, 2, 0, 128)


def test_forward_is_deterministic():
    q, k, v = [t.to(DEV) for t in draw([(1, 4, 1000, 128)] * 3, 9)]
    a, la = sa.attn_segment_fwd(q, k, v, causal_offset=0)
    b, lb = sa.attn_segment_fwd(q, k, v, causal_offset=0)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)


# ------------------------------------------------------------- lse_merge

@pytest.mark.parametrize("b_dtype", [torch.float32, torch.bfloat16])
def test_lse_merge_matches_oracle(b_dtype):
    B, H, N, d = 2, 3, 517, 128
    oa, ob = draw([(B, H, N, d), (B, H, N, d)], 31, torch.float32)
    la, lb = draw([(B, H, N), (B, H, N)], 32, torch.float32)
    la = la * 5
    lb = lb * 5
    la[0, 0, :7] = -math.inf     # a empty
    lb[0, 1, :7] = -math.inf     # b empty
    la[1, 2, :5] = -math.inf     # both empty
    lb[1, 2, :5] = -math.inf
    oa[1, 2, :5] = 0
    ob[1, 2, :5] = 0
    ob = ob.to(b_dtype)
    ro, rl = oracle.lse_merge(oa.numpy(), la.numpy(), ob.float().numpy(), lb.numpy())
    oad, lad = oa.to(DEV), la.to(DEV)
    sa.lse_merge(oad, lad, ob.to(DEV), lb.to(DEV))
    torch.cuda.synchronize()
    assert_parity(to_np(oad), to_np(lad), ro, rl, torch.float32, what="lse_merge")
    assert not torch.isnan(oad).any()


# ------------------------------------------------------------- sweeps

def test_ring_sweep_matches_full_causal_attention_small():
    P, blk, H, d = 4, 96, 2, 128
    n = P * blk
    q, k, v = draw([(1, H, n, d)] * 3, 41)
    o_ref, l_ref = oracle.attn_fwd(_np32(q), _np32(k), _np32(v), delta=0)
    o, lse = emulate.ring_fwd(q.to(DEV), k.to(DEV), v.to(DEV), P, causal=True)
    torch.cuda.synchronize()
    assert_parity(to_np(o), to_np(lse), o_ref, l_ref, torch.bfloat16, what="ring small")


@pytest.mark.parametrize("P,c,H,d", [(4, 96, 2, 128), (3, 70, 2, 64), (1, 128, 1, 128)])
def test_zigzag_ring_matches_full_causal_attention_small(P, c, H, d):
    n = 2 * P * c
    q, k, v = draw([(1, H, n, d)] * 3, 45 + P)
    o_ref, l_ref = oracle.attn_fwd(_np32(q), _np32(k), _np32(v), delta=0)
    order = torch.tensor(emulate.zigzag_order(n, P))
    oz, lz = emulate.zigzag_ring_fwd(*(t[:, :, order].to(DEV) for t in (q, k, v)), P)
    torch.cuda.synchronize()
    o = torch.empty(oz.shape, dtype=oz.dtype)
    lse = torch.empty(lz.shape, dtype=lz.dtype)
    o[:, :, order] = oz.cpu()
    lse[:, :, order] = lz.cpu()
    assert_parity(to_np(o), to_np(lse), o_ref, l_ref, torch.bfloat16, what="zigzag ring small")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("delta", [None, 0, 150])
def test_growing_scores_take_the_rescale_path(delta, d):
    """Keys that line up more and more with the queries: each later block of
    keys scores far above the running maximum of the earlier ones, so the
    kernel's reference maximum is raised and the accumulated O rescaled
    several times per row (random inputs never get there).  At d = 128 the
    jumps at keys 300, 500 and 700 fall in later key tiles, where the
    exponentials against the old reference overflow the lazy bound and the
    tile is redone with its max."""
    H, N = 2, 900
    g = torch.Generator().manual_seed(31)
    u = torch.randn(H, 1, d, generator=g)
    q = (u.expand(H, N, d) + 0.1 * torch.randn(H, N, d, generator=g)).to(torch.bfloat16)
    a = torch.zeros(N)
    for j0, amp in ((100, 1.0), (300, 2.5), (500, 4.0), (700, 6.0)):
        a[j0:] = amp
    k = (a[None, :, None] * u + torch.randn(H, N, d, generator=g)).to(torch.bfloat16)
    v = torch.randn(H, N, d, generator=g).to(torch.bfloat16)
    dl = oracle.NONCAUSAL if delta is None else delta
    o_ref, l_ref = oracle.attn_fwd(_np32(q), _np32(k), _np32(v), delta=dl)
    o, lse = sa.attn_segment_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal_offset=delta,
                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    sc = _np32(q)[0] @ _np32(k)[0].T / np.sqrt(d)  # head 0 scores
    assert sc[:, 700:].max() - sc[:, :100].max() > 25  # far beyond the 2^8 slack
    assert_parity(to_np(o), to_np(lse), o_ref, l_ref, torch.bfloat16, what="growing scores")


@pytest.mark.parametrize("causal", [True, False])
def test_ring_lanes_give_identical_results(causal):
    """Splitting the ranks over streams keeps every rank's merge order, so the
    result is bit-identical to the one-stream sweep."""
    q, k, v = (t.to(DEV) for t in draw([(1, 4, 1024, 128)] * 3, 3))
    o1, l1 = emulate.ring_fwd(q, k, v, 8, causal=causal, lanes=1)
    for lanes in (2, 3, 4, 8):
        o, l = emulate.ring_fwd(q, k, v, 8, causal=causal, lanes=lanes)
        torch.cuda.synchronize()
        assert torch.equal(o, o1) and torch.equal(l, l1), lanes
    if causal:
        order = torch.tensor(emulate.zigzag_order(1024, 8), device=DEV)
        qz, kz, vz = (t[:, :, order].contiguous() for t in (q, k, v))
        z1 = emulate.zigzag_ring_fwd(qz, kz, vz, 8, lanes=1)
        for lanes in (2, 4, 8):
            z = emulate.zigzag_ring_fwd(qz, kz, vz, 8, lanes=lanes)
            torch.cuda.synchronize()
            assert torch.equal(z[0], z1[0]) and torch.equal(z[1], z1[1]), lanes


def _sampled_check(q, k, v, o, lse, delta, rows_per_head, seed, must_rows=(0, -1)):
    """Oracle on a seeded row subset of every head; compare the GPU rows."""
    B, H, N, d = q.shape
    rows = []
    for h in range(H):
        for i in sample_rows(N, rows_per_head, seed + h, must=must_rows):
            rows.append(h * N + i)
    rows = np.array(rows, np.int64)
    o_ref, l_ref = oracle.attn_fwd(_np32(q), _np32(k), _np32(v), delta=delta, rows=rows)
    o_g = to_np(o).reshape(-1, d)[rows]
    l_g = to_np(lse).reshape(-1)[rows]
    return o_g, l_g, o_ref, l_ref, rows // N


def test_largest_key_extent_sampled():
    """One head whose K and V each span just under 2 GiB (8,388,088 rows of
    d = 128, the largest extent the library accepts, since it addresses a
    head's rows with 32-bit byte offsets), 260 query rows seeing all keys but
    the last few: sampled rows against the oracle, so the offsets near 2^31
    are read correctly."""
    d = 128
    nk = (1 << 31) // (2 * d) - 512 - 8
    nq = 260
    delta = nk - 300
    q, k, v = draw([(1, 1, nq, d), (1, 1, nk, d), (1, 1, nk, d)], 1300)
    o, lse = sa.attn_segment_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal_offset=delta,
                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    og, lg, orf, lrf, heads = _sampled_check(q, k, v, o, lse, delta, 3, 1301,
                                             must_rows=(0, 259))
    assert_parity(og, lg, orf, lrf, torch.bfloat16, rows_heads=heads, what="2 GiB keys")


_RING_REF = {}


def _ring_16k_reference():
    """Full fp64 oracle of the ring workload (every row of all 32 heads,
    134,225,920 visible pairs per head, 2.2 TFLOP: about 25 s on 16 host
    cores), computed once for the plain and the zigzag ring tests."""
    if not _RING_REF:
        w = WORKLOADS["ring_16k_bf16"]
        q, k, v = workload_inputs(w)
        _RING_REF["in"] = (q, k, v)
        _RING_REF["ref"] = oracle.attn_fwd(_np32(q), _np32(k), _np32(v), delta=0)
    return _RING_REF["in"], _RING_REF["ref"]


def test_ring_16k_full_size_full_oracle():
    """32 heads, d=128, 16384 tokens, causal, 8 ranks x 2048 rows swept over 8
    KV segments with fused merges (one batched launch per step): every row
    of every head against the full oracle.  The fp32 accumulator starts as
    NaN, so a row that no step writes fails."""
    w = WORKLOADS["ring_16k_bf16"]
    (q, k, v), (o_ref, l_ref) = _ring_16k_reference()
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full(q.shape[:-1], float("nan"), dtype=torch.float32, device=DEV)
    o, l = emulate.ring_fwd(q.to(DEV), k.to(DEV), v.to(DEV), w.segments, causal=True,
                            out=out, lse=lse)
    torch.cuda.synchronize()
    assert_parity(to_np(o), to_np(l), o_ref, l_ref, torch.bfloat16, what="ring 16k full")


def test_zigzag_ring_16k_full_size_full_oracle():
    """The ring workload (32 heads, d=128, 16384 tokens, causal, 8 ranks) with
    the zigzag split: every row (back in sequence order) against the full
    oracle, accumulator NaN-filled first."""
    w = WORKLOADS["ring_16k_bf16"]
    (q, k, v), (o_ref, l_ref) = _ring_16k_reference()
    order = torch.tensor(emulate.zigzag_order(w.nq, w.segments))
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full(q.shape[:-1], float("nan"), dtype=torch.float32, device=DEV)
    oz, lz = emulate.zigzag_ring_fwd(*(t.to(DEV)[:, :, order.to(DEV)] for t in (q, k, v)),
                                     w.segments, out=out, lse=lse)
    torch.cuda.synchronize()
    o = torch.empty(oz.shape, dtype=oz.dtype)
    lse_s = torch.empty(lz.shape, dtype=lz.dtype)
    o[:, :, order] = oz.cpu()
    lse_s[:, :, order] = lz.cpu()
    assert_parity(to_np(o), to_np(lse_s), o_ref, l_ref, torch.bfloat16,
                  what="zigzag ring 16k full")


def test_ulysses_128k_full_size_sampled():
    """4 heads, d=128, 131072 tokens, causal, one call in the launch
    configuration bench.py times (bf16 O, fp32 LSE), and the same input as 8
    KV segments of 16384 swept through the fused merge into an fp32
    accumulator.  O and LSE start as NaN and every row must come back finite
    (each query sees at least its own key); then one seeded row in every
    32-row slice (one wave's rows of one query tile) of every head, 4096 rows
    per head with rows 0 and N-1, against the oracle (0.55 TFLOP fp64: about
    6 s on 16 host cores, shared by both checks)."""
    w = WORKLOADS["ulysses_128k_bf16"]
    q, k, v = workload_inputs(w)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full(q.shape[:-1], float("nan"), dtype=torch.float32, device=DEV)
    sa.attn_segment_fwd(qd, kd, vd, causal_offset=0, out=out, lse=lse)
    seg_out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
    seg_lse = torch.full(q.shape[:-1], float("nan"), dtype=torch.float32, device=DEV)
    emulate.sweep_fwd(qd, kd, vd, 8, 0, True, seg_out, seg_lse)
    torch.cuda.synchronize()
    del qd, kd, vd
    for o_, l_, what in ((out, lse, "one call"), (seg_out, seg_lse, "8 segments")):
        assert torch.isfinite(o_).all(), f"{what}: unwritten or non-finite O rows"
        assert torch.isfinite(l_).all(), f"{what}: unwritten or non-finite LSE rows"
    rows = []
    for h in range(w.hq):
        rows += [h * w.nq + i for i in
                 sample_rows_per_tile(w.nq, 32, 1, 1000 + w.seed + h, must=(0, w.nq - 1))]
    rows = np.array(rows, np.int64)
    o_ref, l_ref = oracle.attn_fwd(_np32(q), _np32(k), _np32(v), delta=0, rows=rows)
    og = to_np(out).reshape(-1, w.d)[rows]
    lg = to_np(lse).reshape(-1)[rows]
    assert_parity(og, lg, o_ref, l_ref, torch.bfloat16, rows_heads=rows // w.nq,
                  what="ulysses 128k")
    og = to_np(seg_out).reshape(-1, w.d)[rows]
    lg = to_np(seg_lse).reshape(-1)[rows]
    assert_parity(og, lg, o_ref, l_ref, torch.bfloat16, rows_heads=rows // w.nq,
                  what="ulysses 128k as 8 KV segments")


LONG_CASES = [
    # (hq, hkv, nq, nk, delta, out dtype); 24 query heads give the 384-row
    # shape its four workgroups per CU, fewer heads take the 256-row shape
    (24, 8, 16384 + 77, 16384 + 77, 0, torch.bfloat16),      # causal, ragged last tile
    (24, 24, 16384 + 300, 20000, -700, torch.float32),        # early rows see no key
    (24, 4, 17000, 5000, None, torch.bfloat16),               # non-causal, ragged key tail
    (24, 1, 16384, 16384 + 999, 999, torch.float32),          # keys ahead of the queries
    (2, 1, 16384 + 77, 16384 + 77, 0, torch.bfloat16),
    (3, 1, 17000, 5000, None, torch.bfloat16),
]


@pytest.mark.parametrize("hq,hkv,nq,nk,delta,odt", LONG_CASES)
def test_long_call_shape(hq, hkv, nq, nk, delta, odt):
    """Long d = 128 calls that write their own output (at least 16384 query
    rows, and enough query tiles for four workgroups per CU) run with 384-row
    workgroups; with fewer heads the same lengths take 256-row workgroups.
    O and LSE start as NaN; every O row must come back finite, every LSE row
    finite or -inf exactly where the oracle says the row sees no key; one
    seeded row in every 32-row slice of every head against the oracle."""
    d = 128
    q, k, v = draw([(1, hq, nq, d), (1, hkv, nk, d), (1, hkv, nk, d)], 1400 + nq + hq)
    out = torch.full(q.shape, float("nan"), dtype=odt, device=DEV)
    lse = torch.full(q.shape[:-1], float("nan"), dtype=torch.float32, device=DEV)
    sa.attn_segment_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal_offset=delta, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all(), "unwritten or non-finite O rows"
    assert not torch.isnan(lse).any(), "unwritten LSE rows"
    rows = []
    for h in range(hq):
        rows += [h * nq + i for i in sample_rows_per_tile(nq, 32, 1, 1500 + h, must=(0, nq - 1))]
    rows = np.array(rows, np.int64)
    o_ref, l_ref = oracle.attn_fwd(_np32(q), _np32(k), _np32(v), delta=_delta_arg(delta),
                                   rows=rows)
    og = to_np(out).reshape(-1, d)[rows]
    lg = to_np(lse).reshape(-1)[rows]
    if delta is not None and delta < 0:
        # rows with no visible key: O = 0, LSE = -inf (all of them, not only sampled)
        empty = torch.arange(nq) + delta < 0
        assert torch.isneginf(lse.cpu()[0][:, empty]).all()
        assert (out.cpu()[0][:, empty] == 0).all()
    assert_parity(og, lg, o_ref, l_ref, torch.bfloat16, rows_heads=rows // nq,
                  what=f"long call {nq}x{nk}")


SPLIT_CASES = [
    # (hq, hkv, nq, nk, delta, out dtype): short calls (fewer 256-row tiles
    # than two per compute unit, causal, or than one, non-causal; at least
    # 1024 keys) whose tiles' visible keys are cut into 2-8 parts
    (4, 4, 16384, 16384, 0, torch.bfloat16),       # 256 tiles, halves
    (2, 2, 16384, 16384, 0, torch.bfloat16),       # quarters
    (2, 1, 8000, 12000, 4000, torch.float32),      # ragged, keys ahead
    (3, 1, 5000, 9000, None, torch.bfloat16),      # non-causal
    (2, 1, 16384, 16384, -3000, torch.float32),    # early rows see no key
    (4, 4, 2048, 2048, 0, torch.bfloat16),         # parts of at least 512 keys
    (1, 1, 1000, 9000, 8500, torch.bfloat16),      # eight parts
]


@pytest.mark.parametrize("hq,hkv,nq,nk,delta,odt", SPLIT_CASES)
def test_split_short_call(hq, hkv, nq, nk, delta, odt):
    """Short calls split their key ranges over more workgroups and merge the
    fp32 partials by LSE.  O and LSE start as NaN; every O row must come
    back finite and every LSE row finite or -inf exactly where the oracle
    says the row sees no key; one seeded row in every 32-row slice of every
    head against the oracle, and every row against the unsplit call."""
    d = 128
    q, k, v = draw([(1, hq, nq, d), (1, hkv, nk, d), (1, hkv, nk, d)], 1600 + nq + hq)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    outs = []
    for split in (True, False):
        out = torch.full(q.shape, float("nan"), dtype=odt, device=DEV)
        lse = torch.full(q.shape[:-1], float("nan"), dtype=torch.float32, device=DEV)
        sa.attn_segment_fwd(qd, kd, vd, causal_offset=delta, out=out, lse=lse, split=split)
        outs.append((out, lse))
    torch.cuda.synchronize()
    (out, lse), (out1, lse1) = outs
    assert torch.isfinite(out).all(), "unwritten or non-finite O rows"
    assert not torch.isnan(lse).any(), "unwritten LSE rows"
    rows = []
    for h in range(hq):
        rows += [h * nq + i for i in sample_rows_per_tile(nq, 32, 1, 1700 + h, must=(0, nq - 1))]
    rows = np.array(rows, np.int64)
    o_ref, l_ref = oracle.attn_fwd(_np32(q), _np32(k), _np32(v), delta=_delta_arg(delta),
                                   rows=rows)
    og = to_np(out).reshape(-1, d)[rows]
    lg = to_np(lse).reshape(-1)[rows]
    if delta is not None and delta < 0:
        empty = torch.arange(nq) + delta < 0
        assert torch.isneginf(lse.cpu()[0][:, empty]).all()
        assert (out.cpu()[0][:, empty] == 0).all()
    assert_parity(og, lg, o_ref, l_ref, torch.bfloat16, rows_heads=rows // nq,
                  what=f"split call {nq}x{nk}")
    # every row against the unsplit call (same inputs, other merge order)
    assert torch.equal(torch.isneginf(lse), torch.isneginf(lse1))
    fin = torch.isfinite(lse1)
    assert (lse[fin] - lse1[fin]).abs().max().item() <= LSE_TOL
    check_close(out, to_np(out1), TOL[torch.bfloat16], what="split vs unsplit", name="o")


def test_usp_forward_full_size_sampled():
    """GQA 8/2, d=128, query block 7 of 8 (32768 rows) swept over 8 KV blocks
    of 32768, accumulator NaN-filled first (every row must come back
    finite); 2 heads x 512 seeded rows, four in every 256-row query tile,
    against the oracle."""
    w = WORKLOADS["usp_gqa_256k_bf16"]
    q, k, v = workload_inputs(w)
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full(q.shape[:-1], float("nan"), dtype=torch.float32, device=DEV)
    emulate.sweep_fwd(q.to(DEV), k.to(DEV), v.to(DEV), w.segments, w.q_block, True, out, lse)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    blk = w.nk // w.segments
    rows = []
    for h in (1, 6):
        for i in sample_rows_per_tile(w.nq, 256, 4, 2000 + h, must=(0, w.nq - 1)):
            rows.append(h * w.nq + i)
    rows = np.array(rows, np.int64)
    o_ref, l_ref = oracle.attn_fwd(_np32(q), _np32(k), _np32(v), delta=w.q_block * blk,
                                   rows=rows)
    og = to_np(out).reshape(-1, w.d)[rows]
    lg = to_np(lse).reshape(-1)[rows]
    assert_parity(og, lg, o_ref, l_ref, torch.bfloat16, rows_heads=rows // w.nq,
                  what="usp fwd")


@pytest.mark.parametrize("causal", [True, False])
def test_batched_ring_steps_equal_per_rank_launches(causal):
    """One launch per ring step (ranks batched through strided views) gives
    bit-identical results to one launch per (rank, step)."""
    P, blk, H, d = 8, 200, 2, 128
    q, k, v = (t.to(DEV) for t in draw([(1, H, P * blk, d)] * 3, 43))
    a, la = emulate.ring_fwd(q, k, v, P, causal=causal, batched=True)
    b, lb = emulate.ring_fwd(q, k, v, P, causal=causal, batched=False)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)
    if not causal:
        o_ref, l_ref = oracle.attn_fwd(*(t.float().cpu().numpy() for t in (q, k, v)))
        assert_parity(to_np(a), to_np(la), o_ref, l_ref, torch.bfloat16, what="ring noncausal")


def test_sequence_major_layout_views():
    """Q/K/V stored [B, N, H, d] (the sequence-sharded layout before Ulysses'
    all-to-all) and passed as permuted [B, H, N, d] views (stride_n = H*d)."""
    B, N, H, Hkv, d = 2, 700, 4, 2, 128
    qs, ks, vs = draw([(B, N, H, d), (B, N, Hkv, d), (B, N, Hkv, d)], 61)
    q, k, v = (t.permute(0, 2, 1, 3) for t in (qs, ks, vs))
    o_ref, l_ref = oracle.attn_fwd(*(t.contiguous().float().numpy() for t in (q, k, v)), delta=0)
    qd, kd, vd = (t.to(DEV).permute(0, 2, 1, 3) for t in (qs, ks, vs))
    assert qd.stride(2) == H * d
    out = torch.empty((B, N, H, d), dtype=torch.float32, device=DEV).permute(0, 2, 1, 3)
    lse = torch.empty((B, N, H), dtype=torch.float32, device=DEV).permute(0, 2, 1)
    sa.attn_segment_fwd(qd, kd, vd, causal_offset=0, out=out, lse=lse)
    torch.cuda.synchronize()
    assert_parity(to_np(out), to_np(lse), o_ref, l_ref, torch.bfloat16, what="seq-major")
