"""Pins of the fp64 oracle against things other than itself (CPU only).

Every pin is one of: a library routine the definition reduces to (PyTorch's
fp64 CPU scaled_dot_product_attention and its autograd), a closed form or
special case, an invariant of the mathematics, or brute-force finite
differences.  Each is chosen so a plausible mistake in the oracle -- a dropped
scale, a wrong sign, a transposed operand, an off-by-one in the visibility
rule, a wrong head map, a wrong merge weight -- fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from long_sequence_exact_amd.synth import draw

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, quant=None):
    (t,) = draw([shape], seed, torch.float32)
    a = t.numpy()
    if quant is not None:       # values on a 2^-quant grid (exact in float32)
        a = np.round(a * 2.0 ** quant) / 2.0 ** quant
    return a.astype(np.float32)


def _sdpa(q, k, v, mask=None, scale=None):
    """Library attention in fp64 on the CPU (the pin, not the oracle)."""
    qt = torch.from_numpy(np.asarray(q, np.float64))
    kt = torch.from_numpy(np.asarray(k, np.float64))
    vt = torch.from_numpy(np.asarray(v, np.float64))
    m = None if mask is None else torch.from_numpy(mask)
    return F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m,
                                          scale=scale).numpy()


def _causal_mask(nq, nk, delta):
    i = np.arange(nq)[:, None]
    j = np.arange(nk)[None, :]
    return (j - i) <= delta


# --------------------------------------------------------------------------
# forward
# --------------------------------------------------------------------------

def test_fwd_noncausal_matches_library():
    q = _rand((2, 3, 37, 16), 10)
    k = _rand((2, 3, 53, 16), 11)
    v = _rand((2, 3, 53, 16), 12)
    o, lse = oracle.attn_fwd(q, k, v)
    ref = _sdpa(q, k, v)
    assert np.abs(o - ref).max() < 1e-12
    assert o.shape == (2, 3, 37, 16) and lse.shape == (2, 3, 37)


@pytest.mark.parametrize("delta", [-40, -5, 0, 7, 60])
def test_fwd_causal_offset_matches_library(delta):
    nq, nk = 29, 45
    q = _rand((1, 2, nq, 8), 20)
    k = _rand((1, 2, nk, 8), 21)
    v = _rand((1, 2, nk, 8), 22)
    o, lse = oracle.attn_fwd(q, k, v, delta=delta)
    mask = _causal_mask(nq, nk, delta)
    live = mask.any(axis=1)
    if live.any():
        ref = _sdpa(q[:, :, live], k, v, mask=mask[live])
        assert np.abs(o[:, :, live] - ref).max() < 1e-12
    # rows with no visible key: O = 0, LSE = -inf
    assert np.all(o[:, :, ~live] == 0.0)
    assert np.all(np.isneginf(lse[:, :, ~live]))
    assert np.all(np.isfinite(lse[:, :, live]))


def test_fwd_scale_argument_matches_library():
    q = _rand((1, 1, 9, 32), 30)
    k = _rand((1, 1, 11, 32), 31)
    v = _rand((1, 1, 11, 32), 32)
    o, _ = oracle.attn_fwd(q, k, v, scale=0.37)
    assert np.abs(o - _sdpa(q, k, v, scale=0.37)).max() < 1e-12


def test_gqa_head_map_is_contiguous_groups():
    # query head h reads KV head floor(h * Hkv / Hq): heads 0-2 -> 0, 3-5 -> 1
    q = _rand((1, 6, 13, 8), 40)
    k = _rand((1, 2, 17, 8), 41)
    v = _rand((1, 2, 17, 8), 42)
    o, _ = oracle.attn_fwd(q, k, v, delta=3)
    kr = np.repeat(k, 3, axis=1)
    vr = np.repeat(v, 3, axis=1)
    ref = _sdpa(q, kr, vr, mask=_causal_mask(13, 17, 3))
    assert np.abs(o - ref).max() < 1e-12


def test_q_zero_gives_mean_of_visible_values_and_log_count():
    n, d = 50, 8
    q = np.zeros((1, 1, n, d), np.float32)
    k = _rand((1, 1, n, d), 50)
    v = _rand((1, 1, n, d), 51)
    o, lse = oracle.attn_fwd(q, k, v, delta=0)
    for i in range(n):
        assert np.allclose(o[0, 0, i], v[0, 0, : i + 1].astype(np.float64).mean(0),
                           atol=1e-13)
        assert abs(lse[0, 0, i] - math.log(i + 1)) < 1e-13


def test_causal_row0_returns_v0():
    d = 16
    q = _rand((1, 1, 5, d), 60)
    k = _rand((1, 1, 5, d), 61)
    v = _rand((1, 1, 5, d), 62)
    o, lse = oracle.attn_fwd(q, k, v, delta=0)
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0].astype(np.float64))
    s00 = float(np.dot(q[0, 0, 0].astype(np.float64), k[0, 0, 0])) / math.sqrt(d)
    assert abs(lse[0, 0, 0] - s00) < 1e-13


def test_lse_matches_library_logsumexp():
    q = _rand((1, 2, 21, 16), 70)
    k = _rand((1, 2, 33, 16), 71)
    v = _rand((1, 2, 33, 16), 72)
    _, lse = oracle.attn_fwd(q, k, v, delta=4)
    s = torch.from_numpy(q.astype(np.float64)) @ \
        torch.from_numpy(k.astype(np.float64)).transpose(-1, -2) / 4.0
    s = s.masked_fill(~torch.from_numpy(_causal_mask(21, 33, 4)), -math.inf)
    ref = torch.logsumexp(s, dim=-1).numpy()
    assert np.abs(lse - ref).max() < 1e-12


def test_mean_lse_statistics():
    # q, k ~ N(0, I): s = q.k/sqrt(d) has variance ~1, so E[exp(s)] ~ e^(1/2)
    # and the mean LSE over rows is close to ln(n) + 1/2.
    n, d = 2048, 64
    q = _rand((1, 1, 64, d), 80)
    k = _rand((1, 1, n, d), 81)
    v = _rand((1, 1, n, d), 82)
    _, lse = oracle.attn_fwd(q, k, v)
    assert abs(lse.mean() - (math.log(n) + 0.5)) < 0.15


def test_row_subset_equals_full():
    q = _rand((2, 2, 31, 8), 90)
    k = _rand((2, 1, 40, 8), 91)
    v = _rand((2, 1, 40, 8), 92)
    o, lse = oracle.attn_fwd(q, k, v, delta=2)
    rows = [0, 5, 31, 62, 123]
    os_, ls_ = oracle.attn_fwd(q, k, v, delta=2, rows=rows)
    flat_o = o.reshape(-1, 8)
    flat_l = lse.reshape(-1)
    assert np.array_equal(os_, flat_o[rows])
    assert np.array_equal(ls_, flat_l[rows])


def test_empty_shapes():
    q = _rand((1, 1, 4, 8), 95)
    k = np.zeros((1, 1, 0, 8), np.float32)
    o, lse = oracle.attn_fwd(q, k, k)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    o, lse = oracle.attn_fwd(np.zeros((1, 1, 0, 8), np.float32), q, q)
    assert o.shape == (1, 1, 0, 8) and lse.shape == (1, 1, 0)


# --------------------------------------------------------------------------
# merge
# --------------------------------------------------------------------------

def test_merge_closed_forms():
    d = 4
    oa = np.arange(d, dtype=np.float64)[None]
    ob = -np.arange(d, dtype=np.float64)[None] + 10
    # equal LSE: weights 1/2, 1/2 and LSE + ln 2
    o, l = oracle.lse_merge(oa, np.array([0.0]), ob, np.array([0.0]))
    assert np.allclose(o, 0.5 * oa + 0.5 * ob, atol=1e-15)
    assert abs(l[0] - math.log(2.0)) < 1e-15
    # LSE ln 3 vs ln 1: weights 3/4, 1/4, total ln 4
    o, l = oracle.lse_merge(oa, np.array([math.log(3)]), ob, np.array([0.0]))
    assert np.allclose(o, 0.75 * oa + 0.25 * ob, atol=1e-15)
    assert abs(l[0] - math.log(4.0)) < 1e-15
    # very different magnitudes do not overflow
    o, l = oracle.lse_merge(oa, np.array([1000.0]), ob, np.array([-1000.0]))
    assert np.allclose(o, oa) and abs(l[0] - 1000.0) < 1e-12


def test_merge_identity_and_empty():
    oa = _rand((3, 8), 100).astype(np.float64)
    la = np.array([0.3, -2.0, 5.0])
    z = np.zeros_like(oa)
    ninf = np.full(3, -np.inf)
    o, l = oracle.lse_merge(oa, la, z, ninf)
    assert np.array_equal(o, oa) and np.array_equal(l, la)
    o, l = oracle.lse_merge(z, ninf, oa, la)
    assert np.array_equal(o, oa) and np.array_equal(l, la)
    o, l = oracle.lse_merge(z, ninf, z, ninf)
    assert np.all(o == 0) and np.all(np.isneginf(l)) and not np.isnan(o).any()


@pytest.mark.parametrize("delta", [oracle.NONCAUSAL, 0, 30])
def test_segment_merge_equals_full_attention(delta):
    nq, nk, nseg, d = 40, 64, 4, 16
    q = _rand((1, 2, nq, d), 110)
    k = _rand((1, 2, nk, d), 111)
    v = _rand((1, 2, nk, d), 112)
    o_full, l_full = oracle.attn_fwd(q, k, v, delta=delta)
    seg = nk // nseg
    acc_o = np.zeros_like(o_full)
    acc_l = np.full(l_full.shape, -np.inf)
    for s in range(nseg):
        ks = k[:, :, s * seg:(s + 1) * seg]
        vs = v[:, :, s * seg:(s + 1) * seg]
        # global rule j_g <= i + delta with j_g = s*seg + j
        dl = delta if delta == oracle.NONCAUSAL else delta - s * seg
        o_s, l_s = oracle.attn_fwd(q, ks, vs, delta=dl)
        acc_o, acc_l = oracle.lse_merge(acc_o, acc_l, o_s, l_s)
    assert np.abs(acc_o - o_full).max() < 1e-13
    fin = np.isfinite(l_full)
    assert np.abs(acc_l[fin] - l_full[fin]).max() < 1e-13
    assert np.array_equal(np.isneginf(acc_l), np.isneginf(l_full))


def test_ring_sweep_union_equals_full_causal():
    # 4 ranks x 8 rows: rank r's Q block against KV blocks j <= r, merged in
    # step order, reproduces full causal attention over 32 tokens.
    P, blk, d = 4, 8, 8
    n = P * blk
    q = _rand((1, 1, n, d), 120)
    k = _rand((1, 1, n, d), 121)
    v = _rand((1, 1, n, d), 122)
    o_full, l_full = oracle.attn_fwd(q, k, v, delta=0)
    for r in range(P):
        qb = q[:, :, r * blk:(r + 1) * blk]
        acc_o = np.zeros((1, 1, blk, d))
        acc_l = np.full((1, 1, blk), -np.inf)
        for t in range(P):
            j = (r - t) % P
            if j > r:
                continue
            o_s, l_s = oracle.attn_fwd(qb, k[:, :, j * blk:(j + 1) * blk],
                                       v[:, :, j * blk:(j + 1) * blk],
                                       delta=(r - j) * blk)
            acc_o, acc_l = oracle.lse_merge(acc_o, acc_l, o_s, l_s)
        assert np.abs(acc_o - o_full[:, :, r * blk:(r + 1) * blk]).max() < 1e-13
        assert np.abs(acc_l - l_full[:, :, r * blk:(r + 1) * blk]).max() < 1e-13


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------

def _autograd_ref(q, k, v, do, delta, group):
    qt = torch.from_numpy(q.astype(np.float64)).requires_grad_()
    kt = torch.from_numpy(k.astype(np.float64)).requires_grad_()
    vt = torch.from_numpy(v.astype(np.float64)).requires_grad_()
    kr = kt.repeat_interleave(group, dim=1)
    vr = vt.repeat_interleave(group, dim=1)
    mask = torch.from_numpy(_causal_mask(q.shape[2], k.shape[2], delta))
    o = F.scaled_dot_product_attention(qt, kr, vr, attn_mask=mask)
    (o * torch.from_numpy(do.astype(np.float64))).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("delta,group", [(0, 1), (5, 2), (40, 3)])
def test_bwd_matches_library_autograd(delta, group):
    nq, nk, d = 17, 23, 16
    q = _rand((1, 2 * group, nq, d), 200)
    k = _rand((1, 2, nk, d), 201)
    v = _rand((1, 2, nk, d), 202)
    do = _rand((1, 2 * group, nq, d), 203)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, delta=delta)
    rq, rk, rv = _autograd_ref(q, k, v, do, delta, group)
    assert np.abs(dq - rq).max() < 1e-12
    assert np.abs(dk - rk).max() < 1e-12
    assert np.abs(dv - rv).max() < 1e-12


def test_bwd_finite_differences():
    # Brute force: central differences of L = sum(dO * O) computed with the
    # forward oracle, with Richardson extrapolation.  Inputs sit on a 2^-6
    # grid so every perturbed value is exact in float32.
    nq, nk, d, delta = 5, 7, 4, 2
    q = _rand((1, 2, nq, d), 210, quant=6)
    k = _rand((1, 1, nk, d), 211, quant=6)
    v = _rand((1, 1, nk, d), 212, quant=6)
    do = _rand((1, 2, nq, d), 213, quant=6)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, delta=delta)

    def loss(qq, kk, vv):
        o, _ = oracle.attn_fwd(qq, kk, vv, delta=delta)
        return float((o * do.astype(np.float64)).sum())

    def fd(which, idx, h):
        args = [q.copy(), k.copy(), v.copy()]
        args[which][idx] += np.float32(h)
        lp = loss(*args)
        args[which][idx] -= np.float32(2 * h)
        lm = loss(*args)
        return (lp - lm) / (2 * h)

    for which, grad in ((0, dq), (1, dk), (2, dv)):
        arr = (q, k, v)[which]
        for idx in np.ndindex(arr.shape):
            h = 2.0 ** -9
            g = (4 * fd(which, idx, h / 2) - fd(which, idx, h)) / 3
            assert abs(g - grad[idx]) < 1e-8 * max(1.0, abs(grad[idx])), (which, idx)


def test_bwd_invariants():
    # Every row sees >= 1 key: sum_j dV_j = sum_i dO_i (softmax rows sum to
    # 1) and sum_j dK_j = 0 (dS rows sum to 0), per KV head over its group.
    nq, nk, d, group = 24, 40, 8, 4
    q = _rand((1, group, nq, d), 220)
    k = _rand((1, 1, nk, d), 221)
    v = _rand((1, 1, nk, d), 222)
    do = _rand((1, group, nq, d), 223)
    _, dk, dv = oracle.attn_bwd(q, k, v, do, delta=3)
    assert np.abs(dv.sum(axis=2)[0, 0] - do.astype(np.float64).sum(axis=(1, 2))[0]).max() < 1e-12
    assert np.abs(dk.sum(axis=2)).max() < 1e-12


def test_bwd_dq_rows_match_full():
    q = _rand((1, 4, 19, 8), 230)
    k = _rand((1, 2, 25, 8), 231)
    v = _rand((1, 2, 25, 8), 232)
    do = _rand((1, 4, 19, 8), 233)
    dq, _, _ = oracle.attn_bwd(q, k, v, do, delta=6)
    rows = [0, 7, 18, 40, 75]
    dq_r, o_r, l_r = oracle.attn_bwd_dq_rows(q, k, v, do, delta=6, rows=rows)
    assert np.abs(dq_r - dq.reshape(-1, 8)[rows]).max() < 1e-14
    o, l = oracle.attn_fwd(q, k, v, delta=6, rows=rows)
    assert np.abs(o_r - o).max() < 1e-15 and np.abs(l_r - l).max() < 1e-15


# --------------------------------------------------------------------------
# dilated attention
# --------------------------------------------------------------------------

def test_dilated_single_dense_branch_is_full_attention():
    n, d = 48, 8
    q = _rand((1, 2, n, d), 300)
    k = _rand((1, 2, n, d), 301)
    v = _rand((1, 2, n, d), 302)
    o, lse = oracle.dilated_fwd(q, k, v, [n], [1])
    assert np.abs(o - _sdpa(q, k, v)).max() < 1e-12
    o2, l2 = oracle.attn_fwd(q, k, v)
    assert np.abs(lse - l2).max() < 1e-13
    oc, _ = oracle.dilated_fwd(q, k, v, [n], [1], causal=True)
    assert np.abs(oc - _sdpa(q, k, v, mask=_causal_mask(n, n, 0))).max() < 1e-12


def test_dilated_r1_short_segments_is_block_diagonal():
    n, w, d = 48, 12, 8
    q = _rand((1, 1, n, d), 310)
    k = _rand((1, 1, n, d), 311)
    v = _rand((1, 1, n, d), 312)
    o, _ = oracle.dilated_fwd(q, k, v, [w], [1])
    blk = (np.arange(n)[:, None] // w) == (np.arange(n)[None, :] // w)
    assert np.abs(o - _sdpa(q, k, v, mask=blk)).max() < 1e-12


def _multiplicity(n, ws, rs, causal, shift=0):
    """c[p, j]: how many branches let query p attend key j (segment-relative
    dilation: offset inside the length-w segment equal to shift mod r plus a
    multiple of r)."""
    c = np.zeros((n, n))
    pos = np.arange(n)
    for w, r in zip(ws, rs):
        off = pos % w - shift % r
        sel = (off >= 0) & (off % r == 0)
        same = (pos[:, None] // w) == (pos[None, :] // w)
        m = same & sel[:, None] & sel[None, :]
        if causal:
            m &= pos[None, :] <= pos[:, None]
        c += m
    return c


@pytest.mark.parametrize("ws,rs,causal", [
    ((8, 16, 32, 64), (1, 2, 4, 8), False),
    ((8, 16, 32, 64), (1, 2, 4, 8), True),
    ((12, 24, 48), (1, 6, 12), False),   # dilations that do not divide 2^k
    ((16, 64), (2, 4), False),           # odd positions unselected
])
def test_dilated_equals_multiset_union_attention(ws, rs, causal):
    # Folding branch partials with the LSE merge equals one softmax over the
    # multiset union of each query's branch key sets: a library attention with
    # additive bias log(multiplicity).
    n, d = 64, 8
    q = _rand((1, 2, n, d), 320)
    k = _rand((1, 2, n, d), 321)
    v = _rand((1, 2, n, d), 322)
    o, lse = oracle.dilated_fwd(q, k, v, ws, rs, causal=causal)
    c = _multiplicity(n, ws, rs, causal)
    live = c.sum(1) > 0
    with np.errstate(divide="ignore"):
        bias = np.log(c)
    ref = _sdpa(q[:, :, live], k, v, mask=bias[live])
    assert np.abs(o[:, :, live] - ref).max() < 1e-12
    assert np.all(o[:, :, ~live] == 0) and np.all(np.isneginf(lse[:, :, ~live]))
    # LSE pin via Q = 0: LSE_p = ln(sum_j c[p, j])
    _, l0 = oracle.dilated_fwd(np.zeros_like(q), k, v, ws, rs, causal=causal)
    assert np.abs(l0[0, 0, live] - np.log(c.sum(1)[live])).max() < 1e-12


def test_dilated_page_branch_lists_fixture():
    # The page's own mixture (w = 2048..32768, r = {1,2,4,6,12}) scaled down
    # by 1/256 keeps the structure (r = 6, 12 do not divide w) and still pins
    # against the multiset-union formulation.
    with open(os.path.join(GOLDEN, "longnet_branches.json")) as f:
        fx = json.load(f)
    ws = [w // 256 for w in fx["page"]["segment_lengths"]]
    rs = fx["page"]["dilations"]
    assert ws == [8, 16, 32, 64, 128] and rs == [1, 2, 4, 6, 12]
    n, d = 128, 8
    q = _rand((1, 1, n, d), 330)
    k = _rand((1, 1, n, d), 331)
    v = _rand((1, 1, n, d), 332)
    o, _ = oracle.dilated_fwd(q, k, v, ws, rs)
    c = _multiplicity(n, ws, rs, False)
    with np.errstate(divide="ignore"):
        bias = np.log(c)
    assert np.abs(o - _sdpa(q, k, v, mask=bias)).max() < 1e-12


@pytest.mark.parametrize("ws,rs,causal,group", [
    ((8, 16, 32, 64), (1, 2, 4, 8), False, 1),
    ((12, 40, 64), (1, 3, 6), True, 1),      # tails; offsets past a tail's end
    ((16, 64), (2, 4), False, 2),            # no dense branch; GQA
])
def test_dilated_head_shift_equals_per_head_multiset_union(ws, rs, causal, group):
    # With head-dependent offsets, query head h of branch (w, r) selects the
    # positions at offset h mod r (plus multiples of r) inside each segment;
    # per head this is again one softmax over a multiset union, built here
    # from positions alone and checked with a library attention.
    n, d, hq = 64, 8, 8 * group
    q = _rand((1, hq, n, d), 350)
    k = _rand((1, 8, n, d), 351)
    v = _rand((1, 8, n, d), 352)
    o, lse = oracle.dilated_fwd(q, k, v, ws, rs, causal=causal, head_shift=True)
    o0, _ = oracle.dilated_fwd(q, k, v, ws, rs, causal=causal)
    assert np.abs(o - o0).max() > 1e-3          # the option changes the function
    for h in range(hq):
        c = _multiplicity(n, ws, rs, causal, shift=h)
        live = c.sum(1) > 0
        with np.errstate(divide="ignore"):
            bias = np.log(c)
        g = h // group
        ref = _sdpa(q[:, h:h + 1, live], k[:, g:g + 1], v[:, g:g + 1], mask=bias[live])
        assert np.abs(o[:, h:h + 1, live] - ref).max() < 1e-12, h
        assert np.all(o[:, h, ~live] == 0) and np.all(np.isneginf(lse[:, h, ~live]))


def test_dilated_head_shift_single_branch_is_strided_attention():
    # One branch (w = N, r = H): head h attends among positions h, h + r, ...
    # only, so it is plain attention on that strided subsequence, and across
    # heads every position is selected exactly once.
    n, d, r = 60, 8, 4
    q = _rand((1, r, n, d), 360)
    k = _rand((1, r, n, d), 361)
    v = _rand((1, r, n, d), 362)
    o, lse = oracle.dilated_fwd(q, k, v, [n], [r], head_shift=True)
    covered = np.zeros(n, int)
    for h in range(r):
        sub = slice(h, n, r)
        ref = _sdpa(q[:, h:h + 1, sub], k[:, h:h + 1, sub], v[:, h:h + 1, sub])
        assert np.abs(o[:, h:h + 1, sub] - ref).max() < 1e-12
        live = np.isfinite(lse[0, h])
        assert np.array_equal(np.flatnonzero(live), np.arange(h, n, r))
        covered += live
    assert np.all(covered == 1)


def test_dilated_row_subset():
    n, d = 64, 8
    q = _rand((1, 2, n, d), 340)
    k = _rand((1, 2, n, d), 341)
    v = _rand((1, 2, n, d), 342)
    o, l = oracle.dilated_fwd(q, k, v, (16, 32, 64), (1, 2, 4))
    rows = [0, 3, 64, 127]
    o2, l2 = oracle.dilated_fwd(q, k, v, (16, 32, 64), (1, 2, 4), rows=rows)
    assert np.array_equal(o2, o.reshape(-1, d)[rows])
    assert np.array_equal(l2, l.reshape(-1)[rows])


# --------------------------------------------------------------------------
# dilated attention backward
# --------------------------------------------------------------------------

@pytest.mark.parametrize("ws,rs,causal,group", [
    ((8, 16, 32), (1, 2, 4), False, 1),
    ((8, 16, 32), (1, 2, 4), True, 2),
    ((12, 24), (2, 6), False, 1),          # unselected positions, r not 2^k
])
def test_dilated_bwd_matches_library_autograd(ws, rs, causal, group):
    # Library autograd through attention with the additive log-multiplicity
    # bias (the multiset-union form of the branch fold).
    n, d = 32, 8
    q = _rand((1, 2 * group, n, d), 400)
    k = _rand((1, 2, n, d), 401)
    v = _rand((1, 2, n, d), 402)
    do = _rand((1, 2 * group, n, d), 403)
    dq, dk, dv = oracle.dilated_bwd(q, k, v, do, ws, rs, causal=causal)
    c = _multiplicity(n, ws, rs, causal)
    live = c.sum(1) > 0
    with np.errstate(divide="ignore"):
        bias = torch.from_numpy(np.log(c[live]))
    qt = torch.from_numpy(q.astype(np.float64)).requires_grad_()
    kt = torch.from_numpy(k.astype(np.float64)).requires_grad_()
    vt = torch.from_numpy(v.astype(np.float64)).requires_grad_()
    o = F.scaled_dot_product_attention(qt[:, :, live], kt.repeat_interleave(group, 1),
                                       vt.repeat_interleave(group, 1), attn_mask=bias)
    (o * torch.from_numpy(do[:, :, live].astype(np.float64))).sum().backward()
    assert np.abs(dq - qt.grad.numpy()).max() < 1e-12
    assert np.abs(dk - kt.grad.numpy()).max() < 1e-12
    assert np.abs(dv - vt.grad.numpy()).max() < 1e-12
    assert np.all(dq[:, :, ~live] == 0)


@pytest.mark.parametrize("ws,rs,causal,group", [
    ((8, 16, 32), (1, 2, 4), True, 1),
    ((12, 24), (2, 6), False, 2),          # GQA: a KV head serves two offsets
])
def test_dilated_bwd_head_shift_matches_library_autograd(ws, rs, causal, group):
    n, d, hq = 32, 8, 4 * group
    q = _rand((1, hq, n, d), 440)
    k = _rand((1, 4, n, d), 441)
    v = _rand((1, 4, n, d), 442)
    do = _rand((1, hq, n, d), 443)
    dq, dk, dv = oracle.dilated_bwd(q, k, v, do, ws, rs, causal=causal, head_shift=True)
    qt = torch.from_numpy(q.astype(np.float64)).requires_grad_()
    kt = torch.from_numpy(k.astype(np.float64)).requires_grad_()
    vt = torch.from_numpy(v.astype(np.float64)).requires_grad_()
    dot = torch.from_numpy(do.astype(np.float64))
    loss = 0
    for h in range(hq):
        c = _multiplicity(n, ws, rs, causal, shift=h)
        live = c.sum(1) > 0
        with np.errstate(divide="ignore"):
            bias = torch.from_numpy(np.log(c[live]))
        g = h // group
        o = F.scaled_dot_product_attention(qt[:, h:h + 1, live], kt[:, g:g + 1],
                                           vt[:, g:g + 1], attn_mask=bias)
        loss = loss + (o * dot[:, h:h + 1, live]).sum()
    loss.backward()
    assert np.abs(dq - qt.grad.numpy()).max() < 1e-12
    assert np.abs(dk - kt.grad.numpy()).max() < 1e-12
    assert np.abs(dv - vt.grad.numpy()).max() < 1e-12


def test_dilated_bwd_finite_differences():
    n, d = 12, 4
    ws, rs = (4, 12), (1, 3)
    q = _rand((1, 1, n, d), 410, quant=6)
    k = _rand((1, 1, n, d), 411, quant=6)
    v = _rand((1, 1, n, d), 412, quant=6)
    do = _rand((1, 1, n, d), 413, quant=6)
    dq, dk, dv = oracle.dilated_bwd(q, k, v, do, ws, rs)

    def loss(qq, kk, vv):
        o, _ = oracle.dilated_fwd(qq, kk, vv, ws, rs)
        return float((o * do.astype(np.float64)).sum())

    def fd(which, idx, h):
        args = [q.copy(), k.copy(), v.copy()]
        args[which][idx] += np.float32(h)
        lp = loss(*args)
        args[which][idx] -= np.float32(2 * h)
        return (lp - loss(*args)) / (2 * h)

    for which, grad in ((0, dq), (1, dk), (2, dv)):
        arr = (q, k, v)[which]
        for idx in np.ndindex(arr.shape):
            h = 2.0 ** -9
            g = (4 * fd(which, idx, h / 2) - fd(which, idx, h)) / 3
            assert abs(g - grad[idx]) < 1e-8 * max(1.0, abs(grad[idx])), (which, idx)


def test_dilated_bwd_invariants():
    # every position selected by the dense first branch: sum_j dV_j = sum_p dO_p
    # and sum_j dK_j = 0 per KV head
    n, d = 64, 8
    q = _rand((1, 2, n, d), 420)
    k = _rand((1, 1, n, d), 421)
    v = _rand((1, 1, n, d), 422)
    do = _rand((1, 2, n, d), 423)
    _, dk, dv = oracle.dilated_bwd(q, k, v, do, (16, 32, 64), (1, 2, 4), causal=True)
    assert np.abs(dv.sum(axis=2)[0, 0] - do.astype(np.float64).sum(axis=(1, 2))[0]).max() < 1e-12
    assert np.abs(dk.sum(axis=2)).max() < 1e-12


@pytest.mark.parametrize("ws,rs,causal", [
    ((16, 40, 100), (1, 3, 8), True),     # tails, dilations not dividing w
    ((24, 96), (2, 4), False),            # odd positions unselected
])
def test_dilated_bwd_dq_equals_segment_bwd_over_listed_keys(ws, rs, causal):
    # The full-size GPU check of dilated dQ runs the segment backward on each
    # sampled row's listed keys (repeated once per listing branch); on small
    # inputs that equals the dilated backward row by row, and the listing
    # agrees with the multiplicity matrix.
    from tests.parity import dilated_key_list
    n, d = 90, 8
    q = _rand((1, 2, n, d), 430)
    k = _rand((1, 1, n, d), 431)
    v = _rand((1, 1, n, d), 432)
    do = _rand((1, 2, n, d), 433)
    dq, _, _ = oracle.dilated_bwd(q, k, v, do, ws, rs, causal=causal)
    c = _multiplicity(n, ws, rs, causal)
    for p in range(n):
        keys = dilated_key_list(p, n, ws, rs, causal)
        assert np.array_equal(np.bincount(keys, minlength=n), c[p])
        for h in range(2):
            if len(keys) == 0:
                assert np.all(dq[0, h, p] == 0)
                continue
            ref, _, _ = oracle.attn_bwd_dq_rows(q[0, h:h + 1, p:p + 1], k[0][:, keys],
                                                v[0][:, keys], do[0, h:h + 1, p:p + 1])
            assert np.abs(ref[0] - dq[0, h, p]).max() < 1e-12 * max(1.0, np.abs(ref).max())
