"""Host-side logic on the CPU: FLOP accounting, ring schedules, seeded inputs."""
import itertools

import pytest
import torch

from bench import visible_pairs
import numpy as np

from long_sequence_exact_amd.emulate import lane_entries, ring_order, zigzag_order, zigzag_plan
from long_sequence_exact_amd.synth import WORKLOADS, draw, sample_rows


def test_visible_pairs_matches_brute_force():
    for nq, nk, d in itertools.product([0, 1, 5, 17], [0, 1, 4, 19],
                                       [None, -30, -5, -1, 0, 1, 3, 20, 40]):
        brute = sum(1 for i in range(nq) for j in range(nk) if d is None or j <= i + d)
        assert visible_pairs(nq, nk, d) == brute


def test_headline_flop_count():
    # causal 131072 tokens: N(N+1)/2 pairs per head, 4*d flops per pair, 4 heads
    n = 131072
    assert visible_pairs(n, n, 0) == n * (n + 1) // 2 == 8_590_000_128
    assert 4 * 128 * 4 * visible_pairs(n, n, 0) == 17_592_320_262_144


def test_ring_schedule_covers_causal_attention_exactly():
    # 8 ranks x 2048 rows at 16384 tokens: the non-skipped (rank, step) pairs
    # are 36 and their visible pairs sum to causal attention over 16384 tokens.
    P, blk = 8, 2048
    calls, pairs = 0, 0
    for r in range(P):
        order = ring_order(r, P)
        assert sorted(order) == list(range(P)) and order[0] == r
        for j in order:
            delta = (r - j) * blk
            if delta + blk - 1 < 0:
                continue
            calls += 1
            pairs += visible_pairs(blk, blk, delta)
    assert calls == 36
    assert pairs == visible_pairs(P * blk, P * blk, 0) == 134_225_920


@pytest.mark.parametrize("n,P", [(16, 1), (32, 2), (48, 4), (64, 8)])
def test_zigzag_plan_covers_causal_attention_once_and_balances_ranks(n, P):
    """Every causal (query, key) pair of the sequence is issued exactly once,
    no non-causal pair is issued, and each step gives every rank the same
    number of pairs (step 0: c(c+1) + c^2; later steps: 2c^2)."""
    order = np.array(zigzag_order(n, P))
    assert sorted(order) == list(range(n))
    c, step = n // (2 * P), n // P
    hits = np.zeros((n, n), np.int64)
    per_rank_step = np.zeros((P, P), np.int64)
    for t, (q0, qn, cnt), (k0, kn, kcnt), delta, acc in zigzag_plan(n, P):
        assert cnt == kcnt and acc == (t > 0)
        for b in range(cnt):
            qrows = q0 + b * step + np.arange(qn)
            krows = k0 + b * step + np.arange(kn)
            rank = int(qrows[0] // step)
            assert (qrows // step == rank).all()
            assert int(krows[0] // step) == (rank - t) % P  # the ring's KV holder
            for i, gi in enumerate(order[qrows]):
                for j, gj in enumerate(order[krows]):
                    if delta is None or j <= i + delta:
                        hits[gi, gj] += 1
                        per_rank_step[rank, t] += 1
    assert np.array_equal(hits, np.tril(np.ones((n, n), np.int64)))
    assert (per_rank_step[:, 0] == c * (c + 1) + c * c).all()
    assert (per_rank_step[:, 1:] == 2 * c * c).all()
    assert len(zigzag_plan(n, P)) == 2 * P - 1


def test_usp_share_pairs():
    w = WORKLOADS["usp_gqa_256k_bf16"]
    blk = w.nk // w.segments
    total = sum(visible_pairs(w.nq, blk, (w.q_block - j) * blk) for j in range(w.segments))
    assert total == 8_053_080_064


def test_draw_is_seeded_and_rounds_to_bf16():
    a = draw([(3, 5)], 11, torch.bfloat16)[0]
    b = draw([(3, 5)], 11, torch.bfloat16)[0]
    f = draw([(3, 5)], 11, torch.float32)[0]
    assert torch.equal(a, b)
    assert torch.equal(a, f.to(torch.bfloat16))


def test_sample_rows():
    r = sample_rows(1000, 20, 3, must=(0, -1))
    assert len(r) == 20 and 0 in r and 999 in r and r == sorted(set(r))
    assert sample_rows(1000, 20, 3, must=(0, -1)) == r
    assert sample_rows(5, 20, 1) == [0, 1, 2, 3, 4]


def test_bench_refuses_multi_gpu():
    import subprocess
    import sys
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    p = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert p.returncode == 2 and "one GPU" in p.stdout


def test_dilated_pair_count_matches_key_lists():
    from long_sequence_exact_amd.perf import dilated_pairs
    from tests.parity import dilated_key_list
    for n, ws, rs, causal in [(200, (16, 40, 100, 400), (1, 3, 8, 12), True),
                              (96, (24, 96), (2, 4), False),
                              (130, (64,), (6,), True)]:
        for shift in (0, 1, 5, 11):     # head-dependent offsets
            brute = sum(len(dilated_key_list(p, n, ws, rs, causal, shift)) for p in range(n))
            assert dilated_pairs(n, ws, rs, causal, shift) == brute


@pytest.mark.parametrize("n,P,w,r", [(32768, 4, 32768, 12), (32768, 4, 16384, 6),
                                     (1152, 3, 768, 6), (768, 4, 384, 5)])
def test_longnet_split_gathers_each_selected_row_once(n, P, w, r):
    """Every device's selected rows of a long segment land in distinct,
    consecutive slots of that segment's gathered buffer, covering it."""
    from long_sequence_exact_amd.emulate import _gathered_parts
    share = n // P
    segs, devs = _gathered_parts(n, P, share, w, r)
    for s0, count in segs:
        selected = [p for p in range(s0, min(s0 + w, n)) if (p - s0) % r == 0]
        assert len(selected) == count
        slots = []
        for dev, (seg0, p0, cnt, i0) in enumerate(devs):
            if seg0 != s0:
                continue
            mine = [p for p in selected if dev * share <= p < (dev + 1) * share]
            assert mine == list(range(p0, p0 + cnt * r, r))[:len(mine)] and len(mine) == cnt
            assert selected[i0:i0 + cnt] == mine
            slots.extend(range(i0, i0 + cnt))
        assert slots == list(range(count))


@pytest.mark.parametrize("lanes", [1, 2, 3, 4, 8])
def test_stream_lanes_partition_every_rank_batch(lanes):
    """Each launch's rank batch is split over the stream lanes by rank % lanes:
    every entry exactly once, and a rank always on the same lane."""
    for first, count in [(0, 8), (3, 5), (7, 1), (0, 1), (2, 6)]:
        seen = []
        for lane in range(lanes):
            b0, m = lane_entries(first, count, lane, lanes)
            entries = [b0 + i * lanes for i in range(m)]
            assert all((first + b) % lanes == lane for b in entries)
            seen += entries
        assert sorted(seen) == list(range(count))


def test_binding_rejects_host_tensors():
    # the kernels dereference these addresses: a host tensor must be refused
    # before anything reaches the library
    import long_sequence_exact_amd as sa
    x = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        sa.attn_segment_fwd(x, x, x, out=torch.empty(x.shape), lse=torch.empty(x.shape[:-1]))
    with pytest.raises(ValueError, match="GPU"):
        sa.lse_merge(torch.zeros((1, 1, 8, 64)), torch.zeros((1, 1, 8)),
                     torch.zeros((1, 1, 8, 64)), torch.zeros((1, 1, 8)))
    # size queries take host descriptors
    assert sa.workspace_size(3, x, x) == 8 * 4


def test_forward_counters_match_the_kernel_source():
    """The HBM and MFMA counters that bench.py reports as roofline traffic and
    mfma_busy were taken on the current forward kernel source and compile
    flags (else bench.py reports null)."""
    import json, os
    from long_sequence_exact_amd.build import source_digest
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    src = os.path.join(root, "long_sequence_exact_amd", "csrc", "fwd_bf16.hip")
    prof = os.path.join(root, "profiles", "fwd_bf16_ulysses_128k_hbm_counters.json")
    sha = source_digest(src)
    rec = json.load(open(prof))
    assert rec["kernel_source_sha256_16"] == sha
    assert rec["hbm_bytes_per_launch"] > 0
    mfma = json.load(open(prof.replace("hbm_counters", "mfma_counters")))
    assert mfma["kernel_source_sha256_16"] == sha
    assert 0 < mfma["mfma_busy"] < 1
