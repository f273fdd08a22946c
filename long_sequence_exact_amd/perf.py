"""Per-workload timing of the HIP path (one JSON line per workload).

    python -m long_sequence_exact_amd.perf [--workload NAME ...] [--reps R]

For each synthetic workload the whole hot path is timed with HIP events on
the launch stream, inputs already resident in HBM:
  ring_16k_bf16       8 ranks x 8 KV segments, fused-merge ring sweep, one launch
                      per step for all ranks (also timed with the ranks split
                      over 2 streams)
  ring_16k_bf16_zigzag  the same with the load-balanced zigzag split (ranks over
                      2 streams; also timed on one)
  ulysses_128k_bf16   one causal forward launch (the benchmark's step); also the
                      same input as 8 KV segments of 16384 through the fused merge
  longnet_32k_bf16    dilated attention, 5 branches merged by LSE; its backward
  longnet_page_32k_bf16  causal, r = 1,2,4,6,12: single-GPU and split over 4
                      emulated devices (all-gathered long segments), fwd + bwd;
                      also with head-dependent offsets
  usp_gqa_256k_bf16   forward sweep over 8 KV blocks, then backward sweep
  ulysses_relayout    a rank's [16384, 32, 128] bf16 shard to its all-to-all send
                      buffer [8][16384][4][128] and back, in GB/s
  lse_merge           standalone merge of two [32, 16384, 128] partials
                      (fp32 accumulator + bf16 partial), reported in GB/s
  ulysses_len_sweep   the 128K call's shape (4 heads, d = 128, causal, one
                      launch) at 16K, 32K, 64K, 128K and 256K tokens
  short_calls         d = 128 calls with fewer 256-row query tiles than
                      compute units, with the key-range split (default) and
                      without it (split=False): 4 heads causal at 2K, 4K, 8K;
                      1 head causal at 32K; 1 head non-causal at 16K
FLOPs are algorithmic (4*d per visible pair forward, 10*d backward); bytes
for the merge are the tensors read and written.  The ring lines also time
every (rank, step) call alone, as on a device of its own, and report the
critical path (sum over steps of the slowest rank) and the load balance.
"""
from __future__ import annotations

import argparse
import json

import torch

from . import (attn_segment_bwd, attn_segment_fwd, dilated_attn_bwd, dilated_attn_fwd,
               emulate, head_relayout, lse_merge)
from .synth import WORKLOADS, draw, workload_inputs

PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CUs x 4096 FLOP/clk x 2.4 GHz
PEAK_GBS = 8000.0


def pairs(nq, nk, delta):
    """Visible (query, key) pairs with key j visible to query i iff j <= i + delta."""
    if delta is None:
        return nq * nk
    tot = 0
    lo = max(0, -delta - 1)
    hi = min(nq, max(0, nk - delta - 1))
    if hi > lo:
        a, b = lo + delta + 1, hi + delta
        tot += (a + b) * (hi - lo) // 2
    tot += max(0, nq - max(lo, hi)) * nk
    return tot


def dilated_pairs(n, segment_lengths, dilations, causal, shift=0):
    """Visible (query, key) pairs summed over the branches of dilated attention
    (one head; shift: the query head under head-dependent offsets)."""
    tot = 0
    for w, r in zip(segment_lengths, dilations):
        w = min(w, n)
        off = shift % r
        for s0 in range(0, n, w):
            m = max(0, -(-(min(w, n - s0) - off) // r))
            tot += m * (m + 1) // 2 if causal else m * m
    return tot


def source_hashes():
    """sha256 prefix of every HIP/C++ source the library is built from (with
    its extra compile flags, if any)."""
    import glob
    import os
    from .build import source_digest
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    out = {}
    for f in sorted(glob.glob(os.path.join(here, "*"))):
        if f.endswith((".hip", ".cpp", ".h")):
            out[os.path.basename(f)] = source_digest(f)
    return out


def warm_up(seconds=1.0):
    """Run the forward kernel untimed for about `seconds`, so the first timed
    workload does not run at ramping clocks."""
    import time
    q, k, v = (t.to("cuda") for t in draw([(1, 4, 16384, 128)] * 3, 99))
    t0 = time.time()
    while time.time() - t0 < seconds:
        for _ in range(10):
            attn_segment_fwd(q, k, v, causal_offset=0)
        torch.cuda.synchronize()


def timed(fn, reps, warmup=3, blocks=3):
    """Per-call milliseconds: the median over `blocks` timed blocks of `reps`
    back-to-back calls (HIP events on the launch stream), after `warmup`
    untimed calls.  The first calls after another workload run at a lower
    clock; the median of several blocks keeps that out."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    per = []
    for _ in range(blocks):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(s)
        for _ in range(reps):
            fn()
        b.record(s)
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b) / reps)
    return sorted(per)[len(per) // 2]


def ring_critical_path(q, k, v, P, zigzag, reps):
    """Per-rank timing of a causal ring: each (rank, step) call runs alone on
    the GPU (as it would on its own device) and is timed with HIP events.

    Returns (critical-path ms = sum over steps of the slowest rank's call,
    mean per-rank busy ms).  Their ratio is the ring's load balance; transfers
    between ranks are not modelled.
    """
    n = q.shape[-2]
    out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    calls = {}  # (rank, step) -> list of thunks
    if zigzag:
        step_rows = n // P
        for t, (q0, qn, cnt), (k0, kn, _), delta, acc in emulate.zigzag_plan(n, P):
            for b in range(cnt):
                qs = slice(q0 + b * step_rows, q0 + b * step_rows + qn)
                ks = slice(k0 + b * step_rows, k0 + b * step_rows + kn)
                rank = (q0 + b * step_rows) // step_rows
                calls.setdefault((rank, t), []).append(
                    lambda qs=qs, ks=ks, delta=delta, acc=acc: attn_segment_fwd(
                        q[..., qs, :], k[..., ks, :], v[..., ks, :], causal_offset=delta,
                        out=out[..., qs, :], lse=lse[..., qs], accumulate=acc))
    else:
        blk = n // P
        for r in range(P):
            for t, j in enumerate(emulate.ring_order(r, P)):
                delta = (r - j) * blk
                if delta + blk - 1 < 0:
                    continue
                qs, ks = slice(r * blk, (r + 1) * blk), slice(j * blk, (j + 1) * blk)
                calls.setdefault((r, t), []).append(
                    lambda qs=qs, ks=ks, delta=delta, t=t: attn_segment_fwd(
                        q[..., qs, :], k[..., ks, :], v[..., ks, :], causal_offset=delta,
                        out=out[..., qs, :], lse=lse[..., qs], accumulate=t > 0))
    ms = {key: timed(lambda fns=fns: [f() for f in fns], reps) for key, fns in calls.items()}
    crit = sum(max(ms.get((r, t), 0.0) for r in range(P)) for t in range(P))
    busy = sum(ms.values()) / P
    return crit, busy


def run(name, reps):
    dev = "cuda"
    if name == "lse_merge":
        H, N, d = 32, 16384, 128
        oa, ob = draw([(1, H, N, d), (1, H, N, d)], 11, torch.float32)
        la, lb = draw([(1, H, N), (1, H, N)], 12, torch.float32)
        oa, la, lb = oa.to(dev), la.to(dev), lb.to(dev)
        ob = ob.to(torch.bfloat16).to(dev)
        ms = timed(lambda: lse_merge(oa, la, ob, lb), reps)
        nbytes = oa.numel() * 4 * 2 + ob.numel() * 2 + la.numel() * 4 * 2 + lb.numel() * 4
        return {"workload": name, "ms": round(ms, 4), "GB/s": round(nbytes / ms / 1e6, 1),
                "frac_hbm_peak": round(nbytes / ms / 1e6 / PEAK_GBS, 3), "bytes": nbytes}
    if name == "ulysses_relayout":
        # one rank of Ulysses at 8 ranks x 32 heads, 131072 tokens, d = 128:
        # its [16384, 32, 128] bf16 shard <-> the [8][16384][4][128] send buffer
        P, ns, H, d = 8, 16384, 32, 128
        hp = H // P
        x = torch.randn((ns, H, d), device=dev).to(torch.bfloat16)
        buf = torch.empty((P, ns, hp, d), dtype=torch.bfloat16, device=dev)
        xs = x.as_strided((1, H, ns, d), (0, d, H * d, 1))
        bs = buf.as_strided((P, hp, ns, d), (ns * hp * d, d, hp * d, 1))
        ms_p = timed(lambda: head_relayout(xs, bs), reps)
        ms_u = timed(lambda: head_relayout(bs, xs), reps)
        nbytes = 2 * x.numel() * 2
        return {"workload": name, "bytes": nbytes, "pack_ms": round(ms_p, 4),
                "pack_GB/s": round(nbytes / ms_p / 1e6, 1),
                "unpack_ms": round(ms_u, 4), "unpack_GB/s": round(nbytes / ms_u / 1e6, 1),
                "frac_hbm_peak": round(nbytes / max(ms_p, ms_u) / 1e6 / PEAK_GBS, 3)}
    w = WORKLOADS.get(name)
    if name == "ring_16k_bf16":
        q, k, v = (t.to(dev) for t in workload_inputs(w))
        # a few more untimed passes: the first multi-stream passes after another
        # workload run slow
        ms = timed(lambda: emulate.ring_fwd(q, k, v, w.segments, causal=True), reps, warmup=6)
        alt = 2
        ms1 = timed(lambda: emulate.ring_fwd(q, k, v, w.segments, causal=True, lanes=alt), reps,
                    warmup=6)
        fl = 4.0 * w.d * w.hq * pairs(w.nq, w.nk, 0)
        crit, busy = ring_critical_path(q, k, v, w.segments, False, reps)
    elif name == "ring_16k_bf16_zigzag":
        w = WORKLOADS["ring_16k_bf16"]
        order = torch.tensor(emulate.zigzag_order(w.nq, w.segments), device=dev)
        q, k, v = (t.to(dev)[:, :, order].contiguous() for t in workload_inputs(w))
        out = torch.empty(q.shape, dtype=torch.float32, device=dev)
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
        ms = timed(lambda: emulate.zigzag_ring_fwd(q, k, v, w.segments, out=out, lse=lse), reps,
                   warmup=6)
        alt = 1
        ms1 = timed(lambda: emulate.zigzag_ring_fwd(q, k, v, w.segments, out=out, lse=lse,
                                                    lanes=alt), reps, warmup=6)
        fl = 4.0 * w.d * w.hq * pairs(w.nq, w.nk, 0)
        crit, busy = ring_critical_path(q, k, v, w.segments, True, reps)
    elif name == "ulysses_128k_bf16":
        q, k, v = (t.to(dev) for t in workload_inputs(w))
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
        ms = timed(lambda: attn_segment_fwd(q, k, v, causal_offset=0, out=out, lse=lse), reps)
        fl = 4.0 * w.d * w.hq * pairs(w.nq, w.nk, 0)
        # the same input as 8 KV segments of 16384 through the fused merge
        del out
        acc = torch.empty(q.shape, dtype=torch.float32, device=dev)
        ms_s = timed(lambda: emulate.sweep_fwd(q, k, v, 8, 0, True, acc, lse), reps)
    elif name == "ulysses_len_sweep":
        # the 128K call's shape (4 heads, d = 128, causal, one launch) at
        # 16K ... 256K tokens
        w = WORKLOADS["ulysses_128k_bf16"]
        res = {"workload": name}
        for n in (16384, 32768, 65536, 131072, 262144):
            q, k, v = draw([(1, w.hq, n, w.d)] * 3, 20 + n // 16384, torch.bfloat16)
            q, k, v = q.to(dev), k.to(dev), v.to(dev)
            out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
            lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
            ms_n = timed(lambda: attn_segment_fwd(q, k, v, causal_offset=0, out=out, lse=lse),
                         max(2, reps * 131072 // n // 4))
            fl_n = 4.0 * w.d * w.hq * pairs(n, n, 0)
            res[f"{n // 1024}k_ms"] = round(ms_n, 3)
            res[f"{n // 1024}k_TFLOP/s"] = round(fl_n / ms_n / 1e9, 1)
            del q, k, v, out, lse
        return res
    elif name == "short_calls":
        res = {"workload": name}
        for tag, hq, n, delta in (("4h_2k", 4, 2048, 0), ("4h_4k", 4, 4096, 0),
                                  ("4h_8k", 4, 8192, 0), ("1h_32k", 1, 32768, 0),
                                  ("1h_16k_noncausal", 1, 16384, None)):
            q, k, v = draw([(1, hq, n, 128)] * 3, 20 + n // 1024 + hq, torch.bfloat16)
            q, k, v = q.to(dev), k.to(dev), v.to(dev)
            out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
            lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
            ws = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
            fl_n = 4.0 * 128 * hq * pairs(n, n, delta)
            for sp in (True, False):
                ms_n = timed(lambda: attn_segment_fwd(q, k, v, causal_offset=delta, out=out,
                                                      lse=lse, workspace=ws, split=sp),
                             max(4, reps * 4))
                key = tag if sp else tag + "_unsplit"
                res[f"{key}_ms"] = round(ms_n, 4)
                res[f"{key}_TFLOP/s"] = round(fl_n / ms_n / 1e9, 1)
            del q, k, v, out, lse, ws
        return res
    elif name == "longnet_32k_bf16":
        q, k, v, do = (t.to(dev) for t in workload_inputs(w, with_dout=True))
        out = torch.empty(q.shape, dtype=torch.float32, device=dev)
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
        ms = timed(lambda: dilated_attn_fwd(q, k, v, w.segment_lengths, w.dilations,
                                            out=out, lse=lse), reps)
        npairs = dilated_pairs(w.nq, w.segment_lengths, w.dilations, w.causal)
        fl = 4.0 * w.d * w.hq * npairs
        dq = torch.zeros(q.shape, dtype=torch.float32, device=dev)
        dk = torch.empty(k.shape, dtype=torch.float32, device=dev)
        dv = torch.empty(v.shape, dtype=torch.float32, device=dev)
        ms_b = timed(lambda: dilated_attn_bwd(q, k, v, out, lse, do, w.segment_lengths,
                                              w.dilations, dq=dq, dk=dk, dv=dv), reps)
        fl_b = 10.0 * w.d * w.hq * npairs
        return {"workload": name, "ms": round(ms, 3), "TFLOP/s": round(fl / ms / 1e9, 1),
                "frac_peak": round(fl / ms / 1e9 / PEAK_TFLOPS, 3), "flop": fl,
                "bwd_ms": round(ms_b, 3), "bwd_TFLOP/s": round(fl_b / ms_b / 1e9, 1),
                "bwd_frac_peak": round(fl_b / ms_b / 1e9 / PEAK_TFLOPS, 3)}
    elif name == "longnet_page_32k_bf16":
        q, k, v, do = (t.to(dev) for t in workload_inputs(w, with_dout=True))
        ws, rs, P = w.segment_lengths, w.dilations, w.segments
        out = torch.empty(q.shape, dtype=torch.float32, device=dev)
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
        ms = timed(lambda: dilated_attn_fwd(q, k, v, ws, rs, causal=True, out=out, lse=lse),
                   reps)
        dq = torch.zeros(q.shape, dtype=torch.float32, device=dev)
        dk = torch.empty(k.shape, dtype=torch.float32, device=dev)
        dv = torch.empty(v.shape, dtype=torch.float32, device=dev)
        ms_b = timed(lambda: dilated_attn_bwd(q, k, v, out, lse, do, ws, rs, causal=True,
                                              dq=dq, dk=dk, dv=dv), reps)
        ms_sf = timed(lambda: emulate.longnet_split_fwd(q, k, v, ws, rs, P, causal=True), reps)
        ms_sb = timed(lambda: emulate.longnet_split_bwd(q, k, v, out, lse, do, ws, rs, P,
                                                        causal=True), reps)
        # head-dependent offsets: one launch per residue class of heads
        ms_hf = timed(lambda: dilated_attn_fwd(q, k, v, ws, rs, causal=True, out=out, lse=lse,
                                               head_shift=True), reps)
        ms_hb = timed(lambda: dilated_attn_bwd(q, k, v, out, lse, do, ws, rs, causal=True,
                                               dq=dq, dk=dk, dv=dv, head_shift=True), reps)
        hpairs = sum(dilated_pairs(w.nq, ws, rs, True, shift=h) for h in range(w.hq))
        fl_h, fl_hb = 4.0 * w.d * hpairs, 10.0 * w.d * hpairs
        npairs = dilated_pairs(w.nq, ws, rs, True)
        fl, fl_b = 4.0 * w.d * w.hq * npairs, 10.0 * w.d * w.hq * npairs
        return {"workload": name, "ms": round(ms, 3), "TFLOP/s": round(fl / ms / 1e9, 1),
                "frac_peak": round(fl / ms / 1e9 / PEAK_TFLOPS, 3), "flop": fl,
                "bwd_ms": round(ms_b, 3), "bwd_TFLOP/s": round(fl_b / ms_b / 1e9, 1),
                "split_devices": P, "split_fwd_ms": round(ms_sf, 3),
                "split_fwd_TFLOP/s": round(fl / ms_sf / 1e9, 1),
                "split_bwd_ms": round(ms_sb, 3),
                "split_bwd_TFLOP/s": round(fl_b / ms_sb / 1e9, 1),
                "head_shift_fwd_ms": round(ms_hf, 3),
                "head_shift_fwd_TFLOP/s": round(fl_h / ms_hf / 1e9, 1),
                "head_shift_bwd_ms": round(ms_hb, 3),
                "head_shift_bwd_TFLOP/s": round(fl_hb / ms_hb / 1e9, 1)}
    elif name == "usp_gqa_256k_bf16":
        q, k, v, do = (t.to(dev) for t in workload_inputs(w, with_dout=True))
        blk = w.nk // w.segments
        npairs = sum(pairs(w.nq, blk, (w.q_block - j) * blk) for j in range(w.segments))
        out = torch.empty(q.shape, dtype=torch.float32, device=dev)
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
        ms_f = timed(lambda: emulate.sweep_fwd(q, k, v, w.segments, w.q_block, True, out, lse),
                     reps)
        dq = torch.zeros(q.shape, dtype=torch.float32, device=dev)
        dk = torch.empty(k.shape, dtype=torch.float32, device=dev)
        dv = torch.empty(v.shape, dtype=torch.float32, device=dev)
        ms_b = timed(lambda: emulate.usp_bwd(q, k, v, out, lse, do, w.segments, w.q_block,
                                             True, dq=dq, dk=dk, dv=dv), reps)
        fl_f = 4.0 * w.d * w.hq * npairs
        fl_b = 10.0 * w.d * w.hq * npairs
        return {"workload": name, "fwd_ms": round(ms_f, 3), "bwd_ms": round(ms_b, 3),
                "fwd_TFLOP/s": round(fl_f / ms_f / 1e9, 1),
                "bwd_TFLOP/s": round(fl_b / ms_b / 1e9, 1),
                "fwd_frac_peak": round(fl_f / ms_f / 1e9 / PEAK_TFLOPS, 3),
                "bwd_frac_peak": round(fl_b / ms_b / 1e9 / PEAK_TFLOPS, 3)}
    else:
        raise ValueError(name)
    res = {"workload": name, "ms": round(ms, 3), "TFLOP/s": round(fl / ms / 1e9, 1),
           "frac_peak": round(fl / ms / 1e9 / PEAK_TFLOPS, 3), "flop": fl}
    if name == "ulysses_128k_bf16":
        res.update({"segments_8x16k_ms": round(ms_s, 3),
                    "segments_8x16k_TFLOP/s": round(fl / ms_s / 1e9, 1)})
    if name.startswith("ring_16k"):
        # `ms`: the ring function's default stream lanes; the other count for comparison
        res.update({"alt_lanes": alt, "alt_lanes_ms": round(ms1, 3),
                    "alt_lanes_TFLOP/s": round(fl / ms1 / 1e9, 1)})
    if name.startswith("ring_16k"):
        # one device per rank: per-step slowest rank, summed over the steps
        res.update({"rank_critical_path_ms": round(crit, 3),
                    "rank_mean_busy_ms": round(busy, 3),
                    "rank_balance": round(busy / crit, 3)})
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", nargs="*",
                    default=["ulysses_128k_bf16", "ring_16k_bf16", "ring_16k_bf16_zigzag",
                             "longnet_32k_bf16", "longnet_page_32k_bf16",
                             "usp_gqa_256k_bf16", "ulysses_relayout", "lse_merge",
                             "ulysses_len_sweep", "short_calls"])
    ap.add_argument("--reps", type=int, default=10)
    args = ap.parse_args()
    print(json.dumps({"kernel_sources_sha256_16": source_hashes(),
                      "device": torch.cuda.get_device_name(0)}), flush=True)
    warm_up()
    for name in args.workload:
        print(json.dumps(run(name, args.reps)), flush=True)


if __name__ == "__main__":
    main()
