"""Benchmark: causal segmented-attention forward throughput on one MI355X.

Default workload: the Ulysses share -- 4 heads (one GPU's eighth of 32),
d = 128, the full 131072-token sequence, causal, one launch of the segment
forward with causal offset 0.  A step is one such forward over seeded,
HBM-resident bf16 inputs.  FLOPs are algorithmic: 4*d per visible (query,
key) pair, i.e. the causal-adjusted count N(N+1)/2 pairs per head.

Prints ONE JSON line (rank 0) with the throughput, a roofline object for the
forward kernel (HIP-event launch durations on the launch stream), and the
fp64 CPU oracle timed on a bounded, seeded row sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CUs x 4096 FLOP/clk x 2.4 GHz (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)
METRIC = "attention TFLOP/s (causal-adjusted) + % bf16 MFMA peak, 128K tokens, 1 GPU"
COUNTERS = os.path.join(ROOT, "profiles", "fwd_bf16_ulysses_128k_hbm_counters.json")
MFMA_COUNTERS = os.path.join(ROOT, "profiles", "fwd_bf16_ulysses_128k_mfma_counters.json")
FWD_SRC = os.path.join(ROOT, "long_sequence_exact_amd", "csrc", "fwd_bf16.hip")


def visible_pairs(nq: int, nk: int, delta: int | None) -> int:
    """Exact number of (i, j) with j <= i + delta, 0 <= i < nq, 0 <= j < nk."""
    if delta is None:
        return nq * nk
    total = 0
    # rows where the count is clamped at nk vs. growing: count_i = clamp(i+delta+1, 0, nk)
    lo = max(0, -delta - 1)             # first row with a visible key
    hi = min(nq, max(0, nk - delta - 1))  # rows [lo, hi) have count i + delta + 1 < nk
    if hi > lo:
        a, b = lo + delta + 1, hi - 1 + delta + 1
        total += (a + b) * (hi - lo) // 2
    full_from = max(lo, hi)
    if nq > full_from:
        total += (nq - full_from) * nk
    return total


def source_hash(path: str) -> str:
    """sha256 prefix of a kernel source and its extra compile flags."""
    from long_sequence_exact_amd.build import source_digest
    return source_digest(path)


def _fresh_counters(path):
    """A committed rocprofv3 counter summary, if it was taken on the current
    forward kernel source (else None)."""
    try:
        with open(path) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_sha256_16") != source_hash(FWD_SRC):
        return None
    return c


def traffic_from_counters():
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated), or None."""
    c = _fresh_counters(COUNTERS)
    return c.get("hbm_bytes_per_launch") if c else None


def mfma_busy_from_counters():
    """Fraction of SIMD cycles with the matrix core busy, or None."""
    c = _fresh_counters(MFMA_COUNTERS)
    return c.get("mfma_busy") if c else None


def cpu_baseline(q, k, v, delta, d, budget_s: float):
    """Time the fp64 oracle on a seeded row sample (about budget_s seconds)."""
    import numpy as np
    import oracle
    from long_sequence_exact_amd.synth import sample_rows

    H, N = q.shape[1], q.shape[2]
    qn, kn, vn = (t.float().numpy() for t in (q, k, v))

    def run(nrows, seed):
        rows = []
        per = max(1, nrows // H)
        for h in range(H):
            rows += [h * N + i for i in sample_rows(N, per, seed + h)]
        rows = np.array(rows, np.int64)
        flops = float(sum(4 * d * min(N, (r % N) + delta + 1) for r in rows))
        t0 = time.perf_counter()
        oracle.attn_fwd(qn, kn, vn, delta=delta, rows=rows)
        return flops, time.perf_counter() - t0, len(rows)

    f0, t0, _ = run(64, 9000)                      # pilot
    rate = f0 / max(t0, 1e-6)
    avg_row = 4 * d * (N / 2)
    nrows = int(max(64, min(N * H, budget_s * rate / avg_row)))
    f, t, n = run(nrows, 9100)
    return {"value": f / t / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{n} seeded query rows over {H} heads of the same workload "
                      f"({f / 1e9:.1f} GFLOP fp64 in {t:.1f} s); value = sampled FLOPs / time"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="ulysses_128k_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=30.0)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one device copy of this size (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "seqattn runs on one GPU only: the multi-GPU "
                                   "collectives (all-to-all, ring exchange) are not built; "
                                   "run with --gpus 1"}))
        sys.exit(2)

    import torch
    import long_sequence_exact_amd as sa
    from long_sequence_exact_amd.synth import WORKLOADS, workload_inputs

    w = WORKLOADS[args.workload]
    if w.name != "ulysses_128k_bf16":
        raise SystemExit("bench times the Ulysses-share forward; other workloads are "
                         "parity cases")
    q, k, v = workload_inputs(w)
    dev = "cuda:0"
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
    delta = 0
    pairs = visible_pairs(w.nq, w.nk, delta) * w.hq
    flops = 4.0 * w.d * pairs

    def step():
        sa.attn_segment_fwd(qd, kd, vd, causal_offset=delta, out=out, lse=lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_all0.record(stream)
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    t_all1.record(stream)
    torch.cuda.synchronize()
    total_ms = t_all0.elapsed_time(t_all1)
    launch_ms = [a.elapsed_time(b) for a, b in evs]
    ms_per_step = total_ms / args.steps
    avg_launch_ms = sum(launch_ms) / len(launch_ms)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (avg_launch_ms * 1e-3) / 1e12

    if args.calib_copy_mib:
        nbytes = args.calib_copy_mib << 20
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(q, k, v, delta, w.d, args.cpu_budget)

    rec = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "heads": w.hq, "seq_len": w.nq, "head_dim": w.d,
                   "causal": True, "batch": 1, "causal_offset": delta,
                   "visible_pairs": pairs, "flop_per_step": flops},
        "pct_bf16_mfma_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_from_counters(),
                     "mfma_busy": mfma_busy_from_counters(),
                     "kernel": "fwd_bf16_kernel<128, 64, 12, false>",
                     "avg_launch_ms": round(avg_launch_ms, 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
