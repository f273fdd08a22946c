"""Seeded synthetic inputs shared by the GPU path's tests/benchmark and the oracle.

This module draws random numbers and nothing else: it holds none of the
attention arithmetic.  Tensors are drawn on the host with a seeded
``torch.Generator`` as float32 standard normals, in the order the caller lists
them, and then cast (round-to-nearest-even) to the compute dtype.  Both sides
read the same host tensors: the GPU path copies them to the device, the oracle
reads their exact values upcast to float32.

The workloads are shaped like those the pages discuss: segment-per-device
attention at 16K-256K tokens ("Boosting Spec Eagle: USP For Long-Context
Training", The Challenge; "Ultra-Long Sequence Distributed Transformer",
Abstract) and LongNet's segment-length / dilation mixture ("LongNet: Scaling
Transformers to 1,000,000,000 Tokens", Results).  Token values do not change
the cost of exact attention, so iid Gaussian entries stand in for the text
corpora the pages train on.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch


def draw(shapes, seed: int, dtype=torch.bfloat16):
    """Draw one float32 N(0,1) tensor per shape, in order, then cast."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    out = []
    for s in shapes:
        t = torch.randn(tuple(s), generator=g, dtype=torch.float32)
        out.append(t.to(dtype) if dtype != torch.float32 else t)
    return out


def sample_rows(n_total: int, count: int, seed: int, must=()):
    """A sorted seeded subset of row indices [0, n_total), always holding ``must``."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    count = min(count, n_total)
    picked = set(int(m) % n_total for m in must if n_total > 0)
    perm = torch.randperm(n_total, generator=g)
    for x in perm.tolist():
        if len(picked) >= count:
            break
        picked.add(int(x))
    return sorted(picked)


@dataclass(frozen=True)
class Workload:
    """Shapes and seed of one synthetic workload ([B,H,N,d], B = 1)."""
    name: str
    dtype: torch.dtype
    hq: int
    hkv: int
    nq: int
    nk: int
    d: int
    causal: bool
    seed: int
    segments: int = 1            # KV segments swept with LSE merges
    q_block: int = 0             # which KV-block-sized query block (causal offset)
    segment_lengths: tuple = field(default_factory=tuple)
    dilations: tuple = field(default_factory=tuple)


WORKLOADS = {
    # fp32 correctness case: 1 head, d=64, 1024 tokens as 4 KV segments of 256.
    "tiny_fp32_segments": Workload("tiny_fp32_segments", torch.float32, 1, 1,
                                   1024, 1024, 64, False, 0, segments=4),
    # ring step emulation: 32 heads, d=128, 16384 tokens, 8 ranks x 2048 rows.
    "ring_16k_bf16": Workload("ring_16k_bf16", torch.bfloat16, 32, 32, 16384,
                              16384, 128, True, 1, segments=8),
    # Ulysses post-all-to-all share: 4 of 32 heads at the full 131072 tokens.
    "ulysses_128k_bf16": Workload("ulysses_128k_bf16", torch.bfloat16, 4, 4,
                                  131072, 131072, 128, True, 2),
    # LongNet mixture: 16 heads, d=64, 32768 tokens, w = 2048..32768.
    "longnet_32k_bf16": Workload("longnet_32k_bf16", torch.bfloat16, 16, 16,
                                 32768, 32768, 64, False, 3,
                                 segment_lengths=(2048, 4096, 8192, 16384, 32768),
                                 dilations=(1, 2, 4, 8, 16)),
    # LongNet's language-model setting: w = 2048..32768 with r = 1, 2, 4, 6, 12
    # (r does not divide w for the last two branches), causal; split over
    # 4 devices of 8192 tokens for the distributed emulation (segments = 4).
    "longnet_page_32k_bf16": Workload("longnet_page_32k_bf16", torch.bfloat16, 16, 16,
                                      32768, 32768, 64, True, 5, segments=4,
                                      segment_lengths=(2048, 4096, 8192, 16384, 32768),
                                      dilations=(1, 2, 4, 6, 12)),
    # USP share: GQA 8/2 heads, local Q block 7 of 8 (32768 rows) against
    # 8 KV blocks of 32768 (262144 keys), forward + backward.
    "usp_gqa_256k_bf16": Workload("usp_gqa_256k_bf16", torch.bfloat16, 8, 2,
                                  32768, 262144, 128, True, 4, segments=8,
                                  q_block=7),
}


def workload_inputs(w: Workload, with_dout: bool = False):
    """Q [1,Hq,Nq,d], K, V [1,Hkv,Nk,d] (and dO [1,Hq,Nq,d]) on the host."""
    shapes = [(1, w.hq, w.nq, w.d), (1, w.hkv, w.nk, w.d), (1, w.hkv, w.nk, w.d)]
    if with_dout:
        shapes.append((1, w.hq, w.nq, w.d))
    return draw(shapes, w.seed, w.dtype)


def sample_rows_per_tile(n_total: int, tile: int, per_tile: int, seed: int, must=()):
    """A sorted seeded subset of [0, n_total) with ``per_tile`` rows drawn in
    every consecutive block of ``tile`` rows (fewer in a short last block),
    always holding ``must``."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    picked = set(int(m) % n_total for m in must if n_total > 0)
    for t0 in range(0, n_total, tile):
        n = min(tile, n_total - t0)
        perm = torch.randperm(n, generator=g)[:min(per_tile, n)]
        picked.update(t0 + int(x) for x in perm.tolist())
    return sorted(picked)
