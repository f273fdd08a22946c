"""Single-GPU emulation of the sequence-parallel schedules (host loops only).

Every step is one library call; these functions only choose which (query
block, KV segment) pairs are issued, in which order, with which offset.

* Ring attention ("Boosting Spec Eagle: USP For Long-Context Training", The
  Solution: devices in a ring, each with a slice, passing blocks to their
  neighbours): rank r holds query block r; at step t it holds KV block
  j = (r - t) mod P, attends to it with causal offset (r - j) * block and merges
  the partial into its running (O, LSE).  Blocks entirely in the causal future
  are skipped.
* DeepSpeed-Ulysses ("DeepSpeed-Ulysses" article, Wie DeepSpeed-Ulysses
  funktioniert: after the all-to-all a GPU sees the whole sequence): one call
  on the GPU's head subset at full length; ulysses_pipeline_fwd runs P ranks
  end to end, with the re-layouts around both all-to-alls and the
  all-to-alls themselves emulated by the library's head re-layout copy.
* USP ("Boosting Spec Eagle ...", The Solution: Ulysses and Ring combined):
  a head subset swept over KV blocks like a ring rank, forward and backward.
* LongNet as a distributed trainer ("LongNet: Scaling Transformers to
  1,000,000,000 Tokens", LONGNET as a Distributed Trainer): each device holds
  N/P tokens; a branch whose segments fit in a device is computed locally,
  a longer one all-gathers the segment's selected keys/values and the local
  selected queries cross-attend to them; in the backward the all-gather
  becomes a reduce-scatter (here: accumulation into the owners' rows).
* Load-balanced causal ring ("Boosting Spec Eagle ...", Implementation
  Details and Next Steps: load balancing so that every device of the ring is
  used effectively; the plain causal ring leaves rank r idle for the P-1-r
  steps whose KV block lies in its future).  The sequence is cut into 2P
  chunks and rank r holds chunks r and 2P-1-r, so every step gives every
  rank the same number of visible pairs.
"""
from __future__ import annotations

import torch

from . import (attn_segment_bwd, attn_segment_fwd, dilated_attn_bwd, dilated_attn_fwd,
               head_relayout)


def ring_order(rank: int, P: int):
    """KV block held by `rank` at steps t = 0..P-1 of a ring."""
    return [(rank - t) % P for t in range(P)]


def sweep_fwd(q, k, v, n_blocks: int, q_block: int, causal: bool, out, lse, scale=None):
    """Forward of one query block against K/V cut into n_blocks equal blocks.

    q is the query block whose first row sits at global position
    q_block * (Nk / n_blocks); out (fp32) and lse receive the merged result.
    Returns the number of launches issued.
    """
    nk = k.shape[-2]
    if nk % n_blocks:
        raise ValueError("K/V length must split into equal blocks")
    blk = nk // n_blocks
    q_start = q_block * blk
    first = True
    launches = 0
    for j in ring_order(q_block, n_blocks):
        k_start = j * blk
        delta = q_start - k_start
        if causal and delta + q.shape[-2] - 1 < 0:
            continue  # every key of block j is in the future of every query
        kj = k[..., k_start:k_start + blk, :]
        vj = v[..., k_start:k_start + blk, :]
        attn_segment_fwd(q, kj, vj, causal_offset=delta if causal else None, scale=scale,
                         out=out, lse=lse, accumulate=not first)
        first = False
        launches += 1
    if first:  # nothing visible at all: the empty segment writes (0, -inf)
        attn_segment_fwd(q, k[..., :0, :], v[..., :0, :], scale=scale, out=out, lse=lse)
        launches += 1
    return launches


def _rows_batch(t, row0, rows, step, count):
    """View of `count` row ranges [row0 + c*step, row0 + c*step + rows) of t
    ([1,H,N,d] or [1,H,N]) as a batch: [count, H, rows(, d)]."""
    st = t.stride()
    off = t.storage_offset() + row0 * st[2]
    if t.dim() == 4:
        return t.as_strided((count, t.shape[1], rows, t.shape[3]),
                            (step * st[2], st[1], st[2], st[3]), off)
    return t.as_strided((count, t.shape[1], rows), (step * st[2], st[1], st[2]), off)


def lane_entries(first_rank: int, count: int, lane: int, lanes: int):
    """Entries of a rank batch (ranks first_rank .. first_rank + count - 1)
    that belong to stream lane `lane` of `lanes` (rank % lanes == lane):
    (index of the first such entry, how many; they are `lanes` apart)."""
    b0 = (lane - first_rank) % lanes
    return b0, len(range(b0, count, lanes))


def _blocks(t, P, blk, first_block, count):
    """View of `count` consecutive length-blk row blocks of t starting at
    block `first_block`, as a batch: [count, H, blk(, d)]."""
    return _rows_batch(t, first_block * blk, blk, blk, count)


def ring_fwd(q, k, v, P: int, causal: bool = True, scale=None, batched: bool = True,
             lanes: int = 1, out=None, lse=None):
    """All P ranks of a ring, run one after another on one GPU.

    q, k, v: [B,H,N,d]; rank r owns rows [r*N/P, (r+1)*N/P).  Returns the
    merged fp32 output [B,H,N,d] and LSE [B,H,N] of the whole sequence.

    batched=True issues one launch per ring step: at step t the ranks
    r = t..P-1 hold KV block j = r - t, all with the same offset t*N/P, so
    they form one strided batch (ranks r < t hold j = r - t + P, which is in
    the causal future and skipped, or one more batch when non-causal).
    With lanes > 1 the ranks are split by r % lanes, each class running its
    steps as such batches on a stream of its own: the classes' launches
    overlap, so one launch's epilogues (the fused merges) run while another
    computes (one stream measures fastest for the causal 16K ring, whose
    launches use the XCD-grouped work order).  batched=False issues one
    launch per (rank, step).  out, lse: optional fp32 destinations (their
    contents on entry are ignored: the first step writes every row).
    """
    B, H, n, d = q.shape
    blk = n // P
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    if not batched or B != 1 or n % P:
        for r in range(P):
            rows = slice(r * blk, (r + 1) * blk)
            sweep_fwd(q[..., rows, :], k, v, P, r, causal, out[..., rows, :], lse[..., rows],
                      scale=scale)
        return out, lse
    lanes = max(1, min(lanes, P))
    main = torch.cuda.current_stream(q.device)
    streams = [main] if lanes == 1 else [torch.cuda.Stream(q.device) for _ in range(lanes)]
    for st in streams[1:] if lanes == 1 else streams:
        st.wait_stream(main)
    for lane, st in enumerate(streams):
        with torch.cuda.stream(st):
            for t in range(P):
                groups = [(t, P - t, 0)]             # (first rank, ranks, first KV block)
                if not causal and t > 0:
                    groups.append((0, t, P - t))
                for g0, gcnt, j0 in groups:
                    b0, cnt = lane_entries(g0, gcnt, lane, lanes)
                    if cnt == 0:
                        continue
                    r0 = g0 + b0
                    jr = j0 + (r0 - g0)
                    delta = (r0 - jr) * blk if causal else None
                    rb = lambda x, first: _rows_batch(x, first * blk, blk, lanes * blk, cnt)
                    attn_segment_fwd(rb(q, r0), rb(k, jr), rb(v, jr), causal_offset=delta,
                                     scale=scale, out=rb(out, r0), lse=rb(lse, r0),
                                     accumulate=t > 0)
    if lanes > 1:
        for st in streams:
            main.wait_stream(st)
    return out, lse


def zigzag_order(n: int, P: int):
    """Global row of each row of the zigzag layout: rank r's 2n/(2P) rows are
    chunk r followed by chunk 2P-1-r of the sequence (chunks of n/(2P) rows)."""
    c = n // (2 * P)
    rows = []
    for r in range(P):
        rows.extend(range(r * c, (r + 1) * c))
        rows.extend(range((2 * P - 1 - r) * c, (2 * P - r) * c))
    return rows


def zigzag_plan(n: int, P: int):
    """Launches of the zigzag causal ring over P ranks (zigzag layout rows).

    Each launch is (step, q_rows, kv_rows, causal_offset, accumulate), where
    q_rows / kv_rows = (row0, rows, count) name `count` row ranges
    [row0 + i*2c, row0 + i*2c + rows), c = n/(2P), one per rank of the batch.

    Step 0: every rank attends to its own two chunks; in rank-local order the
    causal rule between them is plain j <= i (chunk r precedes chunk 2P-1-r),
    so that is one causal launch over all ranks.  Step t > 0: rank r holds
    the KV of rank j = (r - t) mod P.  For j < r both of r's chunks see all of
    chunk j and none of chunk 2P-1-j; for j > r only r's second chunk sees
    anything, and it sees both of j's chunks.  Each case is one non-causal
    launch over its ranks, and every rank gets 2c^2 pairs per step.
    """
    if n % (2 * P):
        raise ValueError("zigzag ring needs N divisible by 2P")
    c = n // (2 * P)
    plan = [(0, (0, 2 * c, P), (0, 2 * c, P), 0, False)]
    for t in range(1, P):
        # ranks r = t..P-1 hold j = r - t < r: all 2c rows vs j's first chunk
        plan.append((t, (2 * c * t, 2 * c, P - t), (0, c, P - t), None, True))
        # ranks r = 0..t-1 hold j = r - t + P > r: second chunk vs both of j's
        plan.append((t, (c, c, t), (2 * c * (P - t), 2 * c, t), None, True))
    return plan


def zigzag_ring_fwd(q, k, v, P: int, scale=None, out=None, lse=None, lanes: int = 2):
    """Causal ring over P ranks with the zigzag split, all ranks on one GPU.

    q, k, v: [1,H,N,d] in the zigzag layout (zigzag_order; rank r owns rows
    [r*2c, (r+1)*2c)).  Returns the merged fp32 output and LSE in the same
    layout.  Issues the launches of zigzag_plan; with lanes > 1 the ranks of
    each launch are split by r % lanes over as many streams, so every rank's
    steps stay in order on one stream while the classes overlap.
    """
    _, H, n, d = q.shape
    if q.shape[0] != 1:
        raise ValueError("zigzag ring takes B = 1")
    plan = zigzag_plan(n, P)
    step = n // P
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    lanes = max(1, min(lanes, P))
    main = torch.cuda.current_stream(q.device)
    streams = [main] if lanes == 1 else [torch.cuda.Stream(q.device) for _ in range(lanes)]
    if lanes > 1:
        for st in streams:
            st.wait_stream(main)
    for lane, st in enumerate(streams):
        with torch.cuda.stream(st):
            for _, (q0, qn, cnt), (k0, kn, _), delta, acc in plan:
                b0, m = lane_entries(q0 // step, cnt, lane, lanes)  # q0 // step: first rank
                if m == 0:
                    continue
                qs, ks = q0 + b0 * step, k0 + b0 * step
                rb = lambda x, first, rows: _rows_batch(x, first, rows, lanes * step, m)
                attn_segment_fwd(rb(q, qs, qn), rb(k, ks, kn), rb(v, ks, kn), causal_offset=delta,
                                 scale=scale, out=rb(out, qs, qn), lse=rb(lse, qs, qn),
                                 accumulate=acc)
    if lanes > 1:
        for st in streams:
            main.wait_stream(st)
    return out, lse


def ulysses_fwd(q, k, v, causal: bool = True, scale=None, out_dtype=None):
    """Ulysses share: the GPU's head subset, full sequence, one call."""
    return attn_segment_fwd(q, k, v, causal_offset=0 if causal else None, scale=scale,
                            out_dtype=out_dtype)


def _strided(buf, shape, strides):
    return buf.as_strided(shape, strides, buf.storage_offset())


def ulysses_pipeline_fwd(q, k, v, P: int, causal: bool = True, scale=None):
    """Ulysses over P emulated ranks on one GPU.

    q: [N, H, d], k, v: [N, Hkv, d] (sequence-major; rank r holds rows
    [r*N/P, (r+1)*N/P)); H and Hkv divisible by P.  Per rank: pack the shard
    [Ns, H, d] into the send buffer [P][Ns][H/P][d] (chunk g goes to rank g),
    all-to-all, attention of head group g over the whole sequence (read in
    place as [N][H/P][d]), the reverse all-to-all of the output, and the
    unpack to [Ns, H, d].  Here the P ranks' buffers are stacked on a leading
    rank axis, so each step is one launch for all ranks.
    Returns (out [N, H, d] bf16, lse [H, N]).
    """
    n, H, d = q.shape
    Hkv = k.shape[1]
    if n % P or H % P or Hkv % P:
        raise ValueError("N, H and Hkv must be divisible by P")
    ns = n // P
    dev = q.device

    def to_heads(x):
        """pack + all-to-all: [N, h, d] -> recv [P(g)][P(r)][Ns][h/P][d]."""
        h = x.shape[1]
        hp = h // P
        send = torch.empty((P, P, ns, hp, d), dtype=x.dtype, device=dev)
        head_relayout(_strided(x, (P, h, ns, d), (ns * h * d, d, h * d, 1)),
                      _strided(send, (P * P, hp, ns, d), (ns * hp * d, d, hp * d, 1)))
        recv = torch.empty((P, P, ns, hp, d), dtype=x.dtype, device=dev)
        blk = ns * hp * d
        head_relayout(_strided(send, (P, P, ns * hp, d), (blk, P * blk, d, 1)),
                      _strided(recv, (P, P, ns * hp, d), (P * blk, blk, d, 1)))
        # group g's whole sequence, read in place as [g][head][row][d]
        return _strided(recv, (P, hp, n, d), (n * hp * d, d, hp * d, 1))

    qg, kg, vg = to_heads(q), to_heads(k), to_heads(v)
    hp = H // P
    o_heads = torch.empty((P, n, hp, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((P, hp, n), dtype=torch.float32, device=dev)
    attn_segment_fwd(qg, kg, vg, causal_offset=0 if causal else None, scale=scale,
                     out=_strided(o_heads, (P, hp, n, d), (n * hp * d, d, hp * d, 1)), lse=lse)
    # reverse all-to-all: [P(g)][P(r)][Ns][hp][d] -> [P(r)][P(g)][Ns][hp][d]
    blk = ns * hp * d
    back = torch.empty((P, P, ns, hp, d), dtype=torch.bfloat16, device=dev)
    head_relayout(_strided(o_heads, (P, P, ns * hp, d), (blk, P * blk, d, 1)),
                  _strided(back, (P, P, ns * hp, d), (P * blk, blk, d, 1)))
    # unpack: [P(r)][P(g)][Ns][hp][d] -> [N, H, d]
    out = torch.empty((n, H, d), dtype=torch.bfloat16, device=dev)
    head_relayout(_strided(back, (P * P, hp, ns, d), (ns * hp * d, d, hp * d, 1)),
                  _strided(out, (P, H, ns, d), (ns * H * d, d, H * d, 1)))
    return out, lse.reshape(H, n)


def _split_branches(n, P, segment_lengths, dilations):
    """Local (w divides the device share) and gathered (w a multiple of it)
    branches of LongNet's distributed split."""
    if n % P:
        raise ValueError("N must be divisible by the device count")
    share = n // P
    local, gathered = [], []
    for w, r in zip(segment_lengths, dilations):
        w = min(int(w), n)
        if share % w == 0:
            local.append((w, int(r)))
        elif w % share == 0:
            gathered.append((w, int(r)))
        else:
            raise ValueError(f"segment length {w} neither divides nor is a multiple "
                             f"of the device share {share}")
    if not local:
        raise ValueError("at least one branch must fit in a device share")
    return share, local, gathered


def _gathered_parts(n, P, share, w, r):
    """For a gathered branch: per segment (start, selected-row count) and per
    device (segment start, first selected position p0, local selected count,
    index i0 of p0 among the segment's selected rows)."""
    segs = []
    for s0 in range(0, n, w):
        seglen = min(w, n - s0)
        segs.append((s0, -(-seglen // r)))
    devs = []
    for dev in range(P):
        a, b = dev * share, (dev + 1) * share
        s0 = (a // w) * w
        p0 = s0 + (-(-(a - s0) // r)) * r
        cnt = -(-(b - p0) // r) if p0 < b else 0
        devs.append((s0, p0, cnt, (p0 - s0) // r))
    return segs, devs


def _rows(t, start, count, step):
    """Rows start, start+step, ... (count of them) of a [1,H,N(,d)] tensor."""
    st = t.stride()
    off = t.storage_offset() + start * st[2]
    if t.dim() == 4:
        return t.as_strided((t.shape[0], t.shape[1], count, t.shape[3]),
                            (st[0], st[1], step * st[2], st[3]), off)
    return t.as_strided((t.shape[0], t.shape[1], count), (st[0], st[1], step * st[2]), off)


def _all_gather_selected(x, segs, devs, s_start, w, r):
    """Each device's selected rows of segment s_start, placed at its slot of the
    gathered [1,H,count,d] buffer (the all-gather's result)."""
    count = dict(segs)[s_start]
    g = torch.empty((1, x.shape[1], count, x.shape[3]), dtype=x.dtype, device=x.device)
    for seg0, p0, cnt, i0 in devs:
        if seg0 == s_start and cnt > 0:
            head_relayout(_rows(x, p0, cnt, r), g[:, :, i0:i0 + cnt, :])
    return g


def longnet_split_fwd(q, k, v, segment_lengths, dilations, P: int, causal: bool = False,
                      scale=None):
    """Dilated attention with the sequence split over P emulated devices.

    q, k, v: [1,H,N,d] bf16.  Device r holds rows [r*N/P, (r+1)*N/P).  Branches
    whose segment length divides the share run as dilated attention on the
    device's rows; for a longer branch, the selected K/V rows of each segment
    are all-gathered (each device's part copied into its slot) and each
    device's selected queries attend to them with the causal offset of their
    place in the segment, merged into the device's running (O, LSE).
    Returns fp32 O [1,H,N,d] and LSE [1,H,N], equal to dilated_attn_fwd's.
    """
    n = q.shape[-2]
    share, local, gathered = _split_branches(n, P, segment_lengths, dilations)
    out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    lw, lr = [w for w, _ in local], [r for _, r in local]
    # the local branches of all devices in one call: their segments never
    # cross a device boundary (w divides the share), so this is each
    # device's own dilated attention on its rows, batched over the devices
    dilated_attn_fwd(q, k, v, lw, lr, causal=causal, scale=scale, out=out, lse=lse)
    for w, r in gathered:
        segs, devs = _gathered_parts(n, P, share, w, r)
        for s0, _ in segs:
            kg = _all_gather_selected(k, segs, devs, s0, w, r)
            vg = _all_gather_selected(v, segs, devs, s0, w, r)
            for seg0, p0, cnt, i0 in devs:
                if seg0 != s0 or cnt == 0:
                    continue
                attn_segment_fwd(_rows(q, p0, cnt, r), kg, vg,
                                 causal_offset=i0 if causal else None, scale=scale,
                                 out=_rows(out, p0, cnt, r), lse=_rows(lse, p0, cnt, r),
                                 accumulate=True)
    return out, lse


def longnet_split_bwd(q, k, v, out, lse, d_o, segment_lengths, dilations, P: int,
                      causal: bool = False, scale=None):
    """Backward of longnet_split_fwd from its merged (out, lse).

    Local branches: the dilated backward on each device's rows.  Gathered
    branches: each device's selected queries against the gathered K/V; the
    gradients of the gathered rows are summed over the segment's devices and
    land on the rows' owners (the reduce-scatter), emulated by accumulating
    into the global dK/dV rows.  Returns (dq, dk, dv), fp32.
    """
    n = q.shape[-2]
    share, local, gathered = _split_branches(n, P, segment_lengths, dilations)
    dq = torch.zeros(q.shape, dtype=torch.float32, device=q.device)
    dk = torch.empty(k.shape, dtype=torch.float32, device=k.device)
    dv = torch.empty(v.shape, dtype=torch.float32, device=v.device)
    lw, lr = [w for w, _ in local], [r for _, r in local]
    # local branches of all devices in one call (see longnet_split_fwd)
    dilated_attn_bwd(q, k, v, out, lse, d_o, lw, lr, causal=causal, scale=scale,
                     dq=dq, dk=dk, dv=dv)
    for w, r in gathered:
        segs, devs = _gathered_parts(n, P, share, w, r)
        for s0, count in segs:
            kg = _all_gather_selected(k, segs, devs, s0, w, r)
            vg = _all_gather_selected(v, segs, devs, s0, w, r)
            for seg0, p0, cnt, i0 in devs:
                if seg0 != s0 or cnt == 0:
                    continue
                attn_segment_bwd(_rows(q, p0, cnt, r), kg, vg, _rows(out, p0, cnt, r),
                                 _rows(lse, p0, cnt, r), _rows(d_o, p0, cnt, r),
                                 causal_offset=i0 if causal else None, scale=scale,
                                 dq=_rows(dq, p0, cnt, r), dk=_rows(dk, s0, count, r),
                                 dv=_rows(dv, s0, count, r), accumulate_kv=True)
    return dq, dk, dv


def usp_fwd_bwd(q, k, v, d_o, n_blocks: int, q_block: int, causal: bool = True,
                scale=None, grad_dtype=torch.float32):
    """USP share: forward sweep over KV blocks, then the backward sweep.

    Returns (o, lse, dq, dk, dv); dk, dv cover all of K/V ([B,Hkv,Nk,d]).
    """
    out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    sweep_fwd(q, k, v, n_blocks, q_block, causal, out, lse, scale=scale)
    dq, dk, dv = usp_bwd(q, k, v, out, lse, d_o, n_blocks, q_block, causal, scale,
                         grad_dtype=grad_dtype)
    return out, lse, dq, dk, dv


def usp_bwd(q, k, v, out, lse, d_o, n_blocks: int, q_block: int, causal: bool = True,
            scale=None, grad_dtype=torch.float32, dq=None, dk=None, dv=None):
    """Backward sweep: dQ accumulates over blocks, each block writes its dK/dV."""
    nk = k.shape[-2]
    blk = nk // n_blocks
    q_start = q_block * blk
    if dq is None:
        dq = torch.zeros(q.shape, dtype=torch.float32, device=q.device)
    if dk is None:
        dk = torch.empty(k.shape, dtype=grad_dtype, device=k.device)
    if dv is None:
        dv = torch.empty(v.shape, dtype=grad_dtype, device=v.device)
    for j in ring_order(q_block, n_blocks):
        k_start = j * blk
        rows = slice(k_start, k_start + blk)
        delta = q_start - k_start
        # a block wholly in the causal future still gets its call: the kernel
        # finds no visible pair and writes dK = dV = 0
        attn_segment_bwd(q, k[..., rows, :], v[..., rows, :], out, lse, d_o,
                         causal_offset=delta if causal else None, scale=scale, dq=dq,
                         dk=dk[..., rows, :], dv=dv[..., rows, :])
    return dq, dk, dv
