"""Shared helpers of the parity tests: error measures and tolerances.

Tolerances (the problem statement fixes them): outputs match the fp64 oracle
within a normwise relative error of 1e-4 for fp32 and 2e-2 for bf16 (max|x -
ref| / max|ref| per tensor and head; element-wise relative error is unbounded
where an output crosses zero), and LSE within 1e-3 absolute, with -inf
entries matching exactly.
"""
import numpy as np
import torch

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
LSE_TOL = 1e-3


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def normwise_per_head(x, ref, head_axis_rows=None):
    """Max over heads of max|x-ref|/max|ref|.  x, ref: [..., H, N, d] arrays
    (or [rows, d] with head_axis_rows = head id per row)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    if head_axis_rows is not None:
        worst = 0.0
        for h in np.unique(head_axis_rows):
            sel = head_axis_rows == h
            den = np.abs(ref[sel]).max()
            num = np.abs(x[sel] - ref[sel]).max()
            worst = max(worst, num / den if den > 0 else num)
        return worst
    x = x.reshape(-1, x.shape[-2], x.shape[-1]) if x.ndim >= 3 else x[None]
    ref = ref.reshape(x.shape)
    worst = 0.0
    for h in range(x.shape[0]):
        den = np.abs(ref[h]).max() if ref[h].size else 0.0
        num = np.abs(x[h] - ref[h]).max() if ref[h].size else 0.0
        worst = max(worst, num / den if den > 0 else num)
    return worst


def lse_check(lse, ref):
    """(max abs error over finite entries, -inf pattern identical)."""
    lse = np.asarray(lse, np.float64)
    ref = np.asarray(ref, np.float64)
    same_inf = np.array_equal(np.isneginf(lse), np.isneginf(ref))
    fin = np.isfinite(ref)
    err = np.abs(lse[fin] - ref[fin]).max() if fin.any() else 0.0
    if not np.all(np.isfinite(lse[fin])):
        err = float("inf")
    return err, same_inf


def assert_parity(o, lse, o_ref, lse_ref, dtype, rows_heads=None, what=""):
    tol = TOL[dtype]
    e = normwise_per_head(o, o_ref, rows_heads)
    le, same = lse_check(lse, lse_ref)
    assert not np.isnan(np.asarray(o)).any(), f"{what}: NaN in output"
    assert e <= tol, f"{what}: normwise relative error {e:.3e} > {tol}"
    assert le <= LSE_TOL, f"{what}: LSE error {le:.3e} > {LSE_TOL}"
    assert same, f"{what}: -inf LSE pattern differs"
    return e, le


def dilated_key_list(p, n, ws, rs, causal, shift=0):
    """Keys that the dilated branches (w_i, r_i) list for query p, a key once
    per listing branch: branch i selects p when p's offset in its w_i-segment
    is shift mod r_i plus a multiple of r_i, and then lists the selected
    positions of that segment (with causal, those <= p).  shift is the query
    head under head-dependent offsets, else 0."""
    keys = []
    for w, r in zip(ws, rs):
        w = min(w, n)
        s0 = (p // w) * w
        off = shift % r
        if p - s0 < off or (p - s0 - off) % r:
            continue
        ks = np.arange(s0 + off, min(s0 + w, n), r)
        if causal:
            ks = ks[ks <= p]
        keys.append(ks)
    return np.concatenate(keys) if keys else np.zeros(0, np.int64)
