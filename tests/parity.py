"""Shared helpers of the parity tests: error measures and tolerances.

Tolerances (the problem statement fixes them): outputs match the fp64 oracle
within a maximum relative error of 1e-4 for fp32 and 2e-2 for bf16, and LSE
within 1e-3 absolute, with -inf entries matching exactly.

"Relative error" is measured per row: for row i (one query's output vector,
or one key's gradient vector), max_c |x_ic - ref_ic| / max_c |ref_ic|.  A row
whose reference is (nearly) zero is measured against a floor: for outputs
ROW_FLOOR times the largest |ref| of its head, so an exactly-zero reference
row (a query that sees no key) needs an absolute match at that scale.  The
per-row measure is at least as strict as the normwise one per head (max|x -
ref| / max|ref|): a causal row deep in the sequence averages many keys and is
small, so a whole run of wrong late rows can stay under the normwise bound,
never under the per-row one.

dV rows are measured the same way.  dQ and dK rows take a higher floor,
DS_FLOOR times the largest |dQ| or |dK| of the head.  Both are sums over
dS_ij = P_ij (dP_ij - D_i): dQ_i = sigma sum_j dS_ij k_j and dK_j = sigma
sum_i dS_ij q_i.  Where one key holds nearly all of a query's softmax weight
the bracket is a difference of nearly equal terms, so dQ_i, and dK_j of a
key whose gradient comes from such queries (a causal key near the start of
a dilated segment, or a key seen by only a few queries), is tiny while its
absolute error is not.  That error comes from D_i = dO_i . O_i, whose O was
formed with P rounded to bf16 in the forward, and from dS rounded to bf16
before its product; it is bounded by a small fraction of the head's scale,
not of the row's own value (a query row with two keys of weights 1 - e and e
has dQ proportional to e and an error about 2^-9 of the row's scale).

Element-wise relative error is unbounded where an output crosses zero; its
regularised form |x - ref| / (|ref| + 1e-3 max|ref|) is reported beside the
gate as a diagnostic, as is the normwise error.

With SEQATTN_PARITY_LOG set to a file path, every check appends one JSON
line with all three measures.
"""
import json
import os

import numpy as np
import torch

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
LSE_TOL = 1e-3
ROW_FLOOR = 1e-3
DS_FLOOR = 0.25


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _groups(x, ref, heads):
    """(x, ref) pairs of 2-D [rows, d] arrays, one per head."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    if heads is not None:
        heads = np.asarray(heads)
        return [(x[heads == h], ref[heads == h]) for h in np.unique(heads)]
    if x.ndim == 1:
        return [(x[:, None], ref[:, None])]
    if x.ndim == 2:
        return [(x, ref)]
    x = x.reshape(-1, x.shape[-2], x.shape[-1])
    ref = ref.reshape(x.shape)
    return [(x[h], ref[h]) for h in range(x.shape[0])]


def errors(x, ref, heads=None, floor=ROW_FLOOR):
    """Dict of the three measures, each a max over heads (and rows):
    row   -- per-row relative error (the gate), rows below floor x the
             head's largest |ref| measured against that floor,
    norm  -- normwise relative error per head,
    elem  -- regularised element-wise relative error (diagnostic).
    x, ref: [..., H, N, d] arrays, or [rows, d] with heads = head id per row."""
    row = norm = elem = 0.0
    for xs, rs in _groups(x, ref, heads):
        if rs.size == 0:
            continue
        diff = np.abs(xs - rs)
        if not np.all(np.isfinite(xs)):
            return {"row": float("inf"), "norm": float("inf"), "elem": float("inf")}
        mags = np.abs(rs).max(axis=-1)
        top = mags.max()
        den_row = np.maximum(mags, floor * top)
        num_row = diff.max(axis=-1)
        with np.errstate(divide="ignore", invalid="ignore"):
            r = np.where(den_row > 0, num_row / np.where(den_row > 0, den_row, 1), num_row)
        row = max(row, float(r.max()))
        norm = max(norm, float(diff.max() / top) if top > 0 else float(diff.max()))
        e = diff / (np.abs(rs) + 1e-3 * top) if top > 0 else diff
        elem = max(elem, float(e.max()))
    return {"row": row, "norm": norm, "elem": elem}


def max_rel_error(x, ref, heads=None, floor=ROW_FLOOR):
    """The gate measure: largest per-row relative error (see the module text)."""
    return errors(x, ref, heads, floor)["row"]


def _log(rec):
    path = os.environ.get("SEQATTN_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")


def _test_name():
    return os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]


def check_close(x, ref, tol, heads=None, what="", name="o", floor=None):
    """Assert x (array or tensor) matches ref within tol by the per-row
    measure, with no NaN; the message carries all three measures.  floor
    defaults to DS_FLOOR for a tensor named dq or dk, else ROW_FLOOR."""
    if floor is None:
        floor = DS_FLOOR if name in ("dq", "dk") else ROW_FLOOR
    if isinstance(x, torch.Tensor):
        assert not torch.isnan(x).any(), f"{what}: NaN in {name}"
        x = to_np(x)
    x = np.asarray(x, np.float64)
    assert not np.isnan(x).any(), f"{what}: NaN in {name}"
    e = errors(x, ref, heads, floor)
    _log({"test": _test_name(), "what": what, "tensor": name, "tol": tol, "floor": floor, **e})
    assert e["row"] <= tol, (f"{what}: {name} per-row relative error {e['row']:.3e} > {tol} "
                             f"(normwise {e['norm']:.3e}, element-wise {e['elem']:.3e})")
    return e


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
    le, same = lse_check(lse, lse_ref)
    assert not np.isnan(np.asarray(lse)).any(), f"{what}: NaN in LSE"
    e = check_close(o, o_ref, tol, rows_heads, what, "o")
    _log({"test": _test_name(), "what": what, "tensor": "lse", "tol": LSE_TOL, "abs": le})
    assert le <= LSE_TOL, f"{what}: LSE error {le:.3e} > {LSE_TOL}"
    assert same, f"{what}: -inf LSE pattern differs"
    return e["row"], le


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
