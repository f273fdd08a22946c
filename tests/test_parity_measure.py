"""CPU checks of the parity measure itself (no GPU).

The gate is the per-row relative error of tests/parity.py.  These tests plant
mistakes in an oracle result (never in GPU output) and show that the gate
catches the ones a normwise-per-head measure misses on a long causal
sequence, while plain bf16 rounding of a correct result still passes.
"""
import numpy as np
import torch

import oracle
from long_sequence_exact_amd.synth import draw, sample_rows
import pytest

from tests.parity import DS_FLOOR, TOL, ROW_FLOOR, check_close, errors, max_rel_error

TOL_BF16 = TOL[torch.bfloat16]


def _long_causal_sample():
    """Oracle rows of one head at 131072 tokens, d = 128, causal: row 0 plus
    63 seeded rows (their magnitudes fall like 1/sqrt(position))."""
    n, d = 131072, 128
    q, k, v = draw([(1, 1, n, d)] * 3, 2)
    rows = np.array(sample_rows(n, 64, 77, must=(0,)), np.int64)
    o, _ = oracle.attn_fwd(q.float().numpy(), k.float().numpy(), v.float().numpy(),
                           delta=0, rows=rows)
    return rows, o


def test_late_rows_zeroed_or_scaled_fail_the_row_gate():
    rows, o = _long_causal_sample()
    late = rows >= 8192
    assert late.sum() > 50
    zeroed = o.copy()
    zeroed[late] = 0.0
    scaled = o.copy()
    scaled[late] *= 0.9
    # a normwise measure over the head cannot see them: row 0 (= V_0) sets the scale
    assert errors(zeroed, o)["norm"] < TOL_BF16
    assert errors(scaled, o)["norm"] < TOL_BF16
    # the per-row gate does
    assert max_rel_error(zeroed, o) > 0.5
    assert max_rel_error(scaled, o) > 5 * TOL_BF16
    # one wrong late row is enough
    one = o.copy()
    one[np.flatnonzero(late)[-1]] *= 0.95
    assert max_rel_error(one, o) > TOL_BF16


def test_bf16_rounding_of_a_correct_result_passes():
    rows, o = _long_causal_sample()
    rounded = torch.from_numpy(o).to(torch.bfloat16).double().numpy()
    e = errors(rounded, o)
    assert e["row"] <= 2.0 ** -8          # one bf16 rounding per element
    assert e["row"] <= TOL_BF16


def test_zero_reference_rows_use_the_head_floor():
    ref = np.zeros((4, 8))
    ref[0] = 2.0                     # head max 2
    x = ref.copy()
    x[1] = 0.5 * ROW_FLOOR * 2.0     # a zero row off by half the floor
    assert abs(max_rel_error(x, ref) - 0.5) < 1e-12
    x[1] = 0.0
    assert max_rel_error(x, ref) == 0.0


def test_heads_are_measured_separately():
    ref = np.ones((2, 3, 4))
    ref[1] *= 1e-4                   # a head of tiny magnitude
    x = ref.copy()
    x[1] *= 1.1                      # 10% off in that head only
    assert abs(max_rel_error(x, ref) - 0.1) < 1e-9
    # the same arrays as rows with a head id per row
    heads = np.repeat([0, 1], 3)
    assert abs(max_rel_error(x.reshape(6, 4), ref.reshape(6, 4), heads) - 0.1) < 1e-9


def test_non_finite_output_is_an_infinite_error():
    ref = np.ones((3, 4))
    x = ref.copy()
    x[2, 1] = np.inf
    assert max_rel_error(x, ref) == float("inf")


def test_gradient_floor_is_a_quarter_of_the_head_scale():
    ref = np.ones((5, 4))
    ref[0] = 1e-3                    # a near-one-hot row: tiny dQ (or dK)
    x = ref.copy()
    x[0] += 4e-3                     # its absolute error, far above its own size
    assert max_rel_error(x, ref) > 1.0                                  # output rule
    assert abs(max_rel_error(x, ref, floor=DS_FLOOR) - 4e-3 / DS_FLOOR) < 1e-12
    # a wrong typical row still fails under the gradient rule
    x = ref.copy()
    x[3] *= 0.9
    assert max_rel_error(x, ref, floor=DS_FLOOR) > 4 * TOL_BF16


def test_check_close_takes_the_gradient_floor_for_dq_and_dk_only():
    ref = np.ones((5, 4))
    ref[0] = 1e-3
    x = ref.copy()
    x[0] += 4e-3
    for name in ("dq", "dk"):
        check_close(x, ref, TOL_BF16, name=name)
    for name in ("dv", "o"):
        with pytest.raises(AssertionError):
            check_close(x, ref, TOL_BF16, name=name)
    x = ref.copy()
    x[3] *= 0.9                      # a wrong typical row fails for every tensor
    for name in ("dq", "dk", "dv", "o"):
        with pytest.raises(AssertionError):
            check_close(x, ref, TOL_BF16, name=name)
