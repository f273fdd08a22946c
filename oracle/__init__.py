"""fp64 CPU oracle -- test infrastructure only (tests, smoke check, CPU baseline)."""
from .oracle import (NONCAUSAL, attn_bwd, attn_bwd_dq_rows, attn_fwd, build,
                     dilated_bwd, dilated_fwd, lse_merge, num_threads)

__all__ = ["NONCAUSAL", "attn_bwd", "attn_bwd_dq_rows", "attn_fwd", "build",
           "dilated_bwd", "dilated_fwd", "lse_merge", "num_threads"]
