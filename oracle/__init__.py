"""fp64 CPU oracle of the speculative-sampling verify step (and, in
``oracle.tree``, of greedy token-tree verification and the tree mask).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.
"""
from .verify import (FLAG_BAD_DRAFT, FLAG_ZW_ZERO, Result, acceptance_threshold, draw_interval,
                     first_argmax, inverse_cdf, log_normalizer, position_stats, residual, softmax_from, verify,
                     verify_batch, verify_greedy_sequence, verify_sequence, widen)

__all__ = ["FLAG_BAD_DRAFT", "FLAG_ZW_ZERO", "Result", "acceptance_threshold", "draw_interval",
           "first_argmax", "inverse_cdf", "log_normalizer", "position_stats", "residual", "softmax_from", "verify",
           "verify_batch", "verify_greedy_sequence", "verify_sequence", "widen"]
