"""fp64 CPU oracle for batched draft verification — test infrastructure only.

Imported by the tests, the smoke check and the benchmark's CPU-baseline leg; never by the GPU
library.
"""
from .sv_oracle import (AMBIGUOUS_MARGIN, RAGGED_INVALID, TAU_MIN, BatchResult, RequestResult,
                        accept_threshold, argmax_lowest, decode_logits, inverse_cdf,
                        ragged_request_valid, residual_weights, softmax_fp64, verify_batch,
                        verify_greedy, verify_greedy_request, verify_ragged, verify_request)

from .markov_oracle import (AMBIGUOUS_GAP, KERNEL_LOGIT_ABS, KERNEL_LOGIT_REL, MARKOV_INVALID,
                            SAMPLE_EPS, argmax_valid_tokens, draw_valid_tokens, markov_draft,
                            markov_draft_request, markov_sampled, markov_sampled_request,
                            markov_topk, markov_topk_request, round_stored, sample_stored_row,
                            sample_weights, stored_uncertainty, topk_candidates)
from .schedule_oracle import (clamp_confidence, prefix_survival, rank_tokens, row_starts,
                              schedule_hardware_aware, schedule_threshold)

__all__ = [
    "AMBIGUOUS_GAP", "KERNEL_LOGIT_ABS", "KERNEL_LOGIT_REL", "MARKOV_INVALID", "SAMPLE_EPS",
    "argmax_valid_tokens", "draw_valid_tokens", "markov_draft", "markov_draft_request",
    "markov_sampled", "markov_sampled_request", "markov_topk", "markov_topk_request",
    "round_stored", "sample_stored_row", "sample_weights", "stored_uncertainty", "topk_candidates",
    "clamp_confidence", "prefix_survival", "rank_tokens", "row_starts",
    "schedule_hardware_aware", "schedule_threshold",
    "AMBIGUOUS_MARGIN", "RAGGED_INVALID", "TAU_MIN", "BatchResult", "RequestResult",
    "accept_threshold", "argmax_lowest", "decode_logits", "inverse_cdf", "ragged_request_valid",
    "residual_weights", "softmax_fp64", "verify_batch", "verify_greedy", "verify_greedy_request",
    "verify_ragged", "verify_request",
]
