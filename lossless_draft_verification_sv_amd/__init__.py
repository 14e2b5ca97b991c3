"""Batched lossless draft verification for speculative decoding on MI355X (gfx950).

The work runs in hand-written HIP kernels behind the C ABI of include/sv.h (libsv.so, built by
lossless_draft_verification_sv_amd.build); this package only marshals torch tensors to it.
"""
from ._binding import (LIBRARY_PATH, SV_DTYPE_BF16, SV_DTYPE_F32, SV_ERR_HIP,
                       SV_ERR_INVALID_ARG, SV_ERR_UNSUPPORTED, SV_ERR_WORKSPACE, SV_OK,
                       ScheduleOutput, SVError, TopkOutput, VerifyOutput, load_library,
                       sv_last_error, sv_markov_draft, sv_markov_draft_sampled,
                       sv_markov_topk, sv_read_probe,
                       sv_schedule_prefix, sv_status_string, sv_verify_batch, sv_verify_greedy,
                       sv_verify_ragged, sv_workspace_bytes)

__all__ = [
    "LIBRARY_PATH", "SV_DTYPE_BF16", "SV_DTYPE_F32", "SV_ERR_HIP", "SV_ERR_INVALID_ARG",
    "SV_ERR_UNSUPPORTED", "SV_ERR_WORKSPACE", "SV_OK", "ScheduleOutput", "SVError",
    "TopkOutput", "VerifyOutput", "load_library", "sv_last_error", "sv_markov_draft",
    "sv_markov_draft_sampled",
    "sv_markov_topk", "sv_read_probe", "sv_schedule_prefix", "sv_status_string",
    "sv_verify_batch", "sv_verify_greedy", "sv_verify_ragged", "sv_workspace_bytes",
]
