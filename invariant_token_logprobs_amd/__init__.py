"""Batch-invariant token logprobs and the REINFORCE Zero IS loss on MI355X.

The compute lives in the HIP library ``librz.so`` (C ABI declared in
``include/rz.h``); the functions here only marshal torch tensors into it.
Importing the package does not load the library; the first call does, and it
raises if the library has not been built.
"""
from .binding import (  # noqa: F401
    EXPORTS, RZ_DEVERR_CU_ROWS, RZ_DEVERR_GROUP, RZ_DEVERR_TOKEN,
    RUN_SUMMARY_KEYS, RZ_DEVERR_MX_SCALE, RZ_LORA_COLS, RZ_MX_FORMATS,
    RZ_OP_FWD_BWD_LORA, RZ_DTYPE_BF16, lora_augment, lora_merge_head,
    reinforce_zero_fwd_bwd_lora, token_logprobs_mx, sample_tokens_mx, RZ_DTYPE_F32, RZ_OP_DIAGNOSTICS,
    RZ_OP_FWD_BWD, RZ_OP_GRAD_NORMS, RZ_OP_SAMPLE, RZ_OP_TOKEN_LOGPROBS,
    RZ_OP_SCORE_CENTERING, score_centering_fwd_bwd, workspace_bytes_common,
    sample_tokens_noalloc, RZ_NOALLOC_SCRATCH_BYTES, calibrate_mfma,
    RunTracker, RzError, Workspace, dequantize_head, diagnostics, grad_norms,
    library_path,
    load_library, reinforce_zero_fwd_bwd, response_diagnostics, run_summary,
    sample_tokens, timing_enable, timing_read, token_logprobs,
    workspace_bytes,
)
