"""Gated-delta-rule (GatedDeltaNet) decode / draft-verification / chunked-prefill
hot path for MI355X (gfx950): HIP kernels behind the libgdn C ABI
(include/gdn.h), with a thin Python binding of the same names.

The library must be built first (``python -m gateddeltanet_linear_attention_amd.build``);
every entry point raises if it is missing -- there is no fallback path.
"""
from .binding import (  # noqa: F401
    Dims,
    GdnError,
    MAX_K,
    ROUTE_CHUNKED,
    ROUTE_RECURRENT,
    gdn_chunked_prefill_with_checkpoints,
    gdn_chunked_workspace_bytes,
    gdn_commit_accepted,
    gdn_decode_step,
    gdn_plan_transaction,
    gdn_run_transaction,
    gdn_status_str,
    gdn_verify_window,
    gdn_version,
    lib,
)
