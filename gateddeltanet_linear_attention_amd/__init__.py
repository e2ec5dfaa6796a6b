"""Gated-delta-rule (GatedDeltaNet) decode / draft-verification / chunked-prefill
hot path for MI355X (gfx950): HIP kernels behind the libgdn C ABI
(include/gdn.h), with a thin Python binding of the same names.

Every C entry point is exported here under its own name, with a ``prepare_*``
form for the ones a decode loop calls repeatedly (arguments marshalled once, the
call replayed, e.g. under HIP graph capture).

The library must be built first (``python -m gateddeltanet_linear_attention_amd.build``);
every entry point raises if it is missing -- there is no fallback path.
"""
from .binding import (  # noqa: F401
    Dims,
    GdnError,
    MAX_K,
    QK_L2NORM,
    ROUTE_CHUNKED,
    ROUTE_RECURRENT,
    STATIC_WS_BYTES,
    delta_shape,
    gdn_chunked_prefill_with_checkpoints,
    gdn_chunked_prefill_with_checkpoints_static,
    gdn_chunked_workspace_bytes,
    gdn_commit_accepted,
    gdn_commit_delta,
    gdn_commit_replay,
    gdn_commit_select,
    gdn_decode_step,
    gdn_plan_transaction,
    gdn_run_transaction,
    gdn_status_str,
    gdn_verify_tree,
    gdn_verify_window,
    gdn_verify_window_delta,
    gdn_verify_window_delta_fold,
    gdn_verify_window_select,
    gdn_verify_window_select_commit,
    gdn_version,
    lib,
    prepare_commit_accepted,
    prepare_commit_delta,
    prepare_commit_replay,
    prepare_commit_select,
    prepare_decode_step,
    prepare_verify_tree,
    prepare_verify_window,
    prepare_verify_window_delta,
    prepare_verify_window_delta_fold,
    prepare_verify_window_select,
    prepare_verify_window_select_commit,
)
