"""Exact tiled scaled-dot-product attention for AMD Instinct MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of include/attn.h
(lib/libattn.so); this package is the thin Python binding used by tests and the bench.
"""
from ._binding import (  # noqa: F401
    ATTN_BF16, ATTN_F32, ATTN_MASK_NONE, ATTN_MASK_CAUSAL_TOP_LEFT, ATTN_MASK_CAUSAL_BOTTOM_RIGHT,
    ATTN_PATH_AUTO, ATTN_PATH_PREFILL, ATTN_PATH_SPLITK, ATTN_PROBE_BWD_KV, ATTN_PROBE_BWD_Q,
    ATTN_PROBE_BWD_KV_F32, ATTN_PROBE_BWD_Q_F32, ATTN_PROBE_PREFILL, ATTN_PROBE_PREFILL_GENERIC,
    ATTN_PROBE_SPLITK, EXPORTS, SEQLENS_ERRORS, AttnError, attn_bwd, attn_bwd_dropout,
    attn_bwd_workspace_size, attn_check_seqlens, attn_describe_plan, attn_dropout_probe,
    attn_fwd, attn_fwd_dropout, attn_fwd_dropout_workspace_size, attn_fwd_no_workspace,
    attn_fwd_workspace_size, attn_mask_probe, attn_mask_probe_ex, attn_status_string, attn_version,
    library_path, load, use_library)
