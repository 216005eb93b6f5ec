"""Speculative-decoding attention hot path for AMD Instinct MI355X (gfx950).

The work happens in ``libspecattn.so`` (hand-written HIP kernels behind the C
ABI of ``include/spec_attn.h``); this package only marshals torch tensors into
that ABI.  Build the library with ``python -m sparse_kv_attention_sink_amd.build``.
"""
from ._lib import (  # noqa: F401
    EXPORTED, LIB_PATH, SPEC_BF16, SPEC_DEV_CACHE_LEN, SPEC_DEV_COMMIT, SPEC_DEV_DEPTH,
    SPEC_DEV_INDEX, SPEC_DEV_PARENT, SPEC_E_DEVICE_RANGE, SPEC_E_HIP, SPEC_E_INVALID,
    SPEC_E_UNSUPPORTED, SPEC_E_WORKSPACE, SPEC_F32, SPEC_FLAG_DETERMINISTIC, SPEC_OK, SpecDims, SpecError, SpecKV,
    accept_workspace_bytes, commit_workspace_bytes, compact_workspace_bytes, draft_workspace_bytes,
    load, make_dims,
    new_workspace, spec_accept_greedy, spec_attn_draft_ring, spec_attn_draft_sparse,
    spec_attn_verify_tree, spec_attn_verify_tree_noalloc, spec_kv_compact,
    SPEC_VERIFY_FULL, SPEC_VERIFY_PARTIAL, spec_block_means, spec_device_status, spec_kv_commit,
    spec_kv_gather, spec_select_blocks, spec_verify_mode, select_workspace_bytes,
    verify_workspace_bytes,
)
