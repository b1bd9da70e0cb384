"""MI355X-native speculative-decoding verification step.

The compute lives in libspecverify.so (hand-written HIP kernels for gfx950
behind the C ABI in include/spec_verify.h and include/sv_ceilings.h).  This package is its Python
binding: the functions carry the C names and only marshal arguments.
"""
from ._lib import (EXPORTS, LIB_PATH, SV_ERR_INVALID, SV_ERR_LAUNCH, SV_ERR_UNSUPPORTED,
                   SV_ERR_WORKSPACE, SV_KV_BF16, SV_KV_FP8_E4M3, SV_OK, SvAppendParams,
                   SvAttnParams, SvError, abi_version, last_error, library, make_append_params,
                   make_attn_params, spec_accept, spec_accept_noalloc, spec_kv_append, spec_draft_signals,
                   spec_draft_signals_workspace_size, spec_verify_attn_tree, spec_accept_tree,
                   spec_kv_commit_tree,
                   spec_accept_sampled, spec_accept_sampled_workspace_size,
                   spec_accept_workspace_size, spec_verify_attn, spec_verify_attn_workspace_size,
                   status_string, sv_ceiling_exp2, sv_ceiling_mfma_bf16, sv_ceiling_read)

__all__ = [
    "EXPORTS", "LIB_PATH", "SV_OK", "SV_ERR_INVALID", "SV_ERR_WORKSPACE", "SV_ERR_UNSUPPORTED",
    "SV_ERR_LAUNCH", "SV_KV_BF16", "SV_KV_FP8_E4M3", "SvAppendParams", "SvAttnParams", "SvError",
    "abi_version", "last_error", "library", "make_append_params", "make_attn_params",
    "spec_accept", "spec_accept_noalloc", "spec_accept_sampled", "spec_kv_append", "spec_draft_signals",
    "spec_draft_signals_workspace_size", "spec_verify_attn_tree", "spec_accept_tree",
    "spec_kv_commit_tree",
    "spec_accept_sampled_workspace_size", "spec_accept_workspace_size",
    "spec_verify_attn", "spec_verify_attn_workspace_size", "status_string",
    "sv_ceiling_read", "sv_ceiling_mfma_bf16", "sv_ceiling_exp2",
]
