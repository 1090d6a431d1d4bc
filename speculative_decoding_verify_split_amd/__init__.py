"""rapid_verify for AMD MI355X (gfx950): the target model's speculative
verification step for long-context decoding -- split-KV history attention,
masked draft-block attention, log-sum-exp merge, and RAPID's acceptance with
the retrieval-augmented target -- as a C-ABI HIP library with a thin Python
binding.  The library is loaded on first use and every call fails loudly if
it has not been built.
"""

from .rapid_verify import (  # noqa: F401
    LIB_PATH,
    RapidVerifyError,
    load_library,
    lse_merge,
    RV_ACCEPT_PRINTED_RESIDUAL,
    RV_ACCEPT_TAIL_PRESERVE,
    rapid_accept,
    rapid_accept_ex,
    rapid_accept_noalloc,
    rapid_accept_workspace_size,
    rapid_tree_accept,
    rapid_tree_accept_workspace_size,
    rv_prefix_balanced_split,
    rv_prefix_default_split,
    rv_status_string,
    rv_verify_single_launch,
    rv_version,
    spec_attn_block,
    spec_attn_block_merge,
    spec_attn_block_merge_ev,
    spec_attn_prefix,
    spec_attn_prefix_ev,
    spec_attn_verify,
    spec_attn_verify_sync_size,
    spec_attn_window,
    spec_attn_window_workspace_size,
)
