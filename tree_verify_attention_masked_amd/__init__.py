"""MI355X-native tree verification for speculative decoding.

The hot path of verifying a flattened draft tree in one target pass, as three
calls into libspectree (hand-written HIP for gfx950, C ABI in
include/spectree.h):

  spec_tree_attn    tree-masked verify attention over a paged KV prefix
  spec_tree_reject  tree rejection sampling (greedy / with / without replacement)
  spec_kv_compact   keep only the accepted path in the KV cache

and spec_tree_reject_compact, the last two in one launch; spec_tree_kv_write
writes the tree's K/V rows into the paged cache (rotated for their tree
positions) before the attention; spec_tree_truncate applies top-k / top-p to
the target logits before the sampler, and spec_tree_reject_truncated applies
them inside the sampler to the rows its walk visits; spec_sequoia_tree builds the Sequoia-optimal
tree shape for a per-rank acceptance vector (host code).

This package is the thin PyTorch binding: tensors in, device pointers and the
current HIP stream out to the library.
"""
from .binding import (  # noqa: F401
    DEV_ERRORS,
    LIB_PATH,
    SPEC_BF16,
    SPEC_F32,
    SpecError,
    header_functions,
    load_library,
    spec_kv_compact,
    spec_sequoia_tree,
    spec_status_string,
    spec_tree_attn,
    spec_tree_attn_workspace_size,
    spec_tree_reject,
    spec_tree_reject_compact,
    spec_tree_reject_compact_noalloc,
    spec_tree_reject_max_resident,
    spec_tree_reject_plan,
    spec_tree_reject_truncated,
    spec_tree_reject_truncated_plan,
    spec_tree_reject_truncated_workspace_size,
    spec_tree_kv_write,
    spec_tree_truncate,
    spec_tree_write_attn,
    spec_tree_write_attn_workspace_size,
    spec_version,
)
