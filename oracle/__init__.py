"""fp64 CPU oracle -- test infrastructure only (see tree_oracle.py)."""
from .tree_oracle import (  # noqa: F401
    ANC_WORDS, MAX_NODES, is_valid_tree, root_path, ancestor_matrix, pack_bitset,
    build_ancestor_mask, gather_prefix, tree_attention, tree_attention_paged_tree, argmax_first, target_choice,
    accept_one, tree_accept, commit_accepted, draft_children, build_tree,
)
