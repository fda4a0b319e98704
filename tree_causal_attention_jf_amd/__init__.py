"""MI355X-native tree-causal attention and greedy tree acceptance.

The compute path is a C-ABI HIP library (libjf_tree.so, built for gfx950);
`tree_causal_attention_jf_amd.binding` is a thin ctypes layer over it.
"""
