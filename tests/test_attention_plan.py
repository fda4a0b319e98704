"""The attention launch plan (host logic, through jf_tree_attention_plan; no
GPU): 32-row blocks with four key groups at budget 16, 64-row streaming blocks
once many tiles fall to each workgroup, a grid that never exceeds one
workgroup per CU unless the 1024-page split limit binds (room kept for the
tree's own split), 128-row blocks for one sequence with few items and for
ragged budgets, 7/8 of the CUs for one sequence in 256-row blocks, and the
batch schedule for 2..64 sequences."""

import itertools

import pytest

from test_abi import JF_ERR_NULL, JF_ERR_UNSUPPORTED, _shape


@pytest.fixture(scope="module")
def jf():
    from tree_causal_attention_jf_amd import binding
    return binding


def plan(jf, max_prefix, **kw):
    d = dict(B=1, N=16, Hq=32, Hkv=8, D=128, page_size=16)
    d.update(kw)
    pages = (max_prefix + 15) // 16 + 1
    s = _shape(jf, num_pages=max(1, pages * d["B"]), max_pages_per_seq=max(1, pages), **d)
    return jf.tree_attention_plan(s, max_prefix)


def test_budget16_plan(jf):
    p = plan(jf, 2048)
    # 64 packed rows per KV head: two 32-row blocks, four key groups; 8 prefix splits + the tree's
    assert (p["rows_per_workgroup"], p["key_groups"], p["splits"], p["tree_split"]) == (32, 4, 9, 1)
    assert p["workgroups"] == 8 * 2 * 9 == 144


def test_streaming_plan_for_long_prefixes(jf):
    # batch 8 x 16384 at 16 nodes: one 64-row block (both row groups share every tile), two key groups
    p = plan(jf, 16384, B=8)
    assert (p["rows_per_workgroup"], p["key_groups"], p["balanced"]) == (64, 2, 1)
    # one sequence switches at 32 tiles per workgroup, batches at 8
    assert plan(jf, 16384)["rows_per_workgroup"] == 32
    assert plan(jf, 32768)["rows_per_workgroup"] == 64
    assert plan(jf, 2048, B=4)["rows_per_workgroup"] == 64
    assert plan(jf, 2048, B=2)["rows_per_workgroup"] == 32


def test_one_sequence_grid_never_exceeds_the_cus(jf):
    for L, N, Hkv, G in itertools.product((16, 700, 2048, 4096, 8192, 32768, 100000), (1, 16, 64, 256),
                                         (1, 4, 8), (1, 4, 8)):
        p = plan(jf, L, N=N, Hkv=Hkv, Hq=Hkv * G)
        # unless a split's page list (at most 1024 pages) forces more splits
        pages = (L + 15) // 16
        assert p["workgroups"] <= 256 or p["splits"] == (pages + 1023) // 1024, (L, N, Hkv, G, p)
        assert p["splits"] >= 1 and p["pages_per_split"] % 4 == 0


def test_one_sequence_few_items_take_128_row_blocks(jf):
    # 1 x 256 nodes, 8 KV heads: 256-row blocks would give 32 items (7 splits each);
    # 128-row blocks with two key groups give 64 items x 4 splits
    p = plan(jf, 8192, N=256)
    assert (p["rows_per_workgroup"], p["key_groups"], p["splits"], p["workgroups"]) == (128, 2, 4, 256)
    # the 4 tree tiles count as 16 pages when the splits are sized: (512 + 16) / 4 = 132 pages
    # per split, so the last split holds 116 prefix pages plus the tree (33 tiles each)
    assert p["pages_per_split"] == 132 and p["tree_split"] == 0


def test_tree_pages_never_change_the_split_count(jf):
    for L, N in itertools.product((700, 2048, 4096, 8192, 8200, 32768), (64, 128, 256)):
        p = plan(jf, L, N=N)
        pages = (L + 15) // 16
        assert (pages + p["pages_per_split"] - 1) // p["pages_per_split"] == p["splits"] - p["tree_split"], (L, N, p)


def test_one_sequence_256_row_blocks_leave_cus_free(jf):
    # enough items for 256-row blocks (16 KV heads: 64 items): 7/8 of the CUs
    p = plan(jf, 8192, N=256, Hkv=16, Hq=64)
    assert p["rows_per_workgroup"] == 256 and p["workgroups"] <= 224, p


def test_batches_of_full_trees_keep_256_row_blocks(jf):
    for B, L in ((8, 4096), (4, 32768)):
        assert plan(jf, L, B=B, N=256)["rows_per_workgroup"] == 256


def test_ragged_budgets_take_128_row_blocks(jf):
    d = dict(B=8, N=256, Hq=32, Hkv=8, D=128, page_size=16)
    pages = 4096 // 16 + 256 // 16 + 1
    s = _shape(jf, num_pages=pages * 8, max_pages_per_seq=pages, **d)
    full, ragged = jf.tree_attention_plan(s, 4096), jf.tree_attention_plan(s, 4096, paged_tree=True)
    assert full["rows_per_workgroup"] == 256 and ragged["rows_per_workgroup"] == 128 and ragged["key_groups"] == 2
    # one workspace serves both entry points
    import ctypes
    need = jf._lib.jf_tree_attention_workspace_bytes(ctypes.byref(s), 4096)
    assert need > 0
    # budget-16 shapes: the same plan either way
    s16 = _shape(jf, num_pages=200, max_pages_per_seq=200, B=1, N=16, Hq=32, Hkv=8, D=128, page_size=16)
    assert jf.tree_attention_plan(s16, 2048) == jf.tree_attention_plan(s16, 2048, paged_tree=True)


def test_batches_use_the_device_schedule(jf):
    assert plan(jf, 4096, B=8, N=256)["balanced"] == 1
    assert plan(jf, 4096, B=65, N=16)["balanced"] == 0
    assert plan(jf, 4096, B=1, N=256)["balanced"] == 0


def test_plan_host_errors(jf):
    import ctypes
    s = _shape(jf)
    assert jf._lib.jf_tree_attention_plan(ctypes.byref(s), 2048, None) == JF_ERR_NULL
    out = (ctypes.c_int32 * 8)()
    assert jf._lib.jf_tree_attention_plan(ctypes.byref(_shape(jf, dtype=jf.JF_F32)), 2048, out) == JF_ERR_UNSUPPORTED
