"""Rows of a full-size attention workload that compare every item of its launch
plan: shared by the GPU parity tests (which compare those rows against the
oracle) and by a CPU test of the selection itself.

An item is one (sequence, KV head, row block) of the plan: row r = node * G + g
of a (sequence, KV head) lies in row block r // RB, where RB is the plan's rows
per workgroup. Every split (or piece) of an item is merged into that item's own
rows, so one compared row covers all of the item's workgroups."""

import numpy as np


def plan_items(jf, wl, tree_len=None):
    """The items of the plan jf_tree_attention uses for workload `wl` (anything
    with q [B, N, Hq, D], k_pages, block_table, sm_scale, max_prefix_len), the
    plan's rows per workgroup, and the plan. With tree_len (ragged budgets, run
    through jf_tree_attention_paged_tree, whose plan is asked for), row blocks
    holding no node of sequence b's tree are not items (the kernel skips them)."""
    B, N, Hq, _ = wl.q.shape
    Hkv = wl.k_pages.shape[1]
    shape = jf.attn_shape(wl.q, wl.k_pages, wl.block_table, wl.sm_scale)
    plan = jf.tree_attention_plan(shape, wl.max_prefix_len, paged_tree=tree_len is not None)
    G = Hq // Hkv
    RB = plan["rows_per_workgroup"]
    items = []
    for b in range(B):
        nb = N if tree_len is None else int(tree_len[b])
        nrb = (G * nb + RB - 1) // RB
        items += [(b, g, rb) for g in range(Hkv) for rb in range(nrb)]
    return items, RB, plan


def item_rows(jf, wl, seed, tree_len=None):
    """Rows (b, node, head): per item, the first and the last node whose rows
    fall in its row block and one random node between them, each with all G
    query heads of the item's KV head. Returns (rows, items, plan)."""
    items, RB, plan = plan_items(jf, wl, tree_len)
    B, N, Hq, _ = wl.q.shape
    G = Hq // wl.k_pages.shape[1]
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = set()
    for b, g, rb in items:
        nb = N if tree_len is None else int(tree_len[b])
        n0 = (rb * RB) // G
        n1 = min(nb, ((rb + 1) * RB + G - 1) // G) - 1
        for node in {n0, n1, int(rng.integers(n0, n1 + 1))}:
            rows |= {(b, node, g * G + j) for j in range(G)}
    return sorted(rows), items, plan


def assert_items_covered(wl, rows, items, plan):
    """Every item has a node whose G heads of the item's KV head are all compared."""
    Hq = wl.q.shape[2]
    Hkv = wl.k_pages.shape[1]
    G = Hq // Hkv
    RB = plan["rows_per_workgroup"]
    heads = {}
    for b, node, h in rows:
        heads.setdefault((b, node), set()).add(h)
    covered = set()
    for (b, node), hs in heads.items():
        for g in range(Hkv):
            if all(g * G + j in hs for j in range(G)):
                covered.add((b, g, (node * G) // RB))
                covered.add((b, g, (node * G + G - 1) // RB))
    missing = [it for it in items if it not in covered]
    assert not missing, f"{len(missing)} of {len(items)} launch-plan items have no fully compared node"
