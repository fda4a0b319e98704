"""The row selection of the full-size GPU parity tests (tests/plan_items.py):
for each full-size workload's launch plan (from jf_tree_attention_plan, host
only), the selected rows give every (sequence, KV head, row block) item a node
with all of its query heads, and a selection that misses one item is caught.
Only shapes are needed, so the tensors here are zero-stride stand-ins."""

import os
import sys
from types import SimpleNamespace

import pytest
import torch

from conftest import ROOT

sys.path.insert(0, os.path.join(ROOT, "tests"))
from plan_items import assert_items_covered, item_rows  # noqa: E402


@pytest.fixture(scope="module")
def jf():
    from tree_causal_attention_jf_amd import binding
    return binding


def _shape_only(B, N, Hq, Hkv, D, max_prefix, pages=None):
    mp = (max_prefix + 15) // 16
    P = pages if pages is not None else B * mp + 4
    e = torch.empty(1, dtype=torch.bfloat16)
    return SimpleNamespace(q=e.expand(B, N, Hq, D), k_pages=e.expand(P, Hkv, 16, D),
                           block_table=torch.empty(1, dtype=torch.int32).expand(B, mp),
                           sm_scale=D ** -0.5, max_prefix_len=max_prefix)


WORKLOADS = {
    # name: (B, N, Hq, Hkv, D, longest prefix)
    "c2_bf256_b8": (8, 256, 32, 8, 128, 4096),
    "c3_bf64_b32": (32, 64, 32, 4, 128, 8192),
    "c4_bf256_32k": (4, 256, 32, 8, 128, 32768),
    "draft_head_b1": (1, 256, 32, 8, 128, 8192),
    "streaming_b1_32k": (1, 16, 32, 8, 128, 32768),
    "streaming_b8_16k": (8, 16, 32, 8, 128, 16384),
}


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_selection_covers_every_plan_item(jf, name):
    B, N, Hq, Hkv, D, L = WORKLOADS[name]
    wl = _shape_only(B, N, Hq, Hkv, D, L)
    rows, items, plan = item_rows(jf, wl, 1)
    G = Hq // Hkv
    assert len(items) == B * Hkv * ((G * N + plan["rows_per_workgroup"] - 1) // plan["rows_per_workgroup"])
    assert_items_covered(wl, rows, items, plan)
    # a planted gap: drop every row of one item's nodes and the check must fail
    b, g, rb = items[len(items) // 2]
    RB = plan["rows_per_workgroup"]
    gone = [r for r in rows if not (r[0] == b and g * G <= r[2] < (g + 1) * G and (r[1] * G) // RB == rb
                                    or r[0] == b and g * G <= r[2] < (g + 1) * G and (r[1] * G + G - 1) // RB == rb)]
    with pytest.raises(AssertionError):
        assert_items_covered(wl, gone, items, plan)
    # one missing head of a node is enough to leave its item uncovered when it is the item's only node
    if len(items) > 1:
        one = [r for r in rows if (r[0], r[2] // G) == (b, g) and r[1] * G // RB == rb]
        partial = [r for r in rows if r not in one] + one[:-1]
        nodes = {r[1] for r in one}
        if len(nodes) == 1:
            with pytest.raises(AssertionError):
                assert_items_covered(wl, partial, items, plan)


def test_ragged_budgets_skip_row_blocks_past_the_tree(jf):
    budgets = [58, 211, 172, 235, 137, 162, 249, 16]
    wl = _shape_only(8, 256, 32, 8, 128, 4096 + 256)
    rows, items, plan = item_rows(jf, wl, 5, tree_len=budgets)
    assert_items_covered(wl, rows, items, plan)
    RB, G = plan["rows_per_workgroup"], 4
    assert {rb for b, g, rb in items if b == 7} == set(range((16 * G + RB - 1) // RB))
    assert all(node < budgets[b] for b, node, h in rows)
