"""Host-side launch plans of the bf16 attention (no GPU needed: the plan query
runs the same host code the entry points use and launches nothing).

Pins the plan choices the kernels are built around, per workload shape:
  * few rows per KV head (budget 16): 32-row blocks with four key groups, one
    round of four tiles per split, the tree in a split of its own;
  * 256-node trees in batches: 256-row blocks, one key group, planned inside the
    kernel from the prefix lengths (balanced);
  * one sequence of 256 nodes (the draft head's pass): 128-row blocks, two key
    groups, equal splits that fill the CUs;
  * ragged budgets: 128-row blocks;
  * few rows with long prefixes: 64-row blocks with two key groups;
and the invariants every plan keeps (page ranges in whole tiles, within the
per-split page limit, covering the longest prefix)."""
import pytest

from tree_causal_attention_jf_amd import binding as jf

ENV_KNOBS = ("JF_RW", "JF_RPW", "JF_SPLITS", "JF_BALANCED", "JF_TARGET_WG", "JF_BAL_CUT", "JF_BAL_HT",
             "JF_STREAM_TILES", "JF_STREAM_TILES1")


@pytest.fixture(autouse=True)
def _no_knobs(monkeypatch):
    for k in ENV_KNOBS:
        monkeypatch.delenv(k, raising=False)


def plan(B, N, Hq, Hkv, maxp, D=128, paged=False):
    s = jf.AttnShape(B=B, N=N, Hq=Hq, Hkv=Hkv, D=D, page_size=16, num_pages=1 << 20,
                     max_pages_per_seq=(maxp + 15) // 16, dtype=jf.JF_BF16, sm_scale=0.1)
    p = jf.tree_attention_plan(s, maxp, paged)
    # invariants of every plan
    max_pages = (maxp + 15) // 16
    assert p["pages_per_split"] % 4 == 0 and 4 <= p["pages_per_split"] <= 1024
    assert p["splits"] >= 1 and p["splits"] * p["pages_per_split"] >= max_pages
    rows = N * (Hq // Hkv)
    items = B * Hkv * -(-rows // p["rows_per_workgroup"])
    assert p["workgroups"] == items * p["splits"]
    assert p["rows_per_workgroup"] in (32, 64, 128, 256)
    return p


def test_budget16_plan():
    p = plan(1, 16, 32, 8, 2048)
    assert (p["rows_per_workgroup"], p["key_groups"], p["splits"], p["tree_split"], p["balanced"]) == (32, 4, 9, 1, 0)
    assert p["pages_per_split"] == 16 and p["workgroups"] == 144


@pytest.mark.parametrize("B,N,Hq,Hkv,maxp", [(8, 256, 32, 8, 4096), (32, 64, 32, 4, 8192), (4, 256, 32, 8, 32768)],
                         ids=["budget256", "budget64", "long_context"])
def test_batches_of_full_trees_plan(B, N, Hq, Hkv, maxp):
    p = plan(B, N, Hq, Hkv, maxp)
    assert (p["rows_per_workgroup"], p["key_groups"], p["balanced"], p["tree_split"]) == (256, 1, 1, 0)


def test_draft_head_plan():
    p = plan(1, 256, 32, 8, 8192)
    assert (p["rows_per_workgroup"], p["key_groups"], p["balanced"]) == (128, 2, 0)
    assert p["workgroups"] == 256


def test_ragged_budgets_plan():
    p = plan(8, 256, 32, 8, 4096, paged=True)
    assert (p["rows_per_workgroup"], p["key_groups"], p["balanced"]) == (128, 2, 1)


@pytest.mark.parametrize("B,maxp", [(8, 16384), (1, 32768)], ids=["batch8_16k", "one_32k"])
def test_few_rows_long_prefix_plan(B, maxp):
    p = plan(B, 16, 32, 8, maxp)
    assert (p["rows_per_workgroup"], p["key_groups"]) == (64, 2)
    assert p["workgroups"] <= 256


def test_env_knobs_override_the_plan(monkeypatch):
    monkeypatch.setenv("JF_RW", "8")
    assert plan(1, 16, 32, 8, 2048)["rows_per_workgroup"] == 256
    monkeypatch.setenv("JF_RW", "1")
    monkeypatch.setenv("JF_SPLITS", "3")
    p = plan(1, 16, 32, 8, 2048)
    assert p["rows_per_workgroup"] == 32 and p["splits"] <= 4
