"""GPU parity of jf_tree_attention_paged_tree (ragged budgets, tree K/V in the
paged cache after the prefix) against the oracle, through the C ABI.

Bars as for jf_tree_attention: bf16 within 1e-2 absolute and 1e-2 of max|ref|
(the derived 2^-7 max|V| bar for unscaled data), lse within 2^-8 + 1e-4;
padding rows untouched; with full budgets, bit-identical to jf_tree_attention
given the same K/V as separate tree arrays.
"""

import numpy as np
import pytest
import torch

import oracle
from tree_causal_attention_jf_amd import workloads as W
from plan_items import assert_items_covered, item_rows

pytestmark = pytest.mark.gpu

DEV = "cuda"
SENTINEL = 7.0


@pytest.fixture(scope="module")
def jf():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from tree_causal_attention_jf_amd import binding
    return binding


def _run(jf, case, tree_len=None):
    t = {k: getattr(case, k).to(DEV) for k in ("q", "k_pages", "v_pages", "block_table", "prefix_len", "parent")}
    anc, _, bad = jf.build_ancestor_mask(t["parent"])
    out = torch.full_like(t["q"], SENTINEL)
    lse = torch.full(case.q.shape[:3], SENTINEL, dtype=torch.float32, device=DEV)
    tl = (case.tree_len if tree_len is None else tree_len).to(DEV)
    jf.tree_attention_paged_tree(t["q"], t["k_pages"], t["v_pages"], t["block_table"], t["prefix_len"], anc,
                                 tree_len=tl, sm_scale=case.sm_scale, max_prefix_len=case.max_prefix_len,
                                 out=out, lse=lse)
    torch.cuda.synchronize()
    assert not bad.any()
    return out, lse


def _check(case, out, lse, rows=None, what=""):
    ref, lref = oracle.tree_attention_paged_tree(case.q, case.k_pages, case.v_pages, case.block_table,
                                                 case.prefix_len, case.tree_len, case.parent, case.sm_scale,
                                                 rows=rows)
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    nb = case.tree_len.tolist()
    vmax = float(case.v_pages.float().abs().max())
    bar = max(1e-2, 2.0 ** -7 * vmax)
    worst = 0.0
    sel = rows if rows is not None else [(b, n, h) for b in range(len(nb)) for n in range(nb[b])
                                         for h in range(case.q.shape[2])]
    for (b, n, h) in sel:
        worst = max(worst, float(np.abs(o[b, n, h] - ref[b, n, h]).max()))
        assert abs(l[b, n, h] - lref[b, n, h]) <= 2.0 ** -8 + 1e-4, (what, b, n, h)
    scale = max(float(np.nanmax(np.abs(ref))), 1e-30)
    print(f"  {what}: max|err| {worst:.3e} (bar {bar:.3e}), rel {worst / scale:.3e}", flush=True)
    assert worst <= bar, what
    assert worst <= 1e-2 * scale, what
    # padding rows were not touched
    for b in range(len(nb)):
        assert (o[b, nb[b]:] == SENTINEL).all() and (l[b, nb[b]:] == SENTINEL).all(), (what, b)


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 8, 2), (64, 16, 2)])
@pytest.mark.parametrize("unscaled", [False, True])
def test_paged_tree_ragged_budgets(jf, D, Hq, Hkv, unscaled):
    # budgets 0, 1, full and in between; prefixes empty, mid-page and on a page edge
    lens = [14, 0, 33, 16, 100]
    budgets = [40, 7, 0, 1, 23]
    case = W.make_paged_tree_case(21, lens, budgets, N=40, Hq=Hq, Hkv=Hkv, D=D, tree=("random", 7),
                                  unscaled=unscaled)
    out, lse = _run(jf, case)
    _check(case, out, lse, what=f"D {D} Hq {Hq} unscaled {unscaled}")


@pytest.mark.parametrize("rw,splits,balanced", [(1, 5, 1), (4, 3, 0), (8, 2, 1), (8, 0, 1), (2, 7, 0)])
def test_paged_tree_forced_plans(jf, rw, splits, balanced, monkeypatch):
    monkeypatch.setenv("JF_RW", str(rw))
    monkeypatch.setenv("JF_SPLITS", str(splits))
    monkeypatch.setenv("JF_BALANCED", str(balanced))
    case = W.make_paged_tree_case(23, [700, 0, 1, 2100], [150, 3, 90, 64], N=150, Hq=8, Hkv=2, D=128,
                                  tree=("random", 9))
    out, lse = _run(jf, case)
    _check(case, out, lse, what=f"rw {rw} splits {splits} balanced {balanced}")


@pytest.mark.parametrize("balanced", [1, 0])
def test_paged_tree_row_blocks_past_the_budget(jf, balanced, monkeypatch):
    # N 256 at G 4 gives four 256-row blocks per KV head; budgets 3, 0 and 70 leave
    # whole blocks without a node of the tree (they exit), 256 leaves none
    monkeypatch.setenv("JF_BALANCED", str(balanced))
    case = W.make_paged_tree_case(29, [40, 300, 17, 129], [3, 0, 70, 256], N=256, Hq=8, Hkv=2, D=128,
                                  tree=("random", 11))
    out, lse = _run(jf, case)
    _check(case, out, lse, what=f"balanced {balanced}")


@pytest.mark.parametrize("rw,cus", [(4, 256), (4, 24), (8, 256), (8, 40)])
def test_paged_tree_live_row_blocks_only(jf, rw, cus, monkeypatch):
    # the balanced schedule gives workgroups to the row blocks that hold rows of a
    # tree only, packed per XCD in rank order; with few CUs (JF_TARGET_WG) each XCD
    # holds several units one after another, and in 256-row blocks long sequences
    # may be cut into head and tail. Budgets 0, 1, 3 and full beside ragged ones.
    monkeypatch.setenv("JF_RW", str(rw))
    monkeypatch.setenv("JF_TARGET_WG", str(cus))
    lens = [900, 40, 2000, 300, 17, 1500, 640, 1100, 64, 2600]
    budgets = [256, 3, 130, 0, 70, 1, 200, 47, 256, 90]
    case = W.make_paged_tree_case(37, lens, budgets, N=256, Hq=8, Hkv=2, D=128, tree=("best_first", 4, 12, 2.0))
    assert jf.tree_attention_plan(jf.attn_shape(case.q, case.k_pages, case.block_table, case.sm_scale),
                                  case.max_prefix_len, paged_tree=True)["balanced"] == 1
    out, lse = _run(jf, case)
    _check(case, out, lse, what=f"rw {rw} cus {cus}")


def test_full_budgets_match_the_separate_tree_kernel_bit_for_bit(jf):
    case = W.make_paged_tree_case(25, [300, 17, 64], [24, 24, 24], N=24, Hq=8, Hkv=2, D=128, tree=("random", 6))
    out, lse = _run(jf, case)
    t = {k: getattr(case, k).to(DEV) for k in ("q", "k_pages", "v_pages", "block_table", "prefix_len", "parent",
                                                "k_tree", "v_tree")}
    anc, _, _ = jf.build_ancestor_mask(t["parent"])
    out2, lse2 = jf.tree_attention(t["q"], t["k_pages"], t["v_pages"], t["block_table"], t["prefix_len"],
                                   t["k_tree"], t["v_tree"], anc, sm_scale=case.sm_scale,
                                   max_prefix_len=case.max_prefix_len, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse, lse2)


def test_paged_tree_budget256_sampled(jf):
    # batch 8, best-first trees of ragged budgets up to 256, prefixes U[1024, 4096]
    rng = np.random.Generator(np.random.PCG64(31))
    lens = rng.integers(1024, 4097, size=8).tolist()
    budgets = rng.integers(16, 257, size=8).tolist()
    case = W.make_paged_tree_case(31, lens, budgets, N=256, Hq=32, Hkv=8, D=128, tree=("best_first", 4, 12, 2.0))
    out, lse = _run(jf, case)
    # every live (sequence, KV head, row block) item of the plan has a node with all heads compared
    rows, items, plan = item_rows(jf, case, 5, tree_len=budgets)
    assert_items_covered(case, rows, items, plan)
    rows = sorted(set(rows) | {(b, budgets[b] - 1, 31) for b in range(8)})
    _check(case, out, lse, rows=rows, what=f"budgets {budgets}, {len(items)} plan items")


def test_paged_tree_bad_lengths_and_missing_pages_give_nan(jf):
    case = W.make_paged_tree_case(27, [20, 20, 20], [8, 8, 8], N=8, Hq=4, Hkv=2, D=128)
    tl = torch.tensor([9, -1, 8], dtype=torch.int32)          # b0, b1: bad tree lengths
    table = case.block_table.clone()
    table[2, (20 + 7) // 16] = case.k_pages.shape[0]            # b2: a tree page past the pool
    case.block_table = table
    out, lse = _run(jf, case, tree_len=tl)
    assert torch.isnan(out[:, :].float()).all() and torch.isnan(lse).all()


def test_paged_tree_default_streaming_plan(jf):
    # 16-node frames at 4 query heads per KV head (64 rows) over prefixes long enough that
    # the default plan takes one 64-row block with two key groups; budgets ragged
    from tree_causal_attention_jf_amd import binding
    case = W.make_paged_tree_case(31, [2100, 1990, 2048, 1500], [16, 9, 1, 12], N=16, Hq=32, Hkv=8, D=128,
                                  tree=("random", 6))
    shape = binding.attn_shape(case.q, case.k_pages, case.block_table, case.sm_scale)
    assert binding.tree_attention_plan(shape, case.max_prefix_len)["rows_per_workgroup"] == 64
    out, lse = _run(jf, case)
    _check(case, out, lse, what="default streaming plan")
