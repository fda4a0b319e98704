"""Pins of the oracle's tree attention with ragged budgets and the tree's K/V
in the paged cache (node j of sequence b is cached token prefix_len[b] + j)."""

import numpy as np
import pytest
import torch

import oracle
from tree_causal_attention_jf_amd import workloads as W


def _paged(case, tree_len=None):
    return oracle.tree_attention_paged_tree(case.q, case.k_pages, case.v_pages, case.block_table, case.prefix_len,
                                            case.tree_len if tree_len is None else tree_len, case.parent,
                                            case.sm_scale)


def test_full_budgets_equal_the_separate_tree_oracle():
    # the generator also hands out the tree's K/V as separate arrays (sliced from
    # the same token runs); with every budget full the two oracles must agree
    case = W.make_paged_tree_case(2, [14, 0, 33, 16], [12, 12, 12, 12], N=12, Hq=4, Hkv=2, D=64)
    out, lse = _paged(case)
    ref, lref = oracle.tree_attention(case.q, case.k_pages, case.v_pages, case.block_table, case.prefix_len,
                                      case.k_tree, case.v_tree, case.parent, case.sm_scale)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lref, rtol=0, atol=1e-13)


def test_a_smaller_budget_leaves_the_remaining_nodes_unchanged():
    # nodes see only their ancestors (smaller indices), so cutting the tree after
    # node n - 1 (same cache, same parent array) changes no row below n
    case = W.make_paged_tree_case(4, [20, 7, 40], [16, 16, 16], N=16, Hq=4, Hkv=2, D=64, tree=("random", 8))
    full, lfull = _paged(case)
    cut = torch.tensor([5, 1, 16], dtype=torch.int32)
    part, lpart = _paged(case, tree_len=cut)
    for b, n in enumerate(cut.tolist()):
        # (equal up to fp64 summation order: the masked products have other shapes)
        np.testing.assert_allclose(part[b, :n], full[b, :n], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lpart[b, :n], lfull[b, :n], rtol=0, atol=1e-13)
        assert np.isnan(part[b, n:]).all()


@pytest.mark.parametrize("lens,budgets", [([30, 0, 17], [9, 5, 1]), ([16], [16])])
def test_chain_trees_are_causal_attention_over_the_cached_run(lens, budgets):
    # a chain of N_b nodes after an L_b-token prefix is ordinary causal attention
    # over the first L_b + N_b cached tokens (torch SDPA in fp64)
    N = max(budgets)
    case = W.make_paged_tree_case(6, lens, budgets, N=N, Hq=4, Hkv=2, D=64, tree=("chain",))
    out, _ = _paged(case)
    G = 2
    for b, (L, n) in enumerate(zip(lens, budgets)):
        kp = oracle.gather_prefix(case.k_pages.double().numpy(), case.block_table[b].numpy(), L + n, 16)
        vp = oracle.gather_prefix(case.v_pages.double().numpy(), case.block_table[b].numpy(), L + n, 16)
        K = torch.from_numpy(kp).permute(1, 0, 2).repeat_interleave(G, 0)        # [Hq, L+n, D]
        V = torch.from_numpy(vp).permute(1, 0, 2).repeat_interleave(G, 0)
        qfull = torch.zeros((case.q.shape[2], L + n, case.q.shape[3]), dtype=torch.float64)
        qfull[:, L:] = case.q[b, :n].double().permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(qfull, K, V, is_causal=True, scale=case.sm_scale)
        np.testing.assert_allclose(out[b, :n], ref[:, L:].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
