"""Pins for the oracle's tree-causal attention.

The pages print no worked attention example, so the oracle is pinned by
hand-derived fixtures, by special cases that reduce to a library routine
(torch's scaled_dot_product_attention in fp64), and by invariants the mask
definition fixes (gist.science technical summary of "JetFlow: Breaking the
Scaling Ceiling of Speculative Decoding with Parallel Tree Drafting",
section 2: the mask, and the branch factorisation under which a node depends
only on its own root-to-node path).
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from conftest import read_golden
from tree_causal_attention_jf_amd import workloads as W

F64 = torch.float64


def _wl(seed, tree, N=8, L=40, Hq=4, Hkv=2, D=64, B=1, prefix=None, **kw):
    return W.make_workload("c1_chain16", seed, B=B, N=N, prefix=prefix or ("fixed", L), tree=tree,
                           Hq=Hq, Hkv=Hkv, D=D, dtype=torch.float32, with_accept=False, **kw)


def _run(wl, **kw):
    return oracle.tree_attention(wl.q, wl.k_pages, wl.v_pages, wl.block_table, wl.prefix_len,
                                 wl.k_tree, wl.v_tree, wl.parent, wl.sm_scale, **kw)


def _contig(wl, b):
    """Prefix + tree keys of sequence b, from the generator's contiguous copy."""
    K = torch.cat([wl.k_prefix[b].to(F64), wl.k_tree[b].to(F64)], 0)
    V = torch.cat([wl.v_prefix[b].to(F64), wl.v_tree[b].to(F64)], 0)
    return K, V


def _sdpa(q, k, v, scale, causal=False):
    # q [H, Tq, D], k/v [H, Tk, D] in fp64 on the CPU
    return F.scaled_dot_product_attention(q.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0),
                                          is_causal=causal, scale=scale)[0]


# ---------------------------------------------------------------- fixtures

def _golden_inputs(tree_v, prefix_v, parent, q_val=0.0, k_vals=None, D=1):
    N, L = len(tree_v), len(prefix_v)
    q = torch.full((1, N, 1, D), q_val, dtype=F64)
    k_tree = torch.zeros((1, N, 1, D), dtype=F64)
    if k_vals is not None:
        k_tree[0, :, 0, 0] = torch.tensor(k_vals, dtype=F64)
    v_tree = torch.tensor(tree_v, dtype=F64).reshape(1, N, 1, 1).expand(1, N, 1, D).clone()
    npages = max(1, (L + 15) // 16)
    k_pages = torch.zeros((npages, 1, 16, D), dtype=F64)
    v_pages = torch.zeros((npages, 1, 16, D), dtype=F64)
    for t, x in enumerate(prefix_v):
        v_pages[t // 16, 0, t % 16, :] = x
    table = torch.arange(npages, dtype=torch.int32).reshape(1, -1)
    plen = torch.tensor([L], dtype=torch.int32)
    par = torch.tensor([parent], dtype=torch.int32)
    return q, k_pages, v_pages, table, plen, k_tree, v_tree, par


def test_golden_equal_scores_is_mean_of_visible_values():
    g = read_golden("tree7.txt")
    parent = [int(x) for x in g["parent"]]
    inp = _golden_inputs([float(x) for x in g["attn.tree_v"]], [float(x) for x in g["attn.prefix_v"]],
                         parent)
    out, lse = oracle.tree_attention(*inp, sm_scale=1.0)
    np.testing.assert_allclose(out[0, :, 0, 0], [float(x) for x in g["attn.out"]], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, :, 0], np.log([float(x) for x in g["attn.visible_count"]]),
                               rtol=0, atol=1e-12)


def test_golden_weighted_pair():
    g = read_golden("tree7.txt")
    inp = _golden_inputs([8.0, 4.0], [], [-1, 0], q_val=1.0, k_vals=[math.log(3.0), 0.0])
    out, lse = oracle.tree_attention(*inp, sm_scale=1.0)
    np.testing.assert_allclose(out[0, :, 0, 0], [float(x) for x in g["weighted.out"]], atol=1e-12)
    np.testing.assert_allclose(np.exp(lse[0, :, 0]), [float(x) for x in g["weighted.lse_exp"]], atol=1e-12)


# ---------------------------------------------------------------- reductions to a library routine

@pytest.mark.parametrize("seed,N,L,Hq,Hkv", [(0, 8, 40, 4, 2), (1, 16, 64, 4, 1), (2, 5, 1, 2, 2),
                                               (3, 12, 0, 8, 2), (4, 33, 17, 2, 1)])
def test_chain_equals_causal_attention(seed, N, L, Hq, Hkv):
    """A chain-shaped tree is ordinary causal attention: run the library's
    causal attention over all L + N positions and keep the last N rows."""
    wl = _wl(seed, ("chain",), N=N, L=L, Hq=Hq, Hkv=Hkv)
    out, _ = _run(wl)
    G = Hq // Hkv
    K, V = _contig(wl, 0)                                       # [L+N, Hkv, D]
    rng = torch.Generator().manual_seed(seed)
    qfull = torch.randn((L + N, Hq, wl.D), generator=rng, dtype=F64)
    qfull[L:] = wl.q[0].to(F64)
    kh = K.repeat_interleave(G, dim=1).permute(1, 0, 2)          # [Hq, L+N, D]
    vh = V.repeat_interleave(G, dim=1).permute(1, 0, 2)
    ref = _sdpa(qfull.permute(1, 0, 2), kh, vh, wl.sm_scale, causal=True)  # [Hq, L+N, D]
    np.testing.assert_allclose(out[0], ref[:, L:].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed,tree", [(0, ("random", 6)), (1, ("random", 4)), (2, ("best_first", 4, 10, 2.0))])
def test_each_node_is_attention_over_its_own_path(seed, tree):
    """Branch factorisation: node v's row equals plain (unmasked) attention of
    its query over the prefix plus the K/V of its root-to-v path alone."""
    wl = _wl(seed, tree, N=16, L=37, Hq=4, Hkv=2)
    out, lse = _run(wl)
    G = wl.G
    parent = wl.parent[0].tolist()
    Kp, Vp = wl.k_prefix[0].to(F64), wl.v_prefix[0].to(F64)
    for v in range(wl.N):
        path = []
        u = v
        while u != -1:
            path.append(u)
            u = parent[u]
        path = sorted(path)
        K = torch.cat([Kp, wl.k_tree[0, path].to(F64)], 0)
        V = torch.cat([Vp, wl.v_tree[0, path].to(F64)], 0)
        for h in range(wl.Hq):
            q = wl.q[0, v, h].to(F64).reshape(1, 1, -1)
            ref = _sdpa(q, K[:, h // G].unsqueeze(0), V[:, h // G].unsqueeze(0), wl.sm_scale)
            np.testing.assert_allclose(out[0, v, h], ref[0, 0].numpy(), rtol=0, atol=1e-12)
            s = wl.sm_scale * (K[:, h // G] @ wl.q[0, v, h].to(F64))
            assert abs(lse[0, v, h] - torch.logsumexp(s, 0).item()) < 1e-12


def test_single_node_is_decode_attention():
    wl = _wl(5, ("chain",), N=1, L=77, Hq=8, Hkv=2)
    out, _ = _run(wl)
    K, V = _contig(wl, 0)
    for h in range(wl.Hq):
        ref = _sdpa(wl.q[0, 0, h].to(F64).reshape(1, 1, -1), K[:, h // 4].unsqueeze(0),
                    V[:, h // 4].unsqueeze(0), wl.sm_scale)
        np.testing.assert_allclose(out[0, 0, h], ref[0, 0].numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- invariants

def test_gqa_equals_mha_with_repeated_kv():
    wl = _wl(6, ("random", 5), N=12, L=50, Hq=8, Hkv=2)
    out, lse = _run(wl)
    G = wl.G
    rep = lambda t, dim: t.repeat_interleave(G, dim=dim)
    out2, lse2 = oracle.tree_attention(wl.q, rep(wl.k_pages, 1), rep(wl.v_pages, 1), wl.block_table,
                                       wl.prefix_len, rep(wl.k_tree, 2), rep(wl.v_tree, 2), wl.parent,
                                       wl.sm_scale)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def _subtree(parent, v):
    kids = {}
    for i, p in enumerate(parent):
        kids.setdefault(p, []).append(i)
    out, stack = [], [v]
    while stack:
        u = stack.pop()
        out.append(u)
        stack.extend(kids.get(u, []))
    return sorted(out)


def test_sibling_subtree_permutation_permutes_outputs():
    # a tree where the root has three child subtrees; renumber nodes by visiting
    # the subtrees in reverse order (still topological) and permute inputs alike
    parent = [-1, 0, 0, 0, 1, 1, 2, 3, 3, 4, 6, 7]
    wl = _wl(7, ("chain",), N=len(parent), L=21, Hq=4, Hkv=2)
    wl.parent[0] = torch.tensor(parent, dtype=torch.int32)
    out, lse = _run(wl)
    order = [0]
    for c in (3, 2, 1):
        order += _subtree(parent, c)
    new_of = {old: new for new, old in enumerate(order)}
    new_parent = [-1] * len(parent)
    for old, new in new_of.items():
        if parent[old] >= 0:
            new_parent[new] = new_of[parent[old]]
    assert oracle.is_valid_tree(new_parent)
    perm = torch.tensor(order)
    out2, lse2 = oracle.tree_attention(wl.q[:, perm], wl.k_pages, wl.v_pages, wl.block_table, wl.prefix_len,
                                       wl.k_tree[:, perm], wl.v_tree[:, perm],
                                       torch.tensor([new_parent], dtype=torch.int32), wl.sm_scale)
    np.testing.assert_allclose(out2, out[:, order], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, lse[:, order], rtol=0, atol=1e-12)


def test_mask_leak_non_ancestors_do_not_matter():
    wl = _wl(8, ("random", 6), N=16, L=30, Hq=4, Hkv=1)
    out, lse = _run(wl)
    parent = wl.parent[0].tolist()
    A = oracle.ancestor_matrix(parent)
    v = 13
    hidden = [j for j in range(wl.N) if not A[v, j]]
    k2, v2 = wl.k_tree.clone(), wl.v_tree.clone()
    k2[0, hidden] = torch.randn_like(k2[0, hidden]) * 100
    v2[0, hidden] = torch.randn_like(v2[0, hidden]) * 100
    out2, lse2 = oracle.tree_attention(wl.q, wl.k_pages, wl.v_pages, wl.block_table, wl.prefix_len,
                                       k2, v2, wl.parent, wl.sm_scale)
    np.testing.assert_array_equal(out2[0, v], out[0, v])
    np.testing.assert_array_equal(lse2[0, v], lse[0, v])
    changed = [j for j in range(wl.N) if any(A[j, h] for h in hidden)]
    assert changed and not np.allclose(out2[0, changed], out[0, changed])


def test_page_order_does_not_matter():
    wl = _wl(9, ("random", 6), N=10, L=70, Hq=2, Hkv=1)
    out, _ = _run(wl)
    # re-page the same contiguous prefix into a fresh pool in sequential order
    L, D = 70, wl.D
    npg = (L + 15) // 16
    kp = torch.zeros((npg + 3, 1, 16, D))
    vp = torch.zeros((npg + 3, 1, 16, D))
    for t in range(L):
        kp[3 + t // 16, :, t % 16] = wl.k_prefix[0][t]
        vp[3 + t // 16, :, t % 16] = wl.v_prefix[0][t]
    table = (torch.arange(npg, dtype=torch.int32) + 3).reshape(1, -1)
    out2, _ = oracle.tree_attention(wl.q, kp, vp, table, wl.prefix_len, wl.k_tree, wl.v_tree, wl.parent,
                                    wl.sm_scale)
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-13)


def test_constant_values_give_that_constant():
    wl = _wl(10, ("random", 6), N=16, L=45, Hq=4, Hkv=2)
    c = torch.linspace(-3, 3, wl.D)
    vp = torch.zeros_like(wl.v_pages) + c
    vt = torch.zeros_like(wl.v_tree) + c
    out, _ = oracle.tree_attention(wl.q, wl.k_pages, vp, wl.block_table, wl.prefix_len, wl.k_tree, vt,
                                   wl.parent, wl.sm_scale)
    np.testing.assert_allclose(out, np.broadcast_to(c.double().numpy(), out.shape), rtol=0, atol=1e-13)


def test_one_dominant_key_selects_its_value():
    # node 5's own key is aligned with its query and scaled up: output -> its V
    wl = _wl(11, ("chain",), N=6, L=20, Hq=1, Hkv=1)
    wl.k_tree[0, 5, 0] = wl.q[0, 5, 0] * 1e3
    out, _ = _run(wl)
    np.testing.assert_allclose(out[0, 5, 0], wl.v_tree[0, 5, 0].double().numpy(), rtol=0, atol=1e-12)


def test_row_subset_matches_full():
    wl = _wl(12, ("random", 6), N=16, L=33, Hq=4, Hkv=2, B=2, prefix=("list", [33, 5]))
    out, lse = _run(wl)
    rows = [(0, 3, 1), (1, 15, 3), (1, 0, 0)]
    out2, lse2 = _run(wl, rows=rows)
    for (b, n, h) in rows:
        # a single-row matmul may sum in another order than the full block
        np.testing.assert_allclose(out2[b, n, h], out[b, n, h], rtol=0, atol=1e-14)
        assert abs(lse2[b, n, h] - lse[b, n, h]) < 1e-14
    assert np.isnan(out2[0, 0, 0]).all()


def test_poisoned_unused_slots_are_never_read():
    clean = _wl(13, ("random", 6), N=8, L=37, Hq=2, Hkv=1, extra_pages=3)
    dirty = _wl(13, ("random", 6), N=8, L=37, Hq=2, Hkv=1, extra_pages=3, poison=True)
    assert torch.isnan(dirty.k_pages).any()
    o1, l1 = _run(clean)
    o2, l2 = _run(dirty)
    np.testing.assert_array_equal(o1, o2)
    assert np.isfinite(o2).all()


def test_softmax_weights_sum_to_one_via_lse():
    # sum_t exp(s_t - lse) = 1 over the visible keys, with s from torch matmul
    wl = _wl(14, ("random", 6), N=16, L=25, Hq=2, Hkv=1)
    _, lse = _run(wl)
    A = oracle.ancestor_matrix(wl.parent[0].tolist())
    K, _ = _contig(wl, 0)
    for v in range(wl.N):
        keys = list(range(25)) + [25 + j for j in range(wl.N) if A[v, j]]
        for h in range(wl.Hq):
            s = wl.sm_scale * (K[keys, 0] @ wl.q[0, v, h].to(F64))
            assert abs(torch.exp(s - lse[0, v, h]).sum().item() - 1.0) < 1e-12
