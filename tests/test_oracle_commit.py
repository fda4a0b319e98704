"""Pins of the oracle's commit of accepted paths into the paged cache.

The main pin goes through attention rather than through the commit's own
indexing: once the accepted path is in the cache, a one-node tree made of the
path's end node, attending to the committed prefix, must reproduce that node's
tree attention of the step before (its visible keys are the old prefix plus
its root-to-node path in both cases).
"""

import numpy as np
import pytest
import torch

import oracle
from tree_causal_attention_jf_amd import workloads as W


def _bits(t):
    return t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.numpy()


def _accept(case):
    return oracle.tree_accept(case.parent.numpy(), case.draft.numpy(), case.target_ids.numpy())


def _commit(case, alen, nodes, table=None, plen=None):
    kp, vp, new = oracle.commit_accepted(_bits(case.k_tree), _bits(case.v_tree), alen, nodes,
                                         case.block_table.numpy() if table is None else table,
                                         case.prefix_len.numpy() if plen is None else plen,
                                         _bits(case.k_pages), _bits(case.v_pages))
    to = (lambda a: torch.from_numpy(a).view(torch.bfloat16)) if case.k_pages.dtype == torch.bfloat16 \
        else torch.from_numpy
    return to(kp), to(vp), new


@pytest.mark.parametrize("lens", [[14, 0, 33, 200], [1, 16, 47]])
def test_committed_path_reproduces_the_end_nodes_attention(lens):
    case = W.make_commit_case(3, lens, N=12, Hq=4, Hkv=2, D=64, max_path_nodes=6, p_agree=0.9)
    alen, nodes, _ = _accept(case)
    assert alen.max() >= 2, "the case should accept paths of several nodes"
    B, N, Hq = case.q.shape[0], case.q.shape[1], case.q.shape[2]
    scale = 0.125
    ends = [int(nodes[b, alen[b]]) for b in range(B)]
    rows = [(b, ends[b], h) for b in range(B) for h in range(Hq)]
    ref, lref = oracle.tree_attention(case.q, case.k_pages, case.v_pages, case.block_table, case.prefix_len,
                                      case.k_tree, case.v_tree, case.parent, scale, rows=rows)
    kp, vp, new_len = _commit(case, alen, nodes)
    assert np.array_equal(new_len, case.prefix_len.numpy() + alen + 1)
    # next step: a one-node tree (the end node itself) over the committed prefix minus its own token
    idx = torch.tensor(ends)
    ar = torch.arange(B)
    q1 = case.q[ar, idx].unsqueeze(1).contiguous()
    k1 = case.k_tree[ar, idx].unsqueeze(1).contiguous()
    v1 = case.v_tree[ar, idx].unsqueeze(1).contiguous()
    p1 = torch.full((B, 1), -1, dtype=torch.int32)
    out1, lse1 = oracle.tree_attention(q1, kp, vp, case.block_table, torch.from_numpy(new_len - 1), k1, v1, p1,
                                       scale)
    for b in range(B):
        for h in range(Hq):
            np.testing.assert_allclose(out1[b, 0, h], ref[b, ends[b], h], rtol=0, atol=1e-12)
            assert abs(lse1[b, 0, h] - lref[b, ends[b], h]) < 1e-12


def test_zero_accepted_tokens_append_the_root_only():
    case = W.make_commit_case(5, [20, 5], N=8, Hq=2, Hkv=2, D=64)
    B, N = 2, 8
    alen = np.zeros(B, dtype=np.int32)
    nodes = np.full((B, N), -1, dtype=np.int32)
    nodes[:, 0] = 0
    kp, vp, new_len = _commit(case, alen, nodes)
    assert new_len.tolist() == [21, 6]
    for b, L in enumerate([20, 5]):
        page = int(case.block_table[b, L // 16])
        assert torch.equal(kp[page, :, L % 16], case.k_tree[b, 0])
        assert torch.equal(vp[page, :, L % 16], case.v_tree[b, 0])


def test_only_the_path_slots_change_and_pages_are_crossed():
    # prefix 14: the path's tokens 14..18 run over the end of page 0 into page 1
    case = W.make_commit_case(7, [14], N=10, Hq=2, Hkv=2, D=64)
    alen = np.array([4], dtype=np.int32)
    nodes = np.full((1, 10), -1, dtype=np.int32)
    nodes[0, :5] = [0, 2, 5, 6, 9]            # any node ids in range; the commit copies what it is given
    kp, vp, new_len = _commit(case, alen, nodes)
    assert new_len.tolist() == [19]
    changed = set()
    for i, n in enumerate(nodes[0, :5]):
        pos = 14 + i
        page, slot = int(case.block_table[0, pos // 16]), pos % 16
        changed.add((page, slot))
        assert torch.equal(kp[page, :, slot], case.k_tree[0, n])
        assert torch.equal(vp[page, :, slot], case.v_tree[0, n])
    assert len({p for p, _ in changed}) == 2
    mask = torch.ones(kp.shape[0], kp.shape[2], dtype=torch.bool)
    for page, slot in changed:
        mask[page, slot] = False
    assert torch.equal(kp.permute(0, 2, 1, 3)[mask], case.k_pages.permute(0, 2, 1, 3)[mask])
    assert torch.equal(vp.permute(0, 2, 1, 3)[mask], case.v_pages.permute(0, 2, 1, 3)[mask])


def test_invalid_sequences_are_left_untouched():
    lens = [10, 10, 10, 10, 10]
    case = W.make_commit_case(9, lens, N=6, Hq=2, Hkv=2, D=64)
    B, N = len(lens), 6
    alen = np.array([2, 6, 1, 1, 2], dtype=np.int32)        # b1: accept_len == N
    nodes = np.full((B, N), -1, dtype=np.int32)
    nodes[:, :3] = [0, 1, 2]
    nodes[2, 1] = N                                          # b2: node id out of range
    table = case.block_table.numpy().copy()
    table[3, (10 + 1) // 16] = -1                            # b3: a page of the new tokens is missing
    plen = case.prefix_len.numpy().copy()
    plen[4] = -1                                             # b4: negative prefix
    kp, vp, new_len = _commit(case, alen, nodes, table=table, plen=plen)
    assert new_len.tolist() == [13, -1, -1, -1, -1]
    for b in range(1, B):
        for p in set(case.block_table[b].tolist()) - {-1}:
            assert torch.equal(kp[p], case.k_pages[p]) and torch.equal(vp[p], case.v_pages[p])
