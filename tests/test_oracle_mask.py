"""Pins for the oracle's tree structure: ancestor sets, depths, bitset encoding.

Definition: gist.science technical summary of "JetFlow: Breaking the Scaling
Ceiling of Speculative Decoding with Parallel Tree Drafting", section 2,
tree-causal attention mask (a node sees its ancestors and itself, never its
descendants or sibling branches).
"""

import itertools

import numpy as np
import pytest

import oracle
from conftest import read_golden
from tree_causal_attention_jf_amd import workloads as W


def _ints(xs):
    return [int(x) for x in xs]


def test_golden_tree7_visible_sets_depths_bits():
    g = read_golden("tree7.txt")
    parent = _ints(g["parent"])
    A = oracle.ancestor_matrix(parent)
    for i in range(len(parent)):
        assert sorted(np.nonzero(A[i])[0].tolist()) == _ints(g[f"visible.{i}"])
    anc, depth, bad = oracle.build_ancestor_mask(np.array([parent]))
    assert bad.tolist() == [0]
    assert depth[0].tolist() == _ints(g["depth"])
    assert [int(w) for w in anc[0, :, 0]] == _ints(g["anc_word0"])
    assert not anc[0, :, 1:].any()


def test_chain_is_lower_triangular():
    for n in (1, 2, 16, 100, 256):
        A = oracle.ancestor_matrix(W.tree_chain(n))
        assert np.array_equal(A, np.tril(np.ones((n, n), dtype=bool)))


def test_star_sees_root_and_itself():
    n = 40
    parent = [-1] + [0] * (n - 1)
    A = oracle.ancestor_matrix(parent)
    for i in range(n):
        assert set(np.nonzero(A[i])[0].tolist()) == ({0, i} if i else {0})


def test_complete_binary_tree_closed_form():
    # BFS numbering of a complete binary tree: with 1-based labels m = i + 1,
    # the ancestors of m are m >> s for s >= 0 (classic heap indexing).
    n = 255
    parent = [-1] + [(i - 1) // 2 for i in range(1, n)]
    A = oracle.ancestor_matrix(parent)
    for i in range(n):
        m = i + 1
        expect = set()
        while m:
            expect.add(m - 1)
            m >>= 1
        assert set(np.nonzero(A[i])[0].tolist()) == expect
    _, depth, _ = oracle.build_ancestor_mask(np.array([parent]))
    assert depth[0].tolist() == [int(i + 1).bit_length() for i in range(n)]


def _trees(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    yield W.tree_random_recursive(16, 6, rng)
    yield W.tree_random_recursive(200, 12, rng)
    yield W.tree_chain(256)
    yield W.tree_best_first(64, 4, 10, 2048, 2.0, rng)[0]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_relation_invariants(seed):
    for parent in _trees(seed):
        n = len(parent)
        A = oracle.ancestor_matrix(parent)
        # reflexive, only earlier nodes, contains the parent
        assert A.diagonal().all()
        assert not np.triu(A, 1).any()
        for i in range(1, n):
            assert A[i, parent[i]]
        # recursion: visible(i) = visible(parent(i)) + {i}
        for i in range(1, n):
            expect = A[parent[i]].copy()
            expect[i] = True
            assert np.array_equal(A[i], expect)
        # transitive
        Ai = A.astype(np.int64)
        assert np.array_equal((Ai @ Ai) > 0, A)
        # siblings never see each other, nor a node its descendants
        for i in range(n):
            for j in range(n):
                if i != j and parent[i] == parent[j]:
                    assert not A[i, j]


def test_bitset_word_and_bit_positions():
    # a 256-node chain: node 255 sees every node, so all four words are full
    anc, depth, bad = oracle.build_ancestor_mask(np.array([W.tree_chain(256)]))
    full = np.uint64(0xFFFFFFFFFFFFFFFF)
    assert (anc[0, 255] == full).all()
    # node 64 sees 0..64: word 0 full, word 1 only bit 0
    assert anc[0, 64, 0] == full and anc[0, 64, 1] == 1 and anc[0, 64, 2] == 0
    # node 63 sees 0..63: word 0 full, nothing else
    assert anc[0, 63, 0] == full and not anc[0, 63, 1:].any()
    assert depth[0, 200] == 201 and bad[0] == 0
    # a star of 256: node 200 = bit 0 of word 0 and bit 8 of word 3
    star = np.array([[-1] + [0] * 255])
    anc, depth, _ = oracle.build_ancestor_mask(star)
    assert anc[0, 200].tolist() == [1, 0, 0, 1 << 8]
    assert depth[0, 200] == 2


@pytest.mark.parametrize("bad_parent", [
    [0, 0, 1],          # root must have parent -1
    [-1, 1, 1],         # parent must come earlier
    [-1, 0, 3, 1],      # forward reference
    [-1, 0, -1],        # a second root
    [-1, -2, 0],        # negative index
])
def test_invalid_trees_flagged(bad_parent):
    assert not oracle.is_valid_tree(bad_parent)
    anc, depth, bad = oracle.build_ancestor_mask(np.array([[-1, 0, 0, 1], bad_parent + [0] * (4 - len(bad_parent))]))
    assert bad.tolist() == [0, 1]


def test_all_small_topological_trees():
    # every labelled tree in creation order with n <= 6 nodes: (n-1)! of them
    for n in range(1, 7):
        count = 0
        for choice in itertools.product(*[range(i) for i in range(1, n)]):
            parent = [-1] + list(choice)
            A = oracle.ancestor_matrix(parent)
            for i in range(n):
                # walk up with an explicit loop counter as an independent check
                seen, u, steps = set(), i, 0
                while u != -1 and steps <= n:
                    seen.add(u)
                    u = parent[u]
                    steps += 1
                assert set(np.nonzero(A[i])[0].tolist()) == seen
            count += 1
        assert count == max(1, int(np.prod(range(1, n))))
