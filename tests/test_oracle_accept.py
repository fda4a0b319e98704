"""Pins for the oracle's target choice (argmax) and greedy tree acceptance.

Acceptance rule: the lay summary on the gist.science pages of "JetFlow:
Breaking the Scaling Ceiling of Speculative Decoding with Parallel Tree
Drafting" and the qxai.app commentary (the target keeps the drafted tokens up
to the first disagreement); the tree form keeps the longest agreeing
root-to-node path. Where two agreeing siblings carry the same token the pages
are silent; the reading taken is "longest path, smallest end index".
"""

import itertools

import numpy as np
import pytest
import torch

import oracle
from conftest import read_golden


def _ints(xs):
    return [int(x) for x in xs]


def test_golden_tree7_cases():
    g = read_golden("tree7.txt")
    parent = _ints(g["parent"])
    nxt = _ints(g["next"])
    for c in "abcd":
        alen, nodes, bonus = oracle.accept_one(parent, _ints(g[f"case.{c}.draft"]), nxt)
        want_nodes = _ints(g[f"case.{c}.nodes"])
        assert alen == int(g[f"case.{c}.accept_len"][0])
        assert nodes == want_nodes + [-1] * (len(parent) - len(want_nodes))
        assert bonus == int(g[f"case.{c}.bonus"][0])


# ---------------------------------------------------------------- argmax

def test_argmax_matches_numpy_first_occurrence():
    rng = np.random.Generator(np.random.PCG64(0))
    for _ in range(50):
        x = rng.integers(-4, 5, size=300).astype(np.float64)  # many ties
        assert oracle.argmax_first(x) == int(np.argmax(x))
    x = torch.randn(151936, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    assert oracle.argmax_first(x) == int(np.argmax(x.float().numpy()))


def test_argmax_special_values():
    nan, inf = float("nan"), float("inf")
    assert oracle.argmax_first([nan, nan, nan]) == 0
    assert oracle.argmax_first([nan, -inf, nan]) == 1
    assert oracle.argmax_first([nan, 1.0, nan, 2.0, 2.0]) == 3
    assert oracle.argmax_first([-0.0, 0.0]) == 0
    assert oracle.argmax_first([0.0, -0.0, -1.0]) == 0
    assert oracle.argmax_first([-1.0, -0.0, 0.0]) == 1
    assert oracle.argmax_first([1.0, inf, nan, inf]) == 1
    assert oracle.argmax_first([-inf, -inf]) == 0


def test_target_choice_batched():
    lg = torch.tensor([[[0.0, 3.0, 3.0], [5.0, float("nan"), 1.0]]], dtype=torch.bfloat16)
    assert oracle.target_choice(lg).tolist() == [[1, 0]]


# ---------------------------------------------------------------- acceptance

def _greedy_descent(parent, draft, nxt):
    """Walk down from the root, each time taking the child whose draft token is
    the target's choice at the current node; stop when none does. Valid when
    at most one child of any node agrees."""
    kids = {}
    for i in range(1, len(parent)):
        kids.setdefault(parent[i], []).append(i)
    path = [0]
    while True:
        u = path[-1]
        nxt_child = [c for c in kids.get(u, []) if draft[c] == nxt[u]]
        assert len(nxt_child) <= 1
        if not nxt_child:
            return path
        path.append(nxt_child[0])


def _agreeing_depths(parent, draft, nxt):
    """Breadth-first over agreeing children: {node: path length} for every node
    whose whole root path agrees."""
    kids = {}
    for i in range(1, len(parent)):
        kids.setdefault(parent[i], []).append(i)
    reach, frontier = {0: 1}, [0]
    while frontier:
        nf = []
        for u in frontier:
            for c in kids.get(u, []):
                if draft[c] == nxt[u]:
                    reach[c] = reach[u] + 1
                    nf.append(c)
        frontier = nf
    return reach


def test_exhaustive_small_trees_all_agreement_patterns():
    for n in range(1, 7):
        for choice in itertools.product(*[range(i) for i in range(1, n)]):
            parent = [-1] + list(choice)
            nxt = [100 + i for i in range(n)]                # distinct target choices
            for pattern in itertools.product([True, False], repeat=n - 1):
                agree = (True,) + pattern
                # agreeing children copy the parent's choice: siblings may collide
                draft = [-1] + [nxt[parent[u]] if agree[u] else 900 + u for u in range(1, n)]
                alen, nodes, bonus = oracle.accept_one(parent, draft, nxt)
                reach = _agreeing_depths(parent, draft, nxt)
                best = max(reach.values())
                end = min(v for v, d in reach.items() if d == best)
                assert alen == best - 1
                assert bonus == nxt[end]
                path = [x for x in nodes if x >= 0]
                assert path[-1] == end and len(path) == best
                assert all(parent[path[i]] == path[i - 1] for i in range(1, len(path)))
                assert nodes[len(path):] == [-1] * (n - len(path))


def test_distinct_sibling_tokens_equal_greedy_descent():
    rng = np.random.Generator(np.random.PCG64(3))
    for trial in range(200):
        n = int(rng.integers(2, 40))
        parent = [-1] + [int(rng.integers(0, i)) for i in range(1, n)]
        nxt = [int(x) for x in rng.integers(0, 5, size=n)]
        kids = {}
        for i in range(1, n):
            kids.setdefault(parent[i], []).append(i)
        draft = [-1] * n
        for u, cs in kids.items():
            toks = rng.permutation(8)[: len(cs)] if len(cs) <= 8 else None
            for c, t in zip(cs, toks if toks is not None else range(len(cs))):
                draft[c] = int(t)
        alen, nodes, bonus = oracle.accept_one(parent, draft, nxt)
        path = _greedy_descent(parent, draft, nxt)
        assert nodes[: len(path)] == path and alen == len(path) - 1 and bonus == nxt[path[-1]]


def test_closed_forms():
    # all agree on a random tree -> the deepest node, smallest index on ties
    rng = np.random.Generator(np.random.PCG64(4))
    parent = [-1] + [int(rng.integers(0, i)) for i in range(1, 30)]
    nxt = list(range(30))
    draft = [-1] + [nxt[parent[u]] for u in range(1, 30)]
    depth = [len(oracle.root_path(parent, v)) for v in range(30)]
    deepest = min(v for v in range(30) if depth[v] == max(depth))
    alen, nodes, bonus = oracle.accept_one(parent, draft, nxt)
    assert alen == max(depth) - 1 and bonus == nxt[deepest]
    # nothing agrees -> 0 accepted, bonus is the root's choice
    draft = [-1] + [nxt[parent[u]] + 1000 for u in range(1, 30)]
    assert oracle.accept_one(parent, draft, nxt) == (0, [0] + [-1] * 29, nxt[0])
    # chain with its first disagreement at node k -> k - 1 accepted
    for k in range(1, 10):
        parent = list(range(-1, 9))
        nxt = [7 * i for i in range(10)]
        draft = [-1] + [nxt[u - 1] if u < k else -5 for u in range(1, 10)]
        alen, nodes, bonus = oracle.accept_one(parent, draft, nxt)
        assert alen == k - 1 and nodes[:k] == list(range(k)) and bonus == nxt[k - 1]


def test_batched_accept_matches_per_sequence():
    parent = np.array([[-1, 0, 0, 1], [-1, 0, 1, 2]])
    draft = np.array([[-1, 5, 5, 6], [-1, 5, 9, 9]])
    nxt = np.array([[5, 6, 7, 8], [5, 9, 1, 2]])
    alen, nodes, bonus = oracle.tree_accept(parent, draft, nxt)
    assert alen.tolist() == [2, 2]
    assert nodes.tolist() == [[0, 1, 3, -1], [0, 1, 2, -1]]
    assert bonus.tolist() == [8, 1]
    with pytest.raises(ValueError):
        oracle.tree_accept(np.array([[0, 0]]), np.array([[0, 0]]), np.array([[0, 0]]))
