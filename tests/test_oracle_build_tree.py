"""Pins of the oracle's best-first tree construction.

The pins do not re-run the oracle's heap: they check a hand-worked example,
closed forms (uniform rows give the complete k-ary tree in breadth-first
order; top-1 gives the greedy chain), the depth cap, and, on random rows, the
properties that define best-first growth, each computed independently with
scipy's log-softmax and a stable argsort.
"""

import math

import numpy as np
import pytest
import torch
from scipy.special import log_softmax

import oracle
from tree_causal_attention_jf_amd import workloads as W


def test_hand_worked_example():
    # probabilities chosen so that the tree can be followed by hand:
    #   root offers token 0 (p .5) and token 1 (p .3);
    #   node 1 (token 0) offers token 0 with p .9: .5 * .9 = .45 beats .3;
    #   node 2 offers token 0 with p .6: .45 * .6 = .27 loses to .3;
    #   so node 3 is the root's second child
    p = np.array([[[.5, .3, .2], [.9, .05, .05], [.6, .3, .1], [1 / 3, 1 / 3, 1 / 3]]])
    parent, token, score, n = oracle.build_tree(np.log(p), topk=2, max_path_nodes=10)
    assert parent.tolist() == [[-1, 0, 1, 0]]
    assert token.tolist() == [[-1, 0, 0, 1]]
    np.testing.assert_allclose(score[0], np.log([1.0, .5, .45, .3]), rtol=0, atol=1e-15)
    assert n.tolist() == [4]


@pytest.mark.parametrize("k,V,N", [(3, 50, 40), (4, 7, 22), (1, 5, 6)])
def test_uniform_rows_give_the_complete_tree_in_breadth_first_order(k, V, N):
    # every token has probability 1/V: all candidates of one depth tie, so the
    # parent's join order and then the token id decide
    case = W.make_draft_logits_case(0, 2, N, V, topk=k, max_path_nodes=64, kind="uniform")
    parent, token, score, n = oracle.build_tree(case.logits, k, 64)
    for i in range(1, N):
        assert parent[0, i] == (i - 1) // k and token[0, i] == (i - 1) % k
        d = 0
        j = i
        while j > 0:
            j, d = (j - 1) // k, d + 1
        assert abs(score[0, i] + d * math.log(V)) < 1e-12
    assert (parent[1] == parent[0]).all() and n.tolist() == [N, N]


def test_top1_gives_the_greedy_chain():
    case = W.make_draft_logits_case(3, 2, 12, 300, topk=1, max_path_nodes=64)
    parent, token, score, _ = oracle.build_tree(case.logits, 1, 64)
    z = case.logits.double().numpy()
    for b in range(2):
        assert parent[b].tolist() == list(range(-1, 11))
        s = 0.0
        for i in range(1, 12):
            row = z[b, i - 1]
            assert token[b, i] == int(np.argmax(row))          # first index of the maximum
            s += float(log_softmax(row)[token[b, i]])
            assert abs(score[b, i] - s) < 1e-12


def test_depth_cap():
    case = W.make_draft_logits_case(5, 1, 20, 100, topk=3)
    parent, token, _, n = oracle.build_tree(case.logits, 3, 2)      # root and its children only
    assert n.tolist() == [4] and parent[0, 1:4].tolist() == [0, 0, 0]
    assert (parent[0, 4:] == 0).all() and (token[0, 4:] == -1).all()
    _, _, _, n1 = oracle.build_tree(case.logits, 3, 1)               # the root alone
    assert n1.tolist() == [1]


def test_budgets_zero_and_one():
    case = W.make_draft_logits_case(6, 3, 9, 40, topk=2, budgets=[0, 1, 9])
    parent, token, score, n = oracle.build_tree(case.logits, 2, 8, case.budget)
    assert n.tolist() == [0, 1, 9]
    assert parent[0].tolist() == [-1] + [0] * 8 and (token[0] == -1).all() and np.isneginf(score[0]).all()
    assert parent[1].tolist() == [-1] + [0] * 8 and score[1, 0] == 0 and np.isneginf(score[1, 1:]).all()


def test_nan_and_infinite_logits():
    V = 6
    z = np.zeros((1, 4, V))
    z[0, 0] = [1.0, np.nan, 3.0, -np.inf, 2.0, np.nan]     # NaN counts as -inf, -inf is never offered
    z[0, 1] = -np.inf                                        # offers nothing
    z[0, 2] = [0, 0, np.inf, 0, 0, 0]                        # +inf: offers nothing
    parent, token, score, n = oracle.build_tree(z, 5, 8)
    # only the root's three finite tokens can join, best logit first
    assert n.tolist() == [4] and token[0].tolist() == [-1, 2, 4, 0]
    lse = math.log(math.exp(1) + math.exp(3) + math.exp(2))
    np.testing.assert_allclose(score[0, 1:], [3 - lse, 2 - lse, 1 - lse], rtol=0, atol=1e-15)


def _check_best_first(z, k, cap, nb, parent, token, score, n):
    """The defining properties of best-first growth, from scipy's log-softmax."""
    N = z.shape[0]
    zz = np.where(np.isnan(z), -np.inf, z)
    lists = []
    for i in range(N):
        row = zz[i]
        if not np.isfinite(row.max()):
            lists.append(([], None))
            continue
        order = [int(t) for t in np.argsort(-row, kind="stable") if row[t] > -np.inf][:k]
        lists.append((order, log_softmax(row)))
    depth = [1]
    rank = [-1]
    key = [(0.0, -1, -1)]
    for i in range(1, n):
        p, t = int(parent[i]), int(token[i])
        assert 0 <= p < i and depth[p] < cap
        toks, lsm = lists[p]
        assert t in toks
        assert abs(score[i] - (score[p] + lsm[t])) < 1e-12
        depth.append(depth[p] + 1)
        rank.append(toks.index(t))
        key.append((-score[i], p, rank[i]))
    # join order is the candidate order: score, then parent's join order, then
    # rank. Scores within 1e-12 that are not bit-equal are equal up to rounding
    # (sums taken in another order), and either order is then correct.
    def before(a, b, exact_tie):
        if abs(a[0] - b[0]) > 1e-12:
            return a[0] < b[0]
        return a[1:] < b[1:] if exact_tie else True

    for i in range(2, n):
        assert before(key[i - 1], key[i], score[i - 1] == score[i]), i
    # nothing better was left behind; if growth stopped short, nothing was left at all
    taken = {(int(parent[i]), int(token[i])) for i in range(1, n)}
    for v in range(n):
        if depth[v] >= cap:
            continue
        toks, lsm = lists[v]
        for r, t in enumerate(toks):
            if (v, t) in taken:
                continue
            assert n == nb, "growth stopped while candidates remained"
            cand = (-(score[v] + lsm[t]), v, r)
            assert before(key[n - 1], cand, v == parent[n - 1]), (v, t)
    # padding (node 0 keeps parent -1 even when the budget is 0)
    assert parent[0] == -1 and token[0] == -1
    assert (parent[max(n, 1):] == 0).all() and (token[n:] == -1).all() and np.isneginf(score[n:]).all()


@pytest.mark.parametrize("kind", ["normal", "ties", "small_ints", "uniform"])
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_random_rows_satisfy_the_best_first_properties(kind, seed):
    budgets = [30, 17, 1, 0, 25]
    k, cap = 3, 5
    case = W.make_draft_logits_case(seed, 5, 30, 64, topk=k, max_path_nodes=cap, budgets=budgets, kind=kind)
    parent, token, score, n = oracle.build_tree(case.logits, k, cap, case.budget)
    z = case.logits.double().numpy()
    for b in range(5):
        assert n[b] <= budgets[b] and (budgets[b] == 0 or n[b] >= 1)
        _check_best_first(z[b], k, cap, budgets[b], parent[b], token[b], score[b], int(n[b]))


def test_running_out_of_candidates_stops_early():
    # top-2 with paths of at most 3 nodes holds at most 1 + 2 + 4 = 7 nodes
    case = W.make_draft_logits_case(7, 1, 12, 30, topk=2, max_path_nodes=3)
    parent, token, score, n = oracle.build_tree(case.logits, 2, 3)
    assert n.tolist() == [7]
    _check_best_first(case.logits.double().numpy()[0], 2, 3, 12, parent[0], token[0], score[0], 7)


def test_property_check_catches_a_planted_mistake():
    # the checker itself must reject a wrong score (as a dropped or misplaced
    # normaliser would give): plant one in a copy of the oracle's scores
    case = W.make_draft_logits_case(8, 1, 20, 64, topk=3, max_path_nodes=6)
    parent, token, score, n = oracle.build_tree(case.logits, 3, 6)
    bad = score.copy()
    bad[0, 5] += 0.25
    with pytest.raises(AssertionError):
        _check_best_first(case.logits.double().numpy()[0], 3, 6, 20, parent[0], token[0], bad[0], int(n[0]))
