"""GPU parity of jf_build_tree (through the C ABI) against the oracle.

Bars: parent, token and tree_len bit-exact (both sides take every decision in
fp64: the logsumexp, each child's log-probability and the cumulative score);
scores within 1e-9 absolute (a row's logsumexp sums up to 151,936 terms in
another order: at most V * 2^-53 relative each, over at most 12 levels).
"""

import numpy as np
import pytest
import torch

import oracle
from tree_causal_attention_jf_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"
SCORE_TOL = 1e-9


@pytest.fixture(scope="module")
def jf():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from tree_causal_attention_jf_amd import binding
    return binding


def _run(jf, logits, topk, cap, budget=None):
    par, tok, sc, n = jf.build_tree(logits.to(DEV), topk, cap, None if budget is None else budget.to(DEV))
    torch.cuda.synchronize()
    return par.cpu().numpy(), tok.cpu().numpy(), sc.cpu().numpy(), n.cpu().numpy()


def _compare(jf, logits, topk, cap, budget=None, what=""):
    par, tok, sc, n = _run(jf, logits, topk, cap, budget)
    rp, rt, rs, rn = oracle.build_tree(logits, topk, cap, budget)
    assert np.array_equal(n, rn), (what, n, rn)
    for b in range(len(rn)):
        if not np.array_equal(par[b], rp[b]) or not np.array_equal(tok[b], rt[b]):
            bad = int(np.nonzero((par[b] != rp[b]) | (tok[b] != rt[b]))[0][0])
            raise AssertionError(f"{what}: sequence {b} first differs at node {bad}: gpu ({par[b, bad]}, "
                                 f"{tok[b, bad]}) oracle ({rp[b, bad]}, {rt[b, bad]})")
    fin = np.isfinite(rs)
    assert np.array_equal(np.isfinite(sc), fin) and (sc[~fin] == rs[~fin]).all(), what
    err = float(np.abs(sc[fin] - rs[fin]).max()) if fin.any() else 0.0
    print(f"  {what}: trees equal, tree_len {n.tolist()}, max|d score| {err:.2e}", flush=True)
    assert err <= SCORE_TOL, what
    return par, tok, sc, n


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("kind", ["normal", "ties", "uniform"])
@pytest.mark.parametrize("V", [70000, 70001])          # several chunks and a ragged tail; 70001: unaligned rows
def test_build_tree_matches_oracle(jf, dtype, kind, V):
    case = W.make_draft_logits_case(11, 3, 40, V, topk=4, max_path_nodes=6, budgets=[40, 17, 2], dtype=dtype,
                                    kind=kind)
    _compare(jf, case.logits, 4, 6, case.budget, what=f"{kind} {dtype} V {V}")


@pytest.mark.parametrize("topk", [1, 2, 3, 5, 8])
def test_build_tree_topk(jf, topk):
    case = W.make_draft_logits_case(13, 2, 64, 5000, topk=topk, max_path_nodes=10)
    _compare(jf, case.logits, topk, 10, None, what=f"topk {topk}")


def test_build_tree_budget256_full_vocabulary(jf):
    # batch 8, 256-node budgets (ragged), top-4, paths of at most 12 nodes, 151,936-way bf16 draft logits
    budgets = [256, 256, 200, 129, 64, 256, 3, 255]
    case = W.make_draft_logits_case(17, 8, 256, W.QWEN3_VOCAB, topk=4, max_path_nodes=12, budgets=budgets)
    par, _, _, n = _compare(jf, case.logits, 4, 12, case.budget, what="budget 256, V 151936")
    assert n.tolist() == budgets


def test_build_tree_chain_budget16(jf):
    case = W.make_draft_logits_case(19, 1, 16, W.QWEN3_VOCAB, topk=1, max_path_nodes=16)
    par, tok, _, n = _compare(jf, case.logits, 1, 16, None, what="top-1 chain of 16")
    assert par[0].tolist() == list(range(-1, 15))


def test_build_tree_edge_budgets_and_caps(jf):
    case = W.make_draft_logits_case(23, 5, 12, 3000, topk=3, max_path_nodes=4, budgets=[0, 1, 12, 2, 12])
    _compare(jf, case.logits, 3, 4, case.budget, what="budgets 0/1/2/full")
    _compare(jf, case.logits, 3, 1, case.budget, what="cap 1: roots only")
    _compare(jf, case.logits, 3, 2, case.budget, what="cap 2: stars")
    _compare(jf, case.logits, 3, 3, None, what="cap 3: 13 nodes possible, budget 12")
    # budgets outside [0, N]: tree_len -1, every node padding
    bad = torch.tensor([-1, 13, 5, 0, 12], dtype=torch.int32)
    par, tok, sc, n = _run(jf, case.logits, 3, 4, bad)
    assert n.tolist()[:2] == [-1, -1]
    for b in (0, 1):
        assert par[b].tolist() == [-1] + [0] * 11 and (tok[b] == -1).all() and np.isneginf(sc[b]).all()
    rp, rt, _, rn = oracle.build_tree(case.logits[2:], 3, 4, bad[2:])
    assert np.array_equal(par[2:], rp) and np.array_equal(tok[2:], rt) and np.array_equal(n[2:], rn)


def test_build_tree_nan_and_infinite_rows(jf):
    case = W.make_draft_logits_case(29, 2, 20, 4096, topk=4, max_path_nodes=8)
    z = case.logits.clone()
    top = int(z[0, 0].float().argmax())
    z[0, 0, 7] = float("nan")
    z[0, 0, top] = float("nan")                              # the largest logit becomes NaN
    z[0, 1] = float("-inf")                                  # offers nothing
    z[0, 2, 100] = float("inf")                              # offers nothing
    z[1, 0, :4000] = float("-inf")                           # only 96 finite tokens
    z[1, 3, 5] = float("-inf")
    _compare(jf, z, 4, 8, None, what="NaN / inf rows")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_build_tree_signalling_nan_patterns(jf, dtype):
    # NaNs with the quiet bit clear (the one input that makes a hardware max3 NaN),
    # of both signs, some beside the row's largest values: they count as -inf
    case = W.make_draft_logits_case(43, 2, 24, 40000, topk=4, max_path_nodes=8, dtype=dtype)
    z = case.logits.clone()
    if dtype == torch.bfloat16:
        bits, pos, neg = z.view(torch.int16), 0x7F81, -127                   # 0x7f81, 0xff81
    else:
        bits, pos, neg = z.view(torch.int32), 0x7F800001, -8388607           # 0x7f800001, 0xff800001
    rng = np.random.Generator(np.random.PCG64(43))
    for b in range(2):
        for r in range(0, 24, 3):
            top = int(z[b, r].float().argmax())
            bits[b, r, top] = pos                                            # the largest logit becomes NaN
            for c in rng.choice(40000, size=5, replace=False):
                bits[b, r, int(c)] = neg if c % 2 else pos
            bits[b, r, min(top + 1, 39999)] = neg
    _compare(jf, z, 4, 8, None, what=f"signalling NaN {dtype}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_build_tree_negative_and_mixed_sign_rows(jf, dtype):
    # every logit negative (log-probability-like rows: each thread's largest value is
    # negative and the chunk's threshold is below zero), and rows whose best values sit
    # around zero (-0.0 and +0.0 among them)
    case = W.make_draft_logits_case(47, 2, 24, 70000, topk=4, max_path_nodes=8, dtype=dtype)
    z = case.logits.clone()
    z[0] = z[0] - 40.0
    z[1] = z[1] - float(z[1].float().max()) + 0.5
    z[1, :, 5] = 0.0
    z[1, :, 6] = -0.0
    z[1, 3, 7] = 0.0
    _compare(jf, z, 4, 8, None, what=f"negative / mixed-sign rows {dtype}")


def test_build_tree_workspace_reused_across_shapes(jf):
    # the arrival counters clean themselves: calls of different shapes share one workspace
    big = W.make_draft_logits_case(31, 4, 64, 40000, topk=4, max_path_nodes=8)
    small = W.make_draft_logits_case(37, 1, 9, 300, topk=2, max_path_nodes=3)
    for _ in range(2):
        _compare(jf, big.logits, 4, 8, None, what="reuse: 4 x 64 x 40000")
        _compare(jf, small.logits, 2, 3, None, what="reuse: 1 x 9 x 300")


def test_build_tree_exact_ties_across_batches(jf):
    # one-hot rows (a single finite logit: that child's log-probability is exactly 0,
    # so it scores what its parent scores) and two-way rows (two equal finite maxima:
    # -ln 2 each) make candidates tie exactly with the children of nodes grown in the
    # same batch; the grown tree must still follow the serial tie rule (the parent that
    # joined first, then the child's rank). Sequence 2 is all one-hot: every score is 0.
    case = W.make_draft_logits_case(41, 3, 48, 500, topk=3, max_path_nodes=10)
    z = case.logits.clone()
    rng = np.random.Generator(np.random.PCG64(41))
    for b, rows in ((0, [0, 2, 5, 9, 11, 20]), (1, [1, 3, 4, 8]), (2, list(range(48)))):
        for r in rows:
            keep = rng.choice(500, size=1, replace=False)
            row = torch.full((500,), float("-inf"), dtype=z.dtype)
            row[keep] = z[b, r, keep]
            z[b, r] = row
    for b, r in ((0, 3), (0, 7), (1, 0), (1, 6)):
        keep = rng.choice(500, size=2, replace=False)
        row = torch.full((500,), float("-inf"), dtype=z.dtype)
        row[keep] = 1.5
        z[b, r] = row
    _compare(jf, z, 3, 10, None, what="exact ties across batches")
    _compare(jf, z, 3, 48, None, what="exact ties, no depth cap")
