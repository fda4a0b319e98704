"""GPU parity over seeded random configurations of the bf16 attention: batch,
tree size and shape, GQA group, head size, prefix lengths (empty, mid-page and
page-edge ones included), separate or cached tree K/V with ragged budgets, and
the schedule's knobs (the CU count the plan divides the work by, head-and-tail
pieces on or off). Each case compares a sample of (sequence, node) pairs, with
every query head of each, against the fp64 oracle at the bf16 bar, and checks
that every output row of the tree is finite (padding rows untouched).

The configurations come from numpy's PCG64 with fixed seeds, so a failing case
is named by its index and reproduces on the CPU side exactly."""
import numpy as np
import pytest
import torch

import oracle
from tree_causal_attention_jf_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"
SENTINEL = 7.0            # exact in bf16 and fp32
N_CASES = 24


@pytest.fixture(scope="module")
def jf():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from tree_causal_attention_jf_amd import binding
    return binding


def config(i):
    rng = np.random.Generator(np.random.PCG64(7000 + i))
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 8]))
    N = int(rng.choice([1, 5, 16, 40, 64, 100, 200, 256]))
    B = int(rng.integers(1, 13))
    lens = rng.integers(0, 3000, size=B)
    for b in range(B):                      # some empty, some on a page edge or a tile edge
        u = rng.random()
        if u < 0.12:
            lens[b] = 0
        elif u < 0.25:
            lens[b] = 16 * int(rng.integers(1, 150))
        elif u < 0.35:
            lens[b] = 64 * int(rng.integers(1, 40))
    kind = rng.choice(["random", "best_first", "chain"])
    tree = {"random": ("random", int(rng.integers(2, 9))), "best_first": ("best_first", 4, 12, 2.0),
            "chain": ("chain",)}[kind]
    paged = bool(rng.random() < 0.4)
    budgets = [int(x) for x in rng.integers(0, N + 1, size=B)] if paged else None
    env = {"JF_TARGET_WG": str(int(rng.choice([256, 256, 64, 24]))), "JF_BAL_HT": str(rng.choice(["1.1", "0"]))}
    return dict(D=D, Hkv=Hkv, Hq=Hkv * G, N=N, B=B, lens=[int(x) for x in lens], tree=tree, paged=paged,
                budgets=budgets, env=env, seed=8000 + i)


def sample_rows(rng, B, N, Hq, nodes_of):
    rows = []
    for b in range(B):
        n = nodes_of(b)
        if n == 0:
            continue
        pick = {0, n - 1} | set(int(x) for x in rng.integers(0, n, size=min(n, 4)))
        rows += [(b, v, h) for v in sorted(pick) for h in range(Hq)]
    return rows


def compare(out, lse, ref, lref, rows, vmax, what):
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    idx = tuple(np.array(rows).T)
    err = float(np.abs(o[idx] - ref[idx]).max())
    lerr = float(np.abs(l[idx] - lref[idx]).max())
    scale = max(float(np.abs(ref[idx]).max()), 1e-30)
    bar = max(1e-2, 2.0 ** -7 * vmax)
    print(f"  {what}: {len(rows)} rows, max|err| {err:.3e} (bar {bar:.3e}), rel {err / scale:.3e}, "
          f"lse {lerr:.3e}", flush=True)
    assert err <= bar and err <= 1e-2 * scale, what
    assert lerr <= 2.0 ** -8 + 1e-4, what


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_configuration(jf, i, monkeypatch):
    c = config(i)
    for k, v in c["env"].items():
        monkeypatch.setenv(k, v)
    what = (f"case {i}: B {c['B']} N {c['N']} Hq {c['Hq']} Hkv {c['Hkv']} D {c['D']} tree {c['tree']} "
            f"paged {c['paged']} env {c['env']}")
    print(what, f"lens {c['lens']} budgets {c['budgets']}", flush=True)
    rng = np.random.Generator(np.random.PCG64(c["seed"]))
    if c["paged"]:
        case = W.make_paged_tree_case(c["seed"], c["lens"], c["budgets"], N=c["N"], Hq=c["Hq"], Hkv=c["Hkv"],
                                      D=c["D"], tree=c["tree"])
        t = {k: getattr(case, k).to(DEV) for k in ("q", "k_pages", "v_pages", "block_table", "prefix_len",
                                                    "tree_len", "parent")}
        anc, _, bad = jf.build_ancestor_mask(t["parent"])
        out = torch.full_like(t["q"], SENTINEL)
        lse = torch.full(case.q.shape[:3], SENTINEL, dtype=torch.float32, device=DEV)
        jf.tree_attention_paged_tree(t["q"], t["k_pages"], t["v_pages"], t["block_table"], t["prefix_len"], anc,
                                     tree_len=t["tree_len"], sm_scale=case.sm_scale,
                                     max_prefix_len=case.max_prefix_len, out=out, lse=lse)
        torch.cuda.synchronize()
        assert not bad.any()
        rows = sample_rows(rng, c["B"], c["N"], c["Hq"], lambda b: c["budgets"][b])
        o = out.float().cpu().numpy()
        l = lse.cpu().numpy()
        for b, n in enumerate(c["budgets"]):
            assert np.isfinite(o[b, :n]).all(), (what, b)
            assert (o[b, n:] == SENTINEL).all() and (l[b, n:] == SENTINEL).all(), (what, b)
        if not rows:
            return
        ref, lref = oracle.tree_attention_paged_tree(case.q, case.k_pages, case.v_pages, case.block_table,
                                                     case.prefix_len, case.tree_len, case.parent, case.sm_scale,
                                                     rows=rows)
        vmax = float(case.v_pages.float().abs().max())
    else:
        wl = W.make_workload("c1_chain16", c["seed"], with_accept=False, B=c["B"], N=c["N"],
                             prefix=("list", c["lens"]), Hq=c["Hq"], Hkv=c["Hkv"], D=c["D"], tree=c["tree"])
        d = {k: getattr(wl, k).to(DEV) for k in ("q", "k_pages", "v_pages", "block_table", "prefix_len", "k_tree",
                                                  "v_tree", "parent")}
        anc, _, _ = jf.build_ancestor_mask(d["parent"])
        out, lse = jf.tree_attention(d["q"], d["k_pages"], d["v_pages"], d["block_table"], d["prefix_len"],
                                     d["k_tree"], d["v_tree"], anc, sm_scale=wl.sm_scale,
                                     max_prefix_len=wl.max_prefix_len, return_lse=True)
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all(), what
        rows = sample_rows(rng, c["B"], c["N"], c["Hq"], lambda b: c["N"])
        ref, lref = oracle.tree_attention(wl.q, wl.k_pages, wl.v_pages, wl.block_table, wl.prefix_len, wl.k_tree,
                                          wl.v_tree, wl.parent, wl.sm_scale, rows=rows)
        vmax = max([float(v.float().abs().max()) for v in wl.v_prefix if v.numel()] +
                   [float(wl.v_tree.float().abs().max())])
    compare(out, lse, ref, lref, rows, vmax, what)
