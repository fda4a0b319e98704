"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Bars
  * masks, depths, bad-tree flags, target choices, accepted paths, lengths and
    bonus tokens: bit-exact;
  * attention, fp32 inputs: max |out - ref| <= 1e-5 (and lse);
  * attention, bf16 inputs (fp32 accumulation): max |out - ref| <= 1e-2 and,
    because 1/sqrt(128)-scaled data gives |out| ~ 1e-2, also
    max |out - ref| <= 1e-2 * max |ref|, plus unscaled N(0,1) variants held to
    the absolute bar. The GPU rounds P to bf16 for the P.V product and rounds
    the output to bf16: each contributes at most 2^-8 relative, well inside
    1e-2. The row sums add the same bf16-rounded weights, so log-sum-exp is
    held to 2^-8 (+1e-4 for fp32 summation).
"""

import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from tree_causal_attention_jf_amd import workloads as W
from plan_items import assert_items_covered, item_rows

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def jf():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from tree_causal_attention_jf_amd import binding
    return binding


def say(*a):
    print(*a, flush=True)


def to_dev(wl):
    d = {}
    for k in ("q", "k_pages", "v_pages", "block_table", "prefix_len", "k_tree", "v_tree", "parent"):
        d[k] = getattr(wl, k).to(DEV)
    for k in ("draft", "target_ids", "logits"):
        v = getattr(wl, k)
        d[k] = None if v is None else v.to(DEV)
    return d


def anc_np(anc_dev):
    return anc_dev.view(torch.int64).cpu().numpy().view(np.uint64)


def run_attention(jf, wl, d, anc=None, **kw):
    if anc is None:
        anc, _, _ = jf.build_ancestor_mask(d["parent"])
    out, lse = jf.tree_attention(d["q"], d["k_pages"], d["v_pages"], d["block_table"], d["prefix_len"],
                                 d["k_tree"], d["v_tree"], anc, sm_scale=wl.sm_scale,
                                 max_prefix_len=wl.max_prefix_len, return_lse=True, **kw)
    torch.cuda.synchronize()
    return out, lse


def check_bf16(out, ref, lse=None, lse_ref=None, what="", abs_tol=1e-2):
    o = out.float().cpu().numpy().astype(np.float64)
    err = np.abs(o - ref)
    scale = np.abs(ref).max()
    say(f"  {what}: max|err| {err.max():.3e} (bar {abs_tol:.3e})  max|ref| {scale:.3e}  rel {err.max() / scale:.3e}")
    assert np.isfinite(o).all()
    assert err.max() <= abs_tol, what
    assert err.max() <= 1e-2 * scale, what
    if lse is not None:
        # the row sum adds the bf16-rounded weights (relative error <= 2^-8 each),
        # so log-sum-exp is off by at most 2^-8
        lerr = np.abs(lse.cpu().numpy().astype(np.float64) - lse_ref).max()
        say(f"  {what}: max|lse err| {lerr:.3e}")
        assert lerr <= 2.0 ** -8 + 1e-4, what


# ------------------------------------------------------------------ mask (bit-exact)

def test_mask_matches_oracle_on_configs(jf):
    for name in ("c0_tiny_fp32", "c1_chain16", "c2_bf256_b8", "c3_bf64_b32", "c4_bf256_32k"):
        for seed in (0, 1):
            B = W.CONFIGS[name]["B"]
            N = W.CONFIGS[name]["N"]
            parent = np.stack([W.make_tree(W.CONFIGS[name]["tree"], N, seed, b)[0] for b in range(B)])
            anc, depth, bad = jf.build_ancestor_mask(torch.from_numpy(parent).to(DEV))
            ra, rd, rb = oracle.build_ancestor_mask(parent)
            assert np.array_equal(anc_np(anc), ra), name
            assert np.array_equal(depth.cpu().numpy(), rd), name
            assert np.array_equal(bad.cpu().numpy(), rb), name
    say("  mask: configs c0-c4 x 2 seeds bit-exact")


def test_mask_exhaustive_small_trees_and_bad_trees(jf):
    for n in range(1, 7):
        parents = [[-1] + list(c) for c in itertools.product(*[range(i) for i in range(1, n)])]
        P = np.array(parents, dtype=np.int32)
        anc, depth, bad = jf.build_ancestor_mask(torch.from_numpy(P).to(DEV))
        ra, rd, rb = oracle.build_ancestor_mask(P)
        assert np.array_equal(anc_np(anc), ra) and np.array_equal(depth.cpu().numpy(), rd)
        assert not bad.cpu().numpy().any()
    badp = np.array([[-1, 0, 1, 2], [0, 0, 1, 2], [-1, 1, 1, 2], [-1, 0, 5, 2], [-1, 0, -1, 1]], dtype=np.int32)
    _, _, bad = jf.build_ancestor_mask(torch.from_numpy(badp).to(DEV))
    assert bad.cpu().numpy().tolist() == oracle.build_ancestor_mask(badp)[2].tolist() == [0, 1, 1, 1, 1]
    # full 256-node chain and star
    for P in (W.tree_chain(256)[None], np.array([[-1] + [0] * 255], dtype=np.int32)):
        anc, depth, _ = jf.build_ancestor_mask(torch.from_numpy(P).to(DEV))
        assert np.array_equal(anc_np(anc), oracle.build_ancestor_mask(P)[0])


# ------------------------------------------------------------------ acceptance (bit-exact)

def _accept_check(jf, parent, draft, next_ref, logits=None, target_ids=None):
    P = torch.from_numpy(np.asarray(parent, dtype=np.int32)).to(DEV)
    anc, _, _ = jf.build_ancestor_mask(P)
    alen, nodes, bonus, nxt = jf.tree_accept(P, anc, torch.from_numpy(np.asarray(draft, dtype=np.int32)).to(DEV),
                                             logits=logits, target_ids=target_ids)
    torch.cuda.synchronize()
    ra, rn, rb = oracle.tree_accept(parent, draft, next_ref)
    assert np.array_equal(nxt.cpu().numpy(), np.asarray(next_ref))
    assert np.array_equal(alen.cpu().numpy(), ra)
    assert np.array_equal(nodes.cpu().numpy(), rn)
    assert np.array_equal(bonus.cpu().numpy(), rb)
    return ra


def test_accept_ids_mode_c0_seeds(jf):
    for seed in range(5):
        wl = W.make_workload("c0_tiny_fp32", seed)
        _accept_check(jf, wl.parent.numpy(), wl.draft.numpy(), wl.target_ids.numpy(),
                      target_ids=wl.target_ids.to(DEV))
    say("  accept ids: c0 seeds 0-4 bit-exact")


def test_accept_exhaustive_small_trees(jf):
    for n in range(2, 7):
        parents, drafts, nexts = [], [], []
        for choice in itertools.product(*[range(i) for i in range(1, n)]):
            parent = [-1] + list(choice)
            nxt = [100 + i for i in range(n)]
            for pattern in itertools.product([True, False], repeat=n - 1):
                agree = (True,) + pattern
                parents.append(parent)
                nexts.append(nxt)
                drafts.append([-1] + [nxt[parent[u]] if agree[u] else 900 + u for u in range(1, n)])
        nx = np.array(nexts, dtype=np.int32)
        _accept_check(jf, np.array(parents), np.array(drafts), nx, target_ids=torch.from_numpy(nx).to(DEV))
    say("  accept: every tree with n <= 6 and every agreement pattern bit-exact")


def test_accept_logits_ties_nan_and_alignment(jf):
    rng = np.random.Generator(np.random.PCG64(5))
    # (2, 40, 151936): 200 workgroups per sequence, which arrive in groups
    for B, N, vocab, dtype in ((2, 24, 5000, torch.bfloat16), (2, 24, 4099, torch.bfloat16),
                               (2, 24, 151936, torch.bfloat16), (2, 40, 151936, torch.bfloat16),
                               (2, 24, 3001, torch.float32), (2, 24, 20000, torch.float32)):
        parent = np.stack([W.tree_random_recursive(N, 6, rng) for _ in range(B)])
        z = torch.from_numpy(rng.integers(-3, 4, size=(B, N, vocab)).astype(np.float32)).to(dtype)  # many ties
        z[0, 1] = float("nan")                              # all-NaN row -> 0
        z[0, 2, :7] = float("nan")
        z[0, 3] = -float("inf")
        z[0, 3, vocab - 1] = float("nan")
        z[1, 4] = 0.0
        z[1, 4, 0] = -0.0                                    # -0 == +0 -> index 0
        z[1, 5, vocab - 1] = 100.0                            # last element wins
        nxt = oracle.target_choice(z)
        draft = np.full((B, N), -1, dtype=np.int32)
        for b in range(B):
            for u in range(1, N):
                draft[b, u] = nxt[b, parent[b, u]] if rng.random() < 0.7 else 77777
        _accept_check(jf, parent, draft, nxt, logits=z.to(DEV))
    say("  accept logits: ties / NaN / -0 / unaligned rows bit-exact")


def test_accept_logits_c4(jf):
    wl = W.make_workload("c4_bf256_32k", 0, prefix=("fixed", 16))   # only the acceptance inputs matter here
    nxt = oracle.target_choice(wl.logits)
    assert np.array_equal(nxt, wl.planted_target.numpy())
    ra = _accept_check(jf, wl.parent.numpy(), wl.draft.numpy(), nxt, logits=wl.logits.to(DEV))
    say(f"  accept logits c4: bit-exact, accept_len {ra.tolist()}")


# ------------------------------------------------------------------ attention

def _oracle_full(wl, rows=None):
    return oracle.tree_attention(wl.q, wl.k_pages, wl.v_pages, wl.block_table, wl.prefix_len, wl.k_tree,
                                 wl.v_tree, wl.parent, wl.sm_scale, rows=rows)


def test_attention_fp32_c0(jf):
    for seed in range(5):
        wl = W.make_workload("c0_tiny_fp32", seed)
        out, lse = run_attention(jf, wl, to_dev(wl))
        ref, lref = _oracle_full(wl)
        err = np.abs(out.cpu().numpy() - ref).max()
        lerr = np.abs(lse.cpu().numpy() - lref).max()
        say(f"  c0 seed {seed}: max|err| {err:.3e}  lse {lerr:.3e}")
        assert err <= 1e-5 and lerr <= 1e-5


@pytest.mark.parametrize("D", [64, 128])
def test_attention_fp32_ragged(jf, D):
    wl = W.make_workload("c0_tiny_fp32", 3, B=3, N=70, prefix=("list", [0, 45, 130]), Hq=6, Hkv=2, D=D,
                         tree=("random", 9))
    out, lse = run_attention(jf, wl, to_dev(wl))
    ref, lref = _oracle_full(wl)
    assert np.abs(out.cpu().numpy() - ref).max() <= 1e-5
    assert np.abs(lse.cpu().numpy() - lref).max() <= 1e-5


SMALL_BF16 = [
    # (name, overrides)
    ("one tile", dict(B=1, N=8, prefix=("fixed", 64), Hq=4, Hkv=1, D=128, tree=("random", 4))),
    ("ragged tails", dict(B=3, N=40, prefix=("list", [1, 100, 333]), Hq=8, Hkv=2, D=128, tree=("random", 7))),
    ("no prefix", dict(B=2, N=19, prefix=("list", [0, 0]), Hq=8, Hkv=8, D=128, tree=("random", 5))),
    ("d64 gqa8", dict(B=2, N=33, prefix=("list", [77, 500]), Hq=16, Hkv=2, D=64, tree=("random", 6))),
    ("full tree", dict(B=1, N=256, prefix=("fixed", 300), Hq=4, Hkv=1, D=128, tree=("best_first", 4, 12, 2.0))),
    ("chain 130", dict(B=1, N=130, prefix=("fixed", 17), Hq=2, Hkv=1, D=128, tree=("chain",))),
]


def derived_bf16_bar(wl):
    """Error bound of the bf16 path from its two roundings: P is rounded to bf16
    (relative 2^-8 per weight, so at most 2^-8 * max|v| on the output) and the
    output is rounded to bf16 (at most 2^-8 * |out| <= 2^-8 * max|v|). The
    configurations' own bar, 1e-2, is kept as the floor."""
    vmax = max([float(v.float().abs().max()) for v in wl.v_prefix if v.numel()] +
               [float(wl.v_tree.float().abs().max())])
    return max(1e-2, 2.0 ** -7 * vmax)


@pytest.mark.parametrize("case", SMALL_BF16, ids=[c[0] for c in SMALL_BF16])
@pytest.mark.parametrize("unscaled", [False, True])
def test_attention_bf16_small(jf, case, unscaled):
    # short prefixes with unscaled data give |out| of order 1, where bf16
    # rounding alone exceeds 1e-2; these stress cases use the derived bar
    name, kw = case
    wl = W.make_workload("c1_chain16", 11, with_accept=False, unscaled=unscaled, **kw)
    out, lse = run_attention(jf, wl, to_dev(wl))
    ref, lref = _oracle_full(wl)
    check_bf16(out, ref, lse, lref, f"{name}{' unscaled' if unscaled else ''}", abs_tol=derived_bf16_bar(wl))


@pytest.mark.parametrize("balanced", [1, 0])
@pytest.mark.parametrize("rw,splits,rpw", [(1, 1, 1), (1, 7, 1), (2, 3, 1), (4, 5, 1), (8, 2, 1), (8, 64, 1),
                                            (4, 0, 1), (8, 1, 2), (8, 3, 2), (8, 64, 2)])
def test_attention_bf16_forced_plans(jf, rw, splits, rpw, balanced, monkeypatch):
    # every row-group layout (rpw 2: four waves of two 32-row blocks), with the
    # prefix cut into several splits merged by the last one to finish (including
    # more splits than some sequences have tiles); balanced 1: the kernel cuts
    # every sequence into that many pieces itself and deals them out longest
    # first, 0: uniform page ranges in id order
    monkeypatch.setenv("JF_RW", str(rw))
    monkeypatch.setenv("JF_SPLITS", str(splits))
    monkeypatch.setenv("JF_RPW", str(rpw))
    monkeypatch.setenv("JF_BALANCED", str(balanced))
    for D, Hq, Hkv in ((128, 8, 2), (64, 16, 2)):
        wl = W.make_workload("c1_chain16", 5, with_accept=False, B=4, N=150, prefix=("list", [700, 0, 1, 2100]),
                             Hq=Hq, Hkv=Hkv, D=D, tree=("random", 9))
        out, lse = run_attention(jf, wl, to_dev(wl))
        ref, lref = _oracle_full(wl)
        check_bf16(out, ref, lse, lref, f"rw {rw} splits {splits} rpw {rpw} balanced {balanced} D {D}",
                   abs_tol=derived_bf16_bar(wl))


@pytest.mark.parametrize("lens", [[3000, 100, 200, 50, 2500, 10], [4000, 0, 17, 4000, 1, 900, 64, 3999]],
                         ids=["skewed6", "skewed8"])
def test_attention_bf16_balanced_skewed(jf, lens):
    # skewed prefix lengths, default plan: the kernel cuts the long sequences into
    # pieces from the lengths it reads (the host sees only the longest) and leaves
    # the short ones whole; unused workgroup ids exit
    for D, Hq, Hkv, N in ((128, 8, 2, 64), (64, 16, 4, 40)):
        wl = W.make_workload("c1_chain16", 17, with_accept=False, B=len(lens), N=N, prefix=("list", lens),
                             Hq=Hq, Hkv=Hkv, D=D, tree=("random", 7))
        out, lse = run_attention(jf, wl, to_dev(wl))
        ref, lref = _oracle_full(wl)
        check_bf16(out, ref, lse, lref, f"lens {lens} D {D}", abs_tol=derived_bf16_bar(wl))


@pytest.mark.parametrize("ht", ["1.1", "0"])
@pytest.mark.parametrize("cus,lens,shape", [
    # four row blocks per (sequence, KV head): three sequences cut (heads of 49 tiles), five whole
    (64, [3904, 3840, 3584, 1344, 1024, 1664, 2304, 2944],
     dict(N=256, Hq=8, Hkv=2, D=128, tree=("best_first", 4, 12, 2.0))),
    # d = 64, one row block per (sequence, KV head): two sequences cut
    (72, [2000, 1500, 1900, 1000, 1300, 1100, 600, 1800], dict(N=80, Hq=16, Hkv=8, D=64, tree=("random", 7))),
], ids=["d128_cut3", "d64_cut2"])
def test_attention_bf16_head_and_tail(jf, cus, lens, shape, ht, monkeypatch):
    # A batch in 256-row blocks whose equal pieces fill the CUs in one round
    # (JF_TARGET_WG sets the CU count the plan divides the work by) takes the
    # head-and-tail rule in the kernel's balanced schedule: a long sequence keeps
    # a head of 1.1x the mean work per CU and hands the rest, with its tree tiles,
    # to a tail piece that starts on a CU a short sequence has freed. JF_BAL_HT=0
    # keeps equal pieces. Every piece layout must give the oracle's result.
    monkeypatch.setenv("JF_TARGET_WG", str(cus))
    monkeypatch.setenv("JF_BAL_HT", ht)
    wl = W.make_workload("c1_chain16", 23, with_accept=False, B=len(lens), prefix=("list", lens), **shape)
    assert jf.tree_attention_plan(jf.attn_shape(wl.q, wl.k_pages, wl.block_table, wl.sm_scale),
                                  wl.max_prefix_len)["balanced"] == 1
    out, lse = run_attention(jf, wl, to_dev(wl))
    ref, lref = _oracle_full(wl)
    check_bf16(out, ref, lse, lref, f"cus {cus} lens {lens} ht {ht}", abs_tol=derived_bf16_bar(wl))


def test_one_workspace_serves_every_shape(jf, monkeypatch):
    # one workspace, used in turn by attention calls whose partial layouts differ
    # and by logits-mode acceptance: each call must find the counter region zero
    # and leave it zero, whatever the previous call wrote past it
    ws = torch.zeros(256 << 20, dtype=torch.uint8, device=DEV)
    cases = [
        (7, dict(B=4, N=150, prefix=("list", [700, 0, 1, 2100]), Hq=8, Hkv=2, D=128, tree=("random", 9))),
        (0, dict(B=8, N=256, prefix=("list", [900, 1500, 64, 3000, 17, 1200, 800, 2500]), Hq=8, Hkv=2, D=128,
                 tree=("best_first", 4, 12, 2.0))),
        (3, dict(B=3, N=40, prefix=("list", [100, 333, 1]), Hq=16, Hkv=2, D=64, tree=("random", 7))),
    ]
    for rnd in range(2):
        for splits, kw in cases:
            if splits:
                monkeypatch.setenv("JF_SPLITS", str(splits))
            else:
                monkeypatch.delenv("JF_SPLITS", raising=False)
            wl = W.make_workload("c1_chain16", 7 + rnd, with_accept=False, **kw)
            out, lse = run_attention(jf, wl, to_dev(wl), workspace=ws)
            rows = _sampled_rows(wl, 40, rnd)
            ref, lref = _oracle_full(wl, rows=rows)
            idx = tuple(np.array(rows).T)
            check_bf16(torch.from_numpy(out.float().cpu().numpy()[idx]), ref[idx], lse.cpu()[idx], lref[idx],
                       f"shared workspace round {rnd} splits {splits}", abs_tol=derived_bf16_bar(wl))
            # acceptance over logits with the same workspace, between the attention calls
            acc = W.make_workload("c1_chain16", 30 + rnd, prefix=("fixed", 16), B=5, N=24,
                                  tree=("random", 6), accept=("logits", 5000, 3.0, 0.8))
            P = acc.parent.to(DEV)
            anc, _, _ = jf.build_ancestor_mask(P)
            alen, nodes, bonus, nxt = jf.tree_accept(P, anc, acc.draft.to(DEV), logits=acc.logits.to(DEV),
                                                     workspace=ws)
            torch.cuda.synchronize()
            nref = oracle.target_choice(acc.logits)
            ra, rn, rb = oracle.tree_accept(acc.parent.numpy(), acc.draft.numpy(), nref)
            assert np.array_equal(nxt.cpu().numpy(), nref)
            assert np.array_equal(alen.cpu().numpy(), ra) and np.array_equal(nodes.cpu().numpy(), rn)
            assert np.array_equal(bonus.cpu().numpy(), rb)
    assert not ws[:4096].any(), "counter region left non-zero"


def test_attention_bf16_c1_full(jf):
    for seed in (0, 1):
        for unscaled in (False, True):
            wl = W.make_workload("c1_chain16", seed, with_accept=False, unscaled=unscaled)
            out, lse = run_attention(jf, wl, to_dev(wl))
            ref, lref = _oracle_full(wl)
            check_bf16(out, ref, lse, lref, f"c1 seed {seed}{' unscaled' if unscaled else ''}")


def _sampled_rows(wl, count, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = {(int(rng.integers(wl.B)), int(rng.integers(wl.N)), int(rng.integers(wl.Hq))) for _ in range(count)}
    # always include the root and the last node of sequence 0, and the deepest chain node
    rows |= {(0, 0, 0), (0, wl.N - 1, wl.Hq - 1), (wl.B - 1, wl.N // 2, 1)}
    return sorted(rows)


@pytest.mark.parametrize("name", ["c2_bf256_b8", "c3_bf64_b32", "c4_bf256_32k", "draft_head_b1"])
def test_attention_bf16_large_sampled(jf, name):
    for unscaled in (False, True):
        wl = W.make_workload(name, 0, with_accept=False, unscaled=unscaled)
        d = to_dev(wl)
        out, lse = run_attention(jf, wl, d)
        rows, items, plan = item_rows(jf, wl, 1 + unscaled)
        assert_items_covered(wl, rows, items, plan)
        say(f"  {name}: plan {plan}, {len(items)} items, {len(rows)} rows compared")
        ref, lref = _oracle_full(wl, rows=rows)
        o = out.float().cpu().numpy()
        idx = tuple(np.array(rows).T)
        check_bf16(torch.from_numpy(o[idx]), ref[idx], lse.cpu()[idx], lref[idx],
                   f"{name}{' unscaled' if unscaled else ''} ({len(rows)} rows)")
        # properties that hold at any size: finite everywhere, lse >= the row's own score term
        assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("B,lens,full", [
    (4, [2048, 1500, 2100, 700], True),      # balanced batch: one 64-row block, two key groups
    (1, [32768], False),                     # one sequence, long splits plus the tree's own split
    (8, [16384] * 8, False),                 # the streaming budget-16 bench size, sampled rows
], ids=["b4_ragged", "b1_32k", "b8_16k"])
def test_attention_bf16_streaming_plan(jf, B, lens, full):
    # 16-node chains x 4 query heads per KV head (64 rows) over prefixes long
    # enough that streaming them sets the time: the plan switches to 64-row blocks
    wl = W.make_workload("c1_chain16", 6, with_accept=False, B=B, prefix=("list", lens))
    for unscaled in ((False, True) if full else (False,)):
        if unscaled:
            wl = W.make_workload("c1_chain16", 6, with_accept=False, B=B, prefix=("list", lens), unscaled=True)
        d = to_dev(wl)
        out, lse = run_attention(jf, wl, d)
        rows = None
        if not full:
            rows, items, plan = item_rows(jf, wl, 2)
            assert_items_covered(wl, rows, items, plan)
            say(f"  streaming B {B}: plan {plan}, {len(items)} items, {len(rows)} rows compared")
        ref, lref = _oracle_full(wl, rows=rows)
        if full:
            check_bf16(out, ref, lse, lref, f"streaming B {B}{' unscaled' if unscaled else ''}",
                       abs_tol=derived_bf16_bar(wl))
        else:
            o = out.float().cpu().numpy()
            idx = tuple(np.array(rows).T)
            check_bf16(torch.from_numpy(o[idx]), ref[idx], lse.cpu()[idx], lref[idx],
                       f"streaming B {B}{' unscaled' if unscaled else ''} ({len(rows)} rows)",
                       abs_tol=derived_bf16_bar(wl))
            assert torch.isfinite(out.float()).all()


def test_attention_bf16_batch_with_long_prefix(jf):
    # a batch whose longest prefix needs more than one split's page list (1024 pages):
    # the balanced plan must give that sequence at least ceil(pages / 1024) pieces
    # whatever the work estimate says, next to short and empty prefixes
    for lens in ([20000, 100, 5000], [16400, 0, 16384, 3]):
        wl = W.make_workload("c1_chain16", 23, with_accept=False, B=len(lens), N=24, prefix=("list", lens),
                             Hq=8, Hkv=2, D=128, tree=("random", 6))
        out, lse = run_attention(jf, wl, to_dev(wl))
        rows = _sampled_rows(wl, 40, 3) + [(0, wl.N - 1, 0), (2, 5, 7)]
        rows = sorted(set(rows))
        ref, lref = _oracle_full(wl, rows=rows)
        idx = tuple(np.array(rows).T)
        check_bf16(torch.from_numpy(out.float().cpu().numpy()[idx]), ref[idx], lse.cpu()[idx], lref[idx],
                   f"lens {lens} ({len(rows)} rows)", abs_tol=derived_bf16_bar(wl))
        assert torch.isfinite(out.float()).all()


def test_attention_bf16_poison_unused_slots(jf):
    kw = dict(B=2, N=50, prefix=("list", [37, 201]), Hq=8, Hkv=2, D=128, tree=("random", 6), extra_pages=5)
    clean = W.make_workload("c1_chain16", 21, with_accept=False, **kw)
    dirty = W.make_workload("c1_chain16", 21, with_accept=False, poison=True, **kw)
    assert torch.isnan(dirty.k_pages.float()).any()
    o1, l1 = run_attention(jf, clean, to_dev(clean))
    o2, l2 = run_attention(jf, dirty, to_dev(dirty))
    assert torch.isfinite(o2.float()).all()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_attention_deterministic(jf):
    wl = W.make_workload("c2_bf256_b8", 2, with_accept=False, B=2)
    d = to_dev(wl)
    o1, l1 = run_attention(jf, wl, d)
    o2, l2 = run_attention(jf, wl, d)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


@pytest.mark.parametrize("rw", [8, 4])
def test_attention_deterministic_many_splits(jf, rw, monkeypatch):
    # eight splits per item, merged by whichever split arrives last: the merged
    # output must not depend on that order (the last arriver merges its own
    # partial as stored, in split order), with and without key groups
    monkeypatch.setenv("JF_RW", str(rw))
    monkeypatch.setenv("JF_SPLITS", "8")
    monkeypatch.setenv("JF_BALANCED", "0")
    wl = W.make_workload("c2_bf256_b8", 4, with_accept=False, B=2)
    d = to_dev(wl)
    o1, l1 = run_attention(jf, wl, d)
    for _ in range(4):
        o2, l2 = run_attention(jf, wl, d)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_attention_mask_leak_exact(jf):
    # randomising K/V of nodes outside a row's path leaves that row bit-identical
    wl = W.make_workload("c1_chain16", 5, with_accept=False, B=1, N=64, prefix=("fixed", 90), Hq=4, Hkv=1,
                         tree=("random", 6))
    d = to_dev(wl)
    o1, _ = run_attention(jf, wl, d)
    parent = wl.parent[0].tolist()
    A = oracle.ancestor_matrix(parent)
    v = 63
    hidden = torch.tensor([j for j in range(wl.N) if not A[v, j]])
    d2 = dict(d)
    d2["k_tree"] = d["k_tree"].clone()
    d2["v_tree"] = d["v_tree"].clone()
    d2["k_tree"][0, hidden.to(DEV)] = torch.randn_like(d2["k_tree"][0, hidden.to(DEV)])
    d2["v_tree"][0, hidden.to(DEV)] = torch.randn_like(d2["v_tree"][0, hidden.to(DEV)])
    o2, _ = run_attention(jf, wl, d2)
    assert torch.equal(o1[0, v].view(torch.int16), o2[0, v].view(torch.int16))


def test_attention_bad_inputs_give_nan_rows(jf):
    wl = W.make_workload("c1_chain16", 6, with_accept=False, B=3, N=16, prefix=("list", [40, 70, 100]), Hq=4,
                         Hkv=1, tree=("random", 5))
    d = to_dev(wl)
    d["prefix_len"] = d["prefix_len"].clone()
    d["prefix_len"][1] = 10_000                          # beyond max_prefix_len
    d["block_table"] = d["block_table"].clone()
    d["block_table"][2, 3] = 999_999                     # page id outside the pool
    out, lse = run_attention(jf, wl, d)
    o = out.float()
    assert torch.isfinite(o[0]).all()
    assert torch.isnan(o[1]).all() and torch.isnan(lse[1]).all()
    assert torch.isnan(o[2]).all() and torch.isnan(lse[2]).all()


@pytest.mark.parametrize("L", [1000, 2048, 7])
def test_attention_one_sequence_table_wider_than_prefix(jf, L):
    # one sequence in the few-row plan (each wave requests its first tile as soon as
    # its page ids land): the host's longest prefix (2048) is above the sequence's own,
    # and the block table is wider than the prefix, its entries past the prefix's
    # pages invalid; those entries are never used, and the ragged last tile reads only
    # its valid keys
    wl = W.make_workload("c1_chain16", 21, with_accept=False, B=1, N=16, prefix=("list", [L]), Hq=32, Hkv=8,
                         tree=("chain",))
    d = to_dev(wl)
    pages = d["block_table"].shape[1]
    wide = torch.full((1, 128), -1, dtype=torch.int32, device=DEV)
    wide[:, :pages] = d["block_table"]
    anc, _, _ = jf.build_ancestor_mask(d["parent"])
    out, lse = jf.tree_attention(d["q"], d["k_pages"], d["v_pages"], wide, d["prefix_len"], d["k_tree"],
                                 d["v_tree"], anc, sm_scale=wl.sm_scale, max_prefix_len=2048, return_lse=True)
    torch.cuda.synchronize()
    ref, lref = _oracle_full(wl)
    check_bf16(out, ref, lse, lref, f"one sequence, prefix {L}, table of 128 pages")


def test_attention_one_sequence_bad_page_in_first_round(jf):
    # an invalid page id inside a split's first round, in the few-row plan: the
    # sequence's rows are NaN (the tile is requested from a clamped id before the page
    # checks run, and the checks still flag it)
    wl = W.make_workload("c1_chain16", 22, with_accept=False, B=1, N=16, prefix=("list", [2048]), Hq=32, Hkv=8,
                         tree=("chain",))
    d = to_dev(wl)
    for bad in (-3, 1 << 30):
        d2 = dict(d)
        d2["block_table"] = d["block_table"].clone()
        d2["block_table"][0, 21] = bad                   # split 1 (pages 16..31), its second tile
        out, lse = run_attention(jf, wl, d2)
        assert torch.isnan(out.float()).all() and torch.isnan(lse).all(), bad
    out, lse = run_attention(jf, wl, d)
    ref, lref = _oracle_full(wl)
    check_bf16(out, ref, lse, lref, "one sequence, valid table")


def test_graph_replay_matches_eager(jf):
    wl = W.make_workload("c1_chain16", 3, with_accept=True)
    d = to_dev(wl)
    s = torch.cuda.Stream()

    def make_bufs():
        return dict(anc=torch.empty((wl.B, wl.N, 4), dtype=torch.uint64, device=DEV),
                    out=torch.empty_like(d["q"]),
                    acc=[torch.empty((wl.B,), dtype=torch.int32, device=DEV),
                         torch.empty((wl.B, wl.N), dtype=torch.int32, device=DEV),
                         torch.empty((wl.B,), dtype=torch.int32, device=DEV),
                         torch.empty((wl.B, wl.N), dtype=torch.int32, device=DEV)])

    def step(o):
        jf.build_ancestor_mask(d["parent"], anc=o["anc"], with_depth=False)
        jf.tree_attention(d["q"], d["k_pages"], d["v_pages"], d["block_table"], d["prefix_len"], d["k_tree"],
                          d["v_tree"], o["anc"], sm_scale=wl.sm_scale, max_prefix_len=wl.max_prefix_len,
                          out=o["out"])
        a = o["acc"]
        jf.tree_accept(d["parent"], o["anc"], d["draft"], logits=d["logits"], accept_len=a[0],
                       accepted_nodes=a[1], bonus_token=a[2], next_tokens=a[3])

    eager, graphed = make_bufs(), make_bufs()
    step(eager)
    torch.cuda.synchronize()
    ref_out = eager["out"].clone()
    ref_acc = [t.clone() for t in eager["acc"]]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(graphed)
    for rep in range(4):
        graphed["out"].zero_()
        for t in graphed["acc"]:
            t.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(graphed["out"].view(torch.int16), ref_out.view(torch.int16)), rep
        for a, b in zip(graphed["acc"], ref_acc):
            assert torch.equal(a, b), rep
        step(eager)                                       # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(eager["out"].view(torch.int16), ref_out.view(torch.int16)), rep


def test_forked_step_graph_matches_serial(jf):
    """Acceptance forked onto a second stream after the mask, beside attention,
    captured in one graph with several steps: every replay equals the serial
    eager step bit for bit."""
    wl = W.make_workload("c1_chain16", 4, with_accept=True)
    d = to_dev(wl)
    s, side = torch.cuda.Stream(), torch.cuda.Stream()

    def make_bufs():
        return dict(anc=torch.empty((wl.B, wl.N, 4), dtype=torch.uint64, device=DEV),
                    out=torch.empty_like(d["q"]),
                    acc=[torch.empty((wl.B,), dtype=torch.int32, device=DEV),
                         torch.empty((wl.B, wl.N), dtype=torch.int32, device=DEV),
                         torch.empty((wl.B,), dtype=torch.int32, device=DEV),
                         torch.empty((wl.B, wl.N), dtype=torch.int32, device=DEV)])

    def accept(o):
        a = o["acc"]
        jf.tree_accept(d["parent"], o["anc"], d["draft"], logits=d["logits"], accept_len=a[0],
                       accepted_nodes=a[1], bonus_token=a[2], next_tokens=a[3])

    def attn(o):
        jf.tree_attention(d["q"], d["k_pages"], d["v_pages"], d["block_table"], d["prefix_len"], d["k_tree"],
                          d["v_tree"], o["anc"], sm_scale=wl.sm_scale, max_prefix_len=wl.max_prefix_len,
                          out=o["out"])

    def forked(o):
        cur = torch.cuda.current_stream()
        jf.build_ancestor_mask(d["parent"], anc=o["anc"], with_depth=False)
        fork = torch.cuda.Event()
        fork.record(cur)
        side.wait_event(fork)
        with torch.cuda.stream(side):
            accept(o)
        attn(o)
        join = torch.cuda.Event()
        join.record(side)
        cur.wait_event(join)

    ref = make_bufs()
    jf.build_ancestor_mask(d["parent"], anc=ref["anc"], with_depth=False)
    attn(ref)
    accept(ref)
    torch.cuda.synchronize()
    bufs = [make_bufs() for _ in range(3)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for o in bufs:
            forked(o)
    for rep in range(4):
        for o in bufs:
            o["out"].zero_()
            for t in o["acc"]:
                t.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for o in bufs:
            assert torch.equal(o["out"].view(torch.int16), ref["out"].view(torch.int16)), rep
            for a, b in zip(o["acc"], ref["acc"]):
                assert torch.equal(a, b), rep
        accept(ref)                                        # eager work between replays
        torch.cuda.synchronize()
