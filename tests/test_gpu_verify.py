"""GPU parity of jf_tree_verify (attention and acceptance in one call, through
the C ABI): bit-identical to jf_tree_attention followed by jf_tree_accept on
the same inputs, in the fused one-launch form and in the two-launch fallback,
with the ancestor bitsets given or built from the parent array inside the
call (then bit-identical to jf_build_ancestor_mask's, broken trees included),
and checked against the fp64 oracle (attention to the bf16 bar of 1e-2 and
1e-2 * max|ref|, or 1e-5 for fp32; acceptance and bitsets bit-exact)."""

import numpy as np
import pytest
import torch

import oracle
from tree_causal_attention_jf_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def jf():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from tree_causal_attention_jf_amd import binding
    return binding


def _dev(wl):
    d = {k: getattr(wl, k).to(DEV) for k in ("q", "k_pages", "v_pages", "block_table", "prefix_len", "k_tree",
                                             "v_tree", "parent", "draft", "logits")}
    return d


def _separate(jf, wl, d, anc):
    out, lse = jf.tree_attention(d["q"], d["k_pages"], d["v_pages"], d["block_table"], d["prefix_len"], d["k_tree"],
                                 d["v_tree"], anc, sm_scale=wl.sm_scale, max_prefix_len=wl.max_prefix_len,
                                 return_lse=True)
    alen, nodes, bonus, nxt = jf.tree_accept(d["parent"], anc, d["draft"], logits=d["logits"])
    return out, lse, alen, nodes, bonus, nxt


def _verify(jf, wl, d, anc):
    # anc None: the call builds the bitsets from the parent array
    return jf.tree_verify(d["q"], d["k_pages"], d["v_pages"], d["block_table"], d["prefix_len"], d["k_tree"],
                          d["v_tree"], anc, d["parent"], d["draft"], d["logits"], sm_scale=wl.sm_scale,
                          max_prefix_len=wl.max_prefix_len, return_lse=True)


def _check(jf, wl, what, tol=1e-2):
    d = _dev(wl)
    anc, _, _ = jf.build_ancestor_mask(d["parent"])
    ref = _separate(jf, wl, d, anc)
    itype = torch.int16 if wl.dtype == torch.bfloat16 else torch.int32
    for given in (True, False):
        got = _verify(jf, wl, d, anc if given else None)
        torch.cuda.synchronize()
        how = f"{what} ({'bitsets given' if given else 'bitsets built in the call'})"
        assert torch.equal(got[0].view(itype), ref[0].view(itype)), how
        assert torch.equal(got[1].view(torch.int32), ref[1].view(torch.int32)), how
        for g, r in zip(got[2:6], ref[2:]):
            assert torch.equal(g, r), how
        assert torch.equal(got[6], anc), how
    # against the oracle
    o, l = oracle.tree_attention(wl.q, wl.k_pages, wl.v_pages, wl.block_table, wl.prefix_len, wl.k_tree, wl.v_tree,
                                 wl.parent, wl.sm_scale)
    err = float(np.abs(got[0].float().cpu().numpy() - o).max())
    assert err <= tol and (wl.dtype != torch.bfloat16 or err <= 1e-2 * np.abs(o).max()), (what, err)
    nxt = oracle.target_choice(wl.logits)
    ra, rn, rb = oracle.tree_accept(wl.parent.numpy(), wl.draft.numpy(), nxt)
    assert np.array_equal(got[5].cpu().numpy(), nxt), what
    assert np.array_equal(got[2].cpu().numpy(), ra) and np.array_equal(got[3].cpu().numpy(), rn), what
    assert np.array_equal(got[4].cpu().numpy(), rb), what
    print(f"  {what}: identical to the separate calls; attention max|err| {err:.2e}, accept_len "
          f"{got[2].cpu().tolist()}", flush=True)


LOGITS = ("logits", 20000, 3.0, 0.8)


@pytest.mark.parametrize("name,kw", [
    ("budget16_fused", dict()),                                                   # one launch, 4 key groups
    ("budget16_full_vocab", dict(accept=("logits", W.QWEN3_VOCAB, 3.0, 0.8))),
    ("streaming_fused", dict(B=4, prefix=("list", [2048, 1500, 2100, 700]), accept=LOGITS)),   # 64-row blocks
    ("ragged_random_tree", dict(B=3, N=24, prefix=("list", [150, 0, 37]), Hq=8, Hkv=2, tree=("random", 6),
                                accept=LOGITS)),
    ("d64_unaligned_vocab", dict(B=2, N=16, prefix=("list", [300, 90]), Hq=8, Hkv=2, D=64, tree=("random", 5),
                                 accept=("logits", 4099, 3.0, 0.8))),              # rows not 16-byte aligned
    ("fallback_256_rows", dict(B=2, N=64, prefix=("list", [700, 1300]), tree=("random", 8), accept=LOGITS)),
    ("one_node_trees", dict(B=3, N=1, prefix=("list", [0, 33, 512]), accept=LOGITS)),       # root only
    ("empty_prefixes", dict(B=2, N=20, prefix=("list", [0, 0]), Hq=8, Hkv=2, tree=("random", 7), accept=LOGITS)),
])
def test_verify_matches_separate_calls_and_oracle(jf, name, kw):
    wl = W.make_workload("c1_chain16", 9, **kw)
    _check(jf, wl, name)


def test_verify_four_wave_row_pairs(jf, monkeypatch):
    # 256-row blocks as four waves of two 32-row blocks: also one launch
    monkeypatch.setenv("JF_RPW", "2")
    wl = W.make_workload("c1_chain16", 10, B=2, N=64, prefix=("list", [400, 999]), tree=("random", 8), accept=LOGITS)
    _check(jf, wl, "rpw2_fused")


def test_verify_builds_bitsets_of_deep_and_broken_trees(jf, monkeypatch):
    # one launch with the bitsets built in the call: a 256-node chain (eight
    # doubling rounds) and star as four-wave 256-row blocks, and trees with broken
    # parent entries, which both the call and jf_build_ancestor_mask read as roots
    monkeypatch.setenv("JF_RPW", "2")
    for tree, B in ((W.tree_chain(256), 1), (np.array([-1] + [0] * 255, dtype=np.int32), 1)):
        wl = W.make_workload("c1_chain16", 13, B=B, N=256, prefix=("list", [300]), Hq=2, Hkv=2, accept=LOGITS)
        wl.parent = torch.from_numpy(np.stack([tree] * B))
        _check(jf, wl, f"256 nodes, depth {int(oracle.build_ancestor_mask(wl.parent.numpy())[1].max())}")
    monkeypatch.delenv("JF_RPW")
    wl = W.make_workload("c1_chain16", 14, B=4, N=24, prefix=("list", [150, 0, 37, 400]), Hq=8, Hkv=2,
                         tree=("random", 6), accept=LOGITS)
    par = wl.parent.numpy().copy()
    par[0, 0] = 3            # the root has a parent
    par[1, 5] = 7            # a parent after its child
    par[2, 9] = -4           # out of range
    par[3, 11] = 11          # its own parent
    d = _dev(wl)
    d["parent"] = torch.from_numpy(par).to(DEV)
    anc, _, bad = jf.build_ancestor_mask(d["parent"])
    assert bad.cpu().tolist() == [1, 1, 1, 1]
    ref = _separate(jf, wl, d, anc)
    got = _verify(jf, wl, d, None)
    torch.cuda.synchronize()
    assert torch.equal(got[6], anc)
    assert torch.equal(got[0].view(torch.int16), ref[0].view(torch.int16))
    for g, r in zip(got[2:6], ref[2:]):
        assert torch.equal(g, r)
    print("  broken trees: bitsets and results identical to the mask kernel's reading", flush=True)


def test_verify_fp32_fallback(jf):
    wl = W.make_workload("c0_tiny_fp32", 2, accept=("logits", 3000, 3.0, 0.7))
    _check(jf, wl, "fp32", tol=1e-5)


def test_verify_graph_replay(jf):
    wl = W.make_workload("c1_chain16", 12, accept=LOGITS)
    d = _dev(wl)
    anc, _, _ = jf.build_ancestor_mask(d["parent"])
    ref = [t.clone() for t in _verify(jf, wl, d, anc)[:6] if t is not None]
    torch.cuda.synchronize()
    bufs = dict(out=torch.empty_like(d["q"]), lse=torch.empty(d["q"].shape[:3], dtype=torch.float32, device=DEV),
                alen=torch.empty((wl.B,), dtype=torch.int32, device=DEV),
                nodes=torch.empty((wl.B, wl.N), dtype=torch.int32, device=DEV),
                bonus=torch.empty((wl.B,), dtype=torch.int32, device=DEV),
                nxt=torch.empty((wl.B, wl.N), dtype=torch.int32, device=DEV))

    anc_built = torch.empty_like(anc)

    def call():
        # bitsets built inside the call (written to anc_built)
        jf.tree_verify(d["q"], d["k_pages"], d["v_pages"], d["block_table"], d["prefix_len"], d["k_tree"],
                       d["v_tree"], None, d["parent"], d["draft"], d["logits"], sm_scale=wl.sm_scale,
                       max_prefix_len=wl.max_prefix_len, out=bufs["out"], lse=bufs["lse"], accept_len=bufs["alen"],
                       accepted_nodes=bufs["nodes"], bonus_token=bufs["bonus"], next_tokens=bufs["nxt"],
                       anc_out=anc_built)

    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
        call()
    for rep in range(4):
        for t in bufs.values():
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        got = [bufs[k] for k in ("out", "lse", "alen", "nodes", "bonus", "nxt")]
        assert torch.equal(got[0].view(torch.int16), ref[0].view(torch.int16)), rep
        for a, b in zip(got[1:], ref[1:]):
            assert torch.equal(a, b), rep
        assert torch.equal(anc_built, anc), rep
        anc_built.zero_()
        _verify(jf, wl, d, anc)                        # eager work between replays
        torch.cuda.synchronize()
