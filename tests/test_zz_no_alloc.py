"""jf_tree_verify_noalloc (the verification call that takes its scratch from the
library's fixed device array) against jf_tree_verify with caller workspaces, on
two calls in a row, the second with a smaller input. Same kernels and plans on
both sides, so every output is compared bit for bit."""

import pytest
import torch

from tree_causal_attention_jf_amd import binding as jf
from tree_causal_attention_jf_amd import workloads as W

pytestmark = pytest.mark.gpu

CASES = [
    # budget 16 (one launch, split prefixes: the attention workspace is used), bitsets built in the call
    ("c1_chain16", dict(), True),
    # smaller: 2 sequences, 24-node random trees, 8q/2kv, ragged short prefixes, bitsets given
    ("c1_chain16", dict(B=2, N=24, prefix=("list", [300, 77]), Hq=8, Hkv=2, tree=("random", 6),
                        accept=("logits", 5000, 3.0, 0.8)), False),
]


def _run(fn, wl, t, from_parent):
    dev = "cuda"
    B, N = wl.B, wl.N
    out = torch.full_like(t["q"], float("nan"))
    nxt = torch.full((B, N), -7, dtype=torch.int32, device=dev)
    alen = torch.full((B,), -7, dtype=torch.int32, device=dev)
    nodes = torch.full((B, N), -7, dtype=torch.int32, device=dev)
    bonus = torch.full((B,), -7, dtype=torch.int32, device=dev)
    anc_out = torch.zeros((B, N, 4), dtype=torch.uint64, device=dev)
    anc_in = None if from_parent else jf.build_ancestor_mask(t["parent"])[0]
    lse = torch.full(t["q"].shape[:3], float("nan"), dtype=torch.float32, device=dev)
    common = (t["q"], t["k_pages"], t["v_pages"], t["block_table"], t["prefix_len"], t["k_tree"], t["v_tree"], anc_in,
              t["parent"], t["draft"], t["logits"])
    if fn == "noalloc":
        jf.tree_verify_noalloc(*common, out, nxt, alen, nodes, bonus, sm_scale=wl.sm_scale,
                               max_prefix_len=wl.max_prefix_len, lse=lse, anc_out=anc_out)
    else:
        jf.tree_verify(*common, sm_scale=wl.sm_scale, max_prefix_len=wl.max_prefix_len, out=out, lse=lse,
                       next_tokens=nxt, accept_len=alen, accepted_nodes=nodes, bonus_token=bonus, anc_out=anc_out)
    torch.cuda.synchronize()
    anc = anc_out if from_parent else anc_in
    return {"out": out.view(torch.int16), "lse": lse.view(torch.int32), "next": nxt, "alen": alen, "nodes": nodes,
            "bonus": bonus, "anc": anc.view(torch.int64)}


def test_noalloc_verify_matches_verify_on_two_calls_in_a_row():
    sizes = []
    for name, kw, from_parent in CASES:
        wl = W.make_workload(name, 3, **kw)
        t = {k: getattr(wl, k).cuda() for k in ("q", "k_pages", "v_pages", "block_table", "prefix_len", "k_tree",
                                                 "v_tree", "parent", "draft", "logits")}
        ref = _run("verify", wl, t, from_parent)
        got = _run("noalloc", wl, t, from_parent)
        for k in ref:
            assert torch.equal(ref[k], got[k]), (name, kw, k)
        # the attention output is not all NaN (it was written)
        assert not torch.isnan(got["out"].view(torch.bfloat16).float()).any()
        sizes.append(wl.B * wl.N * wl.Hq * max(1, wl.max_prefix_len))
    assert sizes[1] < sizes[0]

