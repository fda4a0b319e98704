"""One decoding step end to end on the GPU, each stage through the C ABI and
checked against the oracle: best-first tree from draft logits (jf_build_tree),
one verification launch that builds the ancestor bitsets, runs the tree
attention over the paged prefix and accepts against the target logits
(jf_tree_verify), then the accepted path appended to the paged cache
(jf_commit_accepted). Target logits are planted so that every node's first
child agrees: the accepted path is then the chain of first children from the
root (siblings carry distinct tokens, so no other node agrees)."""

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


@pytest.mark.parametrize("seed,lens,N,topk,cap", [(3, [40, 300], 24, 3, 6), (4, [0, 1000, 77], 40, 2, 9)])
def test_build_verify_commit(jf, seed, lens, N, topk, cap):
    B, V = len(lens), 5000
    c = W.make_commit_case(seed, lens, N=N, Hq=8, Hkv=2, D=128)
    draft_logits = W.make_draft_logits_case(seed, B, N, V, topk=topk, max_path_nodes=cap).logits

    # 1. the draft tree
    par, tok, _, n = jf.build_tree(draft_logits.to(DEV), topk, cap)
    torch.cuda.synchronize()
    rp, rt, _, rn = oracle.build_tree(draft_logits, topk, cap)
    assert np.array_equal(par.cpu().numpy(), rp) and np.array_equal(tok.cpu().numpy(), rt)
    assert np.array_equal(n.cpu().numpy(), rn) and (rn == N).all()
    parent, token = rp, rt

    # target logits: row v's maximum sits on the token of v's first child
    rng = np.random.Generator(np.random.PCG64(seed + 100))
    tl = rng.standard_normal((B, N, V)).astype(np.float32)
    chain = []
    for b in range(B):
        path = [0]
        for v in range(N):
            kids = np.nonzero(parent[b] == v)[0]
            if len(kids):
                tl[b, v, token[b, kids[0]]] = 10.0
                if path[-1] == v:
                    path.append(int(kids[0]))
        chain.append(path)
    target = torch.from_numpy(tl).to(torch.bfloat16)

    # 2. verification: bitsets from the parents, attention, acceptance, one call
    d = {k: getattr(c, k).to(DEV) for k in ("q", "k_pages", "v_pages", "block_table", "prefix_len", "k_tree",
                                             "v_tree")}
    out, lse, alen, nodes, bonus, nxt, anc = jf.tree_verify(
        d["q"], d["k_pages"], d["v_pages"], d["block_table"], d["prefix_len"], d["k_tree"], d["v_tree"], None,
        par, tok, target.to(DEV), max_prefix_len=max(lens), return_lse=True)
    torch.cuda.synchronize()
    ra, _, _ = oracle.build_ancestor_mask(parent)
    assert np.array_equal(anc.view(torch.int64).cpu().numpy().view(np.uint64), ra)
    ref, lref = oracle.tree_attention(c.q, c.k_pages, c.v_pages, c.block_table, c.prefix_len, c.k_tree, c.v_tree,
                                      parent, 1.0 / np.sqrt(128.0))
    err = float(np.abs(out.float().cpu().numpy() - ref).max())
    assert err <= 1e-2 and err <= 1e-2 * np.abs(ref).max(), err
    assert float(np.abs(lse.cpu().numpy() - lref).max()) <= 2.0 ** -8 + 1e-4
    nx = oracle.target_choice(target)
    oa, on, ob = oracle.tree_accept(parent, token, nx)
    assert np.array_equal(nxt.cpu().numpy(), nx)
    assert np.array_equal(alen.cpu().numpy(), oa) and np.array_equal(nodes.cpu().numpy(), on)
    assert np.array_equal(bonus.cpu().numpy(), ob)
    for b in range(B):                       # the chain of first children, and nothing else
        assert on[b, :len(chain[b])].tolist() == chain[b] and oa[b] == len(chain[b]) - 1

    # 3. commit the accepted paths into the cache
    kp, vp = d["k_pages"].clone(), d["v_pages"].clone()
    new = jf.commit_accepted(d["k_tree"], d["v_tree"], alen, nodes, d["block_table"], d["prefix_len"], kp, vp)
    torch.cuda.synchronize()
    bits = lambda x: x.view(torch.int16).cpu().numpy()
    rk, rv, rnew = oracle.commit_accepted(bits(c.k_tree), bits(c.v_tree), oa, on, c.block_table.numpy(),
                                          c.prefix_len.numpy(), bits(c.k_pages), bits(c.v_pages))
    assert np.array_equal(new.cpu().numpy(), rnew)
    assert np.array_equal(bits(kp), rk) and np.array_equal(bits(vp), rv)
    print(f"  step: tree of {N} nodes, attention max|err| {err:.2e}, accepted {oa.tolist()}, "
          f"new prefix lengths {rnew.tolist()}", flush=True)
