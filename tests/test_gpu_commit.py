"""GPU parity of jf_commit_accepted (through the C ABI) against the oracle.

Bars: the whole page pools and the new prefix lengths bit-exact; the
attention of the next step over the committed cache within the bf16 bar of
the attention tests.
"""

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


def _bits(t):
    return t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.numpy()


def _run_both(jf, case, alen, nodes, table=None, plen=None):
    table = case.block_table if table is None else table
    plen = case.prefix_len if plen is None else plen
    kp, vp = case.k_pages.to(DEV), case.v_pages.to(DEV)
    new = jf.commit_accepted(case.k_tree.to(DEV), case.v_tree.to(DEV), torch.as_tensor(alen).to(DEV),
                             torch.as_tensor(nodes).to(DEV), table.to(DEV), plen.to(DEV), kp, vp)
    torch.cuda.synchronize()
    rk, rv, rnew = oracle.commit_accepted(_bits(case.k_tree), _bits(case.v_tree), np.asarray(alen),
                                          np.asarray(nodes), table.numpy(), plen.numpy(), _bits(case.k_pages),
                                          _bits(case.v_pages))
    assert np.array_equal(new.cpu().numpy(), rnew)
    assert np.array_equal(_bits(kp.cpu()), rk)
    assert np.array_equal(_bits(vp.cpu()), rv)
    return new, kp, vp


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.bfloat16, 64), (torch.float32, 128)])
def test_commit_matches_oracle(jf, dtype, D):
    # prefixes ending mid-page, on a page boundary, empty, and long; paths from the
    # acceptance oracle (ids mode), including a forced root-only commit
    lens = [14, 16, 0, 1000, 31]
    case = W.make_commit_case(11, lens, N=24, Hq=8, Hkv=2, D=D, dtype=dtype, max_path_nodes=9, p_agree=0.9)
    alen, nodes, _ = oracle.tree_accept(case.parent.numpy(), case.draft.numpy(), case.target_ids.numpy())
    alen = alen.copy()
    nodes = nodes.copy()
    alen[4] = 0
    nodes[4, 1:] = -1
    new, _, _ = _run_both(jf, case, alen, nodes)
    assert new.cpu().tolist() == [L + int(a) + 1 for L, a in zip(lens, alen)]


def test_commit_rejects_bad_sequences_and_keeps_the_rest(jf):
    lens = [10, 10, 10, 10, 10, 40]
    case = W.make_commit_case(13, lens, N=6, Hq=2, Hkv=2, D=128)
    B, N = len(lens), 6
    alen = np.array([2, 6, 1, 1, 2, 5], dtype=np.int32)        # b1: accept_len == N
    nodes = np.full((B, N), -1, dtype=np.int32)
    nodes[:, :3] = [0, 1, 2]
    nodes[5, :6] = [0, 1, 2, 3, 4, 5]
    nodes[2, 1] = N                                           # b2: node id out of range
    table = case.block_table.clone()
    table[3, (10 + 1) // 16] = -1                             # b3: a page of the new tokens is missing
    table[5, (40 + 5) // 16] = case.k_pages.shape[0]          # b5: page id past the pool
    plen = case.prefix_len.clone()
    plen[4] = -1                                              # b4: negative prefix
    new, _, _ = _run_both(jf, case, alen, nodes, table=table, plen=plen)
    assert new.cpu().tolist() == [13, -1, -1, -1, -1, -1]


def test_accept_commit_then_attend(jf):
    # the full step on the GPU: acceptance, commit, and the next step's one-node tree
    # (the accepted end node) over the committed prefix reproduces that node's tree
    # attention of this step, as the oracle computes it
    lens = [30, 513, 0, 100]
    case = W.make_commit_case(17, lens, N=40, Hq=8, Hkv=2, D=128, max_path_nodes=10, p_agree=0.85)
    B, N, Hq = len(lens), 40, 8
    parent = case.parent.to(DEV)
    anc, _, _ = jf.build_ancestor_mask(parent)
    alen, nodes, _, _ = jf.tree_accept(parent, anc, case.draft.to(DEV), target_ids=case.target_ids.to(DEV))
    kp, vp = case.k_pages.to(DEV), case.v_pages.to(DEV)
    new = jf.commit_accepted(case.k_tree.to(DEV), case.v_tree.to(DEV), alen, nodes, case.block_table.to(DEV),
                             case.prefix_len.to(DEV), kp, vp)
    torch.cuda.synchronize()
    alen_h, nodes_h = alen.cpu().numpy(), nodes.cpu().numpy()
    ra, rn, _ = oracle.tree_accept(case.parent.numpy(), case.draft.numpy(), case.target_ids.numpy())
    assert np.array_equal(alen_h, ra) and np.array_equal(nodes_h, rn)
    assert new.cpu().tolist() == [L + int(a) + 1 for L, a in zip(lens, alen_h)]
    ends = [int(nodes_h[b, alen_h[b]]) for b in range(B)]
    idx, ar = torch.tensor(ends), torch.arange(B)
    q1 = case.q[ar, idx].unsqueeze(1).contiguous()
    k1 = case.k_tree[ar, idx].unsqueeze(1).contiguous()
    v1 = case.v_tree[ar, idx].unsqueeze(1).contiguous()
    p1 = torch.full((B, 1), -1, dtype=torch.int32, device=DEV)
    a1, _, _ = jf.build_ancestor_mask(p1)
    out1, lse1 = jf.tree_attention(q1.to(DEV), kp, vp, case.block_table.to(DEV), (new - 1).contiguous(),
                                   k1.to(DEV), v1.to(DEV), a1, sm_scale=1.0 / np.sqrt(128),
                                   max_prefix_len=int(max(lens) + N), return_lse=True)
    torch.cuda.synchronize()
    rows = [(b, ends[b], h) for b in range(B) for h in range(Hq)]
    ref, lref = oracle.tree_attention(case.q, case.k_pages, case.v_pages, case.block_table, case.prefix_len,
                                      case.k_tree, case.v_tree, case.parent, 1.0 / np.sqrt(128), rows=rows)
    o = out1.float().cpu().numpy()
    err = max(abs(o[b, 0, h] - ref[b, ends[b], h]).max() for b in range(B) for h in range(Hq))
    lerr = max(abs(float(lse1[b, 0, h]) - lref[b, ends[b], h]) for b in range(B) for h in range(Hq))
    print(f"  next-step attention over the committed cache: max|err| {err:.3e}, lse {lerr:.3e}", flush=True)
    assert err <= 1e-2 and lerr <= 2.0 ** -8 + 1e-4
