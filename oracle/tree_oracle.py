"""CPU oracle for tree-causal attention and greedy tree acceptance (fp64).

TEST INFRASTRUCTURE. This module is the checker, not the product: only the
test suite, the smoke check and the benchmark's CPU-baseline leg may import
it. The HIP library never calls it, and it shares no code with the library.

Source of the definitions: "JetFlow: Breaking the Scaling Ceiling of
Speculative Decoding with Parallel Tree Drafting", the gist.science pages
(Japanese and German technical summaries).
  * Section 2 (method), tree-causal attention mask: every node of the draft
    tree attends to the input prefix and to its own ancestors in the tree, and
    never to its descendants or to unrelated sibling branches. The branch
    factorisation printed there conditions each node only on its own
    root-to-node path; we read the path as including the node itself, so a
    chain-shaped tree reduces to ordinary causal attention.
  * Section 3 (contributions): the tree is verified by the target model over
    a paged KV cache.
  * Lay summary and the qxai.app commentary: the target accepts the drafted
    tokens up to the point where it disagrees.

Everything the pages leave open is resolved by the plainest reading:
  - node order is topological: parent[0] = -1 and 0 <= parent[i] < i;
  - query head h reads KV head h // (Hq // Hkv);
  - scores are sm_scale * q.k, softmax over the visible keys, output = P V,
    log-sum-exp in natural log;
  - node 0 is the last committed token (always accepted); a child c agrees
    when its draft token equals the target's choice at its parent; the
    accepted path is the longest root-to-node path on which every node
    agrees, ties to the smallest end-node index; the bonus token is the
    target's choice at the end of that path;
  - the target's choice at a node is the first index of the largest logit;
    NaN never wins; a row of NaN only yields 0;
  - tree construction: row i of the draft logits belongs to the i-th node to
    join the tree; candidates are ordered by cumulative log-probability, then
    by their parent's join order, then by rank (logit, then token id).

Arithmetic is fp64 throughout. Inputs stored in bf16 or fp32 are widened
exactly, so the oracle sees the same rounded values the GPU sees.
"""

from __future__ import annotations

import heapq
import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

ANC_WORDS = 4          # the ancestor bitset is 4 x 64 bits per node
MAX_NODES = 64 * ANC_WORDS


def _f64(x) -> np.ndarray:
    """Widen a torch tensor (any float dtype) or array to float64 exactly."""
    if hasattr(x, "detach"):
        import torch
        return x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _i64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        return x.detach().to("cpu").numpy().astype(np.int64)
    return np.asarray(x, dtype=np.int64)


# --------------------------------------------------------------------------
# Tree structure (section 2, tree-causal attention mask)
# --------------------------------------------------------------------------

def is_valid_tree(parent: Sequence[int]) -> bool:
    """A draft tree in creation order: one root at index 0, every other node's
    parent created before it."""
    p = [int(x) for x in parent]
    if len(p) == 0 or len(p) > MAX_NODES:
        return False
    if p[0] != -1:
        return False
    return all(0 <= p[i] < i for i in range(1, len(p)))


def root_path(parent: Sequence[int], v: int) -> list:
    """Nodes on the path from the root to v, root first, v last (naive walk
    up the parent pointers). Requires a valid tree."""
    path = []
    u = int(v)
    while u != -1:
        path.append(u)
        u = int(parent[u])
    path.reverse()
    return path


def ancestor_matrix(parent: Sequence[int]) -> np.ndarray:
    """Dense visibility among tree nodes: A[i, j] is True iff node j is on
    the root-to-i path (j == i included). Requires a valid tree."""
    n = len(parent)
    A = np.zeros((n, n), dtype=bool)
    for i in range(n):
        for j in root_path(parent, i):
            A[i, j] = True
    return A


def pack_bitset(A: np.ndarray) -> np.ndarray:
    """Encode each row of A as 4 little-endian 64-bit words: node j is bit
    (j % 64) of word (j // 64). Bits at or beyond N are zero."""
    n = A.shape[0]
    words = np.zeros((n, ANC_WORDS), dtype=np.uint64)
    for i in range(n):
        for j in range(n):
            if A[i, j]:
                words[i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
    return words


def build_ancestor_mask(parent) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Batched mask builder: parent int[B, N] ->
    (anc uint64[B, N, 4], depth int32[B, N], bad_tree int32[B]).

    depth counts the nodes on the root-to-node path (root = 1). For a
    sequence whose parent array is not a valid tree only bad_tree (= 1) is
    defined; its anc/depth rows are left zero here."""
    P = _i64(parent)
    B, N = P.shape
    anc = np.zeros((B, N, ANC_WORDS), dtype=np.uint64)
    depth = np.zeros((B, N), dtype=np.int32)
    bad = np.zeros(B, dtype=np.int32)
    for b in range(B):
        if not is_valid_tree(P[b]):
            bad[b] = 1
            continue
        A = ancestor_matrix(P[b])
        anc[b] = pack_bitset(A)
        depth[b] = A.sum(axis=1).astype(np.int32)
    return anc, depth, bad


# --------------------------------------------------------------------------
# Paged prefix (section 3: verification over a paged KV cache)
# --------------------------------------------------------------------------

def gather_prefix(pages: np.ndarray, table_row: np.ndarray, L: int, page_size: int) -> np.ndarray:
    """Prefix token t of a sequence lives in slot t % page_size of page
    table_row[t // page_size]; pages is [P, Hkv, page_size, D].
    Returns [L, Hkv, D]."""
    Hkv, D = pages.shape[1], pages.shape[3]
    out = np.empty((L, Hkv, D), dtype=np.float64)
    for t in range(L):
        out[t] = pages[int(table_row[t // page_size]), :, t % page_size, :]
    return out


# --------------------------------------------------------------------------
# Tree-causal attention (section 2 mask, section 3 paged verification)
# --------------------------------------------------------------------------

def _softmax_attend(qrows: np.ndarray, K: np.ndarray, V: np.ndarray, visible: np.ndarray,
                    sm_scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Masked attention of a few query rows over explicit keys.
    qrows [n, D], K/V [T, D], visible bool [n, T] -> (O [n, D], lse [n])."""
    s = sm_scale * (qrows @ K.T)
    s = np.where(visible, s, -np.inf)
    rowmax = s.max(axis=1, keepdims=True)
    e = np.exp(s - rowmax)
    z = e.sum(axis=1, keepdims=True)
    p = e / z
    return p @ V, rowmax[:, 0] + np.log(z[:, 0])


def _sequence_keys(b, k_pages, v_pages, block_table, prefix_len, k_tree, v_tree, page_size):
    L = int(prefix_len[b])
    Kp = gather_prefix(k_pages, block_table[b], L, page_size)
    Vp = gather_prefix(v_pages, block_table[b], L, page_size)
    K = np.concatenate([Kp, k_tree[b]], axis=0)   # [L + N, Hkv, D]
    V = np.concatenate([Vp, v_tree[b]], axis=0)
    return L, K, V


def tree_attention(q, k_pages, v_pages, block_table, prefix_len, k_tree, v_tree, parent,
                   sm_scale: Optional[float] = None, page_size: int = 16,
                   rows: Optional[Iterable[Tuple[int, int, int]]] = None):
    """Tree-causal attention.

    q [B, N, Hq, D]; k_pages/v_pages [P, Hkv, page, D]; block_table int[B, *];
    prefix_len int[B]; k_tree/v_tree [B, N, Hkv, D]; parent int[B, N].

    Node i of sequence b sees keys 0..L_b-1 of its prefix and the tree keys of
    the nodes on its root-to-i path (itself included) -- an explicit dense
    [N, L_b + N] mask per sequence. Returns (out float64 [B, N, Hq, D],
    lse float64 [B, N, Hq]). With `rows` = iterable of (b, node, head), only
    those entries are computed; the others stay NaN.
    """
    Q = _f64(q)
    KP, VP = _f64(k_pages), _f64(v_pages)
    KT, VT = _f64(k_tree), _f64(v_tree)
    BT, PL, PAR = _i64(block_table), _i64(prefix_len), _i64(parent)
    B, N, Hq, D = Q.shape
    Hkv = KP.shape[1]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    out = np.full((B, N, Hq, D), np.nan)
    lse = np.full((B, N, Hq), np.nan)
    if rows is None:
        want = {(b, h): list(range(N)) for b in range(B) for h in range(Hq)}
    else:
        want = {}
        for (b, n, h) in rows:
            want.setdefault((int(b), int(h)), []).append(int(n))
    by_seq = {}
    for (b, h), nodes in want.items():
        by_seq.setdefault(b, []).append((h, nodes))
    for b, heads in by_seq.items():
        if not is_valid_tree(PAR[b]):
            raise ValueError(f"sequence {b}: parent array is not a valid tree")
        L, K, V = _sequence_keys(b, KP, VP, BT, PL, KT, VT, page_size)
        A = ancestor_matrix(PAR[b])
        mask = np.zeros((N, L + N), dtype=bool)
        mask[:, :L] = True
        mask[:, L:] = A
        for h, nodes in heads:
            g = h // G
            idx = np.asarray(sorted(set(nodes)))
            o, l = _softmax_attend(Q[b, idx, h, :], K[:, g, :], V[:, g, :], mask[idx], sm_scale)
            out[b, idx, h, :] = o
            lse[b, idx, h] = l
    return out, lse


def tree_attention_paged_tree(q, k_pages, v_pages, block_table, prefix_len, tree_len, parent,
                              sm_scale: Optional[float] = None, page_size: int = 16,
                              rows: Optional[Iterable[Tuple[int, int, int]]] = None):
    """Tree-causal attention with ragged budgets and the tree's K/V in the paged cache.

    Sequence b has tree_len[b] = N_b <= N nodes (nodes 0..N_b-1 of q and
    parent; the rest are padding). Its tree K/V follow its prefix in the
    cache: node j's key is prefix token L_b + j, so the keys of the sequence are
    its first L_b + N_b cached tokens, the last N_b of which are the tree's.
    Otherwise the computation is tree_attention's, for nodes 0..N_b-1 of the
    tree parent[b, :N_b]. Rows of padding nodes stay NaN.
    """
    Q = _f64(q)
    TL, PL = _i64(tree_len), _i64(prefix_len)
    BT = _i64(block_table)
    B, N = Q.shape[0], Q.shape[1]
    Hq = Q.shape[2]
    out = np.full(Q.shape, np.nan)
    lse = np.full(Q.shape[:3], np.nan)
    want = {}
    for (b, n, h) in (rows if rows is not None else [(b, n, h) for b in range(B) for n in range(N)
                                                      for h in range(Hq)]):
        if int(n) < int(TL[b]):
            want.setdefault(int(b), []).append((int(n), int(h)))
    for b, pairs in want.items():
        L, nb = int(PL[b]), int(TL[b])
        # the tree's keys and values, gathered from the cache after the prefix
        kt = gather_prefix(_f64(k_pages), BT[b], L + nb, page_size)[L:][None]
        vt = gather_prefix(_f64(v_pages), BT[b], L + nb, page_size)[L:][None]
        o, l = tree_attention(Q[b:b + 1, :nb], k_pages, v_pages, BT[b:b + 1], PL[b:b + 1], kt, vt,
                              _i64(parent)[b:b + 1, :nb], sm_scale, page_size,
                              rows=[(0, n, h) for n, h in pairs])
        for n, h in pairs:
            out[b, n, h] = o[0, n, h]
            lse[b, n, h] = l[0, n, h]
    return out, lse


# --------------------------------------------------------------------------
# Target choice and greedy acceptance (lay summary; qxai.app commentary)
# --------------------------------------------------------------------------

def argmax_first(row) -> int:
    """Index of the largest value, the first one among equal maxima
    (-0 and +0 are equal). NaN never wins; a row of only NaN yields 0."""
    x = _f64(row).reshape(-1)
    ok = ~np.isnan(x)
    if not ok.any():
        return 0
    best = x[ok].max()
    return int(np.nonzero(ok & (x == best))[0][0])


def target_choice(logits) -> np.ndarray:
    """logits [B, N, V] -> int32 [B, N], one argmax_first per row."""
    X = _f64(logits)
    B, N, _ = X.shape
    out = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
        for v in range(N):
            out[b, v] = argmax_first(X[b, v])
    return out


def accept_one(parent: Sequence[int], draft: Sequence[int], next_tok: Sequence[int]):
    """Greedy acceptance for one tree, by a naive walk of every node's path.

    Returns (accept_len, accepted_nodes list padded with -1 to N, bonus)."""
    N = len(parent)
    best_v, best_len = 0, 1
    for v in range(N):
        path = root_path(parent, v)
        agrees = all(int(draft[u]) == int(next_tok[int(parent[u])]) for u in path[1:])
        if agrees and len(path) > best_len:
            best_v, best_len = v, len(path)
    path = root_path(parent, best_v)
    nodes = path + [-1] * (N - len(path))
    return len(path) - 1, nodes, int(next_tok[best_v])


def tree_accept(parent, draft, next_tokens):
    """Batched acceptance: parent/draft/next_tokens int[B, N] ->
    (accept_len int32[B], accepted_nodes int32[B, N], bonus int32[B])."""
    P, Dr, Nx = _i64(parent), _i64(draft), _i64(next_tokens)
    B, N = P.shape
    alen = np.zeros(B, dtype=np.int32)
    nodes = np.full((B, N), -1, dtype=np.int32)
    bonus = np.zeros(B, dtype=np.int32)
    for b in range(B):
        if not is_valid_tree(P[b]):
            raise ValueError(f"sequence {b}: parent array is not a valid tree")
        a, nd, bo = accept_one(P[b], Dr[b], Nx[b])
        alen[b], nodes[b], bonus[b] = a, nd, bo
    return alen, nodes, bonus


def commit_accepted(k_tree, v_tree, accept_len, accepted_nodes, block_table, prefix_len, k_pages, v_pages,
                    page_size: int = 16):
    """Append each sequence's accepted path to its paged cache.

    After verification the kept tokens become part of the prefix the next
    step attends to (lay summary: the target keeps the drafted tokens up to
    its first disagreement; technical summary section 3: that prefix lives in
    a paged KV cache). Node 0 of a tree is the last committed token, whose K/V
    was computed together with the tree, so the path's accept_len + 1 nodes
    are appended: prefix token prefix_len[b] + i receives the K/V of
    accepted_nodes[b, i], for i = 0 .. accept_len[b].

    A sequence is committed only when prefix_len[b] >= 0, 0 <= accept_len[b]
    < N, the path entries are node ids in [0, N), and every page its new
    tokens land in is listed (table slot below the table width, page id in
    [0, num_pages)); otherwise nothing of it is written and its new length is
    -1. Arrays are copied element for element (any dtype, bit patterns kept).

    Returns (k_pages', v_pages', new_prefix_len int32[B]).
    """
    kt, vt = np.asarray(k_tree), np.asarray(v_tree)
    kp, vp = np.array(k_pages, copy=True), np.array(v_pages, copy=True)
    alen, nodes = _i64(accept_len), _i64(accepted_nodes)
    table, plen = _i64(block_table), _i64(prefix_len)
    B, N = nodes.shape
    num_pages, width = kp.shape[0], table.shape[1]
    new_len = np.full(B, -1, dtype=np.int32)
    for b in range(B):
        L, a = int(plen[b]), int(alen[b])
        if L < 0 or not (0 <= a < N):
            continue
        path = [int(n) for n in nodes[b, : a + 1]]
        if any(not (0 <= n < N) for n in path):
            continue
        slots = [(L + i) // page_size for i in range(a + 1)]
        if any(s >= width or not (0 <= int(table[b, s]) < num_pages) for s in slots):
            continue
        for i, n in enumerate(path):
            pos = L + i
            page = int(table[b, pos // page_size])
            kp[page, :, pos % page_size, :] = kt[b, n]
            vp[page, :, pos % page_size, :] = vt[b, n]
        new_len[b] = L + a + 1
    return kp, vp, new_len


# --------------------------------------------------------------------------
# Best-first tree construction (technical summaries, section 2, "tree
# construction": the draft head emits logits for the whole tree in one pass;
# nodes are ranked by their cumulative draft log-probability, and a best-first
# expansion grows the candidate tree to the token budget)
# --------------------------------------------------------------------------

def draft_children(row, topk: int):
    """The children a node offers: its topk most likely next tokens.

    row is the node's draft logits over the vocabulary. NaN entries count as
    -inf. The log-probability of token t is row[t] - logsumexp(row). Tokens
    are ranked by logit, larger first, ties to the smaller token id; tokens of
    -inf logit are never offered, and a row whose largest entry is not finite
    (only -inf / NaN, or any +inf) offers nothing.

    Returns (tokens int list, log-probabilities float list), best first."""
    z = _f64(row).reshape(-1).copy()
    z[np.isnan(z)] = -np.inf
    m = z.max()
    if not np.isfinite(m):
        return [], []
    lse = m + math.log(float(np.exp(z - m).sum()))
    finite = np.nonzero(z > -np.inf)[0]
    k = min(topk, finite.size)
    # the k-th largest logit bounds the candidates; rank those by (-logit, token)
    kth = np.partition(z[finite], finite.size - k)[finite.size - k]
    cand = finite[z[finite] >= kth]
    cand = cand[np.lexsort((cand, -z[cand]))][:k]
    return [int(t) for t in cand], [float(z[t] - lse) for t in cand]


def build_tree(draft_logits, topk: int, max_path_nodes: int, budget=None):
    """Best-first construction of one draft tree per sequence.

    draft_logits [B, N, V]: row i of sequence b is the draft head's output at
    the tree's node i, nodes being numbered in the order they join the tree
    (node 0 is the root, the last committed token). Node i's children are
    draft_children(row i, topk), each scored by the node's cumulative log-
    probability plus the child's log-probability. The candidate with the best
    score joins next, ties to the candidate whose parent joined first, then to
    the better-ranked child; it becomes the next node and, unless its root-to-
    node path already holds max_path_nodes nodes, offers its own children.
    Growth stops at budget[b] nodes (None: N) or when no candidate is left.

    Returns (parent int32[B, N], token int32[B, N], score float64[B, N],
    tree_len int32[B]). Node 0 has parent -1 and token -1 (score 0). Nodes at
    or past tree_len[b] are padding: parent 0 (node 0 keeps -1 when the budget
    is 0), token -1, score -inf.
    """
    X = _f64(draft_logits)
    B, N, _ = X.shape
    nb_all = [N] * B if budget is None else [int(x) for x in _i64(budget).reshape(-1)]
    parent = np.zeros((B, N), dtype=np.int32)
    parent[:, 0] = -1
    token = np.full((B, N), -1, dtype=np.int32)
    score = np.full((B, N), -np.inf)
    tree_len = np.zeros(B, dtype=np.int32)
    for b in range(B):
        nb = nb_all[b]
        if not 0 <= nb <= N:
            raise ValueError(f"sequence {b}: budget {nb} outside [0, {N}]")
        if nb == 0:
            continue
        score[b, 0] = 0.0
        depth = [1]
        heap: list = []

        def offer(v: int) -> None:
            if depth[v] >= max_path_nodes:
                return
            toks, lps = draft_children(X[b, v], topk)
            for r, (t, lp) in enumerate(zip(toks, lps)):
                heapq.heappush(heap, (-(score[b, v] + lp), v, r, t))

        offer(0)
        n = 1
        while n < nb and heap:
            neg, v, _, t = heapq.heappop(heap)
            parent[b, n], token[b, n], score[b, n] = v, t, -neg
            depth.append(depth[v] + 1)
            n += 1
            if n < nb:
                offer(n - 1)
        tree_len[b] = n
    return parent, token, score, tree_len
