"""Seeded synthetic inputs for tree-causal attention and greedy tree acceptance.

This module draws random numbers and lays them out: draft trees (as parent
arrays), a paged KV cache with shuffled page order, queries, the tree's own
K/V, target logits or target ids, and draft tokens. It computes nothing that
the attention or acceptance path computes: no ancestor sets, no attention
scores or weights, no argmax over target logits. Both the CPU oracle's tests
and the GPU path's tests and benchmark take their inputs from here, as plain
CPU tensors.

One exception shapes inputs only: `tree_best_first` grows the best-first
draft trees of the budget-64/256 workloads the way the workload text
describes them, so it normalises its own random draft logits (a log-softmax)
and takes their top-k, i.e. it repeats the arithmetic of tree construction.
Its trees are inputs to attention and acceptance; no expected value comes
from it. Tree construction itself (jf_build_tree) is checked against the
oracle's build_tree on separately drawn logits (make_draft_logits_case), never
against this function.

The workloads stand in for the evaluation set-up of "JetFlow: Breaking the
Scaling Ceiling of Speculative Decoding with Parallel Tree Drafting"
(gist.science technical summary, section 4: Qwen3-8B and Qwen3-30B-A3B, draft
budgets 16 and 256). Only the attention-layer shapes of those models are used;
token content does not enter the attention arithmetic.
"""

from __future__ import annotations

import heapq
import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

PAGE_SIZE = 16
QWEN3_VOCAB = 151936


# --------------------------------------------------------------------------
# Draft trees. Every generator returns a parent array with parent[0] = -1 and
# 0 <= parent[i] < i (nodes are numbered in creation order).
# --------------------------------------------------------------------------

def tree_chain(n: int) -> np.ndarray:
    """A linear draft of n tokens: node i hangs under node i-1."""
    p = np.arange(-1, n - 1, dtype=np.int32)
    return p


def tree_random_recursive(n: int, max_path_nodes: int, rng: np.random.Generator) -> np.ndarray:
    """Node i > 0 picks its parent uniformly among earlier nodes whose
    root-to-node path still has room (fewer than max_path_nodes nodes)."""
    parent = np.full(n, -1, dtype=np.int32)
    level = [1]
    for i in range(1, n):
        cands = [j for j in range(i) if level[j] < max_path_nodes]
        j = int(cands[rng.integers(len(cands))])
        parent[i] = j
        level.append(level[j] + 1)
    return parent


def tree_best_first(n: int, topk: int, max_path_nodes: int, vocab: int, sigma: float,
                    rng: np.random.Generator):
    """Best-first draft tree of n nodes.

    Each expanded node draws i.i.d. N(0, sigma^2) draft logits over the
    vocabulary, normalises them to log-probabilities and offers its top-k
    tokens as children. Candidates are ranked by cumulative draft
    log-probability (ties: creation order); the best candidate joins the tree
    until n nodes exist. A node whose path already holds max_path_nodes nodes
    is not expanded. Returns (parent int32[n], token int32[n]); token[0] = -1.
    """
    parent = [-1]
    token = [-1]
    path_nodes = [1]
    cum = [0.0]
    heap: list = []
    counter = 0

    def expand(v: int) -> None:
        nonlocal counter
        if path_nodes[v] >= max_path_nodes:
            return
        z = rng.standard_normal(vocab, dtype=np.float32).astype(np.float64) * sigma
        zmax = z.max()
        log_norm = zmax + math.log(np.exp(z - zmax).sum())
        top = np.argpartition(-z, topk)[:topk]
        top = top[np.argsort(-z[top], kind="stable")]
        for t in top:
            heapq.heappush(heap, (-(cum[v] + z[t] - log_norm), counter, v, int(t)))
            counter += 1

    expand(0)
    while len(parent) < n:
        if not heap:
            raise ValueError("tree cannot reach the requested size under the path cap")
        neg, _, p, t = heapq.heappop(heap)
        parent.append(p)
        token.append(t)
        path_nodes.append(path_nodes[p] + 1)
        cum.append(-neg)
        if len(parent) < n:
            expand(len(parent) - 1)
    return np.asarray(parent, dtype=np.int32), np.asarray(token, dtype=np.int32)


# --------------------------------------------------------------------------
# Workload container
# --------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    dtype: torch.dtype
    B: int
    N: int
    Hq: int
    Hkv: int
    D: int
    page_size: int
    sm_scale: float
    q: torch.Tensor            # [B, N, Hq, D]
    k_pages: torch.Tensor      # [P, Hkv, page, D]
    v_pages: torch.Tensor      # [P, Hkv, page, D]
    block_table: torch.Tensor  # int32 [B, max_pages_per_seq], unused entries -1
    prefix_len: torch.Tensor   # int32 [B]
    k_tree: torch.Tensor       # [B, N, Hkv, D]
    v_tree: torch.Tensor       # [B, N, Hkv, D]
    parent: torch.Tensor       # int32 [B, N]
    k_prefix: List[torch.Tensor] = field(default_factory=list)  # per b: [L_b, Hkv, D] contiguous
    v_prefix: List[torch.Tensor] = field(default_factory=list)
    # acceptance inputs
    vocab: int = 0
    draft: Optional[torch.Tensor] = None        # int32 [B, N]; column 0 unused
    target_ids: Optional[torch.Tensor] = None   # int32 [B, N] (ids mode)
    logits: Optional[torch.Tensor] = None       # [B, N, vocab] (logits mode)
    planted_target: Optional[torch.Tensor] = None  # int32 [B, N]: the planted unique-max token per row
    planted_leaf: Optional[torch.Tensor] = None    # int32 [B]

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def num_pages(self) -> int:
        return int(self.k_pages.shape[0])

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_prefix_len(self) -> int:
        return int(self.prefix_len.max().item()) if self.B > 0 else 0


def _to_dtype(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """float32 numpy -> torch tensor of dtype (round-to-nearest-even for bf16)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dtype)


def make_paged_kv(prefix_lens, Hkv: int, D: int, dtype: torch.dtype, data_scale: float,
                  rng: np.random.Generator, page_size: int = PAGE_SIZE, extra_pages: int = 0,
                  poison: bool = False):
    """Contiguous per-sequence prefixes scattered into a shuffled page pool.

    Token t of sequence b sits in slot t % page_size of page
    block_table[b, t // page_size]. The pool holds every page the sequences
    need plus `extra_pages` unused ones, in a random order. With poison=True,
    unused slots of partially filled pages and unused pages hold NaN.
    """
    B = len(prefix_lens)
    npages = [(int(L) + page_size - 1) // page_size for L in prefix_lens]
    pool = sum(npages) + extra_pages
    max_pages = max(1, max(npages) if npages else 1)
    perm = rng.permutation(pool).astype(np.int32)
    fill = np.nan if poison else 0.0
    k_pool = np.full((pool, Hkv, page_size, D), fill, dtype=np.float32)
    v_pool = np.full((pool, Hkv, page_size, D), fill, dtype=np.float32)
    table = np.full((B, max_pages), -1, dtype=np.int32)
    k_prefix, v_prefix = [], []
    cursor = 0
    for b, L in enumerate(prefix_lens):
        L = int(L)
        kc = (rng.standard_normal((L, Hkv, D), dtype=np.float32) * data_scale).astype(np.float32)
        vc = (rng.standard_normal((L, Hkv, D), dtype=np.float32) * data_scale).astype(np.float32)
        # round once to the storage dtype so paged and contiguous copies agree bit for bit
        kt = _to_dtype(kc, dtype)
        vt = _to_dtype(vc, dtype)
        k_prefix.append(kt)
        v_prefix.append(vt)
        kc = kt.float().numpy()
        vc = vt.float().numpy()
        for p in range(npages[b]):
            pid = int(perm[cursor])
            cursor += 1
            table[b, p] = pid
            lo, hi = p * page_size, min(L, (p + 1) * page_size)
            k_pool[pid, :, : hi - lo, :] = kc[lo:hi].transpose(1, 0, 2)
            v_pool[pid, :, : hi - lo, :] = vc[lo:hi].transpose(1, 0, 2)
    return (_to_dtype(k_pool, dtype), _to_dtype(v_pool, dtype), torch.from_numpy(table),
            k_prefix, v_prefix)


@dataclass
class CommitCase:
    """Inputs of one commit of accepted paths into a paged cache."""
    k_pages: torch.Tensor          # [P, Hkv, 16, D]
    v_pages: torch.Tensor
    block_table: torch.Tensor      # int32 [B, max_pages]: room for prefix_len[b] + N tokens
    prefix_len: torch.Tensor       # int32 [B]
    k_tree: torch.Tensor           # [B, N, Hkv, D]
    v_tree: torch.Tensor
    q: torch.Tensor                # [B, N, Hq, D] (for attention-based checks)
    parent: torch.Tensor           # int32 [B, N]
    draft: torch.Tensor            # int32 [B, N]
    target_ids: torch.Tensor       # int32 [B, N]


def make_commit_case(seed: int, lens, N: int, Hq: int, Hkv: int, D: int, dtype: torch.dtype = torch.bfloat16,
                     max_path_nodes: int = 8, p_agree: float = 0.8, extra_pages: int = 3) -> CommitCase:
    """A paged cache whose block table lists pages for prefix_len[b] + N tokens
    (the slots past the prefix hold random data, as a reused page would), the
    tree's own Q/K/V, random recursive draft trees, and draft / target ids for
    acceptance (ids mode)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = [int(L) for L in lens]
    scale = 1.0 / math.sqrt(128.0)
    kp, vp, table, _, _ = make_paged_kv([L + N for L in lens], Hkv, D, dtype, scale, rng, extra_pages=extra_pages)
    B = len(lens)
    parent = np.stack([tree_random_recursive(N, max_path_nodes, rng) for _ in range(B)]).astype(np.int32)
    pairs = [make_accept_ids(parent[b], 1000, p_agree, rng) for b in range(B)]
    target = np.stack([t for t, _ in pairs])
    draft = np.stack([d for _, d in pairs])
    q = _to_dtype(rng.standard_normal((B, N, Hq, D), dtype=np.float32) * scale, dtype)
    kt = _to_dtype(rng.standard_normal((B, N, Hkv, D), dtype=np.float32) * scale, dtype)
    vt = _to_dtype(rng.standard_normal((B, N, Hkv, D), dtype=np.float32) * scale, dtype)
    return CommitCase(kp, vp, table, torch.tensor(lens, dtype=torch.int32), kt, vt, q,
                      torch.from_numpy(parent), torch.from_numpy(np.asarray(draft, dtype=np.int32)),
                      torch.from_numpy(np.asarray(target, dtype=np.int32)))


def make_accept_ids(parent: np.ndarray, vocab: int, p_agree: float, rng: np.random.Generator):
    """Ids mode: target token per node uniform in [0, vocab); a child's draft
    token equals its parent's target token with probability p_agree, else a
    uniformly drawn different token. Returns (target_ids, draft)."""
    N = len(parent)
    target = rng.integers(0, vocab, size=N).astype(np.int32)
    draft = np.full(N, -1, dtype=np.int32)
    for u in range(1, N):
        want = int(target[parent[u]])
        if rng.random() < p_agree:
            draft[u] = want
        else:
            other = int(rng.integers(0, vocab - 1))
            draft[u] = other if other < want else other + 1
    return target, draft


def _leaves(parent: np.ndarray) -> np.ndarray:
    has_child = np.zeros(len(parent), dtype=bool)
    has_child[parent[parent >= 0]] = True
    return np.nonzero(~has_child)[0]


def make_accept_logits(parent: np.ndarray, vocab: int, sigma: float, p_agree: float,
                       dtype: torch.dtype, rng: np.random.Generator):
    """Logits mode with a planted path.

    Every row of logits is N(0, sigma^2), rounded to dtype; then one uniformly
    drawn token per row is raised strictly above the row's largest value, so
    the row's target token is known without any argmax. Along one uniformly
    drawn root-to-leaf path, a node's draft token equals its parent's planted
    target token with probability p_agree, else a different uniform token; all
    other nodes get uniform tokens. Returns (logits, planted, draft, leaf).
    """
    N = len(parent)
    z = rng.standard_normal((N, vocab), dtype=np.float32) * np.float32(sigma)
    logits = _to_dtype(z, dtype)
    planted = rng.integers(0, vocab, size=N).astype(np.int32)
    row_top = logits.float().amax(dim=1)
    for v in range(N):
        bump = float(row_top[v]) + max(0.25, abs(float(row_top[v])) * 2.0 ** -5)
        logits[v, int(planted[v])] = bump
    leaves = _leaves(parent)
    leaf = int(leaves[rng.integers(len(leaves))])
    on_path = set()
    u = leaf
    while u > 0:
        on_path.add(u)
        u = int(parent[u])
    draft = np.full(N, -1, dtype=np.int32)
    for u in range(1, N):
        if u in on_path:
            want = int(planted[parent[u]])
            if rng.random() < p_agree:
                draft[u] = want
            else:
                other = int(rng.integers(0, vocab - 1))
                draft[u] = other if other < want else other + 1
        else:
            draft[u] = int(rng.integers(0, vocab))
    return logits, planted, draft, leaf


# --------------------------------------------------------------------------
# Named configurations
# --------------------------------------------------------------------------

CONFIGS = {
    # tiny fp32 case: 64-token prefix, 16-node random tree (<= 6 nodes per path), 4q/1kv, d=64
    "c0_tiny_fp32": dict(dtype=torch.float32, B=1, prefix=("fixed", 64), N=16, Hq=4, Hkv=1, D=64,
                         tree=("random", 6), data_scale=1.0, accept=("ids", 1000, 0.7)),
    # Qwen3-8B attention layer, budget 16 as a linear chain, prefix 2048
    "c1_chain16": dict(dtype=torch.bfloat16, B=1, prefix=("fixed", 2048), N=16, Hq=32, Hkv=8, D=128,
                       tree=("chain",), data_scale=1.0 / math.sqrt(128.0),
                       accept=("logits", QWEN3_VOCAB, 3.0, 0.8)),
    # Qwen3-8B, batch 8, budget 256 best-first, prefix U[1024, 4096]
    "c2_bf256_b8": dict(dtype=torch.bfloat16, B=8, prefix=("uniform", 1024, 4096), N=256, Hq=32, Hkv=8,
                        D=128, tree=("best_first", 4, 12, 2.0), data_scale=1.0 / math.sqrt(128.0),
                        accept=("ids", QWEN3_VOCAB, 0.8)),
    # Qwen3-30B-A3B, batch 32, budget 64 best-first, prefix U[512, 8192], GQA group 8
    "c3_bf64_b32": dict(dtype=torch.bfloat16, B=32, prefix=("uniform", 512, 8192), N=64, Hq=32, Hkv=4,
                        D=128, tree=("best_first", 4, 10, 2.0), data_scale=1.0 / math.sqrt(128.0),
                        accept=("ids", QWEN3_VOCAB, 0.8)),
    # the draft head's own tree-causal pass: one decoder layer in the target's attention shape, all 256
    # nodes of one sequence's tree in one call over its KV cache of the fused target features (8192 tokens)
    "draft_head_b1": dict(dtype=torch.bfloat16, B=1, prefix=("fixed", 8192), N=256, Hq=32, Hkv=8, D=128,
                          tree=("best_first", 4, 12, 2.0), data_scale=1.0 / math.sqrt(128.0),
                          accept=("ids", QWEN3_VOCAB, 0.8)),
    # long-context verification, batch 4, prefix 32768, budget 256, acceptance over full logits
    "c4_bf256_32k": dict(dtype=torch.bfloat16, B=4, prefix=("fixed", 32768), N=256, Hq=32, Hkv=8, D=128,
                         tree=("best_first", 4, 12, 2.0), data_scale=1.0 / math.sqrt(128.0),
                         accept=("logits", QWEN3_VOCAB, 3.0, 0.8)),
}

_TREE_CACHE: dict = {}


def make_tree(spec, N: int, seed: int, b: int):
    """Parent array (and best-first tokens) for sequence b of a workload."""
    key = (spec, N, seed, b)
    if key in _TREE_CACHE:
        return _TREE_CACHE[key]
    rng = np.random.Generator(np.random.PCG64([seed, 7919, b]))
    kind = spec[0]
    if kind == "chain":
        out = (tree_chain(N), None)
    elif kind == "random":
        out = (tree_random_recursive(N, spec[1], rng), None)
    elif kind == "best_first":
        out = tree_best_first(N, spec[1], spec[2], QWEN3_VOCAB, spec[3], rng)
    else:
        raise ValueError(kind)
    _TREE_CACHE[key] = out
    return out


def make_workload(name: str, seed: int = 0, *, unscaled: bool = False, poison: bool = False,
                  with_accept: bool = True, extra_pages: int = 0, B: Optional[int] = None,
                  N: Optional[int] = None, prefix=None, tree=None, dtype=None,
                  Hq: Optional[int] = None, Hkv: Optional[int] = None, D: Optional[int] = None,
                  sm_scale: Optional[float] = None, accept=None) -> Workload:
    """Build the named configuration with the given seed.

    Keyword overrides shrink or reshape a configuration for small parity cases.
    unscaled=True draws Q/K/V from N(0, 1) instead of the configuration's
    scaling; poison=True fills unused page slots and unused pages with NaN.
    """
    cfg = dict(CONFIGS[name])
    for k, v in dict(B=B, N=N, prefix=prefix, tree=tree, dtype=dtype, Hq=Hq, Hkv=Hkv, D=D,
                     accept=accept).items():
        if v is not None:
            cfg[k] = v
    dtype = cfg["dtype"]
    B, N, Hq, Hkv, D = cfg["B"], cfg["N"], cfg["Hq"], cfg["Hkv"], cfg["D"]
    scale = 1.0 if unscaled else cfg["data_scale"]
    rng = np.random.Generator(np.random.PCG64([seed, 1]))
    pspec = cfg["prefix"]
    if pspec[0] == "fixed":
        lens = np.full(B, pspec[1], dtype=np.int32)
    elif pspec[0] == "uniform":
        lens = rng.integers(pspec[1], pspec[2] + 1, size=B).astype(np.int32)
    elif pspec[0] == "list":
        lens = np.asarray(pspec[1], dtype=np.int32)
        assert len(lens) == B
    else:
        raise ValueError(pspec)
    k_pages, v_pages, table, k_prefix, v_prefix = make_paged_kv(
        lens, Hkv, D, dtype, scale, rng, extra_pages=extra_pages, poison=poison)
    q = _to_dtype(rng.standard_normal((B, N, Hq, D), dtype=np.float32) * scale, dtype)
    k_tree = _to_dtype(rng.standard_normal((B, N, Hkv, D), dtype=np.float32) * scale, dtype)
    v_tree = _to_dtype(rng.standard_normal((B, N, Hkv, D), dtype=np.float32) * scale, dtype)
    parents = np.stack([make_tree(cfg["tree"], N, seed, b)[0] for b in range(B)])
    wl = Workload(name=name, dtype=dtype, B=B, N=N, Hq=Hq, Hkv=Hkv, D=D, page_size=PAGE_SIZE,
                  sm_scale=(1.0 / math.sqrt(D)) if sm_scale is None else float(sm_scale),
                  q=q, k_pages=k_pages, v_pages=v_pages, block_table=table,
                  prefix_len=torch.from_numpy(lens.copy()), k_tree=k_tree, v_tree=v_tree,
                  parent=torch.from_numpy(parents.astype(np.int32)),
                  k_prefix=k_prefix, v_prefix=v_prefix)
    if with_accept:
        acc = cfg["accept"]
        arng = np.random.Generator(np.random.PCG64([seed, 2]))
        if acc[0] == "ids":
            tgt, dr = zip(*[make_accept_ids(parents[b], acc[1], acc[2], arng) for b in range(B)])
            wl.vocab = acc[1]
            wl.target_ids = torch.from_numpy(np.stack(tgt))
            wl.draft = torch.from_numpy(np.stack(dr))
        else:
            vocab, sigma, p = acc[1], acc[2], acc[3]
            logits = torch.empty((B, N, vocab), dtype=dtype)
            planted, drafts, leaves = [], [], []
            for b in range(B):
                lg, pl, dr, leaf = make_accept_logits(parents[b], vocab, sigma, p, dtype, arng)
                logits[b] = lg
                planted.append(pl)
                drafts.append(dr)
                leaves.append(leaf)
            wl.vocab = vocab
            wl.logits = logits
            wl.planted_target = torch.from_numpy(np.stack(planted))
            wl.draft = torch.from_numpy(np.stack(drafts))
            wl.planted_leaf = torch.tensor(leaves, dtype=torch.int32)
    return wl


@dataclass
class PagedTreeCase:
    """Ragged tree budgets with each tree's K/V stored in the cache right after
    its prefix (node j of sequence b is cached token prefix_len[b] + j)."""
    q: torch.Tensor                # [B, N, Hq, D]; rows of padding nodes are ordinary data
    k_pages: torch.Tensor          # [P, Hkv, 16, D]: prefix and tree tokens
    v_pages: torch.Tensor
    block_table: torch.Tensor      # int32 [B, max_pages]: pages of prefix_len[b] + tree_len[b] tokens
    prefix_len: torch.Tensor       # int32 [B]
    tree_len: torch.Tensor         # int32 [B], 0 <= tree_len[b] <= N
    parent: torch.Tensor           # int32 [B, N]; padding nodes hang under the root
    draft: torch.Tensor            # int32 [B, N]; -1 for padding nodes
    k_tree: torch.Tensor           # [B, N, Hkv, D]: the same tree keys as separate arrays (0 for padding)
    v_tree: torch.Tensor
    sm_scale: float
    max_prefix_len: int


def make_paged_tree_case(seed: int, lens, budgets, N: int, Hq: int, Hkv: int, D: int, tree=("random", 6),
                         dtype: torch.dtype = torch.bfloat16, unscaled: bool = False,
                         extra_pages: int = 2) -> PagedTreeCase:
    """Sequence b: a prefix of lens[b] tokens followed by its tree's budgets[b]
    nodes, cached as one contiguous run of tokens in a shuffled page pool.
    Trees come from the same generators as the workloads (with budgets[b]
    nodes); padding nodes up to N get parent 0 and draft token -1."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = [int(L) for L in lens]
    budgets = [int(n) for n in budgets]
    assert len(lens) == len(budgets) and all(0 <= n <= N for n in budgets)
    scale = 1.0 if unscaled else 1.0 / math.sqrt(128.0)
    kp, vp, table, kc, vc = make_paged_kv([L + n for L, n in zip(lens, budgets)], Hkv, D, dtype, scale, rng,
                                          extra_pages=extra_pages)
    B = len(lens)
    parent = np.zeros((B, N), dtype=np.int32)
    draft = np.full((B, N), -1, dtype=np.int32)
    k_tree = torch.zeros((B, N, Hkv, D), dtype=dtype)
    v_tree = torch.zeros((B, N, Hkv, D), dtype=dtype)
    for b, (L, n) in enumerate(zip(lens, budgets)):
        parent[b, 0] = -1
        if n > 0:
            par, _ = make_tree(tree, n, seed, b)
            parent[b, :n] = par
            draft[b, 1:n] = rng.integers(0, 1000, size=n - 1)
            k_tree[b, :n] = kc[b][L:L + n]
            v_tree[b, :n] = vc[b][L:L + n]
    q = _to_dtype(rng.standard_normal((B, N, Hq, D), dtype=np.float32) * scale, dtype)
    return PagedTreeCase(q, kp, vp, table, torch.tensor(lens, dtype=torch.int32),
                         torch.tensor(budgets, dtype=torch.int32), torch.from_numpy(parent),
                         torch.from_numpy(draft), k_tree, v_tree, 1.0 / math.sqrt(D), max(lens) if lens else 0)


# --------------------------------------------------------------------------
# Draft logits for best-first tree construction
# --------------------------------------------------------------------------

@dataclass
class DraftLogitsCase:
    logits: torch.Tensor           # [B, N, V]: row i = the draft head's output at the i-th node to join
    topk: int
    max_path_nodes: int
    budget: torch.Tensor           # int32 [B], 0 <= budget[b] <= N


def make_draft_logits_case(seed: int, B: int, N: int, vocab: int, topk: int = 4, max_path_nodes: int = 12,
                           sigma: float = 2.0, budgets=None, dtype: torch.dtype = torch.bfloat16,
                           kind: str = "normal") -> DraftLogitsCase:
    """Draft logits i.i.d. N(0, sigma^2) over the vocabulary (the draft-logit
    recipe of the budget-256 workloads), rounded to dtype. Other kinds:
      "uniform"     all-zero rows;
      "ties"        normal rows in which topk + 2 random positions are raised to
                    the row's largest value, so the best logits of a row tie;
      "small_ints"  integers 0..3, so equal logits are common inside and
                    across rows.
    budgets: per-sequence node budgets (None: N)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if kind in ("normal", "ties"):
        z = rng.standard_normal((B, N, vocab), dtype=np.float32) * np.float32(sigma)
        if kind == "ties":
            z = _to_dtype(z, dtype).float().numpy()
            for row in z.reshape(-1, vocab):
                row[rng.choice(vocab, size=min(vocab, topk + 2), replace=False)] = row.max()
    elif kind == "uniform":
        z = np.zeros((B, N, vocab), dtype=np.float32)
    elif kind == "small_ints":
        z = rng.integers(0, 4, size=(B, N, vocab)).astype(np.float32)
    else:
        raise ValueError(kind)
    bud = [N] * B if budgets is None else [int(x) for x in budgets]
    return DraftLogitsCase(_to_dtype(z, dtype), topk, max_path_nodes, torch.tensor(bud, dtype=torch.int32))
