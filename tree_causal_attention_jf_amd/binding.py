"""ctypes binding over libjf_tree.so (include/jf_tree.h).

Argument marshalling only: every step of the computation runs in the HIP
library. torch supplies device memory (tensor.data_ptr()) and the current HIP
stream. If the library is missing, importing this module raises: there is no
fallback path.
"""

from __future__ import annotations

import ctypes
import math
import os
import threading
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libjf_tree.so")

JF_F32, JF_BF16 = 0, 1
MAX_NODES = 256
PAGE_SIZE = 16
JF_MAX_BATCH = 1024          # sequences per tree_attention call (include/jf_tree.h)
JF_MAX_TOPK = 8              # children per node in build_tree
JF_WORKSPACE_COUNTER_BYTES = 4096   # counter region at the start of every workspace
JF_NOALLOC_SCRATCH_BYTES = 33554432  # fixed scratch array of jf_tree_verify_noalloc (per GPU)
JF_ERR_SCRATCH = 8

EXPORTED = (
    "jf_status_string",
    "jf_version",
    "jf_build_ancestor_mask",
    "jf_tree_attention_workspace_bytes",
    "jf_tree_attention",
    "jf_tree_accept_workspace_bytes",
    "jf_tree_accept",
    "jf_commit_accepted",
    "jf_tree_attention_paged_tree",
    "jf_build_tree_workspace_bytes",
    "jf_build_tree",
    "jf_tree_verify",
    "jf_tree_attention_plan",
    "jf_tree_verify_noalloc",
    "jf_tree_attention_paged_tree_plan",
)


class JfError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class AttnShape(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32),
        ("N", ctypes.c_int32),
        ("Hq", ctypes.c_int32),
        ("Hkv", ctypes.c_int32),
        ("D", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
    ]


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m tree_causal_attention_jf_amd.build` "
            "(hipcc, gfx950). There is no CPU fallback.")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.jf_status_string.restype = ctypes.c_char_p
    lib.jf_status_string.argtypes = [i32]
    lib.jf_version.restype = ctypes.c_char_p
    lib.jf_version.argtypes = []
    lib.jf_build_ancestor_mask.restype = i32
    lib.jf_build_ancestor_mask.argtypes = [vp, i32, i32, vp, vp, vp, vp]
    lib.jf_tree_attention_workspace_bytes.restype = sz
    lib.jf_tree_attention_workspace_bytes.argtypes = [ctypes.POINTER(AttnShape), i32]
    lib.jf_tree_attention_plan.restype = i32
    lib.jf_tree_attention_plan.argtypes = [ctypes.POINTER(AttnShape), i32, ctypes.POINTER(ctypes.c_int32)]
    lib.jf_tree_attention_paged_tree_plan.restype = i32
    lib.jf_tree_attention_paged_tree_plan.argtypes = [ctypes.POINTER(AttnShape), i32, ctypes.POINTER(ctypes.c_int32)]
    lib.jf_tree_attention.restype = i32
    lib.jf_tree_attention.argtypes = [ctypes.POINTER(AttnShape), i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                      vp, sz, vp]
    lib.jf_tree_accept_workspace_bytes.restype = sz
    lib.jf_tree_accept_workspace_bytes.argtypes = [i32, i32, i32]
    lib.jf_tree_accept.restype = i32
    lib.jf_tree_accept.argtypes = [i32, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.jf_tree_verify.restype = i32
    lib.jf_tree_verify.argtypes = [ctypes.POINTER(AttnShape), i32, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp,
                                   vp, sz, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.jf_tree_verify_noalloc.restype = i32
    lib.jf_tree_verify_noalloc.argtypes = [ctypes.POINTER(AttnShape), i32, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp,
                                           vp, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.jf_tree_attention_paged_tree.restype = i32
    lib.jf_tree_attention_paged_tree.argtypes = [ctypes.POINTER(AttnShape), i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                                 vp, vp, sz, vp]
    lib.jf_commit_accepted.restype = i32
    lib.jf_commit_accepted.argtypes = [ctypes.POINTER(AttnShape), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.jf_build_tree_workspace_bytes.restype = sz
    lib.jf_build_tree_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.jf_build_tree.restype = i32
    lib.jf_build_tree.argtypes = [i32, i32, i32, vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    return lib


_lib = load_library()


def status_string(status: int) -> str:
    return _lib.jf_status_string(status).decode()


def version() -> str:
    return _lib.jf_version().decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise JfError(fn, status, status_string(status))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


# ------------------------------------------------------------------ workspaces

class Workspace:
    """Zero-initialised scratch buffers, one per (device, purpose). The
    library leaves the fixed counter region at the start of a workspace zero
    after every call and writes the rest before reading it, so a buffer is
    cleared only when it is first allocated or grown, and serves calls of any
    shape. Not for calls that are in flight concurrently on different streams.

    A buffer replaced by a larger one is kept alive (never returned to the
    caching allocator) for as long as this object lives: a graph captured with
    the old buffer still writes its counters and partials there on replay, and
    no other tensor may own that memory meanwhile."""

    def __init__(self):
        self._bufs = {}
        self._retired = []
        self._lock = threading.Lock()

    def get(self, device: torch.device, key: str, nbytes: int) -> Optional[torch.Tensor]:
        if nbytes == 0:
            return None
        with self._lock:
            k = (str(device), key)
            buf = self._bufs.get(k)
            if buf is None or buf.numel() < nbytes:
                if buf is not None:
                    self._retired.append(buf)
                buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
                self._bufs[k] = buf
            return buf

    def retired(self):
        """Buffers replaced by larger ones and still held (see the class note)."""
        with self._lock:
            return list(self._retired)


_default_ws = Workspace()


# ------------------------------------------------------------------ entry points

def build_ancestor_mask(parent: torch.Tensor, anc: Optional[torch.Tensor] = None,
                        depth: Optional[torch.Tensor] = None, bad_tree: Optional[torch.Tensor] = None,
                        with_depth: bool = True):
    """parent int32 [B, N] -> (anc uint64 [B, N, 4], depth int32 [B, N], bad_tree int32 [B])."""
    _need(parent, "parent", torch.int32)
    B, N = parent.shape
    dev = parent.device
    if anc is None:
        anc = torch.empty((B, N, 4), dtype=torch.uint64, device=dev)
    if depth is None and with_depth:
        depth = torch.empty((B, N), dtype=torch.int32, device=dev)
    if bad_tree is None:
        bad_tree = torch.empty((B,), dtype=torch.int32, device=dev)
    _need(anc, "anc", torch.uint64, (B, N, 4))
    st = _lib.jf_build_ancestor_mask(_ptr(parent), B, N, _ptr(anc), _ptr(depth), _ptr(bad_tree), _stream(dev))
    _check("jf_build_ancestor_mask", st)
    return anc, depth, bad_tree


def attn_shape(q: torch.Tensor, k_pages: torch.Tensor, block_table: torch.Tensor, sm_scale: Optional[float]):
    B, N, Hq, D = q.shape
    P, Hkv, page, Dk = k_pages.shape
    dt = {torch.bfloat16: JF_BF16, torch.float32: JF_F32}.get(q.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    return AttnShape(B=B, N=N, Hq=Hq, Hkv=Hkv, D=D, page_size=page, num_pages=P,
                     max_pages_per_seq=block_table.shape[1], dtype=dt,
                     sm_scale=float(1.0 / math.sqrt(D) if sm_scale is None else sm_scale))


def tree_attention_workspace_bytes(shape: AttnShape, max_prefix_len: int) -> int:
    return int(_lib.jf_tree_attention_workspace_bytes(ctypes.byref(shape), int(max_prefix_len)))


PLAN_FIELDS = ("rows_per_workgroup", "key_groups", "row_blocks_per_wave", "splits", "pages_per_split", "balanced",
               "tree_split", "workgroups")


def tree_attention_plan(shape: AttnShape, max_prefix_len: int, paged_tree: bool = False) -> dict:
    """The launch plan jf_tree_attention (paged_tree: jf_tree_attention_paged_tree)
    would use (bf16; nothing is launched)."""
    out = (ctypes.c_int32 * 8)()
    fn = "jf_tree_attention_paged_tree_plan" if paged_tree else "jf_tree_attention_plan"
    _check(fn, getattr(_lib, fn)(ctypes.byref(shape), int(max_prefix_len), out))
    return dict(zip(PLAN_FIELDS, list(out)))


def tree_attention(q, k_pages, v_pages, block_table, prefix_len, k_tree, v_tree, anc,
                   sm_scale: Optional[float] = None, max_prefix_len: Optional[int] = None,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   return_lse: bool = False, workspace: Optional[torch.Tensor] = None):
    """Tree-causal attention (see include/jf_tree.h). max_prefix_len is a host
    upper bound on prefix_len; when None it is read from the device (a sync)."""
    for t, n in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages"), (k_tree, "k_tree"), (v_tree, "v_tree")):
        _need(t, n, q.dtype)
    _need(block_table, "block_table", torch.int32)
    _need(prefix_len, "prefix_len", torch.int32)
    _need(anc, "anc", torch.uint64)
    shape = attn_shape(q, k_pages, block_table, sm_scale)
    if max_prefix_len is None:
        max_prefix_len = int(prefix_len.max().item()) if prefix_len.numel() else 0
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    need = tree_attention_workspace_bytes(shape, max_prefix_len)
    ws = workspace if workspace is not None else _default_ws.get(dev, "attn", need)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = _lib.jf_tree_attention(ctypes.byref(shape), int(max_prefix_len), _ptr(q), _ptr(k_pages), _ptr(v_pages),
                                _ptr(block_table), _ptr(prefix_len), _ptr(k_tree), _ptr(v_tree), _ptr(anc),
                                _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _stream(dev))
    _check("jf_tree_attention", st)
    return (out, lse) if return_lse else out


def tree_attention_paged_tree(q, k_pages, v_pages, block_table, prefix_len, anc, tree_len=None,
                              sm_scale: Optional[float] = None, max_prefix_len: Optional[int] = None,
                              out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                              return_lse: bool = False, workspace: Optional[torch.Tensor] = None):
    """Tree-causal attention with ragged budgets, the tree's K/V cached right after
    each prefix (see include/jf_tree.h). Rows of padding nodes are left as they are
    in `out` (allocate it yourself to control them)."""
    for t, n in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages")):
        _need(t, n, q.dtype)
    _need(block_table, "block_table", torch.int32)
    _need(prefix_len, "prefix_len", torch.int32)
    _need(anc, "anc", torch.uint64)
    if tree_len is not None:
        _need(tree_len, "tree_len", torch.int32)
    shape = attn_shape(q, k_pages, block_table, sm_scale)
    if max_prefix_len is None:
        max_prefix_len = int(prefix_len.max().item()) if prefix_len.numel() else 0
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    need = tree_attention_workspace_bytes(shape, max_prefix_len)
    ws = workspace if workspace is not None else _default_ws.get(dev, "attn", need)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = _lib.jf_tree_attention_paged_tree(ctypes.byref(shape), int(max_prefix_len), _ptr(q), _ptr(k_pages),
                                           _ptr(v_pages), _ptr(block_table), _ptr(prefix_len), _ptr(tree_len),
                                           _ptr(anc), _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _stream(dev))
    _check("jf_tree_attention_paged_tree", st)
    return (out, lse) if return_lse else out


def tree_accept_workspace_bytes(B: int, N: int, vocab: int) -> int:
    return int(_lib.jf_tree_accept_workspace_bytes(B, N, vocab))


def tree_accept(parent, anc, draft, logits: Optional[torch.Tensor] = None,
                target_ids: Optional[torch.Tensor] = None, next_tokens=None, accept_len=None,
                accepted_nodes=None, bonus_token=None, workspace: Optional[torch.Tensor] = None):
    """Greedy tree acceptance. Exactly one of logits [B, N, V] (bf16/fp32) or
    target_ids int32 [B, N]. Returns (accept_len, accepted_nodes, bonus, next_tokens)."""
    _need(parent, "parent", torch.int32)
    _need(draft, "draft", torch.int32)
    _need(anc, "anc", torch.uint64)
    B, N = parent.shape
    dev = parent.device
    if (logits is None) == (target_ids is None):
        raise ValueError("pass exactly one of logits / target_ids")
    if logits is not None:
        _need(logits, "logits")
        vocab = logits.shape[-1]
        ldt = {torch.bfloat16: JF_BF16, torch.float32: JF_F32}[logits.dtype]
    else:
        _need(target_ids, "target_ids", torch.int32)
        vocab, ldt = 1, JF_F32
    if next_tokens is None:
        next_tokens = torch.empty((B, N), dtype=torch.int32, device=dev)
    if accept_len is None:
        accept_len = torch.empty((B,), dtype=torch.int32, device=dev)
    if accepted_nodes is None:
        accepted_nodes = torch.empty((B, N), dtype=torch.int32, device=dev)
    if bonus_token is None:
        bonus_token = torch.empty((B,), dtype=torch.int32, device=dev)
    ws = workspace
    ws_bytes = 0
    if logits is not None:
        need = tree_accept_workspace_bytes(B, N, vocab)
        if ws is None:
            ws = _default_ws.get(dev, "accept", need)
        ws_bytes = ws.numel() * ws.element_size()
    st = _lib.jf_tree_accept(B, N, vocab, _ptr(logits), ldt, _ptr(target_ids), _ptr(draft), _ptr(parent),
                             _ptr(anc), _ptr(next_tokens), _ptr(accept_len), _ptr(accepted_nodes),
                             _ptr(bonus_token), _ptr(ws), ws_bytes, _stream(dev))
    _check("jf_tree_accept", st)
    return accept_len, accepted_nodes, bonus_token, next_tokens


def tree_verify(q, k_pages, v_pages, block_table, prefix_len, k_tree, v_tree, anc, parent, draft, logits,
                sm_scale: Optional[float] = None, max_prefix_len: Optional[int] = None,
                out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, return_lse: bool = False,
                next_tokens=None, accept_len=None, accepted_nodes=None, bonus_token=None,
                attn_workspace: Optional[torch.Tensor] = None, accept_workspace: Optional[torch.Tensor] = None,
                anc_out: Optional[torch.Tensor] = None):
    """One verification step: tree attention and acceptance over the target logits
    (see include/jf_tree.h). `anc` is the ancestor bitset from build_ancestor_mask,
    or None: the call then builds it from `parent` itself (into `anc_out`, allocated
    when None). Returns (out, lse or None, accept_len, accepted_nodes, bonus_token,
    next_tokens, anc)."""
    for t, n in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages"), (k_tree, "k_tree"), (v_tree, "v_tree")):
        _need(t, n, q.dtype)
    _need(block_table, "block_table", torch.int32)
    _need(prefix_len, "prefix_len", torch.int32)
    _need(parent, "parent", torch.int32)
    _need(draft, "draft", torch.int32)
    _need(logits, "logits")
    from_parent = anc is None
    if from_parent:
        anc = anc_out if anc_out is not None else torch.empty((*parent.shape, 4), dtype=torch.uint64,
                                                              device=parent.device)
    _need(anc, "anc", torch.uint64)
    ldt = {torch.bfloat16: JF_BF16, torch.float32: JF_F32}[logits.dtype]
    shape = attn_shape(q, k_pages, block_table, sm_scale)
    if max_prefix_len is None:
        max_prefix_len = int(prefix_len.max().item()) if prefix_len.numel() else 0
    dev = q.device
    B, N = parent.shape
    vocab = logits.shape[-1]
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    if next_tokens is None:
        next_tokens = torch.empty((B, N), dtype=torch.int32, device=dev)
    if accept_len is None:
        accept_len = torch.empty((B,), dtype=torch.int32, device=dev)
    if accepted_nodes is None:
        accepted_nodes = torch.empty((B, N), dtype=torch.int32, device=dev)
    if bonus_token is None:
        bonus_token = torch.empty((B,), dtype=torch.int32, device=dev)
    need = tree_attention_workspace_bytes(shape, max_prefix_len)
    aws = attn_workspace if attn_workspace is not None else _default_ws.get(dev, "attn", need)
    aws_bytes = 0 if aws is None else aws.numel() * aws.element_size()
    cws = accept_workspace if accept_workspace is not None else \
        _default_ws.get(dev, "accept", tree_accept_workspace_bytes(B, N, vocab))
    cws_bytes = cws.numel() * cws.element_size()
    st = _lib.jf_tree_verify(ctypes.byref(shape), int(max_prefix_len), _ptr(q), _ptr(k_pages), _ptr(v_pages),
                             _ptr(block_table), _ptr(prefix_len), _ptr(k_tree), _ptr(v_tree), _ptr(anc),
                             1 if from_parent else 0, _ptr(out), _ptr(lse), _ptr(aws), aws_bytes, vocab, _ptr(logits), ldt, _ptr(draft), _ptr(parent),
                             _ptr(next_tokens), _ptr(accept_len), _ptr(accepted_nodes), _ptr(bonus_token),
                             _ptr(cws), cws_bytes, _stream(dev))
    _check("jf_tree_verify", st)
    return out, lse, accept_len, accepted_nodes, bonus_token, next_tokens, anc


def tree_verify_noalloc(q, k_pages, v_pages, block_table, prefix_len, k_tree, v_tree, anc, parent, draft, logits,
                        out, next_tokens, accept_len, accepted_nodes, bonus_token, sm_scale: Optional[float] = None,
                        max_prefix_len: int = 0, lse: Optional[torch.Tensor] = None,
                        anc_out: Optional[torch.Tensor] = None):
    """tree_verify for callers that cannot allocate: the library takes its scratch
    from a fixed device array (JF_NOALLOC_SCRATCH_BYTES per GPU), and this wrapper
    allocates nothing either, so every output buffer is the caller's and
    max_prefix_len must be given. anc None: the bitsets are built from parent into
    anc_out. Calls that overlap on one GPU race (see include/jf_tree.h)."""
    for t, n in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages"), (k_tree, "k_tree"), (v_tree, "v_tree"),
                 (out, "out")):
        _need(t, n, q.dtype)
    for t, n in ((block_table, "block_table"), (prefix_len, "prefix_len"), (parent, "parent"), (draft, "draft"),
                 (next_tokens, "next_tokens"), (accept_len, "accept_len"), (accepted_nodes, "accepted_nodes"),
                 (bonus_token, "bonus_token")):
        _need(t, n, torch.int32)
    _need(logits, "logits")
    from_parent = anc is None
    if from_parent:
        if anc_out is None:
            raise ValueError("anc None builds the bitsets into anc_out, which must be given")
        anc = anc_out
    _need(anc, "anc", torch.uint64)
    ldt = {torch.bfloat16: JF_BF16, torch.float32: JF_F32}[logits.dtype]
    shape = attn_shape(q, k_pages, block_table, sm_scale)
    dev = q.device
    st = _lib.jf_tree_verify_noalloc(ctypes.byref(shape), int(max_prefix_len), _ptr(q), _ptr(k_pages),
                                     _ptr(v_pages), _ptr(block_table), _ptr(prefix_len), _ptr(k_tree), _ptr(v_tree),
                                     _ptr(anc), 1 if from_parent else 0, _ptr(out), _ptr(lse), logits.shape[-1],
                                     _ptr(logits), ldt, _ptr(draft), _ptr(parent), _ptr(next_tokens),
                                     _ptr(accept_len), _ptr(accepted_nodes), _ptr(bonus_token), _stream(dev))
    _check("jf_tree_verify_noalloc", st)
    return out, lse, accept_len, accepted_nodes, bonus_token, next_tokens, anc


def commit_accepted(k_tree, v_tree, accept_len, accepted_nodes, block_table, prefix_len, k_pages, v_pages,
                    new_prefix_len: Optional[torch.Tensor] = None):
    """Append each sequence's accepted path (root included) to its paged cache,
    in place in k_pages / v_pages (see include/jf_tree.h). Returns
    new_prefix_len int32 [B] (prefix_len + accept_len + 1, or -1 for a sequence
    that was not committed)."""
    for t, n in ((k_tree, "k_tree"), (v_tree, "v_tree"), (k_pages, "k_pages"), (v_pages, "v_pages")):
        _need(t, n, k_tree.dtype)
    for t, n in ((accept_len, "accept_len"), (accepted_nodes, "accepted_nodes"), (block_table, "block_table"),
                 (prefix_len, "prefix_len")):
        _need(t, n, torch.int32)
    B, N, Hkv, D = k_tree.shape
    P, Hkv_p, page, D_p = k_pages.shape
    if (Hkv_p, D_p) != (Hkv, D) or tuple(v_pages.shape) != tuple(k_pages.shape) or \
            tuple(v_tree.shape) != tuple(k_tree.shape):
        raise ValueError("tree K/V [B, N, Hkv, D] and pages [P, Hkv, 16, D] disagree")
    dt = {torch.bfloat16: JF_BF16, torch.float32: JF_F32}.get(k_tree.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {k_tree.dtype}")
    shape = AttnShape(B=B, N=N, Hq=Hkv, Hkv=Hkv, D=D, page_size=page, num_pages=P,
                      max_pages_per_seq=block_table.shape[1], dtype=dt, sm_scale=1.0)
    dev = k_tree.device
    if new_prefix_len is None:
        new_prefix_len = torch.empty((B,), dtype=torch.int32, device=dev)
    st = _lib.jf_commit_accepted(ctypes.byref(shape), _ptr(k_tree), _ptr(v_tree), _ptr(accept_len),
                                 _ptr(accepted_nodes), _ptr(block_table), _ptr(prefix_len), _ptr(k_pages),
                                 _ptr(v_pages), _ptr(new_prefix_len), _stream(dev))
    _check("jf_commit_accepted", st)
    return new_prefix_len


def build_tree_workspace_bytes(B: int, N: int, vocab: int, topk: int, dtype: torch.dtype = torch.bfloat16) -> int:
    return int(_lib.jf_build_tree_workspace_bytes(B, N, vocab, topk,
                                                  {torch.bfloat16: JF_BF16, torch.float32: JF_F32}[dtype]))


def build_tree(draft_logits, topk: int, max_path_nodes: int, budget: Optional[torch.Tensor] = None,
               parent=None, token=None, score=None, tree_len=None, return_score: bool = True,
               workspace: Optional[torch.Tensor] = None):
    """Best-first draft tree from draft logits [B, N, V] (bf16/fp32), row i being
    the draft head's output at the i-th node to join. Returns (parent int32 [B, N],
    token int32 [B, N], score float64 [B, N] or None, tree_len int32 [B])."""
    _need(draft_logits, "draft_logits")
    dt = {torch.bfloat16: JF_BF16, torch.float32: JF_F32}.get(draft_logits.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {draft_logits.dtype}")
    B, N, V = draft_logits.shape
    dev = draft_logits.device
    if budget is not None:
        _need(budget, "budget", torch.int32, (B,))
    if parent is None:
        parent = torch.empty((B, N), dtype=torch.int32, device=dev)
    if token is None:
        token = torch.empty((B, N), dtype=torch.int32, device=dev)
    if score is None and return_score:
        score = torch.empty((B, N), dtype=torch.float64, device=dev)
    if tree_len is None:
        tree_len = torch.empty((B,), dtype=torch.int32, device=dev)
    need = int(_lib.jf_build_tree_workspace_bytes(B, N, V, topk, dt))
    ws = workspace if workspace is not None else _default_ws.get(dev, "build", max(need, 1))
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    st = _lib.jf_build_tree(B, N, V, _ptr(draft_logits), dt, topk, max_path_nodes, _ptr(budget), _ptr(parent),
                            _ptr(token), _ptr(score), _ptr(tree_len), _ptr(ws), ws_bytes, _stream(dev))
    _check("jf_build_tree", st)
    return parent, token, score, tree_len
