"""C-ABI checks that need no GPU: the library loads, exports every entry point
the header declares, and rejects bad arguments on the host (those checks run
before any HIP call, so they are safe without a device)."""

import ctypes
import os
import re
import subprocess

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "jf_tree.h")
LIB = os.path.join(ROOT, "tree_causal_attention_jf_amd", "libjf_tree.so")

(JF_OK, JF_ERR_NULL, JF_ERR_SHAPE, JF_ERR_DTYPE, JF_ERR_UNSUPPORTED, JF_ERR_WORKSPACE, JF_ERR_LAUNCH, JF_ERR_ALIGN,
 JF_ERR_SCRATCH) = range(9)


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(jf_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def binding():
    if not os.path.exists(LIB):
        pytest.fail("libjf_tree.so is not built (python -m tree_causal_attention_jf_amd.build)")
    from tree_causal_attention_jf_amd import binding as B
    return B


def test_header_declares_the_boundary():
    names = _declared()
    for fn in ("jf_build_ancestor_mask", "jf_tree_attention", "jf_tree_accept", "jf_status_string",
               "jf_tree_attention_workspace_bytes", "jf_tree_accept_workspace_bytes", "jf_version",
               "jf_commit_accepted", "jf_tree_attention_paged_tree", "jf_build_tree",
               "jf_build_tree_workspace_bytes", "jf_tree_verify", "jf_tree_attention_plan",
               "jf_tree_attention_paged_tree_plan", "jf_tree_verify_noalloc"):
        assert fn in names


def test_every_declared_symbol_is_exported(binding):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], stdout=subprocess.PIPE, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (jf_\w+)$", out, flags=re.M))
    for fn in _declared():
        assert fn in exported, fn
        assert hasattr(binding._lib, fn)
    assert set(binding.EXPORTED) == set(_declared())


def test_header_limits_match_the_binding(binding):
    text = open(HEADER).read()
    for name, value in (("JF_MAX_NODES", binding.MAX_NODES), ("JF_PAGE_SIZE", binding.PAGE_SIZE),
                        ("JF_MAX_BATCH", binding.JF_MAX_BATCH), ("JF_MAX_TOPK", binding.JF_MAX_TOPK),
                        ("JF_WORKSPACE_COUNTER_BYTES", binding.JF_WORKSPACE_COUNTER_BYTES),
                        ("JF_NOALLOC_SCRATCH_BYTES", binding.JF_NOALLOC_SCRATCH_BYTES)):
        assert re.search(r"#define %s (\d+)" % name, text).group(1) == str(value), name


def test_status_strings_and_version(binding):
    for code in range(9):
        assert binding.status_string(code)
    assert "JF_NOALLOC_SCRATCH_BYTES" in binding.status_string(JF_ERR_SCRATCH)
    assert binding.status_string(99) == "unknown status"
    assert re.match(r"^\d+\.\d+\.\d+$", binding.version())


def _shape(binding, **kw):
    d = dict(B=1, N=16, Hq=32, Hkv=8, D=128, page_size=16, num_pages=128, max_pages_per_seq=128,
             dtype=binding.JF_BF16, sm_scale=0.088)
    d.update(kw)
    return binding.AttnShape(**d)


def _attn(binding, shape, max_prefix=2048, ptr=16, ws=None, ws_bytes=0, nullify=()):
    args = {n: ctypes.c_void_p(ptr) for n in ("q", "kp", "vp", "bt", "pl", "kt", "vt", "anc", "out")}
    for n in nullify:
        args[n] = None
    return binding._lib.jf_tree_attention(
        ctypes.byref(shape) if shape is not None else None, max_prefix, args["q"], args["kp"], args["vp"],
        args["bt"], args["pl"], args["kt"], args["vt"], args["anc"], args["out"], None, ws, ws_bytes, None)


def test_attention_host_checks(binding):
    L = binding._lib
    assert L.jf_tree_attention(None, 0, *([None] * 10), None, 0, None) == JF_ERR_NULL
    assert _attn(binding, _shape(binding, dtype=7)) == JF_ERR_DTYPE
    assert _attn(binding, _shape(binding, N=0)) == JF_ERR_SHAPE
    assert _attn(binding, _shape(binding, N=257)) == JF_ERR_SHAPE
    assert _attn(binding, _shape(binding, Hq=30)) == JF_ERR_SHAPE          # Hq % Hkv != 0
    assert _attn(binding, _shape(binding, B=-1)) == JF_ERR_SHAPE
    assert _attn(binding, _shape(binding, D=96)) == JF_ERR_UNSUPPORTED
    assert _attn(binding, _shape(binding, page_size=32)) == JF_ERR_UNSUPPORTED
    assert _attn(binding, _shape(binding), max_prefix=2049) == JF_ERR_SHAPE  # beyond the table
    assert _attn(binding, _shape(binding), max_prefix=-1) == JF_ERR_SHAPE
    assert _attn(binding, _shape(binding, num_pages=0)) == JF_ERR_SHAPE
    assert _attn(binding, _shape(binding, sm_scale=0.0)) == JF_ERR_SHAPE
    assert _attn(binding, _shape(binding, sm_scale=float("inf"))) == JF_ERR_SHAPE
    for n in ("q", "pl", "kt", "vt", "anc", "out", "kp", "vp", "bt"):
        assert _attn(binding, _shape(binding), nullify=(n,)) == JF_ERR_NULL, n
    # without a prefix the paged arguments may be NULL; the next check (alignment) fires instead
    assert _attn(binding, _shape(binding), max_prefix=0, ptr=8, nullify=("kp", "vp", "bt")) == JF_ERR_ALIGN
    assert _attn(binding, _shape(binding), ptr=8) == JF_ERR_ALIGN
    # bf16 with many splits needs a workspace
    need = binding.tree_attention_workspace_bytes(_shape(binding), 2048)
    assert need > 0
    assert _attn(binding, _shape(binding)) == JF_ERR_WORKSPACE
    assert _attn(binding, _shape(binding), ws=ctypes.c_void_p(16), ws_bytes=need - 1) == JF_ERR_WORKSPACE
    assert _attn(binding, _shape(binding), ws=ctypes.c_void_p(8), ws_bytes=need) == JF_ERR_ALIGN


def test_workspace_queries(binding):
    # fp32 never needs scratch; an invalid shape reports 0
    assert binding.tree_attention_workspace_bytes(_shape(binding, dtype=binding.JF_F32), 2048) == 0
    assert binding.tree_attention_workspace_bytes(_shape(binding, D=96), 2048) == 0
    # a grid without split prefixes needs none
    assert binding.tree_attention_workspace_bytes(_shape(binding), 0) == 0
    # split prefixes: the fixed counter region, then the partials
    a = binding.tree_attention_workspace_bytes(_shape(binding), 2048)
    assert a > binding.JF_WORKSPACE_COUNTER_BYTES
    c = binding.tree_attention_workspace_bytes(_shape(binding, B=4, N=256, num_pages=8192,
                                                      max_pages_per_seq=2048), 32768)
    assert c > binding.JF_WORKSPACE_COUNTER_BYTES
    # more sequences than one call takes
    assert binding.tree_attention_workspace_bytes(_shape(binding, B=binding.JF_MAX_BATCH + 1), 2048) == 0
    assert binding.tree_accept_workspace_bytes(4, 256, 151936) > 4 * 256 * 4
    assert binding.tree_accept_workspace_bytes(0, 0, 10) == 0


def test_mask_and_accept_host_checks(binding):
    L = binding._lib
    p = ctypes.c_void_p(16)
    assert L.jf_build_ancestor_mask(p, 1, 0, p, None, None, None) == JF_ERR_SHAPE
    assert L.jf_build_ancestor_mask(p, 1, 257, p, None, None, None) == JF_ERR_SHAPE
    assert L.jf_build_ancestor_mask(p, -1, 4, p, None, None, None) == JF_ERR_SHAPE
    assert L.jf_build_ancestor_mask(None, 1, 4, p, None, None, None) == JF_ERR_NULL
    assert L.jf_build_ancestor_mask(p, 1, 4, None, None, None, None) == JF_ERR_NULL
    assert L.jf_build_ancestor_mask(p, 0, 4, p, None, None, None) == JF_OK   # empty batch: no launch

    def acc(B=1, N=8, V=1000, logits=p, dt=1, ids=None, nul=(), ws=None, wsb=0):
        a = {n: p for n in ("draft", "parent", "anc", "next", "alen", "nodes", "bonus")}
        for n in nul:
            a[n] = None
        return L.jf_tree_accept(B, N, V, logits, dt, ids, a["draft"], a["parent"], a["anc"], a["next"],
                                a["alen"], a["nodes"], a["bonus"], ws, wsb, None)

    assert acc(N=0) == JF_ERR_SHAPE
    assert acc(V=0) == JF_ERR_SHAPE
    assert acc(logits=None) == JF_ERR_SHAPE            # neither logits nor ids
    assert acc(ids=p) == JF_ERR_SHAPE                  # both
    assert acc(dt=5) == JF_ERR_DTYPE
    assert acc() == JF_ERR_WORKSPACE
    need = binding.tree_accept_workspace_bytes(1, 8, 1000)
    assert acc(ws=ctypes.c_void_p(8), wsb=need) == JF_ERR_ALIGN
    for n in ("draft", "parent", "anc", "next", "alen", "nodes", "bonus"):
        assert acc(nul=(n,)) == JF_ERR_NULL, n
    assert acc(B=0, ws=ctypes.c_void_p(16), wsb=need) == JF_OK   # empty batch: no launch
    # logits mode keeps one arrival counter per sequence in the fixed counter region
    big = binding.tree_accept_workspace_bytes(binding.JF_MAX_BATCH + 1, 8, 1000)
    assert acc(B=binding.JF_MAX_BATCH + 1, ws=ctypes.c_void_p(16), wsb=big) == JF_ERR_SHAPE


def test_commit_host_checks(binding):
    L = binding._lib
    p = ctypes.c_void_p(16)

    def shape(**kw):
        d = dict(B=2, N=8, Hq=4, Hkv=2, D=128, page_size=16, num_pages=10, max_pages_per_seq=4, dtype=1,
                 sm_scale=1.0)
        d.update(kw)
        return ctypes.byref(binding.AttnShape(**d))

    def commit(s=None, nul=(), align=(), new=None):
        a = {n: p for n in ("kt", "vt", "alen", "nodes", "table", "plen", "kp", "vp")}
        a["new"] = ctypes.c_void_p(32) if new is None else new
        for n in nul:
            a[n] = None
        for n in align:
            a[n] = ctypes.c_void_p(24)
        return L.jf_commit_accepted(shape() if s is None else s, a["kt"], a["vt"], a["alen"], a["nodes"],
                                    a["table"], a["plen"], a["kp"], a["vp"], a["new"], None)

    assert L.jf_commit_accepted(None, p, p, p, p, p, p, p, p, p, None) == JF_ERR_NULL
    assert commit(shape(N=0)) == JF_ERR_SHAPE
    assert commit(shape(N=257)) == JF_ERR_SHAPE
    assert commit(shape(B=binding.JF_MAX_BATCH + 1)) == JF_ERR_SHAPE
    assert commit(shape(Hkv=0)) == JF_ERR_SHAPE
    assert commit(shape(num_pages=-1)) == JF_ERR_SHAPE
    assert commit(shape(dtype=7)) == JF_ERR_DTYPE
    assert commit(shape(D=96)) == JF_ERR_UNSUPPORTED
    assert commit(shape(page_size=32)) == JF_ERR_UNSUPPORTED
    for n in ("kt", "vt", "alen", "nodes", "table", "plen", "kp", "vp", "new"):
        assert commit(nul=(n,)) == JF_ERR_NULL, n
    for n in ("kt", "vt", "kp", "vp"):
        assert commit(align=(n,)) == JF_ERR_ALIGN, n
    assert commit(new=p) == JF_ERR_SHAPE                 # new_prefix_len aliases prefix_len
    assert commit(shape(B=0)) == JF_OK                   # empty batch: no launch


def test_paged_tree_attention_host_checks(binding):
    L = binding._lib
    p = ctypes.c_void_p(16)

    def shape(**kw):
        d = dict(B=2, N=8, Hq=4, Hkv=2, D=128, page_size=16, num_pages=10, max_pages_per_seq=4, dtype=1,
                 sm_scale=0.1)
        d.update(kw)
        return binding.AttnShape(**d)

    def call(s=None, maxp=20, nul=(), align=(), ws=None, wsb=0):
        a = {n: p for n in ("q", "kp", "vp", "table", "plen", "anc", "out")}
        for n in nul:
            a[n] = None
        for n in align:
            a[n] = ctypes.c_void_p(24)
        return L.jf_tree_attention_paged_tree(ctypes.byref(shape() if s is None else s), maxp, a["q"], a["kp"],
                                              a["vp"], a["table"], a["plen"], None, a["anc"], a["out"], None, ws,
                                              wsb, None)

    assert call(shape(dtype=0)) == JF_ERR_UNSUPPORTED              # bf16 only
    assert call(shape(D=96)) == JF_ERR_UNSUPPORTED
    assert call(shape(N=0)) == JF_ERR_SHAPE
    assert call(maxp=65) == JF_ERR_SHAPE                           # beyond the block table
    assert call(shape(num_pages=0), maxp=0) == JF_ERR_SHAPE         # the tree itself must be cached
    for n in ("q", "kp", "vp", "table", "plen", "anc", "out"):
        assert call(nul=(n,)) == JF_ERR_NULL, n
    for n in ("q", "kp", "vp", "out"):
        assert call(align=(n,)) == JF_ERR_ALIGN, n
    assert call(shape(B=0)) == JF_OK


def test_build_tree_host_checks(binding):
    L = binding._lib
    p = ctypes.c_void_p(16)
    need = L.jf_build_tree_workspace_bytes(2, 16, 1000, 4, 1)
    assert need >= binding.JF_WORKSPACE_COUNTER_BYTES
    assert L.jf_build_tree_workspace_bytes(2, 16, 1000, 9, 1) == 0            # topk beyond the limit
    assert L.jf_build_tree_workspace_bytes(2, 16, 1000, 4, 5) == 0            # unknown dtype

    def call(B=2, N=16, V=1000, dt=1, k=4, cap=6, nul=(), ws=None, wsb=None):
        a = {n: p for n in ("logits", "parent", "token", "len")}
        for n in nul:
            a[n] = None
        w = ctypes.c_void_p(4096) if ws is None else ws
        return L.jf_build_tree(B, N, V, a["logits"], dt, k, cap, None, a["parent"], a["token"], None, a["len"],
                               w, need if wsb is None else wsb, None)

    assert call(N=0) == JF_ERR_SHAPE
    assert call(N=257) == JF_ERR_SHAPE
    assert call(B=-1) == JF_ERR_SHAPE
    assert call(B=binding.JF_MAX_BATCH + 1) == JF_ERR_SHAPE
    assert call(V=0) == JF_ERR_SHAPE
    assert call(k=0) == JF_ERR_SHAPE
    assert call(k=binding.JF_MAX_TOPK + 1) == JF_ERR_SHAPE
    assert call(cap=0) == JF_ERR_SHAPE
    assert call(dt=3) == JF_ERR_DTYPE
    for n in ("logits", "parent", "token", "len"):
        assert call(nul=(n,)) == JF_ERR_NULL, n
    assert call(wsb=need - 1) == JF_ERR_WORKSPACE
    assert call(ws=ctypes.c_void_p(0)) == JF_ERR_WORKSPACE
    assert call(ws=ctypes.c_void_p(4104)) == JF_ERR_ALIGN
    assert call(B=0) == JF_OK                                                  # empty batch: no launch


def test_verify_host_checks(binding):
    """jf_tree_verify applies the checks of both calls it stands for, needs the
    logits, and refuses overlapping workspaces; all before any launch."""
    L = binding._lib
    shape = _shape(binding)
    a_need = binding.tree_attention_workspace_bytes(shape, 2048)
    c_need = binding.tree_accept_workspace_bytes(1, 16, 1000)
    p = ctypes.c_void_p(16)

    def ver(shape=shape, max_prefix=2048, logits=p, dt=1, V=1000, aws=0x100000, awsb=a_need, cws=0x800000,
            cwsb=c_need, nul=(), from_parent=0):
        a = {n: p for n in ("q", "kp", "vp", "bt", "pl", "kt", "vt", "anc", "out", "draft", "parent", "next",
                            "alen", "nodes", "bonus")}
        for n in nul:
            a[n] = None
        return L.jf_tree_verify(ctypes.byref(shape), max_prefix, a["q"], a["kp"], a["vp"], a["bt"], a["pl"],
                                a["kt"], a["vt"], a["anc"], from_parent, a["out"], None, ctypes.c_void_p(aws), awsb,
                                V, logits,
                                dt, a["draft"], a["parent"], a["next"], a["alen"], a["nodes"], a["bonus"],
                                ctypes.c_void_p(cws), cwsb, None)

    assert ver(shape=_shape(binding, N=0)) == JF_ERR_SHAPE          # attention's checks
    assert ver(shape=_shape(binding, D=96)) == JF_ERR_UNSUPPORTED
    assert ver(logits=None) == JF_ERR_NULL                          # logits are required
    assert ver(dt=5) == JF_ERR_DTYPE                                # acceptance's checks
    assert ver(V=0) == JF_ERR_SHAPE
    for n in ("q", "anc", "out", "draft", "parent", "next", "alen", "nodes", "bonus"):
        assert ver(nul=(n,)) == JF_ERR_NULL, n
    assert ver(awsb=a_need - 1) == JF_ERR_WORKSPACE
    assert ver(cwsb=c_need - 1) == JF_ERR_WORKSPACE
    assert ver(cws=0x100000 + a_need - 256) == JF_ERR_WORKSPACE     # overlapping workspaces
    assert ver(aws=0x800000 + 256) == JF_ERR_WORKSPACE
    assert ver(from_parent=2) == JF_ERR_SHAPE                       # 0: anc is input, 1: built from parent
    assert ver(from_parent=1, nul=("anc",)) == JF_ERR_NULL          # the built bitsets need somewhere to go
    assert ver(shape=_shape(binding, B=0)) == JF_OK                 # empty batch: no launch
    assert ver(shape=_shape(binding, B=0), from_parent=1) == JF_OK


def test_noalloc_verify_host_checks(binding):
    """jf_tree_verify_noalloc applies jf_tree_verify's checks and refuses a call
    whose two workspaces would not fit its fixed array, all before any HIP call
    (nothing here touches a device)."""
    L = binding._lib
    p = ctypes.c_void_p(16)

    def ver(shape, max_prefix=2048, logits=p, dt=1, V=1000, nul=(), from_parent=0):
        a = {n: p for n in ("q", "kp", "vp", "bt", "pl", "kt", "vt", "anc", "out", "draft", "parent", "next",
                            "alen", "nodes", "bonus")}
        for n in nul:
            a[n] = None
        return L.jf_tree_verify_noalloc(ctypes.byref(shape), max_prefix, a["q"], a["kp"], a["vp"], a["bt"],
                                        a["pl"], a["kt"], a["vt"], a["anc"], from_parent, a["out"], None, V, logits,
                                        dt, a["draft"], a["parent"], a["next"], a["alen"], a["nodes"], a["bonus"],
                                        None)

    shape = _shape(binding)
    assert ver(_shape(binding, N=0)) == JF_ERR_SHAPE
    assert ver(_shape(binding, D=96)) == JF_ERR_UNSUPPORTED
    assert ver(shape, logits=None) == JF_ERR_NULL
    assert ver(shape, dt=5) == JF_ERR_DTYPE
    assert ver(shape, V=0) == JF_ERR_SHAPE
    for n in ("q", "anc", "out", "draft", "parent", "next", "alen", "nodes", "bonus"):
        assert ver(shape, nul=(n,)) == JF_ERR_NULL, n
    assert ver(shape, from_parent=2) == JF_ERR_SHAPE
    assert ver(shape, nul=("q",)) == JF_ERR_NULL
    # batch 32 of 64-node trees at 32q/4kv over prefixes up to 8192 needs more than the array
    big = _shape(binding, B=32, N=64, Hq=32, Hkv=4, num_pages=20000, max_pages_per_seq=512)
    need = binding.tree_attention_workspace_bytes(big, 8192) + binding.tree_accept_workspace_bytes(32, 64, 151936)
    assert need > binding.JF_NOALLOC_SCRATCH_BYTES
    assert ver(big, max_prefix=8192, V=151936) == JF_ERR_SCRATCH
    assert ver(_shape(binding, B=0)) == JF_OK                       # empty batch: nothing looked up or launched


def test_workspace_cache_keeps_replaced_buffers_alive(binding):
    """A workspace replaced by a larger one stays referenced, so a graph that
    captured the old address never writes into memory another tensor owns."""
    import torch
    ws = binding.Workspace()
    dev = torch.device("cpu")
    a = ws.get(dev, "attn", 1000)
    assert ws.get(dev, "attn", 500) is a                # big enough: reused
    assert int(a.sum()) == 0
    b = ws.get(dev, "attn", 5000)                       # grown: a new zeroed buffer
    assert b is not a and b.numel() >= 5000 and int(b.sum()) == 0
    assert any(r is a for r in ws.retired())
    assert ws.get(dev, "accept", 0) is None
