#!/usr/bin/env python3
"""Benchmark of the tree-verification hot path on one MI355X.

A step is one pass of the whole path over one batch of the budget-16 workload
(Qwen3-8B attention layer: 32 query / 8 KV heads, head dim 128, bf16, prefix
2048 in shuffled 16-token pages, a 16-node chain tree):
    jf_tree_verify: one launch that builds the ancestor bitsets from the parent
    array, runs the tree attention, and beside it the argmax over bf16 target
    logits [1, 16, 151936] with the acceptance walk.
Each step runs on its own input set; the sets rotate through more than twice
the 256 MB Infinity Cache so that reads come from HBM. The timed steps are
replayed from HIP graphs holding one pass over the input sets (every kernel
still waits for the one before it). Also reported: the same steps submitted
one graph each (host launch cost included), and the same steps as three
launches (jf_build_ancestor_mask, jf_tree_attention, jf_tree_accept). Prints
one JSON line.

Also measured: each kernel's average duration (HIP events around a graph of
back-to-back launches of that kernel alone, on the stream it runs on), the
roofline fraction of the step's dominant kernel (the verification launch) and
of the attention kernel alone, the budget-256 workload (batch 8, 256-node
best-first trees, prefixes U[1024, 4096]), budget 16 at streaming size, the
long-context workload (attention and acceptance apart), ragged budgets with
the trees' K/V in the paged cache, tree construction, the commit of accepted
paths, and the fp64 CPU oracle on a bounded sample as `cpu_baseline`.

`roofline.traffic` is the verification kernel's HBM bytes per launch from the
FETCH_SIZE / WRITE_SIZE counter summary in profiles/ (each counter scaled by
what it reads for a plain 256 MiB copy in the same run); it is null when the
kernel sources have changed since those counters were taken. The summary is
made by:
    rocprofv3 --pmc FETCH_SIZE -d F -o run --output-format csv -- python bench.py --profile-steps 20
    rocprofv3 --pmc WRITE_SIZE -d W -o run --output-format csv -- python bench.py --profile-steps 20
    python bench.py --summarize-pmc F W
The profile run also reads [4, 256, 151936] bf16 logits once with the
acceptance kernel, a second kernel of known bytes for the FETCH_SIZE factor.

Per-workload summaries in profiles/ (each file records its command):
    rocprofv3 --kernel-trace --stats -d D -o run --output-format csv -- python bench.py --only NAME --no-cpu-baseline
    python bench.py --summarize-stats D NAME
    rocprofv3 --pmc <MFMA_COUNTERS> -d D -o run --output-format csv -- python bench.py --only NAME --no-cpu-baseline --profile-reps 2
    rocprofv3 --pmc <LIMIT_COUNTERS> -d L -o run --output-format csv -- (the same bench.py command)
    python bench.py --summarize-mfma D NAME KERNEL AVERAGE_US --limits L
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
MALL_BYTES = 256 << 20
ROOT = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 256 << 20          # counter calibration: plain copy, reads and writes this much
ATTN_KERNEL = "tree_attn_bf16_kernel"
STEP_KERNEL = "tree_verify_bf16_kernel"   # attention + acceptance of a budget-16 step, one launch


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--config", default="c1_chain16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--eager", action="store_true", help="launch steps eagerly instead of graph replay")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="run a 256 MiB copy (counter calibration), then this many eager steps, and exit")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs of --profile-steps into the traffic summary")
    ap.add_argument("--summarize-stats", nargs=2, metavar=("STATS_DIR", "LABEL"),
                    help="turn a rocprofv3 --kernel-trace --stats run into profiles/kernel_stats_LABEL.txt")
    ap.add_argument("--summarize-mfma", nargs=4, metavar=("PMC_DIR", "LABEL", "KERNEL", "DURATION_US"),
                    help="turn a rocprofv3 --pmc run of the MFMA counters into profiles/KERNEL_LABEL_mfma.txt "
                         "(KERNEL: a substring of the kernel name; DURATION_US: its average duration)")
    ap.add_argument("--limits", default=None, metavar="PMC_DIR",
                    help="with --summarize-mfma: a second rocprofv3 --pmc run of the LDS and VALU counters")
    ap.add_argument("--limits-command", default="",
                    help="with --limits: the profiler command line of that run")
    ap.add_argument("--command", default="",
                    help="with --summarize-*: the profiler command line to record in the summary")
    ap.add_argument("--profile-reps", type=int, default=0,
                    help="sub-workloads replay each graph this many times (short runs under a profiler)")
    ap.add_argument("--only", default=None,
                    help="comma-separated subset of: step (the headline), " + ", ".join(SUBS))
    ap.add_argument("--separate", action="store_true",
                    help="time steps as mask + jf_tree_attention + jf_tree_accept instead of mask + jf_tree_verify")
    return ap.parse_args()


# the verification kernel: attention (its launch plan), acceptance and shared helpers
ATTN_SOURCES = ("attn_bf16.hip", "accept_device.h", "jf_common.h")


def source_digest():
    """sha256 over the attention kernel's sources and the public header (the
    counters go stale when they change)."""
    h = hashlib.sha256()
    files = [os.path.join(ROOT, "tree_causal_attention_jf_amd", "csrc", f) for f in ATTN_SOURCES] + \
        [os.path.join(ROOT, "include", "jf_tree.h")]
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_file(config):
    return os.path.join(ROOT, "profiles", f"{STEP_KERNEL}_{config}_hbm_traffic.txt")


def read_counter_csv(d, counter):
    """{kernel name: [per-dispatch values]} for one counter of a rocprofv3 --pmc csv run."""
    paths = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    assert paths, f"no counter_collection.csv under {d}"
    per = {}
    for path in paths:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return per


def summarize_pmc(fetch_dir, write_dir, config):
    fetch = read_counter_csv(fetch_dir, "FETCH_SIZE")
    write = read_counter_csv(write_dir, "WRITE_SIZE")
    copy_kib = COPY_BYTES / 1024

    def copy_kernel(per):
        # the calibration copy (a device-to-device tensor copy: the runtime's copy
        # kernel) is the dispatch of that kernel moving the most bytes
        cands = [(n, max(v)) for n, v in per.items() if "copybuffer" in n.lower()]
        if not cands:
            cands = [(n, max(v)) for n, v in per.items() if "copy" in n.lower()]
        n, v = max(cands, key=lambda t: t[1])
        return n, v

    cf_name, cf = copy_kernel(fetch)
    cw_name, cw = copy_kernel(write)
    f_fac, w_fac = copy_kib / cf, copy_kib / cw
    # the acceptance kernel over [4, 256, 151936] bf16 logits reads each logit once
    acc = [(n, v) for n, v in fetch.items() if "accept_logits_kernel" in n]
    acc_line = "#   (no acceptance calibration in this run)"
    if acc:
        an, av = max(acc, key=lambda t: max(t[1]))
        acc_kib = max(av)
        logit_kib = 4 * 256 * 151936 * 2 / 1024
        acc_line = (f"#   second calibration: acceptance over [4,256,151936] bf16 logits ({logit_kib:.0f} KiB read once) "
                    f"shows FETCH_SIZE {acc_kib:.0f} KiB: factor {logit_kib / acc_kib:.4f}")
    lines = [f"# HBM traffic of the verification kernel (attention + acceptance), workload {config}",
             "# made by:",
             f"#   rocprofv3 --pmc FETCH_SIZE -d FETCH_DIR -o run --output-format csv -- "
             f"python bench.py --config {config} --profile-steps 20",
             f"#   rocprofv3 --pmc WRITE_SIZE -d WRITE_DIR -o run --output-format csv -- "
             f"python bench.py --config {config} --profile-steps 20",
             f"#   python bench.py --config {config} --summarize-pmc FETCH_DIR WRITE_DIR",
             f"# calibration: a {COPY_BYTES >> 20} MiB copy reads FETCH_SIZE {cf:.0f} KiB and "
             f"WRITE_SIZE {cw:.0f} KiB per dispatch",
             f"#   ({cf_name[:60]}); scale factors fetch {f_fac:.4f}, write {w_fac:.4f}",
             acc_line,
             "# kernel | dispatches | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | scaled bytes/dispatch"]
    attn = None
    for name in sorted(set(fetch) & set(write)):
        if "jf::" not in name:
            continue
        fv, wv = fetch[name], write[name]
        favg, wavg = sum(fv) / len(fv), sum(wv) / len(wv)
        scaled = favg * f_fac * 1024 + wavg * w_fac * 1024
        lines.append(f"# {name} | {len(fv)} | {favg:.1f} | {wavg:.1f} | {scaled:.0f}")
        if STEP_KERNEL in name:
            attn = (name, scaled)
    assert attn is not None, "no verification kernel in the counter runs"
    lines += [f"kernel: {attn[0]}",
              f"traffic_bytes_per_launch: {attn[1]:.0f}",
              f"fetch_factor: {f_fac:.6f}",
              f"write_factor: {w_fac:.6f}",
              f"source_sha256: {source_digest()}"]
    out = traffic_file(config)
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    print(f"wrote {out}")


def _stats_rows(d):
    paths = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    assert paths, f"no kernel_stats.csv under {d}"
    rows = []
    for path in paths:
        with open(path) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def summarize_stats(d, label, command):
    """profiles/kernel_stats_LABEL.txt from a rocprofv3 --kernel-trace --stats run."""
    lines = [f"# Kernel durations, rocprofv3 kernel trace of one bench.py run: {label}",
             "# command (from the repository root; cd /tmp && export TMPDIR=/tmp for the profiler's scratch files):",
             f"#   {command}" if command else "#   (command not given)",
             f"#   python bench.py --summarize-stats <dir> {label}",
             "# kernel | calls | average us | min us | max us | share of GPU time"]
    for r in sorted(_stats_rows(d), key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"]
        if "fill" in name.lower() or "elementwise" in name.lower() or "distribution" in name.lower():
            name = "torch fill / random / elementwise (inputs and workspace set-up): " + name[:40]
        lines.append(f"{name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}%")
    out = os.path.join(ROOT, "profiles", f"kernel_stats_{label}.txt")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    print(f"wrote {out}")


MFMA_COUNTERS = ("SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_VALU",
                 "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "GRBM_GUI_ACTIVE")


# a second pass (the profiler takes at most 8 SQ counters per run): LDS read bytes, exponentials, VALU time
LIMIT_COUNTERS = ("SQ_INSTS_LDS_LOAD_BANDWIDTH", "SQ_INSTS_LDS", "SQ_INSTS_VALU_TRANS_F32", "SQ_ACTIVE_INST_VALU")


def summarize_mfma(d, label, kernel, duration_us, command, limits_dir=None, limits_command=""):
    """profiles/<kernel>_<label>_mfma.txt from a rocprofv3 --pmc run of MFMA_COUNTERS (and, if given, a
    second run of LIMIT_COUNTERS on the same workload)."""
    per = {}
    name = None
    for c in MFMA_COUNTERS:
        for n, v in read_counter_csv(d, c).items():
            if kernel in n:
                per.setdefault(c, []).extend(v)
                name = n
    assert name is not None, f"no dispatch of {kernel} in {d}"
    avg = {k: sum(v) / len(v) for k, v in per.items()}
    simds, xcds = 1024, 8
    mfma_cyc = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / simds
    gpu_cyc = avg["GRBM_GUI_ACTIVE"] / xcds
    clock = gpu_cyc / (duration_us * 1e3)
    short = kernel.replace("<", "_").replace(">", "").replace(", ", "_").replace(",", "_").replace(" ", "")
    lines = [f"# MFMA counters, workload {label}, kernel {name}, {len(per['SQ_INSTS_MFMA'])} dispatches, "
             "averages per dispatch",
             "# command (from the repository root; cd /tmp && export TMPDIR=/tmp first):",
             f"#   {command}" if command else "#   (command not given)",
             f"#   python bench.py --summarize-mfma <dir> {label} '{kernel}' {duration_us}"]
    lines += [f"{k}: {avg[k]:.0f}" for k in sorted(avg)]
    lines += ["# SQ_VALU_MFMA_BUSY_CYCLES is 32 x SQ_INSTS_MFMA (32-cycle 32x32x16 bf16 MFMA), summed over 1024 SIMDs",
              f"mfma_busy_cycles_per_simd: {mfma_cyc:.0f}",
              f"# GRBM_GUI_ACTIVE is summed over the 8 XCDs: busy GPU cycles per XCD {gpu_cyc:.0f}",
              f"mfma_busy_fraction_of_gpu_cycles: {mfma_cyc / gpu_cyc:.3f}",
              f"valu_per_mfma: {avg['SQ_INSTS_VALU'] / avg['SQ_INSTS_MFMA']:.2f}",
              f"lds_bank_conflict_fraction: {avg['SQ_LDS_BANK_CONFLICT'] / max(1.0, avg['SQ_LDS_IDX_ACTIVE']):.3f}",
              f"# clock under load: busy cycles per XCD / the kernel's average duration ({duration_us} us, kernel trace)",
              f"clock_GHz: {clock:.2f}",
              f"mfma_busy_fraction_at_2400MHz: {mfma_cyc / (duration_us * 1e3 * 2.4):.3f}"]
    if limits_dir:
        lim = {}
        for c in LIMIT_COUNTERS:
            for n, v in read_counter_csv(limits_dir, c).items():
                if kernel in n:
                    lim.setdefault(c, []).extend(v)
        lav = {k: sum(v) / len(v) for k, v in lim.items()}
        cus = simds // 4
        lds_bytes = lav["SQ_INSTS_LDS_LOAD_BANDWIDTH"] * 64
        lines += ["# second pass (same workload):",
                  f"#   {limits_command}" if limits_command else "#   (command not given)"]
        lines += [f"{k}: {lav[k]:.0f}" for k in sorted(lav)]
        lines += ["# SQ_INSTS_LDS_LOAD_BANDWIDTH counts 64-byte units read from LDS, summed over all SIMDs",
                  f"lds_read_bytes_per_dispatch: {lds_bytes:.0f}",
                  f"lds_read_bytes_per_cu_per_gpu_cycle: {lds_bytes / cus / gpu_cyc:.1f}",
                  f"lds_insts_per_mfma: {lav['SQ_INSTS_LDS'] / avg['SQ_INSTS_MFMA']:.2f}",
                  f"exp_f32_per_mfma: {lav['SQ_INSTS_VALU_TRANS_F32'] / avg['SQ_INSTS_MFMA']:.2f}",
                  "# SQ_ACTIVE_INST_VALU: quad-cycles that waves spend on VALU instructions, summed over waves",
                  f"valu_wave_cycles_per_simd_cycle: {lav['SQ_ACTIVE_INST_VALU'] * 4 / simds / gpu_cyc:.3f}"]
    out = os.path.join(ROOT, "profiles", f"{short}_{label}_mfma.txt")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    print(f"wrote {out}")


def read_traffic(config):
    """Bytes per launch from the committed counter summary, or None if absent or stale."""
    path = traffic_file(config)
    if not os.path.exists(path):
        return None, "no counter summary"
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_digest():
        return None, "kernel sources changed since the counters were taken"
    return float(kv["traffic_bytes_per_launch"]), os.path.relpath(path, ROOT)


class DeviceSet:
    """One copy of a workload's inputs and outputs in device memory."""

    def __init__(self, wl, src=None):
        dev = "cuda"
        if src is None:
            self.t = {k: getattr(wl, k).to(dev) for k in
                      ("q", "k_pages", "v_pages", "block_table", "prefix_len", "k_tree", "v_tree", "parent")}
            self.t["draft"] = wl.draft.to(dev) if wl.draft is not None else None
            self.t["logits"] = wl.logits.to(dev) if wl.logits is not None else None
            self.t["target_ids"] = wl.target_ids.to(dev) if wl.target_ids is not None else None
        else:
            self.t = {k: (None if v is None else v.clone()) for k, v in src.t.items()}
        B, N = wl.B, wl.N
        self.anc = torch.empty((B, N, 4), dtype=torch.uint64, device=dev)
        self.depth = torch.empty((B, N), dtype=torch.int32, device=dev)
        self.bad = torch.empty((B,), dtype=torch.int32, device=dev)
        self.out = torch.empty_like(self.t["q"])
        self.nxt = torch.empty((B, N), dtype=torch.int32, device=dev)
        self.alen = torch.empty((B,), dtype=torch.int32, device=dev)
        self.nodes = torch.empty((B, N), dtype=torch.int32, device=dev)
        self.bonus = torch.empty((B,), dtype=torch.int32, device=dev)

    def nbytes(self):
        return sum(v.numel() * v.element_size() for v in self.t.values() if v is not None)


def attention_work(wl, depth: np.ndarray):
    """Algorithmic bytes and flops of one attention call: prefix K+V read once
    per KV head, plus Q, tree K/V, output, ancestor bitset, block table; flops
    count only the (query, key) pairs the mask keeps."""
    elt = torch.finfo(wl.dtype).bits // 8
    L = wl.prefix_len.numpy().astype(np.int64)
    kv = int(L.sum()) * wl.Hkv * wl.D * 2 * elt
    q = wl.B * wl.N * wl.Hq * wl.D * elt
    tree_kv = 2 * wl.B * wl.N * wl.Hkv * wl.D * elt
    out = q
    anc = wl.B * wl.N * 32
    table = int(((L + 15) // 16).sum()) * 4 + wl.B * 4
    nbytes = kv + q + tree_kv + out + anc + table
    pairs = int((L[:, None] + depth.astype(np.int64)).sum())
    flops = 4 * wl.D * wl.Hq * pairs
    return nbytes, flops


def plan_graph_chunks(K, per):
    """Split K consecutive steps over `per` rotating input sets into graph
    replays: (first step, step count) per replay, in order. Whole passes over
    the sets are one graph each; a remainder (or K below `per`) is one shorter
    graph that starts where the passes left off. The counts add up to K."""
    if K < 0 or per < 1:
        raise ValueError(f"steps {K} and input sets {per}")
    plan = [(i * per, per) for i in range(K // per)]
    if K % per:
        plan.append((K - K % per, K % per))
    return plan


REPS_OVERRIDE = 0   # --profile-reps: every graph replayed this many times instead


def time_graph(fn_list, reps, stream):
    """Capture fn_list (callables) back to back in one graph, replay `reps`
    times between HIP events on `stream`; returns ms per callable."""
    if REPS_OVERRIDE:
        reps = REPS_OVERRIDE
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for f in fn_list:
            f()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / (reps * len(fn_list))


def make_steps(jf, wl, sets, with_accept=True, fused=True):
    """Per-set callables for mask, attention, accept and the whole step. A step is
    the mask, then attention and acceptance: with `fused`, one jf_tree_verify
    call (attention and acceptance in one launch where the plan allows it),
    otherwise jf_tree_attention followed by jf_tree_accept."""
    def mask(s):
        return lambda: jf.build_ancestor_mask(s.t["parent"], anc=s.anc, depth=s.depth, bad_tree=s.bad)

    def attn(s):
        return lambda: jf.tree_attention(s.t["q"], s.t["k_pages"], s.t["v_pages"], s.t["block_table"],
                                         s.t["prefix_len"], s.t["k_tree"], s.t["v_tree"], s.anc,
                                         sm_scale=wl.sm_scale, max_prefix_len=wl.max_prefix_len, out=s.out)

    def accept(s):
        return lambda: jf.tree_accept(s.t["parent"], s.anc, s.t["draft"], logits=s.t["logits"],
                                      target_ids=s.t["target_ids"] if s.t["logits"] is None else None,
                                      next_tokens=s.nxt, accept_len=s.alen, accepted_nodes=s.nodes,
                                      bonus_token=s.bonus)

    def verify(s):
        # the ancestor bitsets are built inside the call and written to s.anc
        return lambda: jf.tree_verify(s.t["q"], s.t["k_pages"], s.t["v_pages"], s.t["block_table"],
                                      s.t["prefix_len"], s.t["k_tree"], s.t["v_tree"], None, s.t["parent"],
                                      s.t["draft"], s.t["logits"], sm_scale=wl.sm_scale,
                                      max_prefix_len=wl.max_prefix_len, out=s.out, next_tokens=s.nxt,
                                      accept_len=s.alen, accepted_nodes=s.nodes, bonus_token=s.bonus,
                                      anc_out=s.anc)

    def step(s):
        m, a = mask(s), attn(s)
        if not with_accept:
            fs = [m, a]
        elif fused and s.t["logits"] is not None:
            fs = [verify(s)]
        else:
            fs = [m, a, accept(s)]

        def run():
            for f in fs:
                f()
        return run

    return ([mask(s) for s in sets], [attn(s) for s in sets], [accept(s) for s in sets],
            [step(s) for s in sets])


def time_commit(jf, stream, name, lens, N, Hkv, D, path_nodes):
    """Average duration of jf_commit_accepted (graph of back-to-back calls) for
    paths of `path_nodes` nodes; the commit rewrites the same slots each time."""
    from tree_causal_attention_jf_amd import workloads as W
    case = W.make_commit_case(0, lens, N=N, Hq=Hkv, Hkv=Hkv, D=D)
    B = len(lens)
    alen = torch.full((B,), path_nodes - 1, dtype=torch.int32, device="cuda")
    nodes = torch.full((B, N), -1, dtype=torch.int32)
    nodes[:, :path_nodes] = torch.arange(path_nodes, dtype=torch.int32)
    nodes = nodes.cuda()
    kt, vt = case.k_tree.cuda(), case.v_tree.cuda()
    kp, vp = case.k_pages.cuda(), case.v_pages.cuda()
    table, plen = case.block_table.cuda(), case.prefix_len.cuda()
    new = torch.empty((B,), dtype=torch.int32, device="cuda")
    fn = lambda: jf.commit_accepted(kt, vt, alen, nodes, table, plen, kp, vp, new_prefix_len=new)
    with torch.cuda.stream(stream):
        fn()
    torch.cuda.synchronize()
    assert new.cpu().tolist() == [L + path_nodes for L in lens]
    t = time_graph([fn] * 20, 50, stream)
    moved = 2 * 2 * B * path_nodes * Hkv * D * kt.element_size()      # K and V, read and written
    return {"workload": name, "us": round(t * 1e3, 3), "bytes": moved,
            "GBps": round(moved / (t * 1e-3) / 1e9, 1), "bound": "latency"}


def time_paged_tree(jf, stream, seed=0):
    """Ragged budgets with the trees' K/V cached after their prefixes: batch 8,
    best-first trees with budgets U{16..256} (N = 256), prefixes U[1024, 4096],
    32q/8kv, d = 128. Returns the JSON entry."""
    from tree_causal_attention_jf_amd import workloads as W
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(1024, 4097, size=8).tolist()
    budgets = rng.integers(16, 257, size=8).tolist()
    case = W.make_paged_tree_case(seed, lens, budgets, N=256, Hq=32, Hkv=8, D=128, tree=("best_first", 4, 12, 2.0))
    t = {k: getattr(case, k).cuda() for k in ("q", "k_pages", "v_pages", "block_table", "prefix_len", "tree_len",
                                               "parent")}
    anc, depth, _ = jf.build_ancestor_mask(t["parent"])
    out = torch.empty_like(t["q"])
    fn = lambda: jf.tree_attention_paged_tree(t["q"], t["k_pages"], t["v_pages"], t["block_table"],
                                              t["prefix_len"], anc, tree_len=t["tree_len"], sm_scale=case.sm_scale,
                                              max_prefix_len=case.max_prefix_len, out=out)
    with torch.cuda.stream(stream):
        fn()
    torch.cuda.synchronize()
    ms = time_graph([fn] * 10, 20, stream)
    # algorithmic work of the real nodes only: prefix keys plus ancestors, per query head
    dep = depth.cpu().numpy().astype(np.int64)
    L = np.asarray(lens, dtype=np.int64)
    pairs = sum(int((L[b] + dep[b, :budgets[b]]).sum()) for b in range(8))
    flops = 4 * 128 * 32 * pairs
    nodes = int(sum(budgets))
    nbytes = int((L.sum() + nodes) * 8 * 128 * 2 * 2 + 2 * nodes * 32 * 128 * 2 + nodes * 32 +
                 ((L + np.asarray(budgets) + 15) // 16).sum() * 4)
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": f"batch 8, best-first trees of budgets {budgets} (N 256), prefixes {lens}, tree K/V "
                        "cached after each prefix, 32q/8kv, d=128",
            "attention_us": round(ms * 1e3, 3), "tree_tokens_per_s": round(nodes / (ms * 1e-3), 1),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "flops": flops,
                         "algorithmic_bytes": nbytes}}


def time_build_tree(jf, stream, seed=0, B=8, N=256, vocab=151936, topk=4, cap=12):
    """Best-first construction of the budget-256 trees from bf16 draft logits
    [8, 256, 151936] (N(0, 2^2)), top-4 children, paths of at most 12 nodes.
    Two logit sets (1.2 GB, beyond the 256 MB Infinity Cache) alternate.
    Returns the JSON entry."""
    from tree_causal_attention_jf_amd import workloads as W
    case = W.make_draft_logits_case(seed, B, N, vocab, topk=topk, max_path_nodes=cap)
    sets = [case.logits.cuda()]
    sets.append(sets[0].roll(1, dims=0).contiguous())
    outs = [(torch.empty((B, N), dtype=torch.int32, device="cuda"), torch.empty((B, N), dtype=torch.int32,
             device="cuda"), torch.empty((B,), dtype=torch.int32, device="cuda")) for _ in sets]

    def call(i):
        return lambda: jf.build_tree(sets[i], topk, cap, parent=outs[i][0], token=outs[i][1], tree_len=outs[i][2],
                                     return_score=False)
    fns = [call(i) for i in range(len(sets))]
    with torch.cuda.stream(stream):
        for f in fns:
            f()
    torch.cuda.synchronize()
    assert outs[0][2].cpu().tolist() == [N] * B
    ms = time_graph(fns * 10, 20, stream)
    # rows 0 .. N-2 are read (the last node to join offers no children)
    nbytes = B * (N - 1) * vocab * sets[0].element_size()
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"batch {B}, budget {N}, bf16 draft logits [{B},{N},{vocab}] N(0,2^2), top-{topk} children, "
                        f"paths of at most {cap} nodes",
            "us": round(ms * 1e3, 3), "trees_per_s": round(B / (ms * 1e-3), 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": nbytes},
            "input_sets": len(sets)}


def _mfma_entry(flops, nbytes, ms):
    tf = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "hbm_GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "flops": flops,
            "algorithmic_bytes": nbytes}


def _hbm_entry(nbytes, ms, flops=None):
    gbs = nbytes / (ms * 1e-3) / 1e9
    e = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": nbytes}
    if flops is not None:
        e["flops"] = flops
    return e


def _attention_only(jf, W, stream, config, desc, cap, reps, bound="mfma", settle=0, **overrides):
    """Average jf_tree_attention duration on a workload (attention only), over
    rotating copies of its inputs; returns the JSON entry."""
    wl = W.make_workload(config, 0, with_accept=False, **overrides)
    b = DeviceSet(wl)
    sets = rotation_sets(wl, b, cap=cap)
    m, a, _, _ = make_steps(jf, wl, sets, with_accept=False)
    with torch.cuda.stream(stream):
        for f in m + a:
            f()
    torch.cuda.synchronize()
    nb, fl = attention_work(wl, b.depth.cpu().numpy())
    fns = a * max(1, 20 // len(a))
    if settle:
        time_graph(fns, settle, stream)                # settle the clock under sustained load
    ms = time_graph(fns, reps, stream)
    e = {"workload": desc, "tree_tokens_per_s": round(wl.B * wl.N / (ms * 1e-3), 1),
         "attention_us": round(ms * 1e3, 3),
         "roofline": _mfma_entry(fl, nb, ms) if bound == "mfma" else _hbm_entry(nb, ms, fl),
         "input_sets": len(sets)}
    del sets, b, m, a
    return e


def sub_budget256(jf, W, stream):
    return _attention_only(jf, W, stream, "c2_bf256_b8",
                           "c2_bf256_b8: batch 8, 256-node best-first trees, prefix U[1024,4096], 32q/8kv, d=128",
                           cap=8, reps=20)


def sub_c3(jf, W, stream):
    e = _attention_only(jf, W, stream, "c3_bf64_b32",
                        "c3_bf64_b32: Qwen3-30B-A3B attention layer, batch 32, 64-node best-first trees, "
                        "prefix U[512,8192], 32q/4kv (GQA group 8), d=128", cap=4, reps=20)
    # nearly balanced between HBM and MFMA: both fractions are reported
    return e


def sub_streaming(jf, W, stream):
    return _attention_only(jf, W, stream, "c1_chain16",
                           "budget 16 at streaming size: batch 8, 16-node chains, prefix 16384 in shuffled 16-token "
                           "pages, 32q/8kv, d=128 (537 MB of K/V per call, twice the Infinity Cache)",
                           cap=1, reps=20, bound="hbm", B=8, prefix=("fixed", 16384))


def sub_draft_head(jf, W, stream):
    return _attention_only(jf, W, stream, "draft_head_b1",
                           "draft_head_b1: the draft layer's tree-causal pass, batch 1, 256-node best-first tree, "
                           "8192-token cache, 32q/8kv, d=128", cap=16, reps=25)


def sub_long_context(jf, W, stream):
    """Long context: batch 4, prefix 32768, 256-node trees; attention and
    acceptance timed apart."""
    wl = W.make_workload("c4_bf256_32k", 0)
    b = DeviceSet(wl)
    sets = rotation_sets(wl, b, cap=2)
    m, a, acc, _ = make_steps(jf, wl, sets)
    with torch.cuda.stream(stream):
        for f in m + a + acc:
            f()
    torch.cuda.synchronize()
    nb, fl = attention_work(wl, b.depth.cpu().numpy())
    time_graph(a, 50, stream)                          # settle the clock under sustained load
    t = time_graph(a, 300, stream)
    tacc = time_graph(acc, 1000, stream)
    lb = wl.logits.numel() * wl.logits.element_size()
    e = {"workload": "c4_bf256_32k: batch 4, prefix 32768, 256-node best-first trees, 32q/8kv, d=128; "
                     "accept over bf16 logits [4,256,151936]",
         "tree_tokens_per_s": round(wl.B * wl.N / (t * 1e-3), 1), "attention_us": round(t * 1e3, 3),
         "attention_roofline": _mfma_entry(fl, nb, t),
         "accept_us": round(tacc * 1e3, 3),
         "accept_roofline": _hbm_entry(lb, tacc),
         "input_sets": len(sets)}
    e["accept_roofline"]["logit_bytes"] = lb
    del sets, b, m, a, acc
    return e


def sub_commit(jf, W, stream):
    return [time_commit(jf, stream, *spec) for spec in (
        ("budget 16: batch 1, 16-node chain fully accepted, 8 KV heads, d=128", [2048], 16, 8, 128, 16),
        ("budget 256: batch 4, 256-node trees, 12-node accepted paths, 8 KV heads, d=128", [1000] * 4, 256, 8,
         128, 12))]


# the measured workloads beside the headline step, in the order they run; each
# can be run alone (--only NAME) so that a profiler run covers one workload
SUBS = {
    "budget256": sub_budget256,
    "c3_budget64": sub_c3,
    "budget16_streaming": sub_streaming,
    "draft_head_pass": sub_draft_head,
    "long_context": sub_long_context,
    "ragged_budgets": lambda jf, W, stream: time_paged_tree(jf, stream),
    "build_tree": lambda jf, W, stream: time_build_tree(jf, stream),
    "commit": sub_commit,
}


def selected(args, name):
    return args.only is None or name in args.only.split(",")


def rotation_sets(wl, base, budget_bytes=2 * MALL_BYTES, cap=64):
    n = max(1, min(cap, math.ceil(budget_bytes / max(1, base.nbytes()))))
    return [base] + [DeviceSet(wl, src=base) for _ in range(n - 1)]


def cpu_baseline(wl, seconds, threads_limit=None):
    """The oracle on full steps of the workload for about `seconds`; with
    threads_limit, its BLAS pools are held to that many threads."""
    import contextlib

    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    with (threadpool_limits(threads_limit) if threads_limit else contextlib.nullcontext()):
        return _cpu_baseline(oracle, wl, seconds, threadpool_info)


def _cpu_baseline(oracle, wl, seconds, threadpool_info):
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    steps = 0
    t0 = time.perf_counter()
    while True:
        oracle.build_ancestor_mask(wl.parent)
        oracle.tree_attention(wl.q, wl.k_pages, wl.v_pages, wl.block_table, wl.prefix_len, wl.k_tree, wl.v_tree,
                              wl.parent, wl.sm_scale)
        nxt = oracle.target_choice(wl.logits)
        oracle.tree_accept(wl.parent, wl.draft, nxt)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": wl.B * wl.N * steps / el, "unit": "tree-tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{steps} full steps (mask + fp64 attention with dense mask + argmax over "
                      f"{wl.B}x{wl.N}x{wl.vocab} logits + walk) of the same workload, {el:.1f} s, "
                      f"{len(os.sched_getaffinity(0))} host cores visible"}


def run_step(args, jf, W, stream):
    """The headline: K timed steps of the budget-16 workload, per-kernel
    durations and the dominant kernel's roofline. Returns (JSON entries, workload)."""
    log(f"[bench] building workload {args.config}")
    wl = W.make_workload(args.config, 0)
    base = DeviceSet(wl)
    sets = rotation_sets(wl, base)
    log(f"[bench] {len(sets)} input sets x {base.nbytes() / 1e6:.1f} MB")
    masks, attns, accepts, steps = make_steps(jf, wl, sets, fused=not args.separate)
    # the other form of the step, measured beside the timed one
    other_steps = make_steps(jf, wl, sets, fused=args.separate)[3]

    with torch.cuda.stream(stream):
        for i in range(max(1, args.warmup)):
            steps[i % len(sets)]()
    torch.cuda.synchronize()

    if args.profile_steps:
        # counter calibration: a plain copy that reads and writes COPY_BYTES
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        # second calibration: acceptance over [4, 256, 151936] bf16 logits, which reads
        # every logit once (plus a few KB of tree data and chunk keys)
        cal_logits = torch.randn((4, 256, 151936), device="cuda").to(torch.bfloat16)
        cal_parent = torch.arange(-1, 255, dtype=torch.int32, device="cuda").repeat(4, 1).contiguous()
        cal_draft = torch.zeros((4, 256), dtype=torch.int32, device="cuda")
        cal_anc, _, _ = jf.build_ancestor_mask(cal_parent)
        for _ in range(3):
            jf.tree_accept(cal_parent, cal_anc, cal_draft, logits=cal_logits)
        torch.cuda.synchronize()
        del cal_logits
        with torch.cuda.stream(stream):
            for i in range(args.profile_steps):
                steps[i % len(sets)]()
        torch.cuda.synchronize()
        log("[bench] profile run done")
        return None, None

    depth = base.depth.cpu().numpy()
    nbytes, flops = attention_work(wl, depth)

    # ---- timed region: exactly K steps. Each step is mask -> attention -> accept on
    # its own input set; graphs hold up to len(sets) consecutive steps captured from
    # one stream (every kernel still waits for the one before), so the host submits
    # one graph per pass over the input sets instead of one per step.
    K = args.steps
    per = len(sets)
    if K < 1:
        raise SystemExit("--steps must be at least 1")

    def capture(first, count, fns=steps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(first, first + count):
                fns[i % len(sets)]()
        return g

    graphs = {}
    if args.eager:
        chunks = [(lambda i=i: steps[i % len(sets)](), 1) for i in range(K)]
    else:
        plan = plan_graph_chunks(K, per)
        for first, count in plan:
            if (first % per, count) not in graphs:
                graphs[(first % per, count)] = capture(first, count)
        chunks = [(graphs[(first % per, count)].replay, count) for first, count in plan]
        for g in graphs.values():
            g.replay()
        torch.cuda.synchronize()
    assert sum(n for _, n in chunks) == K
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for fn, _ in chunks:
            fn()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K
    value = wl.B * wl.N / (ms_step * 1e-3)
    log(f"[bench] {K} steps: {ms_step * 1e3:.2f} us/step, {value / 1e6:.3f} M tree-tokens/s")
    # the same steps submitted one graph per step (host launch cost included)
    ms_step_single = None
    if not args.eager:
        singles = [capture(i, 1) for i in range(per)]
        for g in singles:
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            for i in range(K):
                singles[i % per].replay()
        torch.cuda.synchronize()
        ms_step_single = (time.perf_counter() - t0) * 1e3 / K
        del singles
    # the same steps in the other form (separate attention and acceptance launches,
    # or the one verification call)
    ms_step_other = None
    if not args.eager:
        g = capture(0, per, other_steps)
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            for _ in range(max(1, K // per)):
                g.replay()
        torch.cuda.synchronize()
        ms_step_other = (time.perf_counter() - t0) * 1e3 / (max(1, K // per) * per)
        del g
    chunks = graphs = None

    # ---- per-kernel durations (graph of back-to-back launches, HIP events on the launch stream)
    reps = max(4, 2000 // len(sets))
    t_mask = time_graph(masks, reps, stream)
    t_attn = time_graph(attns, reps, stream)
    t_acc = time_graph(accepts, reps, stream)
    verifies = [(lambda s=s: jf.tree_verify(s.t["q"], s.t["k_pages"], s.t["v_pages"], s.t["block_table"],
                                            s.t["prefix_len"], s.t["k_tree"], s.t["v_tree"], None, s.t["parent"],
                                            s.t["draft"], s.t["logits"], sm_scale=wl.sm_scale,
                                            max_prefix_len=wl.max_prefix_len, out=s.out, next_tokens=s.nxt,
                                            accept_len=s.alen, accepted_nodes=s.nodes, bonus_token=s.bonus,
                                            anc_out=s.anc))
                for s in sets] if wl.logits is not None else None
    t_ver = time_graph(verifies, reps, stream) if verifies else None
    log(f"[bench] per launch: mask {t_mask * 1e3:.2f} us, attention {t_attn * 1e3:.2f} us, "
        f"accept {t_acc * 1e3:.2f} us, verify (attention + accept) {t_ver * 1e3 if t_ver else 0:.2f} us")
    logit_bytes = wl.logits.numel() * wl.logits.element_size() if wl.logits is not None else 0
    # dominant kernel of the step: the verification launch (attention + acceptance).
    # Its algorithmic bytes: the attention's, plus the logits read once and the
    # acceptance outputs (next tokens, accepted nodes, length, bonus)
    ver_bytes = nbytes + logit_bytes + wl.B * wl.N * 8 + wl.B * 8
    t_dom = t_ver if t_ver else t_attn
    dom_bytes = ver_bytes if t_ver else nbytes
    achieved = dom_bytes / (t_dom * 1e-3) / 1e9
    traffic, traffic_src = read_traffic(args.config)
    rl = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
          "frac": round(achieved / HBM_PEAK_GBS, 4),
          "traffic": None if traffic is None else round(traffic / (t_dom * 1e-3) / 1e9, 1),
          "traffic_bytes_per_launch": None if traffic is None else int(traffic),
          "traffic_source": traffic_src,
          "kernel": STEP_KERNEL if t_ver else ATTN_KERNEL, "algorithmic_bytes": dom_bytes,
          "avg_launch_us": round(t_dom * 1e3, 3),
          "attention_alone": {"kernel": ATTN_KERNEL, "avg_launch_us": round(t_attn * 1e3, 3),
                              "algorithmic_bytes": nbytes, "flops": flops,
                              "achieved_GBps": round(nbytes / (t_attn * 1e-3) / 1e9, 1),
                              "frac": round(nbytes / (t_attn * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}
    result = {
        "metric": "tree-attention tree-tokens/s + % HBM/MFMA roofline at budget 16 and 256",
        "value": round(value, 1),
        "unit": "tree-tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "ms_per_step_one_graph_per_step": round(ms_step_single, 6) if ms_step_single else None,
        ("ms_per_step_verify_call" if args.separate else "ms_per_step_separate_launches"):
            round(ms_step_other, 6) if ms_step_other else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.config}: Qwen3-8B attention layer, batch {wl.B}, {wl.N}-node chain, "
                               f"prefix {wl.max_prefix_len} in shuffled 16-token pages, {wl.Hq}q/{wl.Hkv}kv, "
                               f"d={wl.D}; step = ancestor bitsets + attention + accept over {wl.vocab}-way bf16 logits"
                               + (" (separate launches)" if args.separate else
                                  " (jf_tree_verify: bitsets, attention and acceptance in one launch)"),
                   "graph_replay": not args.eager, "steps_per_graph": 1 if args.eager else per,
                   "input_sets": len(sets)},
        "roofline": rl,
        "kernels_us": {"build_ancestor_mask": round(t_mask * 1e3, 3), "tree_attention": round(t_attn * 1e3, 3),
                       "tree_accept": round(t_acc * 1e3, 3),
                       "tree_verify": round(t_ver * 1e3, 3) if t_ver else None,
                       "accept_GBps": round(logit_bytes / (t_acc * 1e-3) / 1e9, 1) if logit_bytes else None},
    }
    return result, wl


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.config)
        return
    if args.summarize_stats:
        summarize_stats(args.summarize_stats[0], args.summarize_stats[1], args.command)
        return
    if args.summarize_mfma:
        d, label, kernel, dur = args.summarize_mfma
        summarize_mfma(d, label, kernel, float(dur), args.command, args.limits, args.limits_command)
        return
    global REPS_OVERRIDE
    REPS_OVERRIDE = args.profile_reps
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    if "RANK" in os.environ and int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only; launched with WORLD_SIZE > 1", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    from tree_causal_attention_jf_amd import binding as jf
    from tree_causal_attention_jf_amd import workloads as W

    stream = torch.cuda.Stream()
    result, wl = {}, None
    if selected(args, "step"):
        result, wl = run_step(args, jf, W, stream)
        if result is None:
            return
    for name in SUBS:
        if selected(args, name):
            log(f"[bench] {name}")
            result[name] = SUBS[name](jf, W, stream)
            log(f"[bench] {name}: {json.dumps(result[name])[:240]}")

    if not args.no_cpu_baseline and wl is not None:
        log("[bench] timing the CPU oracle")
        # the oracle's NumPy calls are small (one (sequence, head) at a time), so its BLAS
        # pools can lose to a single thread; both are timed and the faster is the baseline
        runs = [cpu_baseline(wl, args.cpu_seconds / 2), cpu_baseline(wl, args.cpu_seconds / 2, threads_limit=1)]
        runs.sort(key=lambda r: -r["value"])
        result["cpu_baseline"] = runs[0]
        result["cpu_baseline_other_threads"] = runs[1]
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
