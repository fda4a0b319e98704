"""Build libjf_tree.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m tree_causal_attention_jf_amd.build
"""

from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libjf_tree.so")
SOURCES = ["api.hip", "mask.hip", "accept.hip", "attn_bf16.hip", "attn_f32.hip", "commit.hip", "tree_build.hip"]
ARCH = "gfx950"

# Packed-fp32 instructions stay off: the compiler must not form v_pk_{add,mul,fma}_f32.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


# Kernels whose loops count their own vector-memory operations (s_waitcnt vmcnt
# with hand-computed limits): a register spill would add scratch loads to that
# count and let a wait return early, so such a kernel must use no scratch.
NO_SCRATCH_KERNELS = ("tree_attn_bf16_kernel", "tree_verify_bf16_kernel")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the gfx feature name: drop that one harmless line
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)
    return out


def check_no_scratch(remarks: str) -> None:
    """Raise if a kernel in NO_SCRATCH_KERNELS reports scratch (from the compiler's
    kernel-resource-usage remarks)."""
    fn = None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            fn = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and fn and any(k in fn for k in NO_SCRATCH_KERNELS) and int(m.group(1)) > 0:
            raise RuntimeError(f"{fn} uses {m.group(1)} bytes of scratch per lane (register spills)")


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every HIP source and link libjf_tree.so next to this file."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = _hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        extra = ["-Rpass-analysis=kernel-resource-usage"] if src == "attn_bf16.hip" else []
        cmds.append([hipcc, *HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(cmds)))) as ex:
        outs = list(ex.map(lambda c: _run(c, verbose and "-Rpass-analysis" not in " ".join(c)), cmds))
    for out in outs:
        check_no_scratch(out)
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
