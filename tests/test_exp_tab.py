"""The tree-construction kernel's fp64 table exponentials (csrc/exp_tab.h),
compiled for the CPU from the same source and measured against the C
library's exp over the kernel's whole input range (tests/c_abi/exp_tab_check.cpp)."""

import os
import re
import subprocess

from conftest import ROOT

SRC = os.path.join(ROOT, "tests", "c_abi", "exp_tab_check.cpp")
CSRC = os.path.join(ROOT, "tree_causal_attention_jf_amd", "csrc")


def test_table_exps_against_the_c_library(tmp_path):
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    exe = str(tmp_path / "exp_tab_check")
    r = subprocess.run([hipcc, "-O2", "-std=c++17", "-x", "hip", "--offload-arch=gfx950", "-I" + CSRC, SRC, "-o", exe],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300)
    assert r.returncode == 0, r.stdout
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300)
    assert r.returncode == 0, r.stdout
    m = re.search(r"points (\d+) max_ulp ([\d.]+) at x=\S+ max_subnormal_steps ([\d.]+) special_bad (\d+) "
                  r"nonpos_rel_near (\S+) nonpos_rel_far (\S+)", r.stdout)
    assert m, r.stdout
    points, max_ulp, max_sub = int(m.group(1)), float(m.group(2)), float(m.group(3))
    assert int(m.group(4)) == 0, r.stdout
    # exp_tab_nonpos: the minimax polynomial (2.4e-14) plus the one-constant reduction
    assert float(m.group(5)) <= 4e-14, r.stdout
    assert float(m.group(6)) <= 1e-13, r.stdout
    print(r.stdout.strip())
    assert points > 16_000_000
    assert max_ulp <= 1.0, r.stdout
    assert max_sub <= 1.0, r.stdout
