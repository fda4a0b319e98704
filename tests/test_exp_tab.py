"""The tree-construction kernel's fp64 table exponential (csrc/exp_tab.h,
exp_tab_nonpos), compiled for the CPU from the same source and measured against
the C library's exp over its whole input range x <= 0, with its special inputs
(tests/c_abi/exp_tab_check.cpp)."""

import os
import re
import subprocess

from conftest import ROOT

SRC = os.path.join(ROOT, "tests", "c_abi", "exp_tab_check.cpp")
CSRC = os.path.join(ROOT, "tree_causal_attention_jf_amd", "csrc")


def test_table_exp_against_the_c_library(tmp_path):
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    exe = str(tmp_path / "exp_tab_check")
    r = subprocess.run([hipcc, "-O2", "-std=c++17", "-x", "hip", "--offload-arch=gfx950", "-I" + CSRC, SRC, "-o", exe],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300)
    assert r.returncode == 0, r.stdout
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300)
    assert r.returncode == 0, r.stdout
    m = re.search(r"points (\d+) rel_near (\S+) rel_far (\S+) below_bad (\d+) special_bad (\d+)", r.stdout)
    assert m, r.stdout
    print(r.stdout.strip())
    assert int(m.group(1)) > 12_000_000
    # the minimax polynomial (2.4e-14) plus the one-constant reduction (3.2e-15 at |x| <= 40)
    assert float(m.group(2)) <= 4e-14, r.stdout
    assert float(m.group(3)) <= 1e-13, r.stdout
    assert int(m.group(4)) == 0 and int(m.group(5)) == 0, r.stdout
