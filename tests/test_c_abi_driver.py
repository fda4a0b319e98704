"""A C++ program that drives one verification step through the C ABI alone
(tests/c_abi/verify_step.cpp: hipMalloc'd buffers, no Python on the path):
it compiles and links against libjf_tree.so on the CPU, and on the GPU the one
jf_tree_verify launch (bitsets built in the call) agrees bit for bit with
jf_build_ancestor_mask + jf_tree_attention + jf_tree_accept."""

import os
import subprocess

import pytest

from conftest import ROOT

SRC = os.path.join(ROOT, "tests", "c_abi", "verify_step.cpp")
LIBDIR = os.path.join(ROOT, "tree_causal_attention_jf_amd")


def _compile(out):
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    cmd = [hipcc, "-O2", "-std=c++17", "-I" + os.path.join(ROOT, "include"), SRC, "-o", out, "-L" + LIBDIR,
           "-ljf_tree", "-Wl,-rpath," + LIBDIR]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300)
    assert r.returncode == 0, r.stdout
    return out


def test_driver_compiles_and_links(tmp_path):
    exe = _compile(str(tmp_path / "verify_step"))
    assert os.access(exe, os.X_OK)


@pytest.mark.gpu
def test_driver_one_launch_equals_three_calls(tmp_path):
    exe = _compile(str(tmp_path / "verify_step"))
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout
    assert r.stdout.strip().endswith("ok")
