"""Host logic of bench.py that needs no GPU: the counter summary (traffic from
FETCH_SIZE / WRITE_SIZE, scaled by what a plain copy of known size reads), its
staleness check against the kernel sources, and the refusal of more than one GPU."""

import csv
import os
import subprocess
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402

VERIFY = "void jf::tree_verify_bf16_kernel<128, 1, 4, 1>(jf::AttnArgs, jf::AcceptArgs, unsigned int)"


def _write_counters(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_summary_scales_counters_by_the_copy_and_detects_stale_sources(tmp_path, monkeypatch):
    copy_kib = bench.COPY_BYTES / 1024
    # the copy's read shows as half its size (factor 2), its write in full (factor 1)
    _write_counters(tmp_path / "F", "FETCH_SIZE", [("__amd_rocclr_copyBuffer", copy_kib / 2),
                                                    (VERIFY, 100.0), (VERIFY, 300.0)])
    _write_counters(tmp_path / "W", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", copy_kib),
                                                    (VERIFY, 10.0), (VERIFY, 30.0)])
    out = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "traffic_file", lambda config: str(out))
    bench.summarize_pmc(str(tmp_path / "F"), str(tmp_path / "W"), "c1_chain16")
    traffic, src = bench.read_traffic("c1_chain16")
    # average fetch 200 KiB x 2 + average write 20 KiB x 1
    assert traffic == pytest.approx((200 * 2 + 20) * 1024, rel=1e-6)
    assert src == os.path.relpath(str(out), ROOT)
    # a change to the kernel's sources makes the summary stale
    monkeypatch.setattr(bench, "source_digest", lambda: "0" * 64)
    assert bench.read_traffic("c1_chain16") == (None, "kernel sources changed since the counters were taken")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], stdout=subprocess.PIPE,
                       stderr=subprocess.PIPE, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("K,per", [(20, 40), (40, 40), (95, 40), (0, 40), (1, 1), (7, 3)])
def test_graph_chunks_cover_exactly_k_steps_in_order(K, per):
    plan = bench.plan_graph_chunks(K, per)
    # consecutive, in order, exactly K steps
    first = 0
    for start, count in plan:
        assert start == first and 1 <= count <= per
        first += count
    assert first == K
    # whole passes start on set 0; at most one shorter replay, and it comes last
    assert all(count == per and start % per == 0 for start, count in plan[:-1])
    assert sum(1 for _, count in plan if count < per) == (1 if K % per else 0)


def test_fewer_steps_than_input_sets_is_one_short_graph():
    assert bench.plan_graph_chunks(20, 40) == [(0, 20)]
    assert bench.plan_graph_chunks(40, 40) == [(0, 40)]
    assert bench.plan_graph_chunks(95, 40) == [(0, 40), (40, 40), (80, 15)]


def test_acceptance_calibration_is_reported_beside_the_copy(tmp_path, monkeypatch, capsys):
    copy_kib = bench.COPY_BYTES / 1024
    logit_kib = 4 * 256 * 151936 * 2 / 1024
    _write_counters(tmp_path / "F", "FETCH_SIZE", [("__amd_rocclr_copyBuffer", copy_kib / 2),
                                                    # a bigger elementwise kernel must not be taken for the copy
                                                    ("void at::native::vectorized_elementwise_kernel<4>", 4 * copy_kib),
                                                    ("void jf::accept_logits_kernel<unsigned short, 2>(jf::AcceptArgs)",
                                                     logit_kib / 2),
                                                    (VERIFY, 100.0)])
    _write_counters(tmp_path / "W", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", copy_kib), (VERIFY, 10.0)])
    monkeypatch.setattr(bench, "traffic_file", lambda config: str(tmp_path / "traffic.txt"))
    bench.summarize_pmc(str(tmp_path / "F"), str(tmp_path / "W"), "c1_chain16")
    text = (tmp_path / "traffic.txt").read_text()
    assert "fetch_factor: 2.000000" in text
    assert "factor 2.0000" in text                      # acceptance: logits read once show at half
    assert bench.read_traffic("c1_chain16")[0] == pytest.approx((100 * 2 + 10) * 1024, rel=1e-6)


def test_stats_and_mfma_summaries(tmp_path, monkeypatch):
    d = tmp_path / "kt"
    d.mkdir()
    with open(d / "run_kernel_stats.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs",
                                           "Percentage"])
        w.writeheader()
        w.writerow(dict(Name=VERIFY, Calls=10, TotalDurationNs=155000, AverageNs=15500, MinNs=15000, MaxNs=16000,
                        Percentage=90.0))
        w.writerow(dict(Name="jf::ancestor_mask_kernel", Calls=10, TotalDurationNs=30000, AverageNs=3000,
                        MinNs=2900, MaxNs=3100, Percentage=10.0))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    bench.summarize_stats(str(d), "step", "rocprofv3 ... -- python3 bench.py --only step")
    text = (tmp_path / "profiles" / "kernel_stats_step.txt").read_text()
    lines = [l for l in text.splitlines() if not l.startswith("#")]
    assert lines[0].startswith(VERIFY) and "| 15.50 |" in lines[0]           # largest total first
    assert "--only step" in text
    # MFMA: 32 busy cycles per MFMA over 1024 SIMDs; GRBM over 8 XCDs
    rows = [("tree_attn_bf16_kernel<128, 8, 1, 1>", {"SQ_INSTS_MFMA": 1024 * 1000, "SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 32000,
                                                     "SQ_BUSY_CYCLES": 1, "SQ_INSTS_VALU": 6 * 1024 * 1000,
                                                     "SQ_LDS_BANK_CONFLICT": 0, "SQ_LDS_IDX_ACTIVE": 5,
                                                     "GRBM_GUI_ACTIVE": 8 * 64000})]
    m = tmp_path / "mfma"
    m.mkdir()
    with open(m / "run_counter_collection.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, cs in rows:
            for c, v in cs.items():
                w.writerow({"Kernel_Name": name, "Counter_Name": c, "Counter_Value": v})
    bench.summarize_mfma(str(m), "budget256", "tree_attn_bf16_kernel<128, 8, 1, 1>", 26.6667, "cmd")
    text = (tmp_path / "profiles" / "tree_attn_bf16_kernel_128_8_1_1_budget256_mfma.txt").read_text()
    assert "mfma_busy_fraction_of_gpu_cycles: 0.500" in text
    assert "valu_per_mfma: 6.00" in text
    assert "clock_GHz: 2.40" in text
