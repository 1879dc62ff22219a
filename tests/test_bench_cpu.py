"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the roofline bound,
the read-ceiling fraction, the source hash that gates committed counters, and the
algorithmic counts on a workload small enough to count by hand."""
import json
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workloads as wl  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_roofline_bound_picks_the_larger_floor():
    # decode-like: 9.13 GFLOP over 604 MB -> the HBM floor (75.6 us) beats the fp32 floor (58 us)
    r = bench.roofline_bound(False, 9.127e9, 604.6e6, 0.110, bench.PEAK_TFLOPS["f32-mfma"])
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["achieved"] - 604.6e6 / 110e-6 / 1e9) < 0.1
    # c4-like: compute-bound on the matrix cores
    r = bench.roofline_bound(False, 1.168e12, 677.7e6, 8.53, bench.PEAK_TFLOPS["f32-mfma"])
    assert r["bound"] == "mfma" and abs(r["frac"] - 1.168e12 / 8.53e-3 / 1e12 / 157.3) < 1e-4
    # the vector path reports "alu"
    assert bench.roofline_bound(True, 1.0e9, 1.0e6, 1.0, bench.PEAK_TFLOPS["f32-valu"])["bound"] == "alu"


def test_read_ceiling_fraction_only_for_memory_bound_lines():
    hbm = {"bound": "hbm", "achieved": 5000.0}
    out = bench.with_ceiling(hbm, {"gbps": 6000.0})
    assert out["read_ceiling_gbps"] == 6000.0 and abs(out["frac_of_read_ceiling"] - 5000 / 6000) < 1e-4
    assert "frac_of_read_ceiling" not in hbm                     # the input is not modified
    assert "frac_of_read_ceiling" not in bench.with_ceiling(hbm, {"gbps": 0.0})
    assert "frac_of_read_ceiling" not in bench.with_ceiling(hbm, None)
    assert "frac_of_read_ceiling" not in bench.with_ceiling({"bound": "mfma", "achieved": 1.0}, {"gbps": 6000.0})


def test_source_hash_ignores_comments_and_blank_lines(tmp_path, monkeypatch):
    csrc = tmp_path / "tree_masked_mla_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in bench.KERNEL_SOURCES["attn_mfma_kernel"]:
        shutil.copy(os.path.join(ROOT, "tree_masked_mla_amd", "csrc", f), csrc / f)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash("attn_mfma_kernel")
    src = csrc / "attn_mfma.hip"
    text = src.read_text()
    src.write_text("// a new comment\n\n/* and a block\n   comment */\n" + text.replace("\n", "\n\n", 3) + "\n// tail\n")
    assert bench.kernel_source_hash("attn_mfma_kernel") == h0
    src.write_text(text.replace("constexpr int kRows = 64;", "constexpr int kRows = 64 ;"))
    assert bench.kernel_source_hash("attn_mfma_kernel") != h0


def test_committed_counters_are_gated_by_the_source_hash():
    for name in ("c4", "c3", "c4_q_len_1", "c5"):
        with open(os.path.join(ROOT, "profiles", f"counters_attn_{name}.json")) as f:
            h = json.load(f)["kernel_source_hash"]
        ctr = bench.load_counters(name, h)
        assert 0.0 < ctr["mfma_busy_per_simd"] < 1.0
        assert 1.0 <= ctr["executed_over_algorithmic_flops"] < 1.05
        assert bench.load_traffic(name, h) > 0
        assert bench.load_counters(name, "0" * 16) is None and bench.load_traffic(name, "0" * 16) is None


def test_algorithmic_counts_by_hand():
    w = wl.config("c1")                      # B=1, H=8, no prefix, 9-node tree
    nbytes, flops, pairs = bench.algorithmic(w)
    depth = wl.tree_depths(w.parent[0])
    assert pairs == w.H * int((depth + 1).sum())          # a node sees its ancestors and itself
    assert flops == pairs * 2 * (576 + 512)
    rows = w.B * w.Q * w.H
    W = (w.Q + 31) // 32
    assert nbytes == (rows * 576 * 4 + w.total_kv * 576 * 4 + rows * 512 * 4 + rows * 4
                      + w.B * w.Q * 4 + w.B * w.Q * W * 4 + w.B * 4)
    # a chain of Q nodes sees 1 + 2 + ... + Q positions per head
    c = wl.c2_chain()
    _, _, pairs_c = bench.algorithmic(c)
    Q = c.Q
    assert pairs_c == c.H * sum(int(p) * Q + Q * (Q + 1) // 2 for p in c.prefix)
