"""FP8 E4M3 caches on the GPU against the oracle.

The kernels widen each FP8 byte exactly to float32 and compute as for a float32
cache, so the bar is the float32 one: |gpu - oracle| <= 1e-4 + 1e-4 |oracle|,
with the oracle reading the same bytes exactly (its FP8 decoding is pinned
against torch's float8_e4m3fn on every code).  Covered: the small workloads on
every path, c4- and c5-shaped reduced workloads with ragged prefixes and forced
splits, the exact single-position case, and the c4 trees at full size (the
benchmark's FP8 launch) on sampled rows.  Workgroup-order invariance on FP8
caches is part of test_attn_gpu.py."""
import numpy as np
import pytest

import oracle
import workloads as wl
from parity import assert_close, assert_lse_close, oracle_rows, say
from test_attn_gpu import check_full, run

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("name", ["c1", "c2"])
@pytest.mark.parametrize("path", [0, 1, 2, 3])
def test_small_workloads_fp8(name, path):
    w = wl.config(name, kv_dtype=wl.FP8)
    r, _, _ = check_full(w, path=path, what=f"{name}-fp8")
    if path in (0, 2, 3) and w.Q * w.H >= 16:
        assert r.plan()[1] == 2          # the fp32 matrix-core kernel, widened


def test_dense_reduced_fp8():
    """c4's shape (H=16, q_len=128, best-first trees) with short ragged prefixes,
    one split and forced splits of 256 positions (the merge)."""
    w = wl.make_workload("c4-small-fp8", 2104, B=3, H=16, Q=128, prefix=[300, 1000, 0], tree="best_first",
                         depth_cap=12, kv_dtype=wl.FP8)
    check_full(w)
    check_full(w, split_len=256, what="c4-small-fp8 split256")


@pytest.mark.parametrize("path", [0, 1])
def test_c5_shaped_fp8(path):
    w = wl.make_workload("c5-small-fp8", 2105, B=3, H=64, Q=64, prefix=[0, 77, 700], tree="uniform",
                         kv_dtype=wl.FP8)
    check_full(w, path=path)


@pytest.mark.parametrize("path", [1, 2])
def test_single_visible_position_is_exact_fp8(path):
    """No prefix: the root sees only itself, so it returns its widened FP8 row bit for bit."""
    w = wl.make_workload("c1-fp8", 1001, B=1, H=8, Q=9, prefix=0, tree="uniform", kv_dtype=wl.FP8)
    r, out, lse = run(w, path=path)
    row0 = wl.fp8_bits_to_f32(w.ckv[0])
    for h in range(w.H):
        assert np.array_equal(out[h], row0), h


def test_c4_trees_fp8_full_size_sampled():
    """The c4 trees and prefixes with an FP8 cache (the benchmark's FP8 call)."""
    say("generate c4-fp8")
    w = wl.config("c4", kv_dtype=wl.FP8)
    bits, _, _ = oracle.build_visibility(w.parent)
    r, out, lse = run(w)
    say(f"  plan {r.plan()}")
    assert np.array_equal(r.bits(), bits)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    rows = wl.sample_rows(w, 48)
    ref, rlse = oracle_rows(w, bits, rows, chunk=4)
    e = assert_close(out[rows], ref, wl.FP8, "c4-fp8")
    assert_lse_close(lse[rows], rlse, wl.FP8, "c4-fp8")
    say(f"  c4-fp8: max abs err {e:.2e} on {len(rows)} sampled rows")
