"""S2..S7 on the GPU against the CPU oracle, element by element.

Bar (tests/parity.py), by the arithmetic that produced the output: fp32
arithmetic (every cache type widened exactly) within 1e-4 + 1e-4 |oracle| on
every element and on lse; the bf16 matrix-core kernel within 2e-2 relative L2
on every query row, every element within 2e-2 of its row's rms plus 2e-2
|oracle|, lse within 2e-2.
Small and reduced workloads are compared in full; the full-size dense workloads
run in the launch configuration the benchmark times and are compared on a
seeded sample of rows (plus properties that hold for every row).
"""
import functools

import numpy as np
import pytest

import oracle
import workloads as wl
from parity import BF16, F32, arithmetic, assert_close, assert_lse_close, oracle_rows, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def run(w, path=0, split_len=0, bits_override=None, parent=None, wg_order=0):
    from tree_masked_mla_amd.runner import DeviceRun
    r = DeviceRun(w, path=path, split_len=split_len, bits_override=bits_override, parent=parent,
                  wg_order=wg_order)
    r.step()
    out, lse = r.results()
    return r, out, lse


def check_full(w, path=0, split_len=0, what=None, wg_order=0):
    what = what or w.name
    say(f"attn {what} path={path} split={split_len} order={wg_order}")
    bits, _, _ = oracle.build_visibility(w.parent)
    r, out, lse = run(w, path, split_len, wg_order=wg_order)
    assert np.array_equal(r.bits(), bits)
    ref, rlse = oracle_rows(w, bits)
    ar = arithmetic(w.kv_dtype, r.plan()[1])
    e = assert_close(out, ref, ar, what)
    assert_lse_close(lse, rlse, ar, what)
    say(f"  {what}: plan={r.plan()} max abs err {e:.2e}")
    return r, out, lse


# ----------------------------------------------------------------------------- the small workloads
@pytest.mark.parametrize("name", ["c1", "c2"])
@pytest.mark.parametrize("path", [0, 1, 2])
def test_small_configs(name, path):
    check_full(wl.config(name), path=path)


@pytest.mark.parametrize("path", [0, 1, 2])
def test_c2_chain_is_causal(path):
    """The chain variant must equal causal attention; the oracle's equality with
    causal SDPA is pinned on the CPU, so parity with the oracle carries it."""
    check_full(wl.c2_chain(), path=path)


def test_c3_full():
    """c3 in the benchmark's plan: 16 splits of 272 rows (8.5 tiles each, the last
    one a half tile) on 256 workgroups; every row against the oracle."""
    r, _, _ = check_full(wl.config("c3"))
    assert r.plan()[2] % 32 == 16, r.plan()


# ----------------------------------------------------------------------------- reduced dense shapes
def test_dense_reduced_f32():
    """c4's shape (H=16, q_len=128, best-first trees) with short ragged prefixes:
    several KV tiles, a tree tail that straddles tiles, a ragged last tile."""
    w = wl.make_workload("c4-small", 2004, B=3, H=16, Q=128, prefix=[300, 1000, 0], tree="best_first",
                         depth_cap=12)
    check_full(w)
    check_full(w, split_len=256, what="c4-small split256")


@pytest.mark.parametrize("path", [0, 1, 3])
def test_dense_reduced_bf16(path):
    """c5's shape (H=64, q_len=64, uniform trees, bf16 cache) with short ragged prefixes,
    on the bf16 matrix cores (auto), the VALU path and the fp32-MFMA path."""
    w = wl.make_workload("c5-small", 2005, B=3, H=64, Q=64, prefix=[0, 77, 700], tree="uniform",
                         kv_dtype=wl.BF16)
    r, out, lse = check_full(w, path=path)
    # the VALU and fp32-MFMA paths widen the bf16 cache exactly: check_full held them
    # to the fp32 bar; auto takes the bf16 matrix cores
    assert (r.plan()[1] == 2) == (path == 0)


def test_bf16_mfma_split_and_ragged():
    w = wl.make_workload("c5-split", 2006, B=2, H=64, Q=64, prefix=[1500, 333], tree="uniform",
                         kv_dtype=wl.BF16)
    check_full(w, split_len=256, what="bf16 split256")


@pytest.mark.parametrize("split_len", [32, 64, 96])
def test_bf16_mfma_short_splits(split_len):
    """Splits of one, two and three 32-position tiles: the bf16 kernel's slot
    pipeline has separate start-up and drain steps for each count (plus the
    merge over many partials)."""
    w = wl.make_workload("c5-short", 2007, B=2, H=8, Q=24, prefix=[5, 70], tree="uniform",
                         kv_dtype=wl.BF16)
    r, _, _ = check_full(w, path=2, split_len=split_len, what=f"bf16 split{split_len}")
    assert r.plan()[2] == split_len


# ----------------------------------------------------------------------------- invariances
def test_split_count_invariance():
    w = wl.config("c3")
    bits, _, _ = oracle.build_visibility(w.parent)
    rows = wl.sample_rows(w, 96)
    ref, rlse = oracle_rows(w, bits, rows)
    outs = []
    for L in (64, 256, 1024, 4224):
        r, out, lse = run(w, split_len=L)
        assert r.plan()[3] == (4160 + L - 1) // L
        assert_close(out[rows], ref, 0, f"split {L}")
        assert_lse_close(lse[rows], rlse, 0, f"split {L}")
        outs.append(out)
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() < 1e-5


# Split lengths that are odd multiples of 16: every split ends mid-tile.  The fp32
# matrix kernel on an fp32 cache runs such a last tile as half a tile (one score
# block, half of P.V); the other kernels mask the unused rows of a whole tile.
@pytest.mark.parametrize("kv_dtype,path,B,H,Q,prefix,split_len", [
    (wl.F32, 2, 2, 16, 64, [600, 300], 112),   # 64-row workgroups, tree rows inside half tiles
    (wl.F32, 2, 1, 8, 9, [40], 48),            # tree nodes 0..7 in split 0's half tile, node 8 alone in split 1
    (wl.F32, 2, 1, 8, 9, [0], 16),             # one split of one half tile (the tree only)
    (wl.F32, 2, 3, 8, 5, [77, 0, 30], 80),     # 40 rows, ragged batch rows, a row with no prefix
    (wl.F32, 1, 2, 8, 9, [100, 37], 48),       # vector path
    (wl.F32, 2, 2, 16, 1, [1000, 3], 48),      # row-half mode (16 rows)
    (wl.F32, 2, 2, 16, 1, [1000, 3], 16),      # row-half, one-half-tile splits: every split's second half is empty
    (wl.F32, 2, 1, 8, 9, [1000], 16),          # 72 rows in 16-row splits: every tile a half tile (63 splits)
    (wl.BF16, 2, 2, 16, 64, [600, 300], 112),  # bf16 matrix kernel
    (wl.FP8, 2, 2, 16, 64, [600, 300], 112),   # FP8 cache on the fp32 matrix kernel (whole tiles)
])
def test_half_tile_splits(kv_dtype, path, B, H, Q, prefix, split_len):
    w = wl.make_workload(f"halftile{B}x{H}x{Q}", 8100 + B * 100 + H * 10 + Q, B=B, H=H, Q=Q, prefix=prefix,
                         tree="uniform", kv_dtype=kv_dtype)
    r, _, _ = check_full(w, path=path, split_len=split_len,
                         what=f"half tiles B{B} H{H} Q{Q} P{prefix} dtype {kv_dtype} split {split_len}")
    assert r.plan()[2] == split_len


# Row-half mode lets a row's last split take a remainder of up to 16 positions
# instead of starting a split for it (rows one position past a split boundary,
# e.g. decode with q_len 1 over a 2^k prefix); the other modes do not.
@pytest.mark.parametrize("kv_dtype,path,B,H,Q,prefix,split_len,n_split", [
    (wl.F32, 2, 2, 16, 1, [3072, 2047], 1024, 3),   # row-half: 3073 = 3 x 1024 + 1 and 2048 = 2 x 1024
    (wl.F32, 2, 2, 16, 4, [524, 100], 128, 5),      # usual mode: 528 = 4 x 128 + 16 keeps a fifth split
    (wl.F32, 2, 1, 16, 64, [490], 272, 3),          # half-tile lengths: 554 = 2 x 272 + 10 keeps a third
    (wl.BF16, 3, 2, 16, 1, [1024, 700], 512, 2),    # widened bf16, row-half: 1025 = 2 x 512 + 1
    (wl.F32, 1, 2, 16, 1, [3072, 2047], 1024, 4),   # vector path: no remainder, 4 splits
])
def test_last_split_takes_the_remainder(kv_dtype, path, B, H, Q, prefix, split_len, n_split):
    w = wl.make_workload(f"absorb{B}x{H}x{Q}", 8300 + B * 100 + H * 10 + Q, B=B, H=H, Q=Q, prefix=prefix,
                         tree="uniform", kv_dtype=kv_dtype)
    r, _, _ = check_full(w, path=path, split_len=split_len,
                         what=f"last split remainder B{B} H{H} Q{Q} P{prefix} dtype {kv_dtype} split {split_len}")
    assert r.plan()[2:4] == (split_len, n_split), r.plan()


# Many partials on few rows: the merge shares a row's partials among 2, 4 or 8
# thread groups and combines their results in LDS (test_split_count_invariance
# covers 1 and 2 groups on c3).
@pytest.mark.parametrize("B,H,Q,prefix,split_len,path", [
    (2, 16, 1, [20000, 3], 256, 2),    # row-half, 79 partials on the long row: 8 groups, 10 each
    (1, 16, 4, [9000], 128, 2),        # 64 rows, 71 splits: 8 groups, the last one short
    (2, 8, 4, [3000, 700], 96, 2),     # row-half, 32 partials: 2 groups of 16
    (1, 4, 4, [2100], 64, 1),          # vector path, 34 splits: 4 groups
])
def test_merge_partial_groups(B, H, Q, prefix, split_len, path):
    w = wl.make_workload(f"mg{B}x{H}x{Q}", 7000 + B * 100 + H * 10 + Q, B=B, H=H, Q=Q, prefix=prefix,
                         tree="uniform")
    r, _, _ = check_full(w, path=path, split_len=split_len,
                         what=f"merge groups B{B} H{H} Q{Q} P{prefix} split {split_len}")
    assert r.plan()[2] == split_len


def test_path_invariance():
    """q_len = 16 sits on the dispatch boundary: both paths must agree with the oracle."""
    w = wl.make_workload("q16", 3016, B=2, H=8, Q=16, prefix=[40, 130], tree="uniform")
    _, o_mfma, _ = check_full(w, path=2)
    _, o_valu, _ = check_full(w, path=1)
    assert np.abs(o_mfma - o_valu).max() < 1e-5
    assert run(w)[0].plan()[1] == 2      # auto: 128 query rows per batch row -> MFMA
    w15 = wl.make_workload("q15", 3015, B=1, H=1, Q=15, prefix=[40], tree="uniform")
    assert run(w15)[0].plan()[1] == 1    # and VALU below 16 rows


@pytest.mark.parametrize("path,kv_dtype", [(1, 0), (2, 0), (2, 1), (1, 2), (2, 2)])
def test_workgroup_order_changes_nothing(path, kv_dtype):
    """The XCD-local and spread work-item orders only change which workgroup
    computes which (batch row, split, query tile): on ragged rows with many
    splits and several query tiles, outputs and lse are bit-identical under both,
    and match the oracle."""
    w = wl.make_workload("ragged", 4100 + 10 * path + kv_dtype, B=5, H=16, Q=24,
                         prefix=[700, 40, 1333, 0, 260], tree="uniform", kv_dtype=kv_dtype)
    res = []
    for order in (1, 2):
        r, out, lse = check_full(w, path=path, split_len=128, what=f"order {order}", wg_order=order)
        assert r.plan()[5] == order and r.plan()[3] > 1
        res.append((out, lse))
    assert np.array_equal(res[0][0], res[1][0])
    assert np.array_equal(res[0][1], res[1][1])


def test_spread_order_many_rows_and_no_order_table():
    """70 ragged batch rows, several KV splits: S1 writes the longest-first row
    table over two launches (up to 64 rows each), and the spread grid visits rows
    through it.  A visibility struct without the table (a caller-made one) runs
    rows in their natural order.
    All three give bit-identical results, equal to the oracle."""
    rng = np.random.default_rng(4170)
    w = wl.make_workload("rows70", 4170, B=70, H=4, Q=8, prefix=[int(x) for x in rng.integers(0, 300, 70)],
                         tree="uniform")
    r1, o1, l1 = check_full(w, split_len=96, what="rows70 local", wg_order=1)
    r2, o2, l2 = check_full(w, split_len=96, what="rows70 spread", wg_order=2)
    assert r2.plan()[5] == 2 and r2.plan()[3] > 1
    r2.vis.vis.order = None                      # drop the row-order table
    r2.verify()
    o3, l3 = r2.results()
    for o, l in ((o2, l2), (o3, l3)):
        assert np.array_equal(o, o1) and np.array_equal(l, l1)


# ----------------------------------------------------------------------------- edge cases
@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("B,H,Q,prefix", [
    (1, 8, 1, [0]),            # a single position
    (2, 16, 1, [1000, 3]),     # autoregressive decode (q_len 1)
    (1, 1, 256, [70]),         # largest tree, one head
    (2, 3, 40, [0, 33]),       # rows not a multiple of 16 / 64, no prefix in one row
    (1, 16, 16, [0]),          # tree only, first tile masked
    (3, 5, 33, [31, 32, 95]),  # two mask words, ragged tails
])
def test_edge_shapes(path, B, H, Q, prefix):
    w = wl.make_workload(f"edge{B}x{H}x{Q}", 4000 + B * 100 + Q, B=B, H=H, Q=Q, prefix=prefix,
                         tree="uniform")
    check_full(w, path=path, what=f"edge B{B} H{H} Q{Q} P{prefix}")


@pytest.mark.parametrize("B,H,Q,prefix", [
    (1, 8, 1, [0]),
    (2, 16, 1, [1000, 3]),
    (1, 1, 256, [70]),
    (2, 3, 40, [0, 33]),
    (1, 16, 16, [0]),
    (3, 5, 33, [31, 32, 95]),
    (1, 64, 64, [129]),
])
def test_edge_shapes_bf16_mfma(B, H, Q, prefix):
    w = wl.make_workload(f"edgeb{B}x{H}x{Q}", 5000 + B * 100 + Q, B=B, H=H, Q=Q, prefix=prefix,
                         tree="uniform", kv_dtype=wl.BF16)
    check_full(w, path=2, what=f"bf16 edge B{B} H{H} Q{Q} P{prefix}")


# Batch rows of at most 32 query rows run the matrix kernel in row-half mode: two
# wave pairs per 16-row group, each over one half of every cache tile, combined in
# the workgroup (one partial per split; with one split the output directly).
@pytest.mark.parametrize("kv_dtype,path", [(wl.F32, 0), (wl.F32, 2), (wl.BF16, 3), (wl.FP8, 0)])
@pytest.mark.parametrize("B,H,Q,prefix,split_len", [
    (2, 16, 1, [1000, 3], 0),          # decode (q_len 1), 16 rows
    (2, 16, 1, [1000, 3], 256),        # the same over several splits
    (3, 8, 4, [200, 0, 77], 0),        # 32 rows, tree masks, a row with no prefix
    (1, 16, 2, [4100], 0),             # 32 rows over a long prefix (planned splits)
    (2, 5, 5, [63, 64], 128),          # 25 rows: pairs 2, 3 hold rows 16..24
    (2, 1, 9, [40, 5], 0),             # 9 rows (the matrix path forced below 16)
    (3, 3, 1, [300, 31, 0], 96),       # 3 rows, ragged tails, a row with no prefix
    (2, 16, 1, [100, 3], 32),          # 16 rows, one-tile splits (the idle waves load nothing ahead)
    (1, 8, 2, [500], 0),               # 16 rows from a two-node tree: idle-wave loads and tree masks
])
def test_row_half_mode(kv_dtype, path, B, H, Q, prefix, split_len):
    if path == 0 and Q * H < 16:
        path = 2
    w = wl.make_workload(f"half{B}x{H}x{Q}", 6000 + B * 100 + H * 10 + Q, B=B, H=H, Q=Q, prefix=prefix,
                         tree="uniform", kv_dtype=kv_dtype)
    check_full(w, path=path, split_len=split_len,
               what=f"row-half B{B} H{H} Q{Q} P{prefix} dtype {kv_dtype} split {split_len}")


def test_row_half_mode_single_visible_position_is_exact():
    """Row-half mode on a lone position: one half holds it (p = 1), the other
    half is empty (weight 0 when the workgroup combines them), so the output is the
    row bit for bit."""
    w = wl.make_workload("half-single", 6900, B=1, H=16, Q=1, prefix=0, tree="uniform")
    r, out, lse = run(w, path=2)
    for h in range(w.H):
        assert np.array_equal(out[h], w.ckv[0]), h


@pytest.mark.parametrize("path", [1, 2])
def test_single_visible_position_is_exact(path):
    """With no prefix the root sees only itself: p = 1, so the output is its latent row bit for bit."""
    w = wl.config("c1")
    r, out, lse = run(w, path=path)
    for h in range(w.H):
        assert np.array_equal(out[h], w.ckv[0]), h


@pytest.mark.parametrize("path", [1, 2, 3])
def test_single_visible_position_is_exact_bf16(path):
    """Same on a bf16 cache: p = 1 is exact in bf16, so every path returns the widened row."""
    w = wl.make_workload("c1-bf16", 1001, B=1, H=8, Q=9, prefix=0, tree="uniform", kv_dtype=wl.BF16)
    r, out, lse = run(w, path=path)
    row0 = wl.bf16_bits_to_f32(w.ckv[0])
    for h in range(w.H):
        assert np.array_equal(out[h], row0), h


@pytest.mark.parametrize("path", [1, 2])
def test_hand_made_masks(path):
    """Caller-built masks: all-ones (dense softmax) and an empty row (out = 0, lse = -inf)."""
    w = wl.make_workload("masks", 4321, B=2, H=4, Q=20, prefix=[10, 0], tree="uniform")
    ones = np.zeros((2, 20, 1), np.uint32)
    ones[...] = (1 << 20) - 1
    ones[1, 3, 0] = 0                 # batch row 1 has no prefix: node 3 sees nothing
    r, out, lse = run(w, path=path, bits_override=ones)
    ref, rlse = oracle.verify_attn(w.q_abs, w.q_rope, w.ckv, w.k_rope, 0, w.prefix, ones, w.scale)
    assert_close(out, ref, 0, "masks")
    assert_lse_close(lse, rlse, 0, "masks")
    empty = (1 * w.Q + 3) * w.H + np.arange(w.H)
    assert (out[empty] == 0).all() and np.isneginf(lse[empty]).all()


def test_malformed_tree_still_runs():
    """A malformed node sees only itself; attention stays defined."""
    w = wl.make_workload("bad", 4444, B=2, H=4, Q=8, prefix=[5, 9], tree="uniform")
    par = w.parent.copy()
    par[1, 4] = 6                     # forward edge
    bits, bad, rc = oracle.build_visibility(par)
    assert rc == oracle.REF_ETREE and list(bad) == [-1, 4]
    r, out, lse = run(w, parent=par)
    assert np.array_equal(r.bits(), bits)
    assert np.array_equal(r.status(), bad)
    ref, rlse = oracle.verify_attn(w.q_abs, w.q_rope, w.ckv, w.k_rope, 0, w.prefix, bits, w.scale)
    assert_close(out, ref, 0, "malformed")


# ----------------------------------------------------------------------------- full sizes, sampled rows
def _full_sampled(name, n_rows, extra_rows=None):
    say(f"generate {name}")
    w = wl.config(name)
    bits, _, _ = oracle.build_visibility(w.parent)
    say(f"run {name}")
    r, out, lse = run(w)
    say(f"  plan {r.plan()}")
    assert np.array_equal(r.bits(), bits)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    # every row is a convex combination of latent rows: bounded by the cache's extremes
    head = w.ckv[:65536]
    kvmax = float(np.abs({0: lambda a: a, 1: wl.bf16_bits_to_f32, 2: wl.fp8_bits_to_f32}[w.kv_dtype](head)).max())
    assert np.abs(out).max() <= 10 * kvmax
    rows = wl.sample_rows(w, n_rows)
    if extra_rows is not None:
        rows = np.unique(np.concatenate([rows, extra_rows(w)]))
    say(f"oracle {name} on {len(rows)} rows")
    ref, rlse = oracle_rows(w, bits, rows, chunk=4)
    ar = arithmetic(w.kv_dtype, r.plan()[1])
    e = assert_close(out[rows], ref, ar, name)
    assert_lse_close(lse[rows], rlse, ar, name)
    say(f"  {name}: max abs err {e:.2e} on {len(rows)} sampled rows")


def _all_heads_of_some_nodes(w):
    """Every head of nodes 0, 1, Q/2 and Q-1 of the batch rows with the longest and
    the shortest prefix."""
    rows = []
    for b in (int(np.argmax(w.prefix)), int(np.argmin(w.prefix))):
        for q in sorted({0, 1, w.Q // 2, w.Q - 1}):
            rows.append((b * w.Q + q) * w.H + np.arange(w.H))
    return np.concatenate(rows).astype(np.int64)


@functools.lru_cache(maxsize=1)
def _beyond_2gib():
    return wl.make_workload("big", 4600, B=2, H=16, Q=16, prefix=[600000, 600000], tree="uniform")


@pytest.mark.parametrize("path", [1, 2])
def test_fp32_cache_beyond_2gib(path):
    """Two 600k-position batch rows: the fp32 latent cache spans 2.46 GB, so the
    second row's cache reaches byte offsets past 2^31.  Sampled query rows of both
    batch rows against the oracle."""
    say("generate beyond-2GiB workload")
    w = _beyond_2gib()
    assert w.ckv.nbytes > 2**31
    bits, _, _ = oracle.build_visibility(w.parent)
    r, out, lse = run(w, path=path)
    say(f"  plan {r.plan()}")
    rows = np.array([0, 37, 255, 256, 300, 511], dtype=np.int64)   # both batch rows, first and last nodes
    ref, rlse = oracle_rows(w, bits, rows, chunk=1)
    e = assert_close(out[rows], ref, 0, f"beyond 2 GiB path {path}")
    assert_lse_close(lse[rows], rlse, 0, f"beyond 2 GiB path {path}")
    say(f"  max abs err {e:.2e}")


def test_c4_full_sampled():
    _full_sampled("c4", 64)


def test_c4_decode_shape_row_half_full_sampled():
    """c4 sizes at q_len 1 (16 query rows per batch row, 262,152 cache rows): the
    row-half mode in the launch the decode probe times (many splits, the halves
    combined in each workgroup, then merged), on every query row of two batch rows
    against the oracle."""
    say("generate c4 at q_len 1")
    w = wl.config("c4", Q=1)
    bits, _, _ = oracle.build_visibility(w.parent)
    r, out, lse = run(w)
    say(f"  plan {r.plan()}")
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    rows = np.concatenate([np.arange(0, 16), np.arange(7 * 16, 8 * 16)]).astype(np.int64)
    ref, rlse = oracle_rows(w, bits, rows, chunk=4)
    e = assert_close(out[rows], ref, 0, "c4 q_len 1")
    assert_lse_close(lse[rows], rlse, 0, "c4 q_len 1")
    say(f"  c4 q_len 1: max abs err {e:.2e} on {len(rows)} rows")


def test_c5_full_sampled():
    """c5 at full size in the benchmark's launch on the bf16 matrix cores: 256
    seeded rows over all batch rows plus all 64 heads of four nodes of the longest
    and the shortest batch row (768 rows), against the bf16-arithmetic bar."""
    _full_sampled("c5", 256, extra_rows=_all_heads_of_some_nodes)


# ----------------------------------------------------------------------------- graph capture
@pytest.mark.parametrize("kv_dtype", [0, 1])
def test_step_replays_from_a_hip_graph(kv_dtype):
    """A whole verify step (visibility build, attention, split merge) captured into a
    HIP graph replays bit-identically to the eager step: the library launches only
    kernels on the caller's stream (no allocation, copy, memset or sync on the path).
    Eager work and a synchronisation run between replays, and every replay is
    checked; the first eager result is also checked against the oracle."""
    w = wl.make_workload("graph", 2100 + kv_dtype, B=2, H=16, Q=32, prefix=[700, 90], tree="uniform",
                         kv_dtype=kv_dtype)
    from tree_masked_mla_amd.runner import DeviceRun
    r = DeviceRun(w, split_len=256)
    assert r.plan()[3] > 1                       # the merge kernel is part of the step
    r.step()
    torch.cuda.synchronize()
    ref_out, ref_lse = r.out.clone(), r.lse.clone()
    bits, _, _ = oracle.build_visibility(w.parent)
    ref, rlse = oracle_rows(w, bits)
    out0, lse0 = r.results()
    ar = arithmetic(kv_dtype, r.plan()[1])
    assert_close(out0, ref, ar, "graph eager")
    assert_lse_close(lse0, rlse, ar, "graph eager")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            r.step()
    torch.cuda.synchronize()
    for i in range(4):
        r.out.fill_(float("nan"))                # eager work between replays
        r.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(r.out, ref_out), f"replay {i}: output differs from the eager step"
        assert torch.equal(r.lse, ref_lse), f"replay {i}: lse differs from the eager step"
    say(f"  graph replay x4 bit-identical (kv_dtype {kv_dtype})")
