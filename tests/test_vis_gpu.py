"""S1 on the GPU: packed ancestor masks must equal the oracle's bit for bit."""
import itertools
import math

import numpy as np
import pytest

import oracle
import workloads as wl
from parity import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def gpu_bits(parent, prefix):
    import tree_masked_mla_amd as dd
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    B, Q = parent.shape
    dev = torch.device("cuda:0")
    par_d = torch.from_numpy(parent).to(dev)
    buf = torch.empty(dd.ddtv_vis_bytes(B, Q), dtype=torch.uint8, device=dev)
    rc, vis = dd.ddtv_build_visibility(par_d, prefix, B, Q, buf)
    assert rc == dd.DDTV_OK
    torch.cuda.synchronize()
    W = (Q + 31) // 32
    raw = buf.cpu().numpy()
    bits = raw[: B * Q * W * 4].view(np.uint32).reshape(B, Q, W).copy()
    rows_off = vis.rows - buf.data_ptr()
    rows = raw[rows_off: rows_off + 16 * B].view(np.int64).reshape(B, 2)
    kv_off = rows[:, 0].copy()
    pk = rows[:, 1].copy().view(np.int32).reshape(B, 2)
    st_off = vis.status - buf.data_ptr()
    status = raw[st_off: st_off + 4 * B].view(np.int32).copy()
    return bits, status, kv_off, pk[:, 0], pk[:, 1], vis, (buf, par_d)


def gpu_order(vis, keep):
    """The row-order table S1 wrote: batch rows by cache length, longest first."""
    buf = keep[0]
    off = vis.order - buf.data_ptr()
    return buf[off: off + 4 * vis.B].cpu().numpy().view(np.int32).copy()


def longest_first(prefix):
    return np.argsort(-np.asarray(prefix, np.int64), kind="stable").astype(np.int32)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_vis_configs_bit_exact(name):
    # trees and prefixes are the first draws of each workload's stream
    say(f"vis {name}")
    parent, prefix = wl.config_trees(name)
    ref, bad, rc = oracle.build_visibility(parent)
    assert rc == 0
    bits, status, kv_off, pk, kvl, vis, keep = gpu_bits(parent, prefix)
    assert np.array_equal(bits, ref)
    assert (status == -1).all()
    assert np.array_equal(gpu_order(vis, keep), longest_first(prefix))
    exp_off = np.concatenate([[0], np.cumsum(prefix.astype(np.int64) + parent.shape[1])[:-1]])
    assert np.array_equal(kv_off, exp_off)
    assert np.array_equal(pk, prefix) and np.array_equal(kvl, prefix + parent.shape[1])
    assert vis.total_kv == int((prefix.astype(np.int64) + parent.shape[1]).sum())
    assert vis.max_kv == int(prefix.max()) + parent.shape[1]


@pytest.mark.parametrize("Q", [1, 2, 3, 4, 5, 6, 7])
def test_vis_bruteforce_all_trees(Q):
    trees = [np.array((-1,) + c, np.int32) for c in itertools.product(*[range(i) for i in range(1, Q)])]
    parent = np.stack(trees)
    assert len(parent) == math.factorial(Q - 1)
    ref, _, _ = oracle.build_visibility(parent)
    bits, status, *_ = gpu_bits(parent, np.zeros(len(trees), np.int32))
    assert np.array_equal(bits, ref)
    assert (status == -1).all()


def test_vis_large_trees_and_many_rows():
    rng = np.random.default_rng(77)
    Q = 256
    trees = [wl.uniform_tree(rng, Q), wl.best_first_tree(rng, Q, 30), wl.chain_tree(Q),
             np.array([-1] + [0] * (Q - 1), np.int32)]          # star
    trees += [wl.uniform_tree(rng, Q) for _ in range(130 - len(trees))]   # > 64 rows: several launches
    parent = np.stack(trees)
    prefix = rng.integers(0, 5000, size=len(trees)).astype(np.int32)
    ref, _, _ = oracle.build_visibility(parent)
    bits, status, kv_off, pk, kvl, vis, keep = gpu_bits(parent, prefix)
    assert np.array_equal(bits, ref)
    assert (status == -1).all()
    order = gpu_order(vis, keep)                  # written chunk by chunk, over several launches
    assert np.array_equal(order, longest_first(prefix))
    assert np.array_equal(np.sort(order), np.arange(len(prefix)))
    assert np.array_equal(kv_off, np.concatenate([[0], np.cumsum(prefix.astype(np.int64) + Q)[:-1]]))
    for Qs in (31, 32, 33, 63, 64, 65, 100):
        par = np.stack([wl.uniform_tree(rng, Qs) for _ in range(3)])
        ref, _, _ = oracle.build_visibility(par)
        assert np.array_equal(gpu_bits(par, np.zeros(3, np.int32))[0], ref), Qs


def test_vis_malformed_trees():
    import tree_masked_mla_amd as dd
    parent = np.stack([
        np.array([-1, 0, 1, 2], np.int32),
        np.array([0, 0, 1, 2], np.int32),
        np.array([-1, 0, 2, 1], np.int32),
        np.array([-1, -1, 5, 0], np.int32),
        np.array([-1, 0, 1, -7], np.int32),
    ])
    ref, bad, rc = oracle.build_visibility(parent)
    assert rc == oracle.REF_ETREE
    bits, status, kv_off, pk, kvl, vis, keep = gpu_bits(parent, np.arange(5, dtype=np.int32))
    assert np.array_equal(status, bad)
    assert np.array_equal(bits, ref)
    rc, row, node = dd.ddtv_read_status(vis)
    assert (rc, row, node) == (dd.DDTV_ETREE, 1, 0)
    good = gpu_bits(parent[:1], np.zeros(1, np.int32))
    assert dd.ddtv_read_status(good[5]) == (dd.DDTV_OK, -1, -1)
