"""External-prefix (tree-tail) mode on the GPU: given each query row's exact
attention over the prefix alone (from the oracle), attending the tree rows and
merging by log-sum-exp must reproduce the oracle's full attention over prefix
and tree (the log-sum-exp merge identity)."""
import numpy as np
import pytest

import oracle
import workloads as wl
from parity import F32, arithmetic, assert_close, assert_lse_close, oracle_rows, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def prefix_results(w):
    """Oracle attention of every query row over its batch row's prefix rows only:
    normalised output [B][Q][H][512] and natural-log lse [B][Q][H] (-inf, zeros
    without prefix)."""
    B, Q, H = w.B, w.Q, w.H
    out = np.zeros((B, Q, H, 512), np.float32)
    lse = np.full((B, Q, H), -np.inf, np.float32)
    off = np.concatenate([[0], np.cumsum(w.prefix.astype(np.int64) + Q)])
    for b in range(B):
        P = int(w.prefix[b])
        if P == 0:
            continue
        idx = off[b] + np.arange(P, dtype=np.int64)
        for q in range(Q):
            for h in range(H):
                m, l, o = oracle.partial(w.q_abs[b, q, h], w.q_rope[b, q, h], w.ckv, w.k_rope, w.kv_dtype, idx,
                                         w.scale)
                out[b, q, h] = o / l
                lse[b, q, h] = m + np.log(l)
    return out, lse


def run_tail(w, split_len=0, want_lse=True, path=0, bits_override=None):
    """path 0 with split_len 0 takes the tree-sparse route; a forced path or split
    length takes the dense route (attention kernels over the tree rows + merge)."""
    import tree_masked_mla_amd as dd
    from tree_masked_mla_amd.runner import DeviceRun
    r = DeviceRun(w, want_lse=want_lse, split_len=split_len, path=path, bits_override=bits_override)
    po, pl = prefix_results(w)
    po_d = torch.from_numpy(po).to(r.device)
    pl_d = torch.from_numpy(pl).to(r.device)
    opts = dd.make_opts(path=path, split_len=split_len)
    need = dd.ddtv_tail_workspace_bytes(r.vis, w.H, w.kv_dtype, opts)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device=r.device)
    r.out.fill_(float("nan"))
    rc = dd.ddtv_verify_attn_tail(r.q_abs, r.q_rope, r.ckv, r.k_rope, w.kv_dtype, w.H, r.vis, w.scale, po_d, pl_d,
                                  r.out, r.lse, ws, opts=opts)
    assert rc == dd.DDTV_OK
    torch.cuda.synchronize()
    out = r.out.cpu().numpy().reshape(-1, 512)
    lse = r.lse.cpu().numpy().reshape(-1) if want_lse else None
    return r, out, lse


@pytest.mark.parametrize("kv_dtype,split_len,want_lse,path", [
    (0, 0, True, 0), (1, 0, True, 0), (2, 0, True, 0), (0, 0, False, 0),     # tree-sparse route
    (0, 32, True, 0), (0, 0, True, 2), (1, 0, True, 2), (2, 0, True, 1),     # dense route
])
def test_tail_mode_equals_full_attention(kv_dtype, split_len, want_lse, path):
    w = wl.make_workload("tail", 3300 + kv_dtype, B=3, H=8, Q=24, prefix=[0, 500, 1300], tree="uniform",
                         kv_dtype=kv_dtype)
    say(f"tail dtype {kv_dtype} split {split_len} lse {want_lse} path {path}")
    r, out, lse = run_tail(w, split_len, want_lse, path)
    bits, _, _ = oracle.build_visibility(w.parent)
    ref, rlse = oracle_rows(w, bits)
    # the sparse route computes in fp32 on every cache dtype: the fp32 bar holds for it
    ar = arithmetic(kv_dtype, r.plan()[1]) if (path or split_len) else F32
    e = assert_close(out, ref, ar, "tail mode")
    if want_lse:
        assert_lse_close(lse, rlse, ar, "tail mode")
    say(f"  max abs err {e:.2e}")


@pytest.mark.parametrize("path", [0, 2])
def test_tail_mode_long_prefix_mfma_rows(path):
    """128-node trees over 4096-position prefixes, 16 heads: the tree rows fill
    several 64-row tiles per batch row, as on the benchmark's shapes (both routes)."""
    w = wl.make_workload("tail-big", 3310, B=2, H=16, Q=128, prefix=[4096, 1000], tree="best_first", depth_cap=12)
    r, out, lse = run_tail(w, path=path)
    bits, _, _ = oracle.build_visibility(w.parent)
    rows = wl.sample_rows(w, 48)
    ref, rlse = oracle_rows(w, bits, rows, chunk=4)
    assert_close(out[rows], ref, 0, "tail mode, long prefix")
    assert_lse_close(lse[rows], rlse, 0, "tail mode, long prefix")


@pytest.mark.parametrize("H", [1, 5, 64])
def test_tail_sparse_heads_and_empty_masks(H):
    """The sparse route with head counts that do not fill its 4-heads-per-wave
    passes, a 256-node chain (8 mask words, up to 256 ancestors), and hand-made
    masks where some nodes see no tree row: with a prefix they return the prefix
    result, without one they return 0 and lse -inf."""
    Q = 256 if H == 1 else 40
    w = wl.make_workload("tail-sparse", 3320 + H, B=2, H=H, Q=Q, prefix=[0, 300], tree="chain" if H == 1 else "uniform")
    bits, _, _ = oracle.build_visibility(w.parent)
    bits = bits.copy()
    bits[:, 3, :] = 0          # node 3 of both batch rows sees no tree row
    bits[1, Q - 1, :] = 0
    r, out, lse = run_tail(w, bits_override=bits)
    ref, rlse = oracle_rows(w, bits)
    assert_close(out, ref, 0, f"sparse tail H={H}")
    assert_lse_close(lse, rlse, 0, f"sparse tail H={H}")
    assert np.isneginf(lse.reshape(2, Q, H)[0, 3]).all() and not out.reshape(2, Q, H, 512)[0, 3].any()
