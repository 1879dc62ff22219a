"""External-prefix (tree-tail) mode on the GPU: given each query row's exact
attention over the prefix alone (from the oracle), attending the tree rows and
merging by log-sum-exp must reproduce the oracle's full attention over prefix
and tree (the log-sum-exp merge identity)."""
import numpy as np
import pytest

import oracle
import workloads as wl
from parity import assert_close, assert_lse_close, oracle_rows, say

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


def run_tail(w, split_len=0, want_lse=True):
    import tree_masked_mla_amd as dd
    from tree_masked_mla_amd.runner import DeviceRun
    r = DeviceRun(w, want_lse=want_lse, split_len=split_len)
    po, pl = prefix_results(w)
    po_d = torch.from_numpy(po).to(r.device)
    pl_d = torch.from_numpy(pl).to(r.device)
    opts = dd.make_opts(split_len=split_len)
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


@pytest.mark.parametrize("kv_dtype,split_len,want_lse", [(0, 0, True), (1, 0, True), (2, 0, True), (0, 32, True),
                                                                (0, 0, False)])
def test_tail_mode_equals_full_attention(kv_dtype, split_len, want_lse):
    w = wl.make_workload("tail", 3300 + kv_dtype, B=3, H=8, Q=24, prefix=[0, 500, 1300], tree="uniform",
                         kv_dtype=kv_dtype)
    say(f"tail dtype {kv_dtype} split {split_len} lse {want_lse}")
    r, out, lse = run_tail(w, split_len, want_lse)
    bits, _, _ = oracle.build_visibility(w.parent)
    ref, rlse = oracle_rows(w, bits)
    e = assert_close(out, ref, kv_dtype, "tail mode")
    if want_lse:
        assert_lse_close(lse, rlse, kv_dtype, "tail mode")
    say(f"  max abs err {e:.2e}")


def test_tail_mode_long_prefix_mfma_rows():
    """128-node trees over 4096-position prefixes, 16 heads: the tree rows fill
    several 64-row tiles per batch row, as on the benchmark's shapes."""
    w = wl.make_workload("tail-big", 3310, B=2, H=16, Q=128, prefix=[4096, 1000], tree="best_first", depth_cap=12)
    r, out, lse = run_tail(w)
    bits, _, _ = oracle.build_visibility(w.parent)
    rows = wl.sample_rows(w, 48)
    ref, rlse = oracle_rows(w, bits, rows, chunk=4)
    assert_close(out[rows], ref, 0, "tail mode, long prefix")
    assert_lse_close(lse[rows], rlse, 0, "tail mode, long prefix")
