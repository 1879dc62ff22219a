"""Greedy tree acceptance and cache compaction on the GPU against their oracle,
bit for bit (predictions, paths, tokens and lengths are integers; compaction
moves bytes), then the whole chain on the device: tree builder, visibility,
verify attention, acceptance and compaction with no host round trip."""
import numpy as np
import pytest

import oracle
import workloads as wl
from parity import assert_close, assert_lse_close, oracle_rows, say
from test_accept_oracle import random_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def run_accept(logits, parent, token, vis=None, ckv=None, k_rope=None, kv_dtype=0, keep=None):
    import tree_masked_mla_amd as dd
    dev = torch.device("cuda:0")
    B, Q, V = logits.shape
    if vis is None:   # a visibility struct for the trees (the accept step reads B, Q and the row table)
        par_d = torch.from_numpy(np.ascontiguousarray(parent, np.int32)).to(dev)
        buf = torch.empty(dd.ddtv_vis_bytes(B, Q), dtype=torch.uint8, device=dev)
        rc, vis = dd.ddtv_build_visibility(par_d, np.zeros(B, np.int32), B, Q, buf)
        assert rc == dd.DDTV_OK
        keep = (par_d, buf)
    lg = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).to(dev)
    par = torch.from_numpy(np.ascontiguousarray(parent, np.int32)).to(dev)
    tok = torch.from_numpy(np.ascontiguousarray(token, np.int32)).to(dev)
    out = {k: torch.full((B, Q), -9, dtype=torch.int32, device=dev) for k in ("pred", "path", "out_tokens")}
    out["accept_len"] = torch.full((B,), -9, dtype=torch.int32, device=dev)
    rc = dd.ddtv_tree_accept(lg, par, tok, vis, out["pred"], out["path"], out["out_tokens"], out["accept_len"],
                             ckv=ckv, k_rope=k_rope, kv_dtype=kv_dtype)
    assert rc == dd.DDTV_OK
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


@pytest.mark.parametrize("seed,B,Q,V", [(1, 6, 32, 64), (2, 4, 128, 1000), (3, 8, 9, 32000), (4, 3, 256, 517),
                                        (5, 70, 16, 33)])
def test_accept_matches_oracle(seed, B, Q, V):
    say(f"accept B{B} Q{Q} V{V}")
    parent, token, logits = random_case(seed, B, Q, V=V)
    rc, ref = oracle.tree_accept(logits, parent, token)
    assert rc == oracle.REF_OK
    got = run_accept(logits, parent, token)
    for k in ("pred", "path", "out_tokens", "accept_len"):
        assert np.array_equal(got[k], ref[k]), k
    assert ref["accept_len"].max() >= 1


def test_accept_unaligned_logits():
    """Logits that start 4 bytes past a 16-byte boundary take the scalar path."""
    import tree_masked_mla_amd as dd
    parent, token, logits = random_case(12, 3, 24, V=64)
    rc, ref = oracle.tree_accept(logits, parent, token)
    dev = torch.device("cuda:0")
    B, Q, V = logits.shape
    flat = torch.zeros(B * Q * V + 4, dtype=torch.float32, device=dev)
    flat[1:1 + B * Q * V] = torch.from_numpy(logits.reshape(-1)).to(dev)
    lg = flat[1:1 + B * Q * V].view(B, Q, V)
    assert lg.data_ptr() % 16 == 4
    par_d = torch.from_numpy(parent).to(dev)
    buf = torch.empty(dd.ddtv_vis_bytes(B, Q), dtype=torch.uint8, device=dev)
    rc, vis = dd.ddtv_build_visibility(par_d, np.zeros(B, np.int32), B, Q, buf)
    o = [torch.empty((B, Q), dtype=torch.int32, device=dev) for _ in range(3)]
    alen = torch.empty(B, dtype=torch.int32, device=dev)
    assert dd.ddtv_tree_accept(lg, par_d, torch.from_numpy(token).to(dev), vis, o[0], o[1], o[2], alen) == dd.DDTV_OK
    torch.cuda.synchronize()
    assert np.array_equal(o[0].cpu().numpy(), ref["pred"])
    assert np.array_equal(alen.cpu().numpy(), ref["accept_len"])


def test_accept_ties_in_logits():
    parent, token, logits = random_case(11, 3, 40, V=64)
    logits = np.round(logits)                     # many equal maxima: the lowest index wins
    logits[1] = 0.0
    rc, ref = oracle.tree_accept(logits.astype(np.float32), parent, token)
    got = run_accept(logits.astype(np.float32), parent, token)
    for k in ("pred", "path", "out_tokens", "accept_len"):
        assert np.array_equal(got[k], ref[k]), k


@pytest.mark.parametrize("kv_dtype", [0, 1, 2])
def test_compaction_matches_oracle(kv_dtype):
    """Compaction in place on the device caches: every batch row's rows equal the
    oracle's out-of-place move, and the other batch rows are untouched."""
    from tree_masked_mla_amd.runner import DeviceRun
    B, H, Q = 5, 4, 64
    parent, token, logits = random_case(21 + kv_dtype, B, Q, V=200, follow=0.9)
    w = wl.make_workload("compact", 3100 + kv_dtype, B=B, H=H, Q=Q, prefix=[100, 0, 2048, 37, 500],
                         tree="uniform", kv_dtype=kv_dtype)
    w.parent[...] = parent
    r = DeviceRun(w)
    rc, ref = oracle.tree_accept(logits, parent, token)
    assert rc == oracle.REF_OK and ref["accept_len"].max() >= 2
    got = run_accept(logits, parent, token, vis=r.vis, ckv=r.ckv, k_rope=r.k_rope, kv_dtype=kv_dtype)
    assert np.array_equal(got["path"], ref["path"])
    def host(t):   # the device cache as its stored bits
        return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t).cpu().numpy()
    ckv, kr = host(r.ckv), host(r.k_rope)
    off = np.concatenate([[0], np.cumsum(w.prefix.astype(np.int64) + Q)])
    for b in range(B):
        lo, hi = off[b], off[b + 1]
        k = int(ref["accept_len"][b])
        want = oracle.compact_rows(np.asarray(w.ckv)[lo:hi], int(w.prefix[b]), ref["path"][b], k)
        assert np.array_equal(ckv[lo:hi].view(want.dtype), want), f"latent rows of batch row {b}"
        want = oracle.compact_rows(np.asarray(w.k_rope)[lo:hi], int(w.prefix[b]), ref["path"][b], k)
        assert np.array_equal(kr[lo:hi].view(want.dtype), want), f"rope rows of batch row {b}"


def test_whole_chain_on_device():
    """Builder -> visibility -> verify attention -> acceptance -> compaction, all on
    the device; each stage equals the oracle's."""
    import tree_masked_mla_amd as dd
    from tree_masked_mla_amd.runner import DeviceRun
    B, H, Q, D, K, V = 4, 8, 40, 9, 4, 256
    lp, tok = wl.drafter_topk(31, B, D, K, vocab=V)
    rc, tree = oracle.build_tree(lp, Q, tok)
    assert rc == oracle.REF_OK
    w = wl.make_workload("chain", 3200, B=B, H=H, Q=Q, prefix=[64, 300, 0, 1000], tree="uniform")
    w.parent[...] = tree["parent"]
    r = DeviceRun(w)
    dev = r.device
    tok_d = torch.empty((B, Q), dtype=torch.int32, device=dev)
    assert dd.ddtv_build_tree(torch.from_numpy(lp).to(dev), Q, r.parent, tokens=torch.from_numpy(tok).to(dev),
                              token=tok_d) == dd.DDTV_OK
    r.step()                                     # S1 .. S7 on the device-built trees
    out, lse = r.results()
    bits, _, _ = oracle.build_visibility(tree["parent"])
    want, wlse = oracle_rows(w, bits)
    assert_close(out, want, 0, "chain attention")
    assert_lse_close(lse, wlse, 0, "chain attention")
    rng = np.random.default_rng(32)
    logits = rng.standard_normal((B, Q, V)).astype(np.float32)
    for b in range(B):                           # the target mostly agrees with the drafter's best child
        for i in range(Q):
            kids = np.nonzero(tree["parent"][b] == i)[0]
            if len(kids) and rng.random() < 0.8:
                logits[b, i, tree["token"][b, kids[0]]] = 9.0
    rc, acc = oracle.tree_accept(logits, tree["parent"], tree["token"])
    assert rc == oracle.REF_OK
    lg = torch.from_numpy(logits).to(dev)
    o = {k: torch.empty((B, Q), dtype=torch.int32, device=dev) for k in ("pred", "path", "out_tokens")}
    alen = torch.empty(B, dtype=torch.int32, device=dev)
    assert dd.ddtv_tree_accept(lg, r.parent, tok_d, r.vis, o["pred"], o["path"], o["out_tokens"], alen,
                               ckv=r.ckv, k_rope=r.k_rope, kv_dtype=0) == dd.DDTV_OK
    torch.cuda.synchronize()
    assert np.array_equal(alen.cpu().numpy(), acc["accept_len"])
    assert np.array_equal(o["out_tokens"].cpu().numpy(), acc["out_tokens"])
    ckv = r.ckv.cpu().numpy()
    off = np.concatenate([[0], np.cumsum(w.prefix.astype(np.int64) + Q)])
    for b in range(B):
        want = oracle.compact_rows(w.ckv[off[b]:off[b + 1]], int(w.prefix[b]), acc["path"][b],
                                   int(acc["accept_len"][b]))
        assert np.array_equal(ckv[off[b]:off[b + 1]], want)
    say(f"  accepted {acc['accept_len'].tolist()}")
