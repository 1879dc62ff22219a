"""One whole tree-verify iteration through every entry point, captured into a HIP
graph: draft-tree builder -> visibility -> the tree's cache rows -> query
preparation -> attention -> value projection -> greedy acceptance with
compaction.  Each replay (after restoring the caches, which the iteration edits
in place) must reproduce the eager iteration bit for bit: the library launches
only kernels on the caller's stream, with no allocation, copy, memset or
synchronisation on the path.  The eager iteration's tree and acceptance are
also checked against the oracle."""
import numpy as np
import pytest

import oracle
import workloads as wl
from parity import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("kv_dtype", [wl.F32, wl.BF16, wl.FP8])
def test_iteration_replays_from_a_hip_graph(kv_dtype):
    import tree_masked_mla_amd as dd
    from tree_masked_mla_amd.runner import to_device_kv
    B, H, Q, D, K, V = 2, 16, 32, 6, 4, 200
    w = wl.make_workload("iter", 2200 + kv_dtype, B=B, H=H, Q=Q, prefix=[700, 90], tree="uniform",
                         kv_dtype=kv_dtype)
    dev = torch.device("cuda")
    lp, tok = wl.drafter_topk(2210, B, D, K)
    nb = wl.neighbour_inputs(2211, B, Q, H)
    logits_h = wl.target_logits(2212, B, Q, V)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    lp_d, tok_d, q, w_kc, w_vc, lat, k_pe, logits = (t(x) for x in (lp, tok, nb.q, nb.w_kc, nb.w_vc, nb.latent,
                                                                    nb.k_pe, logits_h))
    ckv0 = to_device_kv(w.ckv, kv_dtype, dev)
    kr0 = to_device_kv(w.k_rope, kv_dtype, dev)
    ckv, kr = ckv0.clone(), kr0.clone()
    i32 = lambda *shape: torch.full(shape, -7, dtype=torch.int32, device=dev)
    outs = dict(parent=i32(B, Q), token=i32(B, Q), pred=i32(B, Q), path=i32(B, Q), out_tokens=i32(B, Q),
                accept_len=i32(B),
                q_abs=torch.empty((B, Q, H, 512), device=dev), q_rope=torch.empty((B, Q, H, 64), device=dev),
                out=torch.empty((B, Q, H, 512), device=dev), lse=torch.empty((B, Q, H), device=dev),
                v=torch.empty((B, Q, H, 128), device=dev))
    vis_buf = torch.empty(dd.ddtv_vis_bytes(B, Q), dtype=torch.uint8, device=dev)
    prefix = np.ascontiguousarray(w.prefix, dtype=np.int32)
    keep = {}

    def iteration(stream=None):
        o, ok = outs, dd.DDTV_OK
        assert dd.ddtv_build_tree(lp_d, Q, o["parent"], tokens=tok_d, token=o["token"], stream=stream) == ok
        rc, vis = dd.ddtv_build_visibility(o["parent"], prefix, B, Q, vis_buf, stream=stream)
        assert rc == ok
        if "ws" not in keep:
            need = dd.ddtv_workspace_bytes(vis, H, kv_dtype)
            keep["ws"] = (torch.empty(max(need, 1), dtype=torch.uint8, device=dev), need)
        ws, need = keep["ws"]
        assert dd.ddtv_append_kv(lat, k_pe, vis, ckv, kr, kv_dtype, nb.theta, stream=stream) == ok
        assert dd.ddtv_prepare_query(q, w_kc, vis, o["q_abs"], o["q_rope"], nb.theta, stream=stream) == ok
        assert dd.ddtv_verify_attn(o["q_abs"], o["q_rope"], ckv, kr, kv_dtype, H, vis, w.scale, o["out"], o["lse"],
                                   ws, need, stream=stream) == ok
        assert dd.ddtv_value_proj(o["out"], w_vc, o["v"], stream=stream) == ok
        assert dd.ddtv_tree_accept(logits, o["parent"], o["token"], vis, o["pred"], o["path"], o["out_tokens"],
                                   o["accept_len"], ckv=ckv, k_rope=kr, kv_dtype=kv_dtype, stream=stream) == ok
        keep["vis"] = vis

    say(f"iteration eager (kv_dtype {kv_dtype})")
    iteration()
    torch.cuda.synchronize()
    ref = {k: x.clone() for k, x in outs.items()}
    ref_ckv, ref_kr = ckv.clone(), kr.clone()

    # the eager tree and acceptance against the oracle
    rc, tree = oracle.build_tree(lp, Q, tok)
    assert rc == oracle.REF_OK
    assert np.array_equal(ref["parent"].cpu().numpy(), tree["parent"])
    rc, acc = oracle.tree_accept(logits_h, tree["parent"], tree["token"])
    assert rc == oracle.REF_OK
    for k in ("pred", "path", "out_tokens", "accept_len"):
        assert np.array_equal(ref[k].cpu().numpy(), acc[k]), k

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    ckv.copy_(ckv0)
    kr.copy_(kr0)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            iteration()
    torch.cuda.synchronize()
    for i in range(3):
        ckv.copy_(ckv0)                       # eager work between replays: fresh caches, poisoned outputs
        kr.copy_(kr0)
        for x in outs.values():
            x.fill_(-7 if x.dtype == torch.int32 else float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, x in outs.items():
            assert torch.equal(x, ref[k]), f"replay {i}: {k} differs from the eager iteration"
        assert torch.equal(ckv, ref_ckv) and torch.equal(kr, ref_kr), f"replay {i}: caches differ"
    say(f"  iteration graph replay x3 bit-identical (kv_dtype {kv_dtype})")
