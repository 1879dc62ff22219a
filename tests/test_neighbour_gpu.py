"""The steps around the verify attention on the GPU against the oracle: query
preparation (split, NeoX rotation, w_kc absorb), the w_vc value projection, the
tree's appended cache rows, and the whole chain parent -> visibility -> append
-> prepare -> attention -> value projection.

Bars: float32 results within 1e-4 + 1e-4 |ref| (the fp32 tolerance of the verify
step); latents copied into the cache bit-exact (float32) or equal to their
round-to-nearest-even bf16 or FP8 E4M3 codes (narrow caches); rotated narrow keys
within one code of the oracle's value rounded the same way (the rotation's
float64 result is rounded to float32 first on both sides, so the two can straddle
a tie only by float64 rounding noise)."""
import numpy as np
import pytest

import oracle
import workloads as wl
from parity import assert_close, oracle_rows, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def build_vis(parent, prefix):
    import tree_masked_mla_amd as dd
    B, Q = parent.shape
    buf = torch.empty(dd.ddtv_vis_bytes(B, Q), dtype=torch.uint8, device="cuda")
    rc, vis = dd.ddtv_build_visibility(dev(parent.astype(np.int32)), np.ascontiguousarray(prefix, np.int32), B, Q,
                                       buf)
    assert rc == dd.DDTV_OK
    return vis, buf


def trees(seed, B, Q, kind="uniform", depth_cap=12):
    rng = np.random.default_rng(seed)
    if kind == "best_first":
        return np.stack([wl.best_first_tree(rng, Q, depth_cap) for _ in range(B)]).astype(np.int32)
    return np.stack([wl.uniform_tree(rng, Q) for _ in range(B)]).astype(np.int32)


def input_positions(parent, prefix):
    """Explicit positions handed to the kernels (input helper: prefix + depth)."""
    return np.stack([prefix[b] + wl.tree_depths(parent[b]) for b in range(parent.shape[0])]).astype(np.int32)


def run_prepare(nb, vis, positions=None):
    import tree_masked_mla_amd as dd
    B, Q, H, _ = nb.q.shape
    q_abs = torch.full((B, Q, H, 512), float("nan"), device="cuda")
    q_rope = torch.full((B, Q, H, 64), float("nan"), device="cuda")
    rc = dd.ddtv_prepare_query(dev(nb.q), dev(nb.w_kc), vis, q_abs, q_rope, nb.theta,
                               positions=None if positions is None else dev(positions))
    assert rc == dd.DDTV_OK
    torch.cuda.synchronize()
    return q_abs.cpu().numpy(), q_rope.cpu().numpy()


CASES = [
    # (seed, B, Q, H, d_nope, prefix, explicit positions)
    (1, 1, 9, 8, 128, [0], False),
    (2, 3, 9, 8, 128, [37, 37, 37], True),
    (3, 3, 37, 5, 64, [5, 0, 1000], False),        # 111 nodes: a ragged 64-row tile
    (4, 2, 33, 3, 256, [130000, 7], True),          # two mask words, positions past 2^17
    (5, 1, 64, 16, 32, [4096], False),
]


@pytest.mark.parametrize("seed,B,Q,H,d_nope,prefix,explicit", CASES)
def test_prepare_query_matches_oracle(seed, B, Q, H, d_nope, prefix, explicit):
    say(f"prepare_query B={B} Q={Q} H={H} d_nope={d_nope} explicit={explicit}")
    prefix = np.asarray(prefix, np.int32)
    par = trees(seed, B, Q)
    nb = wl.neighbour_inputs(100 + seed, B, Q, H, d_nope=d_nope)
    vis, _buf = build_vis(par, prefix)
    pos_in = input_positions(par, prefix) if explicit else None
    qa, qr = run_prepare(nb, vis, pos_in)
    ra, rr = oracle.prepare_query(nb.q, oracle.tree_positions(par, prefix).reshape(-1), nb.theta, nb.w_kc)
    assert_close(qa, ra, 0, "q_abs")
    err = np.abs(qr - rr)
    assert (err <= 1e-6 + 1e-6 * np.abs(rr)).all(), f"q_rope max abs err {err.max():.3e}"


@pytest.mark.parametrize("name", ["c4", "c5"])
def test_prepare_query_full_size_sampled(name):
    """The verify workloads' node and head counts with d_nope = 128: all nodes on
    the GPU, a seeded sample of 96 (node, head) rows through the oracle."""
    parent, prefix = wl.config_trees(name)
    B, Q = parent.shape
    H = wl.CONFIGS[name]["H"]
    say(f"prepare_query full size {name}: B={B} Q={Q} H={H}")
    nb = wl.neighbour_inputs(7, B, Q, H)
    vis, _buf = build_vis(parent, prefix)
    qa, qr = run_prepare(nb, vis)
    pos = oracle.tree_positions(parent, prefix).reshape(-1)
    rng = np.random.default_rng(9)
    nodes = rng.choice(B * Q, size=96, replace=False)
    heads = rng.integers(0, H, size=96)
    q = nb.q.reshape(B * Q, H, -1)
    for n, h in zip(nodes, heads):
        ra, rr = oracle.prepare_query(q[n:n + 1, h:h + 1], pos[n:n + 1], nb.theta, nb.w_kc[h:h + 1])
        assert_close(qa.reshape(B * Q, H, 512)[n, h], ra[0, 0], 0, f"q_abs node {n} head {h}")
        got = qr.reshape(B * Q, H, 64)[n, h]
        assert np.allclose(got, rr[0, 0], rtol=1e-6, atol=1e-6), (n, h)
    assert np.isfinite(qa).all() and np.isfinite(qr).all()


# (the small grids run the split-K kernel; (640, 4, 128) the narrow one, (1024, 16, 128) the wide one)
@pytest.mark.parametrize("M,H,d_v", [(9, 8, 128), (111, 5, 96), (64, 3, 32), (1, 1, 1), (1024, 16, 128),
                                     (200, 2, 512), (640, 4, 128)])
def test_value_proj_matches_oracle(M, H, d_v):
    import tree_masked_mla_amd as dd
    say(f"value_proj M={M} H={H} d_v={d_v}")
    nb = wl.neighbour_inputs(30 + M, 1, 1, H, d_v=d_v)
    lat = np.random.default_rng(M).standard_normal((M, H, 512), dtype=np.float32)
    v = torch.full((M, H, d_v), float("nan"), device="cuda")
    assert dd.ddtv_value_proj(dev(lat), dev(nb.w_vc), v) == dd.DDTV_OK
    torch.cuda.synchronize()
    assert_close(v.cpu().numpy(), oracle.value_proj(lat, nb.w_vc), 0, "v")


def test_value_proj_empty_is_a_no_op():
    import tree_masked_mla_amd as dd
    w = torch.zeros((2, 128, 512), device="cuda")
    v = torch.full((1,), 5.0, device="cuda")
    lat = torch.zeros((1,), device="cuda")
    assert dd.load().ddtv_value_proj(lat.data_ptr(), 0, 2, 128, w.data_ptr(), v.data_ptr(), None) == dd.DDTV_OK
    torch.cuda.synchronize()
    assert v.item() == 5.0


@pytest.mark.parametrize("kv_dtype", [wl.F32, wl.BF16, wl.FP8])
@pytest.mark.parametrize("explicit", [False, True])
def test_append_kv_matches_oracle(kv_dtype, explicit):
    import tree_masked_mla_amd as dd
    from tree_masked_mla_amd.runner import to_device_kv
    say(f"append_kv dtype={kv_dtype} explicit={explicit}")
    B, Q = 3, 40
    prefix = np.array([17, 0, 300], np.int32)
    par = trees(41, B, Q)
    nb = wl.neighbour_inputs(42, B, Q, 1)
    total = int((prefix + Q).sum())
    rng = np.random.default_rng(43)
    ckv0 = rng.standard_normal((total, 512), dtype=np.float32)
    kr0 = rng.standard_normal((total, 64), dtype=np.float32)
    narrow = {wl.BF16: (wl.round_bf16_bits, wl.bf16_bits_to_f32, torch.int16, np.uint16),
              wl.FP8: (wl.round_fp8_bits, wl.fp8_bits_to_f32, torch.uint8, np.uint8)}.get(kv_dtype)
    if narrow:
        ckv0, kr0 = narrow[0](ckv0), narrow[0](kr0)
    ckv = to_device_kv(ckv0, kv_dtype, "cuda")
    kr = to_device_kv(kr0, kv_dtype, "cuda")
    vis, _buf = build_vis(par, prefix)
    pos_in = dev(input_positions(par, prefix)) if explicit else None
    assert dd.ddtv_append_kv(dev(nb.latent), dev(nb.k_pe), vis, ckv, kr, kv_dtype, nb.theta,
                             positions=pos_in) == dd.DDTV_OK
    torch.cuda.synchronize()
    pos = oracle.tree_positions(par, prefix)
    base_c = narrow[1](ckv0) if narrow else ckv0
    base_k = narrow[1](kr0) if narrow else kr0
    ref_c, ref_k = oracle.append_kv(nb.latent, nb.k_pe, pos, prefix, nb.theta, base_c, base_k)
    if narrow:
        got_c = ckv.view(narrow[2]).cpu().numpy().view(narrow[3])
        got_k = kr.view(narrow[2]).cpu().numpy().view(narrow[3])
        want_c = narrow[0](ref_c.astype(np.float32))
        assert np.array_equal(got_c, want_c), "latent rows differ from their round-to-nearest-even codes"
        want_k = narrow[0](ref_k.astype(np.float32))
        ulps = np.abs(got_k.astype(np.int32) - want_k.astype(np.int32))
        assert ulps.max() <= 1, f"rotated keys off by {ulps.max()} ulps"
        owned = np.zeros(total, bool)
        off = 0
        for b in range(B):
            owned[off + prefix[b]: off + prefix[b] + Q] = True
            off += int(prefix[b]) + Q
        assert np.array_equal(got_k[~owned], kr0[~owned]), "rows outside the trees changed"
    else:
        got_c = ckv.cpu().numpy()
        got_k = kr.cpu().numpy()
        assert np.array_equal(got_c, ref_c.astype(np.float32)), "latent rows must be copied exactly"
        err = np.abs(got_k - ref_k)
        assert (err <= 1e-6 + 1e-6 * np.abs(ref_k)).all(), f"rotated keys max abs err {err.max():.3e}"


@pytest.mark.parametrize("name,d_nope,d_v", [("c2", 128, 128), ("c3", 128, 128), ("c2", 64, 96)])
def test_chain_matches_oracle(name, d_nope, d_v):
    """parent -> visibility -> append -> prepare -> verify attention -> value
    projection, every step through the C ABI, against the oracle's chain."""
    import tree_masked_mla_amd as dd
    from tree_masked_mla_amd.runner import to_device_kv
    w = wl.config(name)
    say(f"chain {name} d_nope={d_nope} d_v={d_v}")
    nb = wl.neighbour_inputs(55, w.B, w.Q, w.H, d_nope=d_nope, d_v=d_v)
    vis, _buf = build_vis(w.parent, w.prefix)
    ckv = to_device_kv(w.ckv, w.kv_dtype, "cuda")
    kr = to_device_kv(w.k_rope, w.kv_dtype, "cuda")
    assert dd.ddtv_append_kv(dev(nb.latent), dev(nb.k_pe), vis, ckv, kr, w.kv_dtype, nb.theta) == dd.DDTV_OK
    q_abs = torch.empty((w.B, w.Q, w.H, 512), device="cuda")
    q_rope = torch.empty((w.B, w.Q, w.H, 64), device="cuda")
    assert dd.ddtv_prepare_query(dev(nb.q), dev(nb.w_kc), vis, q_abs, q_rope, nb.theta) == dd.DDTV_OK
    out = torch.empty((w.B, w.Q, w.H, 512), device="cuda")
    need = dd.ddtv_workspace_bytes(vis, w.H, w.kv_dtype)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    assert dd.ddtv_verify_attn(q_abs, q_rope, ckv, kr, w.kv_dtype, w.H, vis, w.scale, out, None, ws,
                               need) == dd.DDTV_OK
    v = torch.empty((w.B, w.Q, w.H, d_v), device="cuda")
    assert dd.ddtv_value_proj(out, dev(nb.w_vc), v) == dd.DDTV_OK
    torch.cuda.synchronize()

    # the oracle's chain, from the same inputs
    pos = oracle.tree_positions(w.parent, w.prefix)
    ra, rr = oracle.prepare_query(nb.q, pos.reshape(-1), nb.theta, nb.w_kc)
    rc, rk = oracle.append_kv(nb.latent, nb.k_pe, pos, w.prefix, nb.theta, w.ckv, w.k_rope)
    bits, _, _ = oracle.build_visibility(w.parent)
    w2 = wl.Workload(name=w.name, B=w.B, H=w.H, Q=w.Q, prefix=w.prefix, parent=w.parent,
                     q_abs=ra.astype(np.float32), q_rope=rr.astype(np.float32), ckv=rc.astype(np.float32),
                     k_rope=rk.astype(np.float32), kv_dtype=wl.F32, scale=w.scale)
    ref_out, _ = oracle_rows(w2, bits)
    ref_v = oracle.value_proj(ref_out.astype(np.float32).reshape(w.B, w.Q, w.H, 512), nb.w_vc)
    assert_close(out.cpu().numpy().reshape(-1, 512), ref_out, 0, "latent out")
    assert_close(v.cpu().numpy(), ref_v, 0, "value")
