"""Pins for the oracle of the steps around the verify attention.

The steps (pages: "The Query-Split Kernel: A Pivotal Edit in Building a Native
DDTree Inference Engine", sections "The Reasoning Chain" and "Input Knowledge";
"The Verify-Attn Kernel: A Single File Write ...", section "Design Decisions and
Trade-Offs"): the query projection splits into a nope part, absorbed into latent
space through w_kc, and a rope part that gets NeoX rotary embedding; after the
attention, a per-head GEMM with w_vc maps the latent to the value.

What pins them, none of it the oracle's own code:
  - rotary embedding against rotation written as complex multiplication
    (pair i is the complex number x[i] + i x[i+32], turned by pos * theta^(-i/32));
    position 0 is the identity; pair norms are kept; scores depend only on the
    difference of positions;
  - the absorb against the un-absorbed key: q_abs . c must equal nope . (W_kc c)
    for any latent c (numpy matmul); one-hot queries pick a weight row exactly;
  - the value projection against numpy matmul and one-hot latents;
  - the whole chain (positions, query prep, appended keys, masked attention,
    value projection) against naive, un-absorbed multi-head attention in float64
    torch on the CPU, with keys W_kc c_j and values W_vc c_j built per head;
  - tree positions against chains, stars and the popcount of ancestor masks.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

THETAS = (wl.ROPE_THETA, 10000.0)


def complex_rope(x: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotary embedding as complex multiplication (float64)."""
    x = np.asarray(x, dtype=np.float64)
    z = x[:32] + 1j * x[32:]
    freq = theta ** (-np.arange(32, dtype=np.float64) / 32.0)
    w = z * np.exp(1j * (pos * freq))
    return np.concatenate([w.real, w.imag])


@pytest.mark.parametrize("theta", THETAS)
def test_rope_is_complex_rotation(theta):
    rng = np.random.default_rng(3)
    for pos in (0, 1, 2, 7, 100, 4096, 32779, 131135):
        x = rng.standard_normal(64).astype(np.float32)
        y = oracle.rope_neox(x, pos, theta)
        ref = complex_rope(x, pos, theta)
        # the two evaluations may differ by an ulp of the frequency, i.e. pos * 2.2e-16 rad
        tol = 2e-15 * max(1, pos) * np.abs(x).max() + 1e-13
        assert np.allclose(y, ref, rtol=0, atol=tol), (pos, np.abs(y - ref).max())


def test_rope_unit_vectors_closed_form():
    # e_0 at position p turns to cos p e_0 + sin p e_32 (frequency 1 for pair 0);
    # e_32 turns to -sin p e_0 + cos p e_32.
    e = np.eye(64, dtype=np.float32)
    for p in (1, 3, 50):
        y0 = oracle.rope_neox(e[0], p, wl.ROPE_THETA)
        y1 = oracle.rope_neox(e[32], p, wl.ROPE_THETA)
        assert y0[0] == pytest.approx(math.cos(p), abs=1e-15) and y0[32] == pytest.approx(math.sin(p), abs=1e-15)
        assert y1[0] == pytest.approx(-math.sin(p), abs=1e-15) and y1[32] == pytest.approx(math.cos(p), abs=1e-15)
        assert np.count_nonzero(np.delete(y0, [0, 32])) == 0
    # the last pair turns at theta^(-31/32) radians per position
    y = oracle.rope_neox(e[31], 1000, wl.ROPE_THETA)
    a = 1000 * wl.ROPE_THETA ** (-31 / 32)
    assert y[31] == pytest.approx(math.cos(a), abs=1e-14) and y[63] == pytest.approx(math.sin(a), abs=1e-14)


def test_rope_identity_norms_and_relative_positions():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(64).astype(np.float32)
    k = rng.standard_normal(64).astype(np.float32)
    assert np.array_equal(oracle.rope_neox(x, 0, wl.ROPE_THETA), x.astype(np.float64))
    for p in (9, 777):
        y = oracle.rope_neox(x, p, wl.ROPE_THETA)
        xd = x.astype(np.float64)
        assert np.allclose(y[:32] ** 2 + y[32:] ** 2, xd[:32] ** 2 + xd[32:] ** 2, rtol=1e-13, atol=1e-14)
    # <rope(x, m), rope(k, n)> depends on m - n only
    for m, n in ((40, 7), (1000, 900), (5, 5)):
        a = oracle.rope_neox(x, m, wl.ROPE_THETA) @ oracle.rope_neox(k, n, wl.ROPE_THETA)
        b = oracle.rope_neox(x, m - n + 3, wl.ROPE_THETA) @ oracle.rope_neox(k, 3, wl.ROPE_THETA)
        assert a == pytest.approx(b, abs=1e-11)


def test_absorb_equals_unabsorbed_key_and_rope_part():
    B, Q, H = 2, 5, 3
    nb = wl.neighbour_inputs(11, B, Q, H, d_nope=128)
    pos = np.arange(B * Q, dtype=np.int32) * 13
    q_abs, q_rope = oracle.prepare_query(nb.q, pos, nb.theta, nb.w_kc)
    rng = np.random.default_rng(1)
    c = rng.standard_normal((4, 512))
    for b in range(B):
        for i in range(Q):
            for h in range(H):
                nope = nb.q[b, i, h, :128].astype(np.float64)
                k_nope = nb.w_kc[h].astype(np.float64) @ c.T          # un-absorbed keys [128][4]
                assert np.allclose(q_abs[b, i, h] @ c.T, nope @ k_nope, rtol=1e-12, atol=1e-11)
                ref = complex_rope(nb.q[b, i, h, 128:], int(pos[b * Q + i]), nb.theta)
                assert np.allclose(q_rope[b, i, h], ref, atol=1e-10)


def test_absorb_one_hot_picks_weight_rows():
    H, d_nope = 2, 32
    nb = wl.neighbour_inputs(12, 1, 1, H, d_nope=d_nope)
    q = np.zeros((d_nope, H, d_nope + 64), dtype=np.float32)
    for k in range(d_nope):
        q[k, :, k] = 1.0
    q_abs, q_rope = oracle.prepare_query(q, np.zeros(d_nope, np.int32), nb.theta, nb.w_kc)
    for k in range(d_nope):
        for h in range(H):
            assert np.array_equal(q_abs[k, h], nb.w_kc[h, k].astype(np.float64))
    assert not q_rope.any()


def test_value_projection_matmul_and_one_hot():
    H, d_v = 3, 64
    nb = wl.neighbour_inputs(13, 1, 1, H, d_v=d_v)
    rng = np.random.default_rng(2)
    o = rng.standard_normal((6, H, 512)).astype(np.float32)
    v = oracle.value_proj(o, nb.w_vc)
    for m in range(6):
        for h in range(H):
            ref = nb.w_vc[h].astype(np.float64) @ o[m, h].astype(np.float64)
            assert np.allclose(v[m, h], ref, rtol=1e-12, atol=1e-12)
    e = np.zeros((2, H, 512), dtype=np.float32)
    e[0, :, 5] = 1.0
    e[1, :, 511] = 1.0
    v = oracle.value_proj(e, nb.w_vc)
    for h in range(H):
        assert np.array_equal(v[0, h], nb.w_vc[h, :, 5].astype(np.float64))
        assert np.array_equal(v[1, h], nb.w_vc[h, :, 511].astype(np.float64))


def test_tree_positions():
    pre = np.array([0, 17], np.int32)
    chain = np.stack([wl.chain_tree(6)] * 2)
    assert np.array_equal(oracle.tree_positions(chain, pre), pre[:, None] + np.arange(6)[None, :])
    star = np.array([[-1, 0, 0, 0, 0]] * 2, np.int32)
    assert np.array_equal(oracle.tree_positions(star, pre), pre[:, None] + np.array([0, 1, 1, 1, 1])[None, :])
    rng = np.random.default_rng(4)
    par = np.stack([wl.uniform_tree(rng, 40) for _ in range(3)])
    pre = np.array([5, 0, 300], np.int32)
    bits, _, _ = oracle.build_visibility(par)
    depth = np.vectorize(lambda u: bin(int(u)).count("1"))(bits).sum(-1) - 1
    assert np.array_equal(oracle.tree_positions(par, pre), pre[:, None] + depth)


def test_append_kv_rows():
    B, Q, P = 2, 4, np.array([3, 0], np.int32)
    nb = wl.neighbour_inputs(14, B, Q, 1)
    total = int((P + Q).sum())
    ckv = np.full((total, 512), 7.0)
    kr = np.full((total, 64), 7.0)
    pos = np.array([[3, 4, 4, 5], [0, 1, 2, 1]], np.int32)
    c2, k2 = oracle.append_kv(nb.latent, nb.k_pe, pos, P, nb.theta, ckv, kr)
    owned = {3 + i: (0, i) for i in range(Q)}
    owned.update({7 + i: (1, i) for i in range(Q)})
    for r in range(total):
        if r in owned:
            b, i = owned[r]
            assert np.array_equal(c2[r], nb.latent[b, i].astype(np.float64))
            assert np.allclose(k2[r], complex_rope(nb.k_pe[b, i], int(pos[b, i]), nb.theta), atol=1e-12)
        else:
            assert (c2[r] == 7.0).all() and (k2[r] == 7.0).all()


def naive_mla(par, prefix, ckv_pre, kr_pre, nb, scale, d_nope):
    """Un-absorbed multi-head attention of every tree node, float64 torch on the CPU.
    Per head: key_j = [W_kc c_j ; kr_j], value_j = W_vc c_j, query = [nope ; rope(pe, pos)],
    positions and visibility from a Python walk over the parent links."""
    B, Q = par.shape
    H = nb.w_kc.shape[0]
    outs = np.zeros((B, Q, H, nb.w_vc.shape[1]))
    for b in range(B):
        P = int(prefix[b])
        depth = [0] * Q
        anc = [set([0])] + [None] * (Q - 1)
        for i in range(1, Q):
            depth[i] = depth[par[b, i]] + 1
            anc[i] = anc[par[b, i]] | {i}
        c = np.concatenate([ckv_pre[b], nb.latent[b].astype(np.float64)])        # [P+Q][512]
        kr_new = np.stack([complex_rope(nb.k_pe[b, i], P + depth[i], nb.theta) for i in range(Q)])
        kr = np.concatenate([kr_pre[b], kr_new])
        ct = torch.from_numpy(c)
        for h in range(H):
            wk = torch.from_numpy(nb.w_kc[h].astype(np.float64))                  # [d_nope][512]
            wv = torch.from_numpy(nb.w_vc[h].astype(np.float64))                  # [d_v][512]
            K = torch.cat([ct @ wk.T, torch.from_numpy(kr)], dim=1)              # [P+Q][d_nope+64]
            V = ct @ wv.T                                                         # [P+Q][d_v]
            for i in range(Q):
                qn = torch.from_numpy(nb.q[b, i, h, :d_nope].astype(np.float64))
                qr = torch.from_numpy(complex_rope(nb.q[b, i, h, d_nope:], P + depth[i], nb.theta))
                s = scale * (K @ torch.cat([qn, qr]))
                vis = torch.zeros(P + Q, dtype=torch.bool)
                vis[:P] = True
                vis[[P + a for a in anc[i]]] = True
                s = s.masked_fill(~vis, -math.inf)
                outs[b, i, h] = (torch.softmax(s, 0) @ V).numpy()
    return outs


@pytest.mark.parametrize("d_nope,d_v", [(128, 128), (64, 96)])
def test_chain_equals_unabsorbed_attention(d_nope, d_v):
    B, Q, H = 2, 9, 3
    rng = np.random.default_rng(21)
    par = np.stack([wl.uniform_tree(rng, Q) for _ in range(B)])
    prefix = np.array([6, 11], np.int32)
    ckv_pre = [rng.standard_normal((int(p), 512)) * 0.5 for p in prefix]
    kr_pre = [rng.standard_normal((int(p), 64)) for p in prefix]
    nb = wl.neighbour_inputs(22, B, Q, H, d_nope=d_nope, d_v=d_v)
    scale = 1.0 / math.sqrt(d_nope + 64)
    ref = naive_mla(par, prefix, ckv_pre, kr_pre, nb, scale, d_nope)

    pos = oracle.tree_positions(par, prefix)
    q_abs, q_rope = oracle.prepare_query(nb.q, pos.reshape(-1), nb.theta, nb.w_kc)
    total = int((prefix + Q).sum())
    ckv = np.zeros((total, 512))
    kr = np.zeros((total, 64))
    off = 0
    for b in range(B):
        ckv[off:off + prefix[b]] = ckv_pre[b]
        kr[off:off + prefix[b]] = kr_pre[b]
        off += int(prefix[b]) + Q
    ckv, kr = oracle.append_kv(nb.latent, nb.k_pe, pos, prefix, nb.theta, ckv, kr)
    bits, _, _ = oracle.build_visibility(par)
    # the attention oracle takes float32 operands: round once here
    out, _ = oracle.verify_attn(q_abs.astype(np.float32), q_rope.astype(np.float32), ckv.astype(np.float32),
                                kr.astype(np.float32), 0, prefix, bits, scale)
    v = oracle.value_proj(out.astype(np.float32).reshape(B, Q, H, 512), nb.w_vc)
    assert np.allclose(v, ref, rtol=1e-5, atol=1e-5), np.abs(v - ref).max()
