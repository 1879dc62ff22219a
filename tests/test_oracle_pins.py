"""Pins for the CPU oracle: each check compares it with something other than itself.

Sources of truth used here: closed forms written out with Python's math module,
PyTorch's scaled_dot_product_attention in float64 on the CPU (a library routine),
invariants of softmax attention, brute force over every small tree, and the
test shapes printed by the pages (tests/golden/page_test_shapes.txt).

The attention being pinned is the absorbed-MLA tree-verify attention described on
"The Verify-Attn Kernel: A Single File Write That Completed a Critical Piece of
the DDTree Engine" (sections "The Design Journey: From Concept to CUDA",
"Design Decisions and Trade-Offs", "Assumptions and the Path Forward").
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- helpers
def closure_visibility(parent: np.ndarray) -> np.ndarray:
    """Ancestor-or-self matrix of one tree via boolean powers of the parent
    adjacency matrix (independent of the oracle's walk)."""
    Q = len(parent)
    A = np.zeros((Q, Q), dtype=np.int64)
    for i in range(1, Q):
        A[i, parent[i]] = 1
    M = np.eye(Q, dtype=np.int64)
    P = np.eye(Q, dtype=np.int64)
    for _ in range(Q):
        P = (P @ A > 0).astype(np.int64)
        M |= P
    return M.astype(bool)


def bits_to_bool(bits: np.ndarray, Q: int) -> np.ndarray:
    """uint32 [.., W] -> bool [.., Q] (LSB-first unpacking)."""
    W = bits.shape[-1]
    k = np.arange(W * 32)
    full = (bits[..., k // 32] >> (k % 32).astype(np.uint32)) & 1
    return full[..., :Q].astype(bool)


def bool_to_bits(vis: np.ndarray) -> np.ndarray:
    Q = vis.shape[-1]
    W = (Q + 31) // 32
    out = np.zeros(vis.shape[:-1] + (W,), dtype=np.uint32)
    for a in range(Q):
        out[..., a // 32] |= (vis[..., a].astype(np.uint32) << np.uint32(a % 32))
    return out


def kv_f64(a, kv_dtype):
    if kv_dtype == wl.FP8:
        return wl.fp8_bits_to_f32(a).astype(np.float64)
    return (wl.bf16_bits_to_f32(a) if kv_dtype == wl.BF16 else a).astype(np.float64)


def torch_reference(w, vis_tree: np.ndarray):
    """Masked attention per batch row with torch SDPA in float64.

    vis_tree: bool [B][Q][Q] -- which tree nodes each node sees.  The prefix is
    fully visible.  Returns (out [B*Q*H][512], lse [B*Q*H])."""
    outs, lses = [], []
    off = w.kv_off
    for b in range(w.B):
        P = int(w.prefix[b])
        kv = slice(int(off[b]), int(off[b + 1]))
        ckv = torch.from_numpy(kv_f64(w.ckv[kv], w.kv_dtype))
        kr = torch.from_numpy(kv_f64(w.k_rope[kv], w.kv_dtype))
        K = torch.cat([ckv, kr], dim=1)                      # [KV, 576]
        V = ckv                                              # value = latent only
        qa = torch.from_numpy(w.q_abs[b].astype(np.float64))  # [Q, H, 512]
        qr = torch.from_numpy(w.q_rope[b].astype(np.float64))
        Qm = torch.cat([qa, qr], dim=2).reshape(w.Q * w.H, 576)
        mask = np.zeros((w.Q, P + w.Q), dtype=bool)
        mask[:, :P] = True
        mask[:, P:] = vis_tree[b]
        mrow = torch.from_numpy(np.repeat(mask, w.H, axis=0))  # rows are (q, h)
        o = torch.nn.functional.scaled_dot_product_attention(
            Qm[None], K[None], V[None], attn_mask=mrow[None], scale=w.scale)[0]
        s = (Qm @ K.T) * w.scale
        s = s.masked_fill(~mrow, float("-inf"))
        outs.append(o.numpy())
        lses.append(torch.logsumexp(s, dim=1).numpy())
    return np.concatenate(outs), np.concatenate(lses)


def small(name="t", seed=5, B=2, H=3, Q=6, prefix=(4, 0), tree="uniform", kv_dtype=wl.F32,
          scale=wl.SCALE_192, **kw):
    return wl.make_workload(name, seed, B=B, H=H, Q=Q, prefix=list(prefix) if not np.isscalar(prefix) else prefix,
                            tree=tree, kv_dtype=kv_dtype, scale=scale, **kw)


# ----------------------------------------------------------------------------- golden shapes
def read_page_shapes():
    rows = []
    with open(os.path.join(GOLDEN, "page_test_shapes.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tag, B, H, P, q, kv = line.split()
            rows.append((tag, int(B), int(H), int(P), int(q), int(kv)))
    return rows


def test_page_shapes_fix_layout_readings():
    """The printed shapes fix two readings: q_len = budget + 1 (the root is a
    query) and kv_len = prefix + q_len (tree rows follow the prefix)."""
    rows = read_page_shapes()
    assert len(rows) == 3
    for tag, B, H, P, q, kv in rows:
        h, p, bud = tag.split("_")
        assert int(h[1:]) == H and int(p[1:]) == P
        assert q == int(bud[1:]) + 1
        assert kv == P + q


@pytest.mark.parametrize("shape", read_page_shapes(), ids=lambda s: s[0])
def test_page_shapes_match_torch(shape):
    """Oracle on each printed shape (uniform trees, inputs of std 0.05 as the page's
    tests used) against float64 SDPA with the closure mask."""
    tag, B, H, P, q, kv = shape
    w = wl.make_workload(tag, 11, B=B, H=H, Q=q, prefix=P, q_sigma=0.05, kv_sigma=0.05)
    assert w.total_kv == B * kv
    bits, bad, rc = oracle.build_visibility(w.parent)
    assert rc == 0 and (bad == -1).all()
    out, lse = oracle.attend_workload(w, bits=bits)
    vis = np.stack([closure_visibility(w.parent[b]) for b in range(B)])
    ro, rl = torch_reference(w, vis)
    np.testing.assert_allclose(out, ro, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- closed forms
def _two_node_case(qa_vals, qr_vals, scale):
    """H=1, Q=2, P=0, tree 0 <- 1.  Latent rows e0*2 and e1*3; rope rows e0 and -e1."""
    B, H, Q = 1, 1, 2
    q_abs = np.zeros((B, Q, H, 512), np.float32)
    q_rope = np.zeros((B, Q, H, 64), np.float32)
    q_abs[0, 1, 0, :2] = qa_vals
    q_rope[0, 1, 0, :2] = qr_vals
    ckv = np.zeros((2, 512), np.float32)
    ckv[0, 0] = 2.0
    ckv[1, 1] = 3.0
    kr = np.zeros((2, 64), np.float32)
    kr[0, 0] = 1.0
    kr[1, 1] = -1.0
    parent = np.array([[-1, 0]], np.int32)
    bits, _, _ = oracle.build_visibility(parent)
    out, lse = oracle.verify_attn(q_abs, q_rope, ckv, kr, 0, np.zeros(1, np.int32), bits, scale)
    return out, lse


def test_closed_form_latent_scores():
    x, y = 0.75, -1.25
    scale = 0.5
    out, lse = _two_node_case([x, y], [0.0, 0.0], scale)
    s0, s1 = scale * (x * 2.0), scale * (y * 3.0)
    z = math.exp(s0) + math.exp(s1)
    # node 0 sees only itself: its latent row, lse = its score (0 here)
    assert out[0, 0] == 2.0 and np.count_nonzero(out[0]) == 1
    assert lse[0] == 0.0
    assert math.isclose(out[1, 0], 2.0 * math.exp(s0) / z, rel_tol=1e-15)
    assert math.isclose(out[1, 1], 3.0 * math.exp(s1) / z, rel_tol=1e-15)
    assert np.count_nonzero(out[1, 2:]) == 0
    assert math.isclose(lse[1], math.log(z), rel_tol=1e-15)


def test_closed_form_rope_scores_value_excludes_rope():
    """Scores coming only from the rope term; the output holds latent values only."""
    a, c = 1.5, 0.25
    scale = 1.0 / math.sqrt(192.0)
    out, lse = _two_node_case([0.0, 0.0], [a, c], scale)
    s0 = scale * (a * 1.0)
    s1 = scale * (c * -1.0)
    s0, s1 = float(np.float64(s0)), float(np.float64(s1))
    z = math.exp(s0) + math.exp(s1)
    assert math.isclose(out[1, 0], 2.0 * math.exp(s0) / z, rel_tol=1e-14)
    assert math.isclose(out[1, 1], 3.0 * math.exp(s1) / z, rel_tol=1e-14)
    assert math.isclose(lse[1], math.log(z), rel_tol=1e-14)


def test_bf16_widening_exact():
    """bf16 patterns are read as the float32 with the same top 16 bits."""
    B, H, Q = 1, 1, 1
    q_abs = np.ones((B, Q, H, 512), np.float32)
    q_rope = np.ones((B, Q, H, 64), np.float32)
    ckv = np.zeros((1, 512), np.uint16)
    ckv[0, :4] = [0x3F80, 0xC000, 0x3E20, 0x0001]   # 1, -2, 0.15625, smallest subnormal
    kr = np.zeros((1, 64), np.uint16)
    bits, _, _ = oracle.build_visibility(np.array([[-1]], np.int32))
    out, lse = oracle.verify_attn(q_abs, q_rope, ckv, kr, 1, np.zeros(1, np.int32), bits, 1.0)
    assert out[0, 0] == 1.0 and out[0, 1] == -2.0 and out[0, 2] == 0.15625
    assert out[0, 3] == 2.0 ** -133
    assert lse[0] == 1.0 - 2.0 + 0.15625 + 2.0 ** -133


# ----------------------------------------------------------------------------- P1 / P2 library routine
@pytest.mark.parametrize("kv_dtype", [wl.F32, wl.BF16, wl.FP8])
def test_chain_equals_causal(kv_dtype):
    """A chain tree is causal attention offset by the prefix (the prefill mode)."""
    w = small(B=3, H=4, Q=11, prefix=(0, 7, 40), tree="chain", kv_dtype=kv_dtype)
    bits, _, _ = oracle.build_visibility(w.parent)
    out, lse = oracle.attend_workload(w, bits=bits)
    causal = np.tril(np.ones((w.Q, w.Q), bool))
    ro, rl = torch_reference(w, np.stack([causal] * w.B))
    np.testing.assert_allclose(out, ro, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


def test_c2_chain_variant_equals_causal():
    w = wl.c2_chain()
    out, lse = oracle.attend_workload(w)
    causal = np.tril(np.ones((w.Q, w.Q), bool))
    ro, rl = torch_reference(w, np.stack([causal] * w.B))
    np.testing.assert_allclose(out, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


def test_single_query_equals_dense():
    """q_len = 1 (autoregressive decode): dense softmax over the whole cache."""
    w = small(B=2, H=5, Q=1, prefix=(33, 2))
    out, lse = oracle.attend_workload(w)
    ro, rl = torch_reference(w, np.ones((w.B, 1, 1), bool))
    np.testing.assert_allclose(out, ro, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


def test_all_ones_mask_equals_dense():
    w = small(B=2, H=2, Q=37, prefix=(5, 19))
    ones = np.ones((w.B, w.Q, w.Q), bool)
    out, lse = oracle.attend_workload(w, bits=bool_to_bits(ones))
    ro, rl = torch_reference(w, ones)
    np.testing.assert_allclose(out, ro, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_small_configs_match_torch(name):
    w = wl.config(name)
    bits, bad, rc = oracle.build_visibility(w.parent)
    assert rc == 0
    out, lse = oracle.attend_workload(w, bits=bits)
    vis = np.stack([closure_visibility(w.parent[b]) for b in range(w.B)])
    ro, rl = torch_reference(w, vis)
    np.testing.assert_allclose(out, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


def test_ragged_bf16_matches_torch():
    w = small(B=3, H=2, Q=40, prefix=(0, 3, 70), tree="best_first", depth_cap=5, kv_dtype=wl.BF16)
    out, lse = oracle.attend_workload(w)
    vis = np.stack([closure_visibility(w.parent[b]) for b in range(w.B)])
    ro, rl = torch_reference(w, vis)
    np.testing.assert_allclose(out, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- P3 exact special case
def test_single_visible_position_exact():
    """With no prefix the root sees only its own row: the output is that latent row."""
    w = wl.config("c1")
    out, lse = oracle.attend_workload(w, rows=np.arange(w.H))   # node 0, every head
    for h in range(w.H):
        assert np.array_equal(out[h], w.ckv[0].astype(np.float64))
        s = w.scale * (np.dot(w.q_abs[0, 0, h].astype(np.float64), w.ckv[0].astype(np.float64))
                       + np.dot(w.q_rope[0, 0, h].astype(np.float64), w.k_rope[0].astype(np.float64)))
        assert math.isclose(lse[h], s, rel_tol=1e-13, abs_tol=1e-13)


def test_single_bit_mask_exact():
    w = small(B=1, H=3, Q=5, prefix=0)
    one = np.zeros((1, 5, 5), bool)
    one[0, :, 3] = True                   # every node sees only node 3
    out, _ = oracle.attend_workload(w, bits=bool_to_bits(one))
    for r in range(out.shape[0]):
        assert np.array_equal(out[r], w.ckv[3].astype(np.float64))


def test_empty_mask_row():
    w = small(B=1, H=2, Q=4, prefix=0)
    none = np.zeros((1, 4, 4), bool)
    out, lse = oracle.attend_workload(w, bits=bool_to_bits(none))
    assert (out == 0).all() and np.isneginf(lse).all()


# ----------------------------------------------------------------------------- P4..P9 invariants
def test_probabilities_sum_to_one():
    w = small(B=2, H=3, Q=20, prefix=(100, 9), tree="best_first", depth_cap=6)
    bits, _, _ = oracle.build_visibility(w.parent)
    _, _, psum = oracle.verify_attn(w.q_abs, w.q_rope, w.ckv, w.k_rope, w.kv_dtype, w.prefix,
                                    bits, w.scale, want_psum=True)
    assert np.abs(psum - 1.0).max() < 1e-12
    # and the probabilities vanish exactly off the visible set
    vis = closure_visibility(w.parent[1])
    for q in (0, 7, 19):
        row = (1 * w.Q + q) * w.H + 2
        p = oracle.row_probs(w.q_abs, w.q_rope, w.ckv, w.k_rope, w.kv_dtype, w.prefix, bits,
                             w.scale, row)
        P = int(w.prefix[1])
        assert (p[P:][~vis[q]] == 0).all() and (p[:P] > 0).all() and (p[P:][vis[q]] > 0).all()


def test_prefix_permutation_invariance():
    w = small(B=2, H=2, Q=9, prefix=(50, 12))
    out, lse = oracle.attend_workload(w)
    rng = np.random.default_rng(3)
    ckv, kr = w.ckv.copy(), w.k_rope.copy()
    off = w.kv_off
    for b in range(w.B):
        P = int(w.prefix[b])
        perm = rng.permutation(P) + off[b]
        ckv[off[b]:off[b] + P] = w.ckv[perm]
        kr[off[b]:off[b] + P] = w.k_rope[perm]
    w2 = wl.Workload(**{**w.__dict__, "ckv": ckv, "k_rope": kr})
    out2, lse2 = oracle.attend_workload(w2)
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-12)
    assert not np.array_equal(ckv, w.ckv)


def test_locality_appending_nodes():
    """Adding nodes with higher indices leaves existing nodes' outputs bit-identical."""
    Q0, Q1, H, P = 20, 45, 2, 13
    big = wl.make_workload("loc", 21, B=1, H=H, Q=Q1, prefix=P, tree="uniform")
    small_w = wl.Workload(**{**big.__dict__, "Q": Q0, "parent": big.parent[:, :Q0].copy(),
                             "q_abs": big.q_abs[:, :Q0].copy(), "q_rope": big.q_rope[:, :Q0].copy(),
                             "ckv": big.ckv[:P + Q0].copy(), "k_rope": big.k_rope[:P + Q0].copy()})
    o_big, l_big = oracle.attend_workload(big)
    o_small, l_small = oracle.attend_workload(small_w)
    assert np.array_equal(o_big[:Q0 * H], o_small)
    assert np.array_equal(l_big[:Q0 * H], l_small)


def test_scale_zero_is_mean():
    w = small(B=2, H=2, Q=12, prefix=(6, 0), scale=0.0)
    out, lse = oracle.attend_workload(w)
    off = w.kv_off
    for b in range(w.B):
        vis = closure_visibility(w.parent[b])
        P = int(w.prefix[b])
        for q in range(w.Q):
            idx = np.concatenate([np.arange(P), P + np.nonzero(vis[q])[0]]) + off[b]
            mean = w.ckv[idx].astype(np.float64).mean(axis=0)
            for h in range(w.H):
                r = (b * w.Q + q) * w.H + h
                np.testing.assert_allclose(out[r], mean, rtol=0, atol=1e-14)
                assert math.isclose(lse[r], math.log(len(idx)), rel_tol=1e-14)


@pytest.mark.parametrize("kv_dtype", [wl.F32, wl.BF16, wl.FP8])
def test_lse_merge_identity(kv_dtype):
    """Attention over V1 u V2 (u V3 empty) equals the log-sum-exp merge of partials."""
    w = small(B=1, H=1, Q=16, prefix=300, tree="best_first", depth_cap=4, kv_dtype=kv_dtype)
    bits, _, _ = oracle.build_visibility(w.parent)
    full, lse_full = oracle.attend_workload(w, bits=bits)
    vis = closure_visibility(w.parent[0])
    rng = np.random.default_rng(9)
    for q in (0, 5, 15):
        idx = np.concatenate([np.arange(300), 300 + np.nonzero(vis[q])[0]])
        cut = sorted(rng.choice(len(idx), 2, replace=False))
        parts = [idx[:cut[0]], idx[cut[0]:cut[1]], idx[cut[1]:], idx[:0]]
        ms, ls, os_ = zip(*[oracle.partial(w.q_abs[0, q, 0], w.q_rope[0, q, 0], w.ckv, w.k_rope,
                                           kv_dtype, p, w.scale) for p in parts])
        assert ms[3] == -math.inf and ls[3] == 0.0
        o, lse = oracle.merge(np.array(ms), np.array(ls), np.stack(os_))
        np.testing.assert_allclose(o, full[q], rtol=0, atol=1e-14)
        assert math.isclose(lse, lse_full[q], rel_tol=1e-14)
        # a single partial over everything, divided by l, is the full row
        m1, l1, o1 = oracle.partial(w.q_abs[0, q, 0], w.q_rope[0, q, 0], w.ckv, w.k_rope,
                                    kv_dtype, idx, w.scale)
        np.testing.assert_allclose(o1 / l1, full[q], rtol=0, atol=1e-14)


def test_merge_all_empty():
    o, lse = oracle.merge(np.array([-np.inf, -np.inf]), np.zeros(2), np.zeros((2, 512)))
    assert (o == 0).all() and lse == -math.inf


# ----------------------------------------------------------------------------- P6 / P10 brute force + structure
def all_recursive_trees(Q):
    for choice in itertools.product(*[range(i) for i in range(1, Q)]):
        yield np.array((-1,) + choice, dtype=np.int32)


@pytest.mark.parametrize("Q", [1, 2, 3, 4, 5, 6, 7])
def test_bruteforce_masks(Q):
    trees = list(all_recursive_trees(Q))
    assert len(trees) == math.factorial(Q - 1)
    parent = np.stack(trees)
    bits, bad, rc = oracle.build_visibility(parent)
    assert rc == 0 and (bad == -1).all()
    assert bits.shape == (len(trees), Q, 1)
    assert (bits[..., 0] >> np.uint32(Q) == 0).all() if Q < 32 else True
    got = bits_to_bool(bits, Q)
    for t, p in enumerate(trees):
        assert np.array_equal(got[t], closure_visibility(p))


def test_bruteforce_attention_q6():
    trees = list(all_recursive_trees(6))
    base = wl.make_workload("bf", 31, B=1, H=2, Q=6, prefix=3)
    parent = np.stack(trees)
    bits, _, _ = oracle.build_visibility(parent)
    for t, p in enumerate(trees):
        w = base.with_parent(p[None])
        out, lse = oracle.attend_workload(w, bits=bits[t:t + 1])
        ro, rl = torch_reference(w, closure_visibility(p)[None])
        np.testing.assert_allclose(out, ro, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


@pytest.mark.parametrize("Q,cap", [(64, 8), (128, 12), (256, 20), (33, 3)])
def test_mask_structure(Q, cap):
    rng = np.random.default_rng(Q)
    parent = np.stack([wl.best_first_tree(rng, Q, cap), wl.uniform_tree(rng, Q)])
    bits, bad, rc = oracle.build_visibility(parent)
    assert rc == 0
    W = (Q + 31) // 32
    assert bits.shape == (2, Q, W)
    vis = bits_to_bool(bits, Q)
    # padding bits beyond Q are zero
    k = np.arange(W * 32)
    pad = (bits[..., k // 32] >> (k % 32).astype(np.uint32)) & 1
    assert (pad[..., Q:] == 0).all()
    for t in range(2):
        d = wl.tree_depths(parent[t])
        assert (vis[t].sum(axis=1) == d + 1).all()            # popcount = depth + 1
        assert vis[t][np.arange(Q), np.arange(Q)].all()        # self
        for i in range(1, Q):
            pa = parent[t, i]
            expect = bits[t, pa].copy()
            expect[i // 32] |= np.uint32(1 << (i % 32))
            assert np.array_equal(bits[t, i], expect)          # recurrence
        assert np.array_equal(vis[t], closure_visibility(parent[t]))
    if cap < Q:
        assert wl.tree_depths(parent[0]).max() <= cap


def test_invalid_trees_reported():
    parent = np.stack([
        np.array([-1, 0, 1, 2], np.int32),      # fine
        np.array([0, 0, 1, 2], np.int32),       # root has a parent
        np.array([-1, 0, 2, 1], np.int32),      # node 2 is its own parent
        np.array([-1, -1, 5, 0], np.int32),     # second root (node 1) and a forward edge
        np.array([-1, 0, 1, -7], np.int32),     # parent below -1
    ])
    bits, bad, rc = oracle.build_visibility(parent)
    assert rc == oracle.REF_ETREE
    assert list(bad) == [-1, 0, 2, 1, 3]
    vis = bits_to_bool(bits, 4)
    assert vis[1, 0].tolist() == [True, False, False, False]      # bad root: self only
    assert vis[1, 3].tolist() == [True, True, True, True]        # walk stops at bad root
    assert vis[2, 2].tolist() == [False, False, True, False]
    assert vis[2, 3].tolist() == [True, True, False, True]        # 3 -> 1 -> 0 fine
    assert vis[3, 1].tolist() == [False, True, False, False]
    assert vis[3, 2].tolist() == [False, False, True, False]
    assert vis[4, 3].tolist() == [False, False, False, True]


def test_fp8_decode_every_code():
    """FP8 E4M3 decoding of all 256 byte values against torch's float8_e4m3fn
    conversion (a library routine), plus closed forms from the format's definition
    (bias 7, 3 mantissa bits, subnormals m * 2^-9, 0x7F / 0xFF NaN, no infinities)."""
    ref = wl.fp8_bits_to_f32(np.arange(256, dtype=np.uint8)).astype(np.float64)
    got = np.array([oracle.fp8_value(b) for b in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    assert np.array_equal(got[~nan], ref[~nan])
    assert oracle.fp8_value(0x7E) == 448.0
    assert oracle.fp8_value(0x08) == 2.0 ** -6
    assert oracle.fp8_value(0x01) == 2.0 ** -9
    assert oracle.fp8_value(0x07) == 7 * 2.0 ** -9
    assert oracle.fp8_value(0x38) == 1.0
    assert oracle.fp8_value(0xB9) == -1.125
    assert math.copysign(1.0, oracle.fp8_value(0x80)) == -1.0 and oracle.fp8_value(0x80) == 0.0


def test_fp8_cache_matches_torch():
    """A ragged FP8-cache workload against float64 SDPA over the decoded cache."""
    w = small(B=3, H=2, Q=12, prefix=(0, 5, 37), tree="best_first", depth_cap=4, kv_dtype=wl.FP8)
    bits, _, _ = oracle.build_visibility(w.parent)
    out, lse = oracle.attend_workload(w, bits=bits)
    ref, rlse = torch_reference(w, np.stack([closure_visibility(p) for p in w.parent]))
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, rlse, rtol=1e-12, atol=1e-12)
