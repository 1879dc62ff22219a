"""Pins of the greedy tree-accept oracle and of the KV compaction after it (CPU).

Independent formulations checked against the oracle's walk:
- with distinct tokens among siblings, the accepted nodes are exactly the nodes
  whose every edge from the root matches: child token == the parent's
  prediction (numpy argmax, first maximum on ties); they form a chain, and the
  walk returns it root first;
- compaction equals numpy fancy indexing of the original rows;
- special cases: nothing accepted, a whole chain accepted, ties in the logits,
  duplicate sibling tokens (the lower node index wins), malformed trees.
"""
import numpy as np
import pytest

import oracle
import workloads as wl


def random_case(seed, B, Q, V=64, D=10, K=4, follow=0.75):
    """Trees from the builder oracle (sibling tokens distinct), and target logits
    whose argmax follows one of the node's children with probability `follow`."""
    rng = np.random.default_rng(seed)
    lp, tok = wl.drafter_topk(seed, B, D, K, vocab=V)
    rc, t = oracle.build_tree(lp, Q, tok)
    assert rc == oracle.REF_OK
    parent, token = t["parent"], t["token"]
    logits = rng.standard_normal((B, Q, V)).astype(np.float32)
    for b in range(B):
        for i in range(Q):
            kids = np.nonzero(parent[b] == i)[0]
            if len(kids) and rng.random() < follow:
                logits[b, i, token[b, rng.choice(kids)]] = 10.0
    return parent, token, logits


def accepted_set(parent, token, pred):
    ok = np.zeros(len(parent), bool)
    ok[0] = True
    for i in range(1, len(parent)):      # parents come first
        ok[i] = ok[parent[i]] and token[i] == pred[parent[i]]
    return np.nonzero(ok)[0]


@pytest.mark.parametrize("seed,B,Q", [(1, 6, 32), (2, 4, 128), (3, 8, 9), (4, 3, 256)])
def test_walk_equals_matching_edge_set(seed, B, Q):
    parent, token, logits = random_case(seed, B, Q)
    rc, a = oracle.tree_accept(logits, parent, token)
    assert rc == oracle.REF_OK
    pred = np.argmax(logits, axis=-1)
    assert np.array_equal(a["pred"], pred)
    for b in range(B):
        acc = accepted_set(parent[b], token[b], pred[b])
        k = a["accept_len"][b]
        assert k == len(acc) - 1
        assert np.array_equal(a["path"][b, :k + 1], acc)          # a chain, in index (= depth) order
        assert np.all(a["path"][b, k + 1:] == -1)
        assert np.array_equal(a["out_tokens"][b, :k], token[b, acc[1:]])
        assert a["out_tokens"][b, k] == pred[b, acc[-1]]           # bonus token
        assert np.all(a["out_tokens"][b, k + 1:] == -1)


def test_special_cases():
    Q, V = 12, 16
    parent = np.array([[-1] + list(range(Q - 1))], np.int32)        # a chain
    token = np.array([[0] + [3] * (Q - 1)], np.int32)
    logits = np.zeros((1, Q, V), np.float32)
    logits[0, :, 3] = 1.0                                            # every prediction matches
    rc, a = oracle.tree_accept(logits, parent, token)
    assert rc == oracle.REF_OK and a["accept_len"][0] == Q - 1
    assert np.array_equal(a["path"][0], np.arange(Q))
    logits[0, 0, 3] = 0.0
    logits[0, 0, 5] = 2.0                                            # the root's prediction misses
    rc, a = oracle.tree_accept(logits, parent, token)
    assert a["accept_len"][0] == 0 and a["out_tokens"][0, 0] == 5 and np.all(a["out_tokens"][0, 1:] == -1)
    flat = np.zeros((1, Q, V), np.float32)                           # all equal: argmax is token 0
    rc, a = oracle.tree_accept(flat, parent, token)
    assert np.all(a["pred"] == 0) and a["accept_len"][0] == 0
    # duplicate sibling tokens: the lower node index is taken
    parent2 = np.array([[-1, 0, 0, 1, 2]], np.int32)
    token2 = np.array([[0, 7, 7, 4, 4]], np.int32)
    lg = np.zeros((1, 5, 8), np.float32)
    lg[0, 0, 7] = 1.0
    lg[0, 1, 4] = 1.0
    lg[0, 2, 4] = 1.0
    rc, a = oracle.tree_accept(lg, parent2, token2)
    assert np.array_equal(a["path"][0, :3], [0, 1, 3])
    bad = np.array([[-1, 0, 5, 1, 2]], np.int32)                     # parent after child
    assert oracle.tree_accept(lg, bad, token2)[0] == oracle.REF_EINVAL


@pytest.mark.parametrize("dtype", [np.float32, np.uint16])
def test_compaction_equals_fancy_indexing(dtype):
    rng = np.random.default_rng(9)
    P, Q = 37, 20
    rows = rng.integers(0, 60000, (P + Q, 576)).astype(dtype)
    path = np.array([0, 2, 5, 6, 11, 19] + [-1] * (Q - 6), np.int32)
    k = 5
    got = oracle.compact_rows(rows, P, path, k)
    want = rows.copy()
    want[P + 1:P + k + 1] = rows[P + path[1:k + 1]]
    assert np.array_equal(got, want)
    assert np.array_equal(oracle.compact_rows(rows, P, path, 0), rows)
