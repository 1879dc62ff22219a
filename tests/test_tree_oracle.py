"""Pins of the best-first draft-tree builder's oracle (CPU only).

The oracle takes nodes off a binary heap into which every taken node pushes all
K children.  These tests check it against what holds independently of that:
- brute force: with log-probabilities <= 0 a child never scores above its
  parent, and a better-ranked sibling never scores below a worse one, so the
  best-first tree of Q nodes is the root plus the Q-1 highest-scoring nodes of
  the whole lattice of choice paths (enumerated and sorted here), in score
  order -- for choices given in descending order and for shuffled ones;
- shuffling the K choices of a depth (with their token ids) changes nothing:
  the ranking is by value, not by position;
- the tree's own invariants, and the special cases that have a closed form:
  K = 1 gives a chain, D = 1 a star in rank order (equal values ranked by
  index), and a worked example with a positive log-probability, where a
  child outscores the nodes taken before it;
- ties go to the candidate whose parent was taken first, then the better rank;
- argument errors.
"""
import itertools

import numpy as np
import pytest

import oracle


def sorted_logp(rng, B, D, K, vocab=32, sigma=2.0):
    """Per-depth top-K log-softmax of N(0, sigma^2) logits over `vocab` tokens,
    descending (the drafter's output as the builder receives it), and token ids."""
    logits = rng.standard_normal((B, D, vocab)) * sigma
    lp = logits - np.log(np.exp(logits).sum(-1, keepdims=True))
    order = np.argsort(-lp, axis=-1, kind="stable")[..., :K]
    return np.take_along_axis(lp, order, -1).astype(np.float32), order.astype(np.int32)


def paths(t, b, Q, key="rank"):
    """Choice path (tuple of ranks, or of choice indices with key="token" when the
    tree was built without token ids) of every node of batch row b."""
    out = []
    for i in range(Q):
        p = t["parent"][b, i]
        out.append(() if p < 0 else out[p] + (int(t[key][b, i]),))
    return out


def shuffled(lp, tok, seed):
    """The same choices in a random order within each (batch row, depth)."""
    rng = np.random.default_rng(seed)
    perm = np.argsort(rng.random(lp.shape), axis=-1)
    return np.take_along_axis(lp, perm, -1), np.take_along_axis(tok, perm, -1)


def lattice(lp, D, K):
    """Every non-root node of the depth-D lattice with its float32 score,
    accumulated from the root in path order."""
    nodes = []
    for d in range(1, D + 1):
        for path in itertools.product(range(K), repeat=d):
            s = np.float32(0.0)
            for j, r in enumerate(path):
                s = np.float32(s + lp[j, r])
            nodes.append((path, s))
    return nodes


@pytest.mark.parametrize("D,K,Q", [(3, 3, 20), (4, 2, 25), (2, 5, 31), (5, 3, 60), (6, 2, 64)])
def test_bruteforce_top_scores(D, K, Q):
    rng = np.random.default_rng(100 * D + K)
    lp, _ = sorted_logp(rng, 4, D, K)
    rc, t = oracle.build_tree(lp, Q)
    assert rc == oracle.REF_OK
    for b in range(4):
        nodes = lattice(lp[b], D, K)
        scores = np.array([s for _, s in nodes])
        assert len(np.unique(scores)) == len(scores)          # no ties in this draw
        order = np.argsort(-scores, kind="stable")[: Q - 1]
        want = [()] + [nodes[i][0] for i in order]
        assert paths(t, b, Q) == want
        np.testing.assert_array_equal(t["score"][b], [0.0] + [scores[i] for i in order])


@pytest.mark.parametrize("D,K,Q", [(3, 3, 20), (4, 2, 25), (2, 5, 31), (5, 3, 60)])
def test_bruteforce_top_scores_unsorted(D, K, Q):
    """Choices in a random order: the tree, read as paths of choice indices, is
    still the root plus the Q-1 best lattice nodes, enumerated over the choices
    in their given order."""
    rng = np.random.default_rng(200 * D + K)
    lp, tok = sorted_logp(rng, 4, D, K)
    lp, _ = shuffled(lp, tok, 300 + D)
    rc, t = oracle.build_tree(lp, Q)              # no token ids: token = choice index
    assert rc == oracle.REF_OK
    for b in range(4):
        nodes = lattice(lp[b], D, K)
        scores = np.array([s for _, s in nodes])
        assert len(np.unique(scores)) == len(scores)
        order = np.argsort(-scores, kind="stable")[: Q - 1]
        assert paths(t, b, Q, key="token") == [()] + [nodes[i][0] for i in order]
        np.testing.assert_array_equal(t["score"][b], [0.0] + [scores[i] for i in order])


@pytest.mark.parametrize("seed", [0, 1])
def test_shuffled_choices_change_nothing(seed):
    """Permuting the K choices of every depth, together with their token ids,
    leaves parents, depths, ranks, tokens and scores unchanged (values distinct)."""
    rng = np.random.default_rng(40 + seed)
    lp, tok = sorted_logp(rng, 5, 12, 4)
    rc, want = oracle.build_tree(lp, 128, tok)
    assert rc == oracle.REF_OK
    lp2, tok2 = shuffled(lp, tok, 50 + seed)
    assert not np.array_equal(lp2, lp)
    rc, got = oracle.build_tree(lp2, 128, tok2)
    assert rc == oracle.REF_OK
    for k in ("parent", "depth", "rank", "token", "score"):
        np.testing.assert_array_equal(got[k], want[k], err_msg=k)


def test_equal_values_rank_by_index():
    """A star (D = 1) is the choices in rank order; equal log-probabilities rank
    by their index, so the root's children come out as choices 1, 2, 0, 3."""
    lp = np.array([[[-1.0, -0.5, -0.5, -2.0]]], np.float32)
    rc, t = oracle.build_tree(lp, 5)
    assert rc == oracle.REF_OK
    np.testing.assert_array_equal(t["parent"][0], [-1, 0, 0, 0, 0])
    np.testing.assert_array_equal(t["token"][0], [-1, 1, 2, 0, 3])
    np.testing.assert_array_equal(t["rank"][0], [-1, 0, 1, 2, 3])
    np.testing.assert_array_equal(t["score"][0], [0.0, -0.5, -0.5, -1.0, -2.0])


def test_positive_log_prob_worked_example():
    """Best first is not the top-Q lattice set when a choice has a positive value:
    depth 1 offers (-1, -2), depth 2 offers (+5, -1).  Taken in order: the root;
    (-1) from the root; its child +5 scoring 4; then of the two candidates at -2
    the one whose parent (the root) was taken first."""
    lp = np.array([[[-1.0, -2.0], [5.0, -1.0]]], np.float32)
    rc, t = oracle.build_tree(lp, 4)
    assert rc == oracle.REF_OK
    np.testing.assert_array_equal(t["parent"][0], [-1, 0, 1, 0])
    np.testing.assert_array_equal(t["depth"][0], [0, 1, 2, 1])
    np.testing.assert_array_equal(t["rank"][0], [-1, 0, 0, 1])
    np.testing.assert_array_equal(t["token"][0], [-1, 0, 0, 1])
    np.testing.assert_array_equal(t["score"][0], [0.0, -1.0, 4.0, -2.0])


def test_tree_invariants():
    rng = np.random.default_rng(7)
    D, K, Q = 12, 4, 256
    lp, tok = sorted_logp(rng, 6, D, K)
    rc, t = oracle.build_tree(lp, Q, tok)
    assert rc == oracle.REF_OK
    for b in range(6):
        par, dep, rk, sc = t["parent"][b], t["depth"][b], t["rank"][b], t["score"][b]
        assert par[0] == -1 and dep[0] == 0 and rk[0] == -1 and sc[0] == 0.0 and t["token"][b, 0] == -1
        seen = set()
        for i in range(1, Q):
            p = par[i]
            assert 0 <= p < i
            assert dep[i] == dep[p] + 1 <= D
            assert 0 <= rk[i] < K
            assert sc[i] == np.float32(sc[p] + lp[b, dep[i] - 1, rk[i]])
            assert t["token"][b, i] == tok[b, dep[i] - 1, rk[i]]
            assert (p, rk[i]) not in seen
            seen.add((p, rk[i]))
            if rk[i] > 0:                     # the better-ranked sibling came first
                assert (p, rk[i] - 1) in seen
        assert np.all(np.diff(sc) <= 0)       # best first


def test_k1_is_a_chain_and_d1_is_a_star():
    rng = np.random.default_rng(3)
    lp, _ = sorted_logp(rng, 2, 40, 1)
    rc, t = oracle.build_tree(lp, 41)
    assert rc == oracle.REF_OK
    np.testing.assert_array_equal(t["parent"], np.tile(np.arange(-1, 40), (2, 1)))
    np.testing.assert_array_equal(t["depth"], np.tile(np.arange(41), (2, 1)))
    lp, _ = sorted_logp(rng, 2, 1, 30)
    rc, t = oracle.build_tree(lp, 31)
    assert rc == oracle.REF_OK
    np.testing.assert_array_equal(t["parent"][:, 1:], 0)
    np.testing.assert_array_equal(t["rank"][:, 1:], np.tile(np.arange(30), (2, 1)))


def eager_tree(lp, Q):
    """Best-first with every child offered at once, a plain list scanned for its
    best entry each step (ranks from Python's sort of each depth's choices)."""
    D, K = lp.shape
    rank = [{k: r for r, k in enumerate(sorted(range(K), key=lambda k: (-lp[d, k], k)))} for d in range(D)]
    cand = [(np.float32(0.0), -1, 0, -1)]           # (score, parent, depth, rank)
    par, rk = [], []
    score = []
    while len(par) < Q:
        best = min(range(len(cand)), key=lambda i: (-cand[i][0], cand[i][1], cand[i][3]))
        s, p, d, r = cand.pop(best)
        i = len(par)
        par.append(p), rk.append(r), score.append(s)
        if d < D:
            cand += [(np.float32(s + lp[d, k]), i, d + 1, rank[d][k]) for k in range(K)]
    return par, rk, score


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_offering_all_children(seed):
    rng = np.random.default_rng(seed)
    lp, tok = sorted_logp(rng, 3, 5, 4)
    lp[:, :, 2] = lp[:, :, 1]                       # ties between siblings
    lp[1] = np.round(lp[1])                         # many ties across branches
    lp[2] = np.round(lp[2] * 2) / 2
    lp, _ = shuffled(lp, tok, 60 + seed)           # and in no particular order
    rc, t = oracle.build_tree(lp, 90)
    assert rc == oracle.REF_OK
    for b in range(3):
        par, rk, score = eager_tree(lp[b], 90)
        np.testing.assert_array_equal(t["parent"][b], par)
        np.testing.assert_array_equal(t["rank"][b], rk)
        np.testing.assert_array_equal(t["score"][b], score)


def test_ties_go_to_the_earlier_parent_then_rank():
    # every choice equally likely: scores tie within each depth; nodes come out
    # breadth first, parents in the order they were taken, siblings by rank
    D, K = 3, 3
    lp = np.full((1, D, K), np.float32(-np.log(3.0)), np.float32)
    rc, t = oracle.build_tree(lp, 13)
    assert rc == oracle.REF_OK
    np.testing.assert_array_equal(t["parent"][0], [-1, 0, 0, 0, 1, 1, 1, 2, 2, 2, 3, 3, 3])
    np.testing.assert_array_equal(t["rank"][0], [-1, 0, 1, 2, 0, 1, 2, 0, 1, 2, 0, 1, 2])


def test_capacity_and_errors():
    assert oracle.tree_capacity(3, 2) == 15
    assert oracle.tree_capacity(1, 7) == 8
    assert oracle.tree_capacity(200, 8, 300) == 300
    lp = np.zeros((1, 2, 2), np.float32) - 1
    assert oracle.build_tree(lp, 7)[0] == oracle.REF_OK
    assert oracle.build_tree(lp, 8)[0] == oracle.REF_EINVAL      # only 7 nodes exist
    assert oracle.build_tree(lp, 0)[0] == oracle.REF_EINVAL
    assert oracle.build_tree(np.zeros((1, 0, 2), np.float32), 1)[0] == oracle.REF_EINVAL
