"""The best-first draft-tree builder on the GPU against its oracle (bit for bit:
parents, depths, ranks and tokens are integers; scores are float32 sums taken in
the same order), then end to end: trees built on the device feed the visibility
builder and the attention step with no host round trip.

The kernel answers from its level pass when every log-probability is <= 0 and
no scores tie, and from its one-node-per-step pass otherwise (ties, positive
values, more candidates than the level pass holds); the cases below reach both:
drafter log-probs in descending and in shuffled order, tie-heavy and positive
inputs, and the largest staging table."""
import numpy as np
import pytest

import oracle
import workloads as wl
from parity import assert_close, assert_lse_close, oracle_rows, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def gpu_tree(lp, Q, tok=None, outputs=True):
    import tree_masked_mla_amd as dd
    dev = torch.device("cuda:0")
    B = lp.shape[0]
    lp_d = torch.from_numpy(np.ascontiguousarray(lp, np.float32)).to(dev)
    tok_d = None if tok is None else torch.from_numpy(np.ascontiguousarray(tok, np.int32)).to(dev)
    out = {k: torch.full((B, Q), -7, dtype=torch.int32, device=dev) for k in ("parent", "depth", "rank", "token")}
    out["score"] = torch.full((B, Q), 7.0, dtype=torch.float32, device=dev)
    if not outputs:
        for k in ("depth", "rank", "token", "score"):
            out[k] = None
    rc = dd.ddtv_build_tree(lp_d, Q, out["parent"], tokens=tok_d, depth=out["depth"], rank=out["rank"],
                            token=out["token"], score=out["score"])
    assert rc == dd.DDTV_OK
    torch.cuda.synchronize()
    return {k: (None if v is None else v.cpu().numpy()) for k, v in out.items()}


def assert_same_tree(got, ref, what):
    for k in ("parent", "depth", "rank", "token"):
        if got[k] is not None:
            assert np.array_equal(got[k], ref[k]), f"{what}: {k} differs"
    if got["score"] is not None:
        assert np.array_equal(got["score"].view(np.uint32), ref["score"].view(np.uint32)), f"{what}: score bits"


@pytest.mark.parametrize("B,D,K,Q", [
    (8, 12, 4, 128),      # the attention workloads' tree budget
    (4, 6, 8, 256),       # largest tree
    (3, 1, 30, 31),       # star: every node a child of the root
    (2, 255, 1, 256),     # chain: one choice per depth
    (5, 300, 2, 64),      # more depths than nodes
    (1, 4, 64, 200),      # most choices per depth
    (70, 8, 3, 40),       # many batch rows
    (2, 3, 2, 15),        # exactly the full tree of depth 3
    (2, 8, 4, 65),        # just past the smallest register-slot instantiation (Q <= 64)
    (2, 8, 4, 129),       # just past the middle one (Q <= 128)
])
def test_tree_matches_oracle(B, D, K, Q):
    say(f"tree B{B} D{D} K{K} Q{Q}")
    lp, tok = wl.drafter_topk(6000 + B * 7 + D + K + Q, B, D, K)
    rc, ref = oracle.build_tree(lp, Q, tok)
    assert rc == oracle.REF_OK
    assert_same_tree(gpu_tree(lp, Q, tok), ref, f"B{B} D{D} K{K} Q{Q}")


def shuffled(lp, tok, seed):
    rng = np.random.default_rng(seed)
    perm = np.argsort(rng.random(lp.shape), axis=-1)
    return (np.ascontiguousarray(np.take_along_axis(lp, perm, -1)),
            np.ascontiguousarray(np.take_along_axis(tok, perm, -1)))


@pytest.mark.parametrize("B,D,K,Q", [
    (8, 12, 4, 128),      # the benchmarked trees
    (3, 6, 8, 200),
    (2, 1, 30, 31),       # star
    (4, 9, 64, 256),      # most choices, largest tree
    (70, 8, 3, 40),       # many batch rows
])
def test_tree_unsorted_matches_oracle(B, D, K, Q):
    """Choices in no particular order: ranked by value inside the kernel.  With
    token ids, and without them (the token is then the choice's index)."""
    say(f"tree unsorted B{B} D{D} K{K} Q{Q}")
    lp, tok = shuffled(*wl.drafter_topk(6300 + B + D + K + Q, B, D, K), seed=Q)
    rc, ref = oracle.build_tree(lp, Q, tok)
    assert rc == oracle.REF_OK
    assert_same_tree(gpu_tree(lp, Q, tok), ref, f"unsorted B{B} D{D} K{K} Q{Q}")
    rc, ref = oracle.build_tree(lp, Q)
    assert_same_tree(gpu_tree(lp, Q), ref, f"unsorted, no tokens, B{B} D{D} K{K} Q{Q}")


def test_tree_positive_log_probs():
    """Values above 0 (a child can outscore its parent): the one-node-per-step pass."""
    lp, tok = wl.drafter_topk(6400, 5, 10, 4)
    lp = lp.copy()
    lp[:, 3, :] += 3.0                     # depth 4's choices all positive
    lp[1, 0, 2] = 0.5
    lp = np.ascontiguousarray(lp, dtype=np.float32)
    assert (lp > 0).any()
    rc, ref = oracle.build_tree(lp, 100, tok)
    assert rc == oracle.REF_OK
    assert_same_tree(gpu_tree(lp, 100, tok), ref, "positive values")


def test_tree_largest_staging_table():
    """D = 256 depths x K = 64 choices at Q = 256: the rank-ordered tables take
    80 KiB of LDS; shuffled and sorted choices."""
    lp, tok = wl.drafter_topk(6500, 2, 256, 64)
    rc, ref = oracle.build_tree(lp, 256, tok)
    assert rc == oracle.REF_OK
    assert_same_tree(gpu_tree(lp, 256, tok), ref, "largest table, sorted")
    lp2, tok2 = shuffled(lp, tok, 6501)
    rc, ref = oracle.build_tree(lp2, 256, tok2)
    assert_same_tree(gpu_tree(lp2, 256, tok2), ref, "largest table, shuffled")


def test_tree_ties_and_optional_outputs():
    """Rounded log-probabilities tie across branches and between siblings; equal
    scores must resolve exactly as the oracle does (earlier parent, then rank).
    Without a token table the token output is the rank."""
    lp, _ = wl.drafter_topk(6101, 6, 7, 5)
    lp = np.round(lp * 2) / 2
    lp = -np.sort(-lp, axis=-1)
    lp[:, :, 3] = lp[:, :, 2]
    lp = np.ascontiguousarray(lp, dtype=np.float32)
    rc, ref = oracle.build_tree(lp, 180)
    assert rc == oracle.REF_OK
    assert_same_tree(gpu_tree(lp, 180), ref, "ties")
    got = gpu_tree(lp, 180, outputs=False)
    assert np.array_equal(got["parent"], ref["parent"])


def test_tree_argument_errors():
    import tree_masked_mla_amd as dd
    dev = torch.device("cuda:0")
    lp = torch.zeros((1, 2, 2), dtype=torch.float32, device=dev) - 1
    par = torch.zeros((1, 8), dtype=torch.int32, device=dev)
    assert dd.ddtv_build_tree(lp, 8, par) == dd.DDTV_EINVAL          # only 7 nodes exist
    assert dd.ddtv_build_tree(lp, 7, par) == dd.DDTV_OK
    big = torch.zeros((1, 2, 65), dtype=torch.float32, device=dev)
    assert dd.ddtv_build_tree(big, 7, par) == dd.DDTV_EUNSUPPORTED
    torch.cuda.synchronize()


def test_device_trees_feed_visibility_and_attention():
    """Trees built on the device go straight into S1 and S2..S7; the result equals
    the oracle pipeline (oracle trees, oracle masks, oracle attention)."""
    import tree_masked_mla_amd as dd
    from tree_masked_mla_amd.runner import DeviceRun
    B, H, Q, D, K = 3, 8, 48, 10, 4
    lp, tok = wl.drafter_topk(6200, B, D, K)
    rc, ref = oracle.build_tree(lp, Q, tok)
    assert rc == oracle.REF_OK
    w = wl.make_workload("tree-e2e", 6201, B=B, H=H, Q=Q, prefix=[300, 0, 777], tree="uniform")
    w.parent[...] = ref["parent"]                       # the oracle's trees for the oracle side
    r = DeviceRun(w)
    rc = dd.ddtv_build_tree(torch.from_numpy(lp).to(r.device), Q, r.parent)   # overwrite on the device
    assert rc == dd.DDTV_OK
    r.step()
    out, lse = r.results()
    assert np.array_equal(r.parent.cpu().numpy(), ref["parent"])
    bits, _, brc = oracle.build_visibility(ref["parent"])
    assert brc == oracle.REF_OK and np.array_equal(r.bits(), bits)
    want, wlse = oracle_rows(w, bits)
    assert_close(out, want, 0, "device-built trees")
    assert_lse_close(lse, wlse, 0, "device-built trees")
