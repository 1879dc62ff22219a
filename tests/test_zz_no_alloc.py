"""ddtv_verify_attn_noalloc (no workspace argument; split partials in the
library's per-GPU scratch) against ddtv_verify_attn_ex with a caller workspace,
through the C ABI.

Two calls in a row, the second on a smaller input: each must equal the
workspace entry point's result bit for bit (same plan, same kernels) and the
oracle within the fp32 bar.  A third batch needs more partials than the scratch
holds under the workspace entry point's plan: the no-alloc call plans fewer
splits and still matches the oracle.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from parity import assert_close, assert_lse_close, oracle_rows, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _noalloc(r, opts=None):
    import tree_masked_mla_amd as dd
    out = torch.full_like(r.out, float("nan"))
    lse = torch.full_like(r.lse, float("nan"))
    rc = dd.ddtv_verify_attn_noalloc(r.q_abs, r.q_rope, r.ckv, r.k_rope, r.kv_dtype, r.H, r.vis, r.scale, out,
                                     lse, opts=opts)
    assert rc == dd.DDTV_OK, dd.ddtv_status_string(rc)
    return out, lse


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    import tree_masked_mla_amd as dd
    from tree_masked_mla_amd.runner import DeviceRun
    big = wl.config("c3")                                   # 16 splits of 272: 32.1 MiB of partials
    small = wl.make_workload("noalloc-small", 7301, B=3, H=8, Q=20, prefix=[300, 37, 0], tree="uniform")
    cases = [(big, dd.make_opts()), (small, dd.make_opts(split_len=64))]
    runs = []
    for w, opts in cases:
        r = DeviceRun(w, split_len=opts.split_len)
        assert r.plan()[3] > 1                              # the partials and the merge are exercised
        assert 0 < r.ws_bytes <= dd.NOALLOC_SCRATCH_BYTES
        r.step()
        torch.cuda.synchronize()
        runs.append((r, opts, r.out.clone(), r.lse.clone()))
    assert runs[1][0].ws_bytes < runs[0][0].ws_bytes        # the second call is the smaller one
    got = []
    for r, opts, _, _ in runs:                               # the two no-alloc calls back to back
        say(f"noalloc call: B{r.B} Q{r.Q} H{r.H} plan {r.plan()} workspace {r.ws_bytes} B")
        got.append(_noalloc(r, opts))
    torch.cuda.synchronize()
    for (r, _, ref_out, ref_lse), (out, lse) in zip(runs, got):
        assert torch.equal(out, ref_out), "no-alloc output differs from the workspace entry point"
        assert torch.equal(lse, ref_lse), "no-alloc lse differs from the workspace entry point"
        w = r.w
        bits, _, _ = oracle.build_visibility(w.parent)
        rows = wl.sample_rows(w, 256) if w.B * w.Q * w.H > 256 else None
        ref, rlse = oracle_rows(w, bits, rows)
        o = out.cpu().numpy().reshape(-1, 512)
        l = lse.cpu().numpy().reshape(-1)
        if rows is not None:
            o, l = o[rows], l[rows]
        e = assert_close(o, ref, 0, f"noalloc {w.name}")
        assert_lse_close(l, rlse, 0, f"noalloc {w.name}")
        say(f"  {w.name}: bit-identical to the workspace call; max abs err vs oracle {e:.2e}")


def test_noalloc_plans_within_the_scratch():
    """The workspace entry point plans 13 splits (52 MiB of partials) for this
    batch; the no-alloc call must pick a plan whose partials fit and still
    match the oracle."""
    import tree_masked_mla_amd as dd
    from tree_masked_mla_amd.runner import DeviceRun
    w = wl.make_workload("noalloc-cap", 7302, B=2, H=16, Q=64, prefix=[20000, 3000], tree="uniform")
    r = DeviceRun(w)
    assert r.ws_bytes > dd.NOALLOC_SCRATCH_BYTES
    r.build_visibility()
    say(f"noalloc over-cap batch: workspace plan {r.plan()} needs {r.ws_bytes} B")
    out, lse = _noalloc(r)
    torch.cuda.synchronize()
    bits, _, _ = oracle.build_visibility(w.parent)
    rows = wl.sample_rows(w, 128)
    ref, rlse = oracle_rows(w, bits, rows)
    e = assert_close(out.cpu().numpy().reshape(-1, 512)[rows], ref, 0, "noalloc capped plan")
    assert_lse_close(lse.cpu().numpy().reshape(-1)[rows], rlse, 0, "noalloc capped plan")
    say(f"  capped plan: max abs err vs oracle {e:.2e}")
