"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import tree_masked_mla_amd as dd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ddtv.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dd.LIB_PATH):
        from tree_masked_mla_amd import build
        build.build()
    return dd.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ddtv_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 10
    raw = ctypes.CDLL(dd.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert set(names) == set(dd.EXPORTED)


def test_version_and_strings(lib):
    assert dd.ddtv_version() == 800
    for code in range(6):
        assert dd.ddtv_status_string(code)
    assert dd.ddtv_status_string(2).startswith("malformed tree")


def test_vis_bytes(lib):
    assert dd.ddtv_vis_bytes(0, 9) == 0
    assert dd.ddtv_vis_bytes(1, 0) == 0
    assert dd.ddtv_vis_bytes(1, 257) == 0
    assert dd.ddtv_vis_bytes(1, 256) > 0
    for B, Q in [(1, 9), (3, 9), (8, 128), (32, 64), (5, 33)]:
        W = (Q + 31) // 32
        need = B * Q * W * 4 + B * 16 + B * 4
        got = dd.ddtv_vis_bytes(B, Q)
        assert got >= need and got % 256 == 0


FAKE = 1 << 40          # an aligned address that is never dereferenced (checks fail first)


def build_call(lib, parent=FAKE, prefix=None, B=2, Q=9, buf=FAKE, nbytes=1 << 20):
    prefix = np.zeros(max(B, 1), np.int32) if prefix is None else prefix
    vis = dd.ddtv_vis()
    return lib.ddtv_build_visibility(parent, prefix.ctypes.data if prefix is not False else None, B, Q, buf,
                                     nbytes, ctypes.byref(vis), None)


def test_build_visibility_host_errors(lib):
    E = dd.DDTV_EINVAL
    assert build_call(lib, parent=None) == E
    assert build_call(lib, prefix=False) == E
    assert build_call(lib, buf=None) == E
    assert build_call(lib, B=0) == E
    assert build_call(lib, Q=0) == E
    assert build_call(lib, Q=257) == E
    assert build_call(lib, parent=FAKE + 2) == E                     # misaligned parent
    assert build_call(lib, buf=FAKE + 16) == E                       # vis_buf not 256-aligned
    assert build_call(lib, prefix=np.array([3, -1], np.int32)) == E  # negative prefix
    assert build_call(lib, prefix=np.array([2**31 - 5, 0], np.int32)) == E  # P + Q overflows int32
    assert build_call(lib, nbytes=dd.ddtv_vis_bytes(2, 9) - 1) == dd.DDTV_EWORKSPACE
    vis = dd.ddtv_vis()
    assert lib.ddtv_build_visibility(FAKE, np.zeros(2, np.int32).ctypes.data, 2, 9, FAKE, 1 << 20, None,
                                     None) == E


def fake_vis(B=2, Q=9, prefix=(37, 37), order=True):
    v = dd.ddtv_vis()
    v.B, v.Q, v.W = B, Q, (Q + 31) // 32
    pre = np.asarray(prefix, np.int32)
    v.max_kv = int(pre.max()) + Q
    v.total_kv = int((pre.astype(np.int64) + Q).sum())
    v.bits, v.rows, v.status = FAKE, FAKE + 4096, FAKE + 8192
    v.order = FAKE + 12288 if order else None
    v.prefix_host = pre.ctypes.data
    return dd.Visibility(v, (pre,))


def verify_call(lib, vis, q_abs=FAKE, q_rope=FAKE, ckv=FAKE, k_rope=FAKE, kv_dtype=0, H=8, scale=0.07,
                out=FAKE, lse=None, ws=None, ws_bytes=0, opts=None):
    return lib.ddtv_verify_attn_ex(q_abs, q_rope, ckv, k_rope, kv_dtype, H, ctypes.byref(vis.vis),
                                   ctypes.c_float(scale), out, lse, ws, ws_bytes, None,
                                   ctypes.byref(opts) if opts is not None else None)


def test_verify_host_errors(lib):
    vis = fake_vis()
    E, U = dd.DDTV_EINVAL, dd.DDTV_EUNSUPPORTED
    for kw in ("q_abs", "q_rope", "ckv", "k_rope", "out"):
        assert verify_call(lib, vis, **{kw: None}) == E, kw
        assert verify_call(lib, vis, **{kw: FAKE + 4}) == E, kw        # not 16-byte aligned
    assert verify_call(lib, vis, lse=FAKE + 2) == E
    assert verify_call(lib, vis, H=0) == E
    assert verify_call(lib, vis, scale=float("nan")) == E
    assert verify_call(lib, vis, scale=float("inf")) == E
    assert verify_call(lib, vis, kv_dtype=3) == U        # FP8 E4M3 (2) is the last cache dtype
    assert verify_call(lib, vis, opts=dd.make_opts(path=4)) == U
    assert verify_call(lib, vis, opts=dd.make_opts(split_len=100)) == E   # not a multiple of 16
    assert verify_call(lib, vis, opts=dd.make_opts(split_len=-64)) == E
    assert verify_call(lib, vis, opts=dd.make_opts(wg_order=3)) == U
    bad = fake_vis()
    bad.vis.W = 2
    assert verify_call(lib, bad) == E
    bad = fake_vis()
    bad.vis.bits = None
    assert verify_call(lib, bad) == E
    bad = fake_vis(Q=9)
    bad.vis.Q = 300
    assert verify_call(lib, bad) == E
    # splitting needs a workspace
    vis = fake_vis(B=1, Q=64, prefix=(4096,))
    opts = dd.make_opts(split_len=1024)
    need = dd.ddtv_workspace_bytes(vis, 16, 0, opts)
    assert need > 0
    assert verify_call(lib, vis, H=16, opts=opts) == dd.DDTV_EWORKSPACE
    assert verify_call(lib, vis, H=16, opts=opts, ws=FAKE, ws_bytes=need - 1) == dd.DDTV_EWORKSPACE
    assert verify_call(lib, vis, H=16, opts=opts, ws=FAKE + 16, ws_bytes=need) == E


def test_build_tree_argument_checks(lib):
    """The tree builder's host checks come before any HIP call (so no GPU is touched here)."""
    E, U = dd.DDTV_EINVAL, dd.DDTV_EUNSUPPORTED

    def call(logp=FAKE, tokens=None, B=2, D=3, K=4, Q=20, parent=FAKE + 4096, depth=None):
        return lib.ddtv_build_tree(logp, tokens, B, D, K, Q, parent, depth, None, None, None, None)

    assert call(logp=None) == E
    assert call(parent=None) == E
    assert call(parent=FAKE + 2) == E                 # misaligned
    assert call(depth=FAKE + 6) == E
    assert call(B=0) == E
    assert call(D=0) == E
    assert call(Q=0) == E
    assert call(Q=257) == E
    assert call(K=0) == U
    assert call(K=65) == U
    assert call(B=(1 << 26) + 1) == U                 # B x 64 work-items past 2^32
    assert call(D=2, K=2, Q=8) == E                   # the depth-2 binary tree has 7 nodes
    assert call(D=1, K=64, Q=66) == E


def test_tree_accept_argument_checks(lib):
    """Host checks of the accept step come before any HIP call."""
    E, U = dd.DDTV_EINVAL, dd.DDTV_EUNSUPPORTED
    vis = fake_vis(B=2, Q=9)

    def call(logits=FAKE, V=32, v=vis, ckv=None, k_rope=None, dtype=0, pred=FAKE + 4096, accept_len=FAKE + 8192):
        return lib.ddtv_tree_accept(logits, V, FAKE, FAKE, ctypes.byref(v.vis) if v is not None else None, ckv,
                                    k_rope, dtype, pred, FAKE, FAKE, accept_len, None)

    assert call(logits=None) == E
    assert call(pred=None) == E
    assert call(accept_len=FAKE + 2) == E
    assert call(v=None) == E
    assert call(V=0) == E
    assert call(ckv=FAKE) == E                        # one cache without the other
    assert call(ckv=FAKE + 8, k_rope=FAKE) == E       # misaligned cache
    assert call(ckv=FAKE, k_rope=FAKE, dtype=5) == U
    big = fake_vis(B=(1 << 18) + 1, Q=64, prefix=np.zeros((1 << 18) + 1, np.int32))
    assert call(v=big) == U                           # B x Q x 256 work-items past 2^32


def test_tail_mode_argument_checks(lib):
    """The external-prefix call's host checks come before any HIP call."""
    vis = fake_vis(B=2, Q=24, prefix=(100, 0))
    need = dd.ddtv_tail_workspace_bytes(vis, 8, 0)
    assert need >= 2 * 16 + 2 * 24 * 8 * 4

    def call(po=FAKE, pl=FAKE, ws=FAKE, ws_bytes=need):
        return lib.ddtv_verify_attn_tail(FAKE, FAKE, FAKE, FAKE, 0, 8, ctypes.byref(vis.vis), ctypes.c_float(0.07),
                                         po, pl, FAKE, None, ws, ws_bytes, None, None)

    assert call(po=None) == dd.DDTV_EINVAL
    assert call(pl=None) == dd.DDTV_EINVAL
    assert call(po=FAKE + 4) == dd.DDTV_EINVAL            # prefix output must be 16-byte aligned
    assert call(ws=None) == dd.DDTV_EWORKSPACE
    assert call(ws_bytes=need - 1) == dd.DDTV_EWORKSPACE
    assert call(ws=FAKE + 16) == dd.DDTV_EINVAL           # workspace must be 256-byte aligned


def test_neighbour_argument_checks(lib):
    """Host checks of query preparation, value projection and cache append come before any HIP call."""
    E, U = dd.DDTV_EINVAL, dd.DDTV_EUNSUPPORTED
    vis = fake_vis(B=2, Q=9)

    def prep(q=FAKE, d_nope=128, H=8, v=vis, pos=None, theta=50000.0, w=FAKE, qa=FAKE, qr=FAKE):
        return lib.ddtv_prepare_query(q, d_nope, H, ctypes.byref(v.vis) if v is not None else None, pos, theta,
                                      w, qa, qr, None)

    assert prep(q=None) == E
    assert prep(w=None) == E
    assert prep(qa=FAKE + 8) == E                  # 16-byte alignment
    assert prep(pos=FAKE + 2) == E
    assert prep(v=None) == E
    assert prep(H=0) == E
    assert prep(H=1025) == E
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert prep(theta=bad) == E
    for d in (0, 16, 48, 544):
        assert prep(d_nope=d) == U

    def vproj(lat=FAKE, M=18, H=8, d_v=128, w=FAKE, v=FAKE):
        return lib.ddtv_value_proj(lat, M, H, d_v, w, v, None)

    assert vproj(lat=None) == E
    assert vproj(v=None) == E
    assert vproj(lat=FAKE + 4) == E
    assert vproj(M=-1) == E
    assert vproj(H=0) == E
    assert vproj(d_v=0) == U
    assert vproj(d_v=513) == U
    assert vproj(M=(1 << 28) + 1) == U
    assert vproj(M=0) == dd.DDTV_OK                 # nothing to do, nothing launched

    def app(lat=FAKE, kpe=FAKE, v=vis, pos=None, theta=50000.0, ckv=FAKE, kr=FAKE, dtype=0):
        return lib.ddtv_append_kv(lat, kpe, ctypes.byref(v.vis) if v is not None else None, pos, theta, ckv, kr,
                                  dtype, None)

    assert app(lat=None) == E
    assert app(kr=None) == E
    assert app(ckv=FAKE + 8) == E
    assert app(v=None) == E
    assert app(theta=0.0) == E
    assert app(dtype=7) == U
    big = fake_vis(B=(1 << 20) + 1, Q=64, prefix=np.zeros((1 << 20) + 1, np.int32))
    assert app(v=big) == U                            # B x Q x 64 work-items past 2^32


def test_plan_rules(lib):
    # fewer than 16 query rows per batch row (Q * H) -> VALU, else MFMA; forced paths honoured
    for Q, H, want in [(1, 8, dd.DDTV_PATH_VALU), (1, 15, dd.DDTV_PATH_VALU), (15, 1, dd.DDTV_PATH_VALU),
                       (1, 16, dd.DDTV_PATH_MFMA), (16, 1, dd.DDTV_PATH_MFMA), (9, 8, dd.DDTV_PATH_MFMA),
                       (128, 16, dd.DDTV_PATH_MFMA)]:
        vis = fake_vis(B=1, Q=Q, prefix=(100,))
        rc, path, L, ns, wg, order = dd.ddtv_plan_info(vis, H, 0)
        assert rc == 0 and path == want, (Q, H, path)
    vis = fake_vis(B=1, Q=9, prefix=(100,))
    assert dd.ddtv_plan_info(vis, 8, 0, dd.make_opts(path=dd.DDTV_PATH_MFMA))[1] == dd.DDTV_PATH_MFMA
    # at most 32 query rows on the matrix path: row-half mode, 32 rows per workgroup, whose
    # two halves are combined in the workgroup: one partial per split, none with a single
    # split; bf16 caches keep their own kernel
    def ru(x):
        return (x + 255) // 256 * 256
    for Q, H, path in [(1, 16, 0), (2, 16, 0), (9, 1, dd.DDTV_PATH_MFMA), (4, 8, dd.DDTV_PATH_MFMA_F32)]:
        vis = fake_vis(B=2, Q=Q, prefix=(1000, 3))
        opts = dd.make_opts(path=path) if path else None
        rc, p_, L, ns, wg, order = dd.ddtv_plan_info(vis, H, 0, opts)
        assert rc == 0 and p_ == dd.DDTV_PATH_MFMA and wg == 2 * ns, (Q, H, p_, wg, ns)
        rows = 2 * ns * Q * H
        want = ru(rows * 512 * 4) + ru(rows * 8) if ns > 1 else 0
        assert dd.ddtv_workspace_bytes(vis, H, 0, opts) == want, (Q, H)
    vis = fake_vis(B=2, Q=1, prefix=(1000, 3))
    rc, p_, L, ns, wg, order = dd.ddtv_plan_info(vis, 16, dd.DDTV_BF16)
    rows = 2 * ns * 16                                   # one partial per split
    assert rc == 0 and dd.ddtv_workspace_bytes(vis, 16, dd.DDTV_BF16) == (ru(rows * 2048) + ru(rows * 8) if ns > 1 else 0)
    # 33 rows: the usual 64-row mode, one partial per split (none with a single split)
    vis = fake_vis(B=2, Q=3, prefix=(1000, 3))
    for L in (0, 128, 2048):
        opts = dd.make_opts(split_len=L)
        rc, p_, L_, ns, wg, order = dd.ddtv_plan_info(vis, 11, 0, opts)
        rows = 2 * ns * 33
        want = ru(rows * 2048) + ru(rows * 8) if ns > 1 else 0
        assert rc == 0 and wg == 2 * ns and dd.ddtv_workspace_bytes(vis, 11, 0, opts) == want, (L, ns)
    # 32 rows on the same trees: row-half mode (one workgroup per split instead of two),
    # one partial per split, none with a single split
    vis32 = fake_vis(B=2, Q=2, prefix=(1000, 3))
    for L in (128, 2048):
        opts = dd.make_opts(split_len=L)
        rc, p_, L_, ns, wg, order = dd.ddtv_plan_info(vis32, 16, 0, opts)
        rows = 2 * ns * 32
        want = ru(rows * 2048) + ru(rows * 8) if ns > 1 else 0
        assert rc == 0 and wg == 2 * ns, (L, ns, wg)
        assert dd.ddtv_workspace_bytes(vis32, 16, 0, opts) == want, (L, ns)
    # a grid past 2^32 work-items is refused before any launch
    big = fake_vis(B=(1 << 16) + 1, Q=256, prefix=np.zeros((1 << 16) + 1, np.int32))
    assert dd.ddtv_plan_info(big, 128, 0)[0] == dd.DDTV_EUNSUPPORTED
    # a forced split length gives ceil(max_kv / L) splits and a matching workspace
    vis = fake_vis(B=2, Q=64, prefix=(1000, 5000))
    opts = dd.make_opts(split_len=1024)
    rc, path, L, ns, wg, order = dd.ddtv_plan_info(vis, 16, 0, opts)
    assert (L, ns) == (1024, (5064 + 1023) // 1024)
    R = 64 * 16
    assert wg == 2 * ns * ((R + 63) // 64)
    ws = dd.ddtv_workspace_bytes(vis, 16, 0, opts)
    assert ws >= 2 * ns * R * (512 * 4 + 8)
    # single split: no workspace
    opts = dd.make_opts(split_len=8192)
    assert dd.ddtv_workspace_bytes(vis, 16, 0, opts) == 0
    assert dd.ddtv_plan_info(vis, 16, 0, opts)[3] == 1


def test_auto_plan_shapes(lib):
    """The automatic planner fills the device with small grids and keeps big ones whole."""
    vis = fake_vis(B=1, Q=64, prefix=(4096,))          # 16 row tiles: must split
    rc, path, L, ns, wg, order = dd.ddtv_plan_info(vis, 16, 0)
    assert rc == 0 and ns > 1 and wg >= 128
    vis = fake_vis(B=8, Q=128, prefix=(32768,) * 8)    # 256 row tiles of equal work
    rc, path, L, ns, wg, order = dd.ddtv_plan_info(vis, 16, 0)
    assert rc == 0 and wg >= 256
    assert L % 64 == 0


def test_workgroup_order_rules(lib):
    """Equal-length batch rows keep the XCD-local order (each XCD's L2 serves the
    query tiles that share a cache tile); when one row is far longer than the
    rest, XCD-local would leave that row's XCD with most of the work, so the
    planner spreads each row's query tiles over all XCDs.  Forced orders are
    honoured and change nothing else in the plan."""
    vis = fake_vis(B=8, Q=128, prefix=(32768,) * 8)
    rc, path, L, ns, wg, order = dd.ddtv_plan_info(vis, 16, 0)
    assert rc == 0 and order == dd.DDTV_ORDER_XCD_LOCAL
    ragged = fake_vis(B=8, Q=64, prefix=(131072,) + (1024,) * 7)
    for dtype in (0, 1):
        rc, path, L, ns, wg, order = dd.ddtv_plan_info(ragged, 64, dtype)
        assert rc == 0 and order == dd.DDTV_ORDER_SPREAD, dtype
    for want in (dd.DDTV_ORDER_XCD_LOCAL, dd.DDTV_ORDER_SPREAD):
        opts = dd.make_opts(split_len=4096, wg_order=want)
        rc, path, L, ns, wg, order = dd.ddtv_plan_info(ragged, 64, 1, opts)
        assert (rc, L, order) == (0, 4096, want)
        assert ns == (131072 + 64 + 4095) // 4096 and wg == 8 * ns * 64
    assert dd.ddtv_plan_info(ragged, 64, 1, dd.make_opts(wg_order=7))[0] == dd.DDTV_EUNSUPPORTED
    # rows of random length (the long ones anywhere in the batch): with the row-order
    # table the spread grid starts the longest rows first and needs no KV split
    pre = tuple(int(x) for x in np.random.default_rng(5).integers(1024, 131073, 32))
    rc, path, L, ns, wg, order = dd.ddtv_plan_info(fake_vis(B=32, Q=64, prefix=pre), 64, 1)
    assert (rc, order, ns) == (0, dd.DDTV_ORDER_SPREAD, 1)


def test_oracle_shares_error_contract(lib):
    """The oracle rejects the same shapes the library rejects."""
    o = oracle._load()
    bits = np.zeros(4, np.uint32)
    out = np.zeros(512)
    lse = np.zeros(1)
    pre = np.array([-1], np.int32)
    q = np.zeros((1, 1, 1, 512), np.float32)
    rc = o.ddtvref_verify_attn_rows(q.ctypes.data, q.ctypes.data, q.ctypes.data, q.ctypes.data, 0, 1, 1, 1,
                                    pre.ctypes.data, bits.ctypes.data, 1.0, None, 0, out.ctypes.data,
                                    lse.ctypes.data, None)
    assert rc == oracle.REF_EINVAL == dd.DDTV_EINVAL
    b, _, rc = oracle.build_visibility(np.array([[0, 0]], np.int32))
    assert rc == oracle.REF_ETREE == dd.DDTV_ETREE


def test_plan_cache_is_thread_safe(lib):
    """Plans come from a small shared cache (more shapes than entries here, so
    entries are evicted while other threads read): every thread must get exactly
    the plan a lone caller gets, and repeated calls must agree."""
    from concurrent.futures import ThreadPoolExecutor
    shapes = [(B, Q, H, tuple(int(p) for p in np.random.default_rng(B * 1000 + Q).integers(0, 40000, B)))
              for B in (1, 3, 8) for Q in (16, 64, 128) for H in (8, 16, 64)]
    keep = {}

    def plan(shape):
        B, Q, H, prefix = shape
        vis = fake_vis(B=B, Q=Q, prefix=prefix)
        keep[shape] = vis                 # the borrowed prefix array must outlive the call
        return dd.ddtv_plan_info(vis, H, 0)

    expected = {s: plan(s) for s in shapes}
    with ThreadPoolExecutor(8) as ex:
        for _ in range(3):
            got = list(ex.map(plan, shapes * 4))
            assert got == [expected[s] for s in shapes * 4]


def test_header_is_c11_and_links_from_c(lib, tmp_path):
    """include/ddtv.h compiles as C11 (gcc, warnings as errors) and a C program links
    against libddtv.so and calls it: the version, a status string and an argument
    error reported before any HIP call (no GPU needed)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = tmp_path / "use_ddtv.c"
    src.write_text(r'''
#include <stdio.h>
#include <string.h>
#include "ddtv.h"
int main(void) {
    ddtv_vis vis;
    memset(&vis, 0, sizeof vis);
    if (ddtv_version() <= 0) return 1;
    if (strcmp(ddtv_status_string(DDTV_EINVAL), "invalid argument") != 0) return 2;
    /* null inputs and an empty visibility: rejected on the host */
    if (ddtv_verify_attn(NULL, NULL, NULL, NULL, DDTV_F32, 8, &vis, 0.07f, NULL, NULL, NULL, 0, NULL) != DDTV_EINVAL)
        return 3;
    if (ddtv_vis_bytes(0, 9) != 0 || ddtv_vis_bytes(1, 9) == 0) return 4;
    printf("%d\n", (int)ddtv_version());
    return 0;
}
''')
    exe = tmp_path / "use_ddtv"
    libdir = os.path.dirname(dd.LIB_PATH)
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), str(src), "-L" + libdir, "-lddtv", "-Wl,-rpath," + libdir,
           "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stderr)
    assert int(r.stdout.strip()) == dd.ddtv_version()


def test_noalloc_host_errors(lib):
    """ddtv_verify_attn_noalloc checks its arguments like ddtv_verify_attn_ex and
    refuses, before any HIP call, a plan whose partials exceed the scratch."""
    vis = fake_vis(B=2, Q=64, prefix=(20000, 3000))
    E = dd.DDTV_EINVAL

    def call(q_abs=FAKE, out=FAKE, scale=0.07, H=16, opts=None):
        return lib.ddtv_verify_attn_noalloc(q_abs, FAKE, FAKE, FAKE, 0, H, ctypes.byref(vis.vis),
                                            ctypes.c_float(scale), out, None, None,
                                            ctypes.byref(opts) if opts is not None else None)
    assert call(q_abs=None) == E
    assert call(out=FAKE + 4) == E
    assert call(scale=float("nan")) == E
    assert call(H=0) == E
    assert call(opts=dd.make_opts(split_len=100)) == E
    # 32-position splits: 626 splits x 2 batch rows x 1024 query rows of partials, far past the scratch
    assert call(opts=dd.make_opts(split_len=32)) == dd.DDTV_EWORKSPACE
    need = dd.ddtv_workspace_bytes(vis, 16, 0, dd.make_opts(split_len=32))
    assert need > dd.NOALLOC_SCRATCH_BYTES


def workload_vis(name, q_len=None):
    """A visibility struct with the geometry of a named workload (fake device
    pointers: planning reads only the host-side fields)."""
    import workloads as wl
    parent, pre = wl.config_trees(name)
    B, Q = parent.shape
    if q_len is not None:
        Q = q_len
    H = {"c1": 8, "c2": 8, "c3": 16, "c4": 16, "c5": 64}[name]
    return fake_vis(B, Q, tuple(int(x) for x in pre)), H


@pytest.mark.parametrize("name,q_len,dtype,want", [
    ("c3", None, 0, (2, 272, 16, 256, dd.DDTV_ORDER_XCD_LOCAL)),
    ("c4", None, 0, (2, 32896, 1, 256, dd.DDTV_ORDER_XCD_LOCAL)),
    ("c4", 1, 0, (2, 1024, 32, 256, dd.DDTV_ORDER_XCD_LOCAL)),
    ("c5", None, 1, (2, None, 1, 2048, dd.DDTV_ORDER_SPREAD)),
])
def test_plans_of_the_benchmarked_workloads(lib, name, q_len, dtype, want):
    """The split plans the measurements were taken with: c3 in 16 splits of 272
    rows (the last tile of each a half tile) on 256 workgroups, c4 unsplit, c4
    sizes at q_len 1 in 32 splits (row-half mode), c5 unsplit in the spread order."""
    vis, H = workload_vis(name, q_len)
    rc, path, split_len, n_split, wgs, order = dd.ddtv_plan_info(vis, H, dtype)
    assert rc == dd.DDTV_OK
    got = (path, split_len, n_split, wgs, order)
    for g, w in zip(got, want):
        assert w is None or g == w, (name, got, want)


@pytest.mark.parametrize("name,q_len,dtype", [("c5", None, 1), ("c4", 1, 0), ("c3", None, 0), ("c4", None, 0)])
def test_uncached_planning_is_cheap(lib, name, q_len, dtype):
    """A verify loop whose prefixes grow every step misses the plan cache each
    call; planning must stay far below the GPU step it plans.  Median of 25
    calls, each on prefixes one position longer than the last."""
    import statistics
    import time
    vis0, H = workload_vis(name, q_len)
    pre = np.ctypeslib.as_array(ctypes.cast(vis0.vis.prefix_host, ctypes.POINTER(ctypes.c_int32)), (vis0.vis.B,))
    ts = []
    for i in range(25):
        vis = fake_vis(vis0.vis.B, vis0.vis.Q, tuple(int(x) + i + 1 for x in pre))
        t0 = time.perf_counter()
        rc = dd.ddtv_plan_info(vis, H, dtype)[0]
        ts.append(time.perf_counter() - t0)
        assert rc == dd.DDTV_OK
    med = statistics.median(ts)
    print(f"{name} q_len {q_len or vis0.vis.Q}: uncached plan {med * 1e6:.1f} us")
    assert med < 200e-6, f"{name}: uncached planning took {med * 1e6:.0f} us"


def test_split_lengths_off_the_tile_grid(lib):
    """Split lengths are multiples of 16; the planner takes one off the 32-row grid
    (an odd multiple of 16) only for the fp32 matrix kernel on an fp32 cache, whose
    last tile of at most 16 rows then runs as half a tile, and only when the grid
    starts in one round (c3's shape: 16 splits of 272 rows on 256 workgroups)."""
    vis = fake_vis(B=1, Q=64, prefix=(4096,))
    assert verify_call(lib, vis, opts=dd.make_opts(split_len=40)) == dd.DDTV_EINVAL
    rc, path, L, ns, wg, order = dd.ddtv_plan_info(vis, 16, 0, dd.make_opts(split_len=48))
    assert rc == 0 and (L, ns) == (48, (4160 + 47) // 48)
    rc, path, L, ns, wg, order = dd.ddtv_plan_info(vis, 16, 0)   # (256 CUs: MI355X, or no device)
    assert rc == 0 and (L, ns, wg) == (272, 16, 256), (L, ns, wg)
    # a half tile has to beat the tile-aligned length by the planner's 2 % margin: a c4-sized
    # batch whose longest prefix grew by 5 rows keeps one tile-aligned split
    grown = fake_vis(B=8, Q=128, prefix=(32768 + 5,) + (32768,) * 7)
    rc, path, L, ns, wg, order = dd.ddtv_plan_info(grown, 16, 0)
    assert rc == 0 and (L, ns) == (32928, 1), (L, ns)
    small = fake_vis(B=1, Q=64, prefix=(1000,))           # 3.5 tiles beat 4 by more than that
    assert dd.ddtv_plan_info(small, 16, 0)[2:4] == (112, 10)
    # in row-half mode a row's last split takes a remainder of up to 16 positions: decode rows one
    # position past 32 x 1024 keep 32 splits of 1024, 17 past need a 33rd; the vector path, the
    # usual matrix mode and the bf16 matrix kernel end every split at the split length
    for extra, want in ((1, 32), (16, 32), (17, 33)):
        dec = fake_vis(B=8, Q=1, prefix=(32767 + extra,) * 8)
        assert dd.ddtv_plan_info(dec, 16, 0, dd.make_opts(split_len=1024))[2:4] == (1024, want), extra
    dec = fake_vis(B=8, Q=1, prefix=(32768,) * 8)
    assert dd.ddtv_plan_info(dec, 16, 0)[2:4] == (1024, 32)
    assert dd.ddtv_plan_info(dec, 16, 0, dd.make_opts(split_len=1024, path=dd.DDTV_PATH_VALU))[2:4] == (1024, 33)
    bfv = fake_vis(B=2, Q=64, prefix=(2048 + 8 - 64,) * 2)   # 2 x 1024 + 8 positions per row
    assert dd.ddtv_plan_info(bfv, 16, dd.DDTV_BF16, dd.make_opts(split_len=1024))[2:4] == (1024, 3)
    assert dd.ddtv_plan_info(bfv, 16, 0, dd.make_opts(split_len=1024))[2:4] == (1024, 3)
    # the other kernels keep 32-row split lengths: bf16 matrix kernel, FP8 cache, vector path
    for dtype, opts in [(dd.DDTV_BF16, None), (dd.DDTV_FP8_E4M3, None), (0, dd.make_opts(path=dd.DDTV_PATH_VALU))]:
        rc, path, L, ns, wg, order = dd.ddtv_plan_info(vis, 16, dtype, opts)
        assert rc == 0 and L % 32 == 0, (dtype, L)
