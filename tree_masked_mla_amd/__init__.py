"""Python binding of libddtv (DDTree tree-verify MLA-absorb attention on MI355X).

Argument marshalling only: every step of the computation runs in the HIP kernels
of ``libddtv.so``.  PyTorch supplies device memory and the HIP stream.  The
functions carry the names of the C entry points declared in include/ddtv.h.

Importing this package does not need a GPU; calling into the library does need
the built ``libddtv.so`` (``python -m tree_masked_mla_amd.build``) and raises
``DdtvLibraryMissing`` if it is absent -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libddtv.so")

DDTV_OK, DDTV_EINVAL, DDTV_ETREE, DDTV_EUNSUPPORTED, DDTV_EWORKSPACE, DDTV_EDEVICE = range(6)
DDTV_F32, DDTV_BF16, DDTV_FP8_E4M3 = 0, 1, 2
DDTV_PATH_AUTO, DDTV_PATH_VALU, DDTV_PATH_MFMA, DDTV_PATH_MFMA_F32 = 0, 1, 2, 3
DDTV_ORDER_AUTO, DDTV_ORDER_XCD_LOCAL, DDTV_ORDER_SPREAD = 0, 1, 2
D_LATENT, D_ROPE, MAX_Q = 512, 64, 256
NOALLOC_SCRATCH_BYTES = 40 << 20   # DDTV_NOALLOC_SCRATCH_BYTES

EXPORTED = (
    "ddtv_vis_bytes", "ddtv_build_visibility", "ddtv_read_status", "ddtv_workspace_bytes",
    "ddtv_workspace_bytes_ex", "ddtv_verify_attn", "ddtv_verify_attn_ex", "ddtv_plan_info",
    "ddtv_status_string", "ddtv_version", "ddtv_build_tree", "ddtv_tree_accept",
    "ddtv_tail_workspace_bytes", "ddtv_verify_attn_tail", "ddtv_prepare_query", "ddtv_value_proj",
    "ddtv_append_kv", "ddtv_verify_attn_noalloc",
)


class DdtvLibraryMissing(RuntimeError):
    pass


class DdtvError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = code
        super().__init__(f"{what}: {ddtv_status_string(code)} ({code})" if what else ddtv_status_string(code))


class ddtv_vis(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Q", ctypes.c_int32), ("W", ctypes.c_int32),
                ("max_kv", ctypes.c_int32), ("total_kv", ctypes.c_int64),
                ("bits", ctypes.c_void_p), ("rows", ctypes.c_void_p), ("status", ctypes.c_void_p),
                ("order", ctypes.c_void_p), ("prefix_host", ctypes.c_void_p)]


class ddtv_opts(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("split_len", ctypes.c_int32),
                ("attn_begin", ctypes.c_void_p), ("attn_end", ctypes.c_void_p), ("wg_order", ctypes.c_int32)]


_lib = None


def share_hip_runtime_with_torch() -> None:
    """Import torch (when installed) before any of this package's HIP libraries is
    loaded.  torch ships its own copy of the HIP runtime under the same soname as
    the system's: whichever loads first serves the library, and a process that
    loads the library first ends up holding two runtimes, the library's blind to
    the device memory (and, on some drivers, the devices) the other one owns."""
    try:
        import torch  # noqa: F401
    except ImportError:
        pass


def load(path: str = LIB_PATH):
    """Load libddtv.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise DdtvLibraryMissing(f"{path} not found; build it with `python -m tree_masked_mla_amd.build`")
    share_hip_runtime_with_torch()
    lib = ctypes.CDLL(path)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    VP, OP = ctypes.POINTER(ddtv_vis), ctypes.POINTER(ddtv_opts)
    lib.ddtv_vis_bytes.argtypes = [i32, i32]
    lib.ddtv_vis_bytes.restype = sz
    lib.ddtv_build_visibility.argtypes = [P, P, i32, i32, P, sz, VP, P]
    lib.ddtv_build_visibility.restype = ctypes.c_int
    lib.ddtv_read_status.argtypes = [VP, ctypes.POINTER(i32), ctypes.POINTER(i32), P]
    lib.ddtv_read_status.restype = ctypes.c_int
    lib.ddtv_workspace_bytes.argtypes = [VP, i32, ctypes.c_int]
    lib.ddtv_workspace_bytes.restype = sz
    lib.ddtv_workspace_bytes_ex.argtypes = [VP, i32, ctypes.c_int, OP]
    lib.ddtv_workspace_bytes_ex.restype = sz
    lib.ddtv_verify_attn.argtypes = [P, P, P, P, ctypes.c_int, i32, VP, ctypes.c_float, P, P, P, sz, P]
    lib.ddtv_verify_attn.restype = ctypes.c_int
    lib.ddtv_verify_attn_ex.argtypes = [P, P, P, P, ctypes.c_int, i32, VP, ctypes.c_float, P, P, P, sz, P, OP]
    lib.ddtv_verify_attn_ex.restype = ctypes.c_int
    lib.ddtv_verify_attn_noalloc.argtypes = [P, P, P, P, ctypes.c_int, i32, VP, ctypes.c_float, P, P, P, OP]
    lib.ddtv_verify_attn_noalloc.restype = ctypes.c_int
    lib.ddtv_plan_info.argtypes = [VP, i32, ctypes.c_int, OP, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                   ctypes.POINTER(i32), ctypes.POINTER(i64), ctypes.POINTER(i32)]
    lib.ddtv_plan_info.restype = ctypes.c_int
    lib.ddtv_build_tree.argtypes = [P, P, i32, i32, i32, i32, P, P, P, P, P, P]
    lib.ddtv_build_tree.restype = ctypes.c_int
    lib.ddtv_tree_accept.argtypes = [P, i32, P, P, VP, P, P, ctypes.c_int, P, P, P, P, P]
    lib.ddtv_tree_accept.restype = ctypes.c_int
    lib.ddtv_tail_workspace_bytes.argtypes = [VP, i32, ctypes.c_int, OP]
    lib.ddtv_tail_workspace_bytes.restype = sz
    lib.ddtv_verify_attn_tail.argtypes = [P, P, P, P, ctypes.c_int, i32, VP, ctypes.c_float, P, P, P, P, P, sz, P, OP]
    lib.ddtv_verify_attn_tail.restype = ctypes.c_int
    f64 = ctypes.c_double
    lib.ddtv_prepare_query.argtypes = [P, i32, i32, VP, P, f64, P, P, P, P]
    lib.ddtv_prepare_query.restype = ctypes.c_int
    lib.ddtv_value_proj.argtypes = [P, ctypes.c_int64, i32, i32, P, P, P]
    lib.ddtv_value_proj.restype = ctypes.c_int
    lib.ddtv_append_kv.argtypes = [P, P, VP, P, f64, P, P, ctypes.c_int, P]
    lib.ddtv_append_kv.restype = ctypes.c_int
    lib.ddtv_status_string.argtypes = [ctypes.c_int]
    lib.ddtv_status_string.restype = ctypes.c_char_p
    lib.ddtv_version.argtypes = []
    lib.ddtv_version.restype = i32
    _lib = lib
    return lib


# ----------------------------------------------------------------------------- marshalling helpers
def _ptr(x) -> int | None:
    """Device/host address of a torch tensor, numpy array, int or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _event(ev) -> int | None:
    if ev is None:
        return None
    if isinstance(ev, int):
        return ev
    return ev.cuda_event


def make_opts(path: int = DDTV_PATH_AUTO, split_len: int = 0, attn_begin=None, attn_end=None,
              wg_order: int = DDTV_ORDER_AUTO) -> ddtv_opts:
    return ddtv_opts(path, split_len, _event(attn_begin), _event(attn_end), wg_order)


class Visibility:
    """Holds the C struct plus the Python objects its pointers borrow from."""

    def __init__(self, vis: ddtv_vis, keep: tuple):
        self.vis = vis
        self._keep = keep

    def __getattr__(self, name):
        return getattr(self.vis, name)


# ----------------------------------------------------------------------------- entry points
def ddtv_version() -> int:
    return load().ddtv_version()


def ddtv_status_string(code: int) -> str:
    return load().ddtv_status_string(int(code)).decode()


def ddtv_vis_bytes(B: int, Q: int) -> int:
    return load().ddtv_vis_bytes(B, Q)


def ddtv_build_visibility(parent, prefix_len, B: int, Q: int, vis_buf, vis_buf_bytes: int | None = None,
                          stream=None):
    """parent: device int32 [B][Q]; prefix_len: host int32 [B] (numpy); vis_buf: device buffer.
    Returns (status, Visibility)."""
    prefix = np.ascontiguousarray(prefix_len, dtype=np.int32)
    if vis_buf_bytes is None:
        vis_buf_bytes = vis_buf.numel() * vis_buf.element_size()
    vis = ddtv_vis()
    rc = load().ddtv_build_visibility(_ptr(parent), _ptr(prefix), B, Q, _ptr(vis_buf), vis_buf_bytes,
                                      ctypes.byref(vis), _stream(stream))
    return rc, Visibility(vis, (prefix, vis_buf, parent))


def ddtv_read_status(vis: Visibility, stream=None):
    """Returns (status, bad_row, bad_node)."""
    r, n = ctypes.c_int32(-1), ctypes.c_int32(-1)
    rc = load().ddtv_read_status(ctypes.byref(vis.vis), ctypes.byref(r), ctypes.byref(n), _stream(stream))
    return rc, r.value, n.value


def ddtv_workspace_bytes(vis: Visibility, H: int, kv_dtype: int, opts: ddtv_opts | None = None) -> int:
    lib = load()
    if opts is None:
        return lib.ddtv_workspace_bytes(ctypes.byref(vis.vis), H, kv_dtype)
    return lib.ddtv_workspace_bytes_ex(ctypes.byref(vis.vis), H, kv_dtype, ctypes.byref(opts))


def ddtv_plan_info(vis: Visibility, H: int, kv_dtype: int, opts: ddtv_opts | None = None):
    """Returns (status, path, split_len, n_split, workgroups, wg_order)."""
    p, L, ns, order = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    wg = ctypes.c_int64()
    rc = load().ddtv_plan_info(ctypes.byref(vis.vis), H, kv_dtype,
                               ctypes.byref(opts) if opts is not None else None,
                               ctypes.byref(p), ctypes.byref(L), ctypes.byref(ns), ctypes.byref(wg),
                               ctypes.byref(order))
    return rc, p.value, L.value, ns.value, wg.value, order.value


def ddtv_build_tree(logp, Q: int, parent, tokens=None, depth=None, rank=None, token=None, score=None,
                    stream=None) -> int:
    """logp: device float32 [B][D][K]; outputs: device [B][Q] tensors (parent required)."""
    B, D, K = (int(x) for x in logp.shape)
    return load().ddtv_build_tree(_ptr(logp), _ptr(tokens), B, D, K, Q, _ptr(parent), _ptr(depth), _ptr(rank),
                                  _ptr(token), _ptr(score), _stream(stream))


def ddtv_tree_accept(logits, parent, token, vis: Visibility, pred, path, out_tokens, accept_len, ckv=None,
                     k_rope=None, kv_dtype: int = DDTV_F32, stream=None) -> int:
    """logits: device float32 [B][Q][V]; parent/token: device int32 [B][Q]; outputs: device int32 tensors."""
    V = int(logits.shape[-1])
    return load().ddtv_tree_accept(_ptr(logits), V, _ptr(parent), _ptr(token), ctypes.byref(vis.vis), _ptr(ckv),
                                   _ptr(k_rope), kv_dtype, _ptr(pred), _ptr(path), _ptr(out_tokens),
                                   _ptr(accept_len), _stream(stream))


def ddtv_tail_workspace_bytes(vis: Visibility, H: int, kv_dtype: int, opts: ddtv_opts | None = None) -> int:
    return load().ddtv_tail_workspace_bytes(ctypes.byref(vis.vis), H, kv_dtype,
                                            ctypes.byref(opts) if opts is not None else None)


def ddtv_verify_attn_tail(q_abs, q_rope, ckv, k_rope, kv_dtype: int, H: int, vis: Visibility, scale: float,
                          prefix_out, prefix_lse, out, lse, workspace, workspace_bytes: int | None = None,
                          stream=None, opts: ddtv_opts | None = None) -> int:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return load().ddtv_verify_attn_tail(_ptr(q_abs), _ptr(q_rope), _ptr(ckv), _ptr(k_rope), kv_dtype, H,
                                        ctypes.byref(vis.vis), ctypes.c_float(scale), _ptr(prefix_out),
                                        _ptr(prefix_lse), _ptr(out), _ptr(lse), _ptr(workspace), workspace_bytes,
                                        _stream(stream), ctypes.byref(opts) if opts is not None else None)


def ddtv_verify_attn(q_abs, q_rope, ckv, k_rope, kv_dtype: int, H: int, vis: Visibility, scale: float, out,
                     lse=None, workspace=None, workspace_bytes: int | None = None, stream=None,
                     opts: ddtv_opts | None = None) -> int:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = load()
    args = (_ptr(q_abs), _ptr(q_rope), _ptr(ckv), _ptr(k_rope), kv_dtype, H, ctypes.byref(vis.vis),
            ctypes.c_float(scale), _ptr(out), _ptr(lse), _ptr(workspace), workspace_bytes, _stream(stream))
    if opts is None:
        return lib.ddtv_verify_attn(*args)
    return lib.ddtv_verify_attn_ex(*args, ctypes.byref(opts))


def ddtv_verify_attn_noalloc(q_abs, q_rope, ckv, k_rope, kv_dtype: int, H: int, vis: Visibility, scale: float,
                             out, lse=None, stream=None, opts: ddtv_opts | None = None) -> int:
    """ddtv_verify_attn_ex without a workspace: split partials go to the library's
    per-GPU scratch (DDTV_NOALLOC_SCRATCH_BYTES)."""
    return load().ddtv_verify_attn_noalloc(_ptr(q_abs), _ptr(q_rope), _ptr(ckv), _ptr(k_rope), kv_dtype, H,
                                           ctypes.byref(vis.vis), ctypes.c_float(scale), _ptr(out), _ptr(lse),
                                           _stream(stream), ctypes.byref(opts) if opts is not None else None)


def ddtv_prepare_query(q, w_kc, vis: Visibility, q_abs, q_rope, rope_theta: float, positions=None,
                       stream=None) -> int:
    """q: device float32 [B][Q][H][d_nope + 64]; w_kc: [H][d_nope][512]; outputs [B][Q][H][512], [B][Q][H][64]."""
    H, row = int(q.shape[-2]), int(q.shape[-1])
    return load().ddtv_prepare_query(_ptr(q), row - 64, H, ctypes.byref(vis.vis), _ptr(positions),
                                     float(rope_theta), _ptr(w_kc), _ptr(q_abs), _ptr(q_rope), _stream(stream))


def ddtv_value_proj(latent, w_vc, v, stream=None) -> int:
    """latent: device float32 [..., H, 512]; w_vc: [H][d_v][512]; v: [..., H, d_v]."""
    H, d_v = int(w_vc.shape[0]), int(w_vc.shape[1])
    M = latent.numel() // (H * 512)
    return load().ddtv_value_proj(_ptr(latent), M, H, d_v, _ptr(w_vc), _ptr(v), _stream(stream))


def ddtv_append_kv(latent, k_pe, vis: Visibility, ckv, k_rope, kv_dtype: int, rope_theta: float, positions=None,
                   stream=None) -> int:
    """latent: device float32 [B][Q][512]; k_pe: [B][Q][64]; caches [total_kv][512], [total_kv][64]."""
    return load().ddtv_append_kv(_ptr(latent), _ptr(k_pe), ctypes.byref(vis.vis), _ptr(positions),
                                 float(rope_theta), _ptr(ckv), _ptr(k_rope), kv_dtype, _stream(stream))


ddtv_verify_attn_ex = ddtv_verify_attn
ddtv_workspace_bytes_ex = ddtv_workspace_bytes


def check(code: int, what: str = "") -> None:
    if code != DDTV_OK:
        raise DdtvError(code, what)
