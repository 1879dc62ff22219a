"""CPU oracle for DDTree tree-verify MLA-absorb attention (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library never does.  The
arithmetic lives in ``ddtv_oracle.c`` (plain fp64 C, single-threaded); this file
only compiles it with gcc, marshals numpy arrays and returns numpy results.
The best-first draft-tree builder's oracle lives in ``ddtv_tree_oracle.c``
(plain C, a binary heap) and the greedy tree-accept step's in
``ddtv_accept_oracle.c``, and the steps around the attention (query split with
rotary embedding and absorb, value projection, appended key rows) in
``ddtv_neighbour_oracle.c``, all compiled into the same library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ddtv_oracle.c")
_SRC_TREE = os.path.join(_HERE, "ddtv_tree_oracle.c")
_SRC_ACCEPT = os.path.join(_HERE, "ddtv_accept_oracle.c")
_SRC_NEIGHBOUR = os.path.join(_HERE, "ddtv_neighbour_oracle.c")
SOURCES = (_SRC, _SRC_TREE, _SRC_ACCEPT, _SRC_NEIGHBOUR)
_LIB = os.path.join(_HERE, "libddtv_oracle.so")

REF_OK, REF_EINVAL, REF_ETREE = 0, 1, 2
D_LATENT, D_ROPE = 512, 64

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc -O2 (no fast-math).  Returns the library path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall",
                               "-Wextra", "-o", tmp, *SOURCES, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def configure(lib):
    """Declare the C signatures on a loaded oracle library."""
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.ddtvref_build_visibility.argtypes = [P, i32, i32, P, P]
    lib.ddtvref_verify_attn_rows.argtypes = [P, P, P, P, i32, i32, i32, i32, P, P, f64,
                                             P, i64, P, P, P]
    lib.ddtvref_row_probs.argtypes = [P, P, P, P, i32, i32, i32, i32, P, P, f64, i64, P]
    lib.ddtvref_partial.argtypes = [P, P, P, P, i32, P, i64, f64, P, P, P]
    lib.ddtvref_merge.argtypes = [i32, P, P, P, P, P]
    lib.ddtvref_build_tree_row.argtypes = [P, P, i32, i32, i32, P, P, P, P, P]
    lib.ddtvref_build_tree_row.restype = ctypes.c_int
    lib.ddtvref_tree_capacity.argtypes = [i32, i32, i64]
    lib.ddtvref_tree_capacity.restype = i64
    lib.ddtvref_tree_accept_row.argtypes = [P, i32, P, P, i32, P, P, P, P]
    lib.ddtvref_tree_accept_row.restype = ctypes.c_int
    lib.ddtvref_compact_rows.argtypes = [P, P, i64, i64, i32, P, i32]
    lib.ddtvref_compact_rows.restype = None
    lib.ddtvref_fp8_value.argtypes = [ctypes.c_uint8]
    lib.ddtvref_fp8_value.restype = f64
    lib.ddtvref_rope_neox.argtypes = [P, i32, f64, P]
    lib.ddtvref_rope_neox.restype = None
    lib.ddtvref_tree_positions.argtypes = [P, P, i32, i32, P]
    lib.ddtvref_prepare_query.argtypes = [P, i32, i32, i32, P, f64, P, P, P]
    lib.ddtvref_value_proj.argtypes = [P, i32, i32, i32, P, P]
    lib.ddtvref_append_kv.argtypes = [P, P, P, P, i32, i32, f64, P, P]
    for name in ("ddtvref_tree_positions", "ddtvref_prepare_query", "ddtvref_value_proj",
                 "ddtvref_append_kv"):
        getattr(lib, name).restype = ctypes.c_int
    for name in ("ddtvref_build_visibility", "ddtvref_verify_attn_rows",
                 "ddtvref_row_probs", "ddtvref_partial", "ddtvref_merge", "ddtvref_words"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(os.path.getmtime(f) for f in SOURCES):
            build()
        _lib = configure(ctypes.CDLL(_LIB))
    return _lib


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def words(q: int) -> int:
    return (q + 31) // 32


def build_visibility(parent: np.ndarray):
    """parent int32 [B][Q] -> (bits uint32 [B][Q][W], bad int32 [B], rc)."""
    parent = _c(parent, np.int32)
    B, Q = parent.shape
    bits = np.zeros((B, Q, words(Q)), dtype=np.uint32)
    bad = np.zeros(B, dtype=np.int32)
    rc = _load().ddtvref_build_visibility(_p(parent), B, Q, _p(bits), _p(bad))
    return bits, bad, rc


def _kv(a, kv_dtype):
    return _c(a, {0: np.float32, 1: np.uint16, 2: np.uint8}[kv_dtype])


def fp8_value(b: int) -> float:
    """The oracle's decoding of one FP8 E4M3 byte."""
    return float(_load().ddtvref_fp8_value(int(b)))


def verify_attn(q_abs, q_rope, ckv, k_rope, kv_dtype, prefix, bits, scale, rows=None,
                want_psum=False):
    """Attention of the given flat query rows (all rows when ``rows`` is None).

    Returns (out float64 [n][512], lse float64 [n]) plus psum [n] when asked.
    """
    q_abs = _c(q_abs, np.float32)
    q_rope = _c(q_rope, np.float32)
    B, Q, H, _ = q_abs.shape
    ckv, k_rope = _kv(ckv, kv_dtype), _kv(k_rope, kv_dtype)
    prefix = _c(prefix, np.int32)
    bits = _c(bits, np.uint32)
    if rows is None:
        n = B * Q * H
        rows_p = None
    else:
        rows = _c(rows, np.int64)
        n = rows.shape[0]
        rows_p = rows
    out = np.zeros((n, D_LATENT), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    psum = np.zeros(n, dtype=np.float64) if want_psum else None
    rc = _load().ddtvref_verify_attn_rows(_p(q_abs), _p(q_rope), _p(ckv), _p(k_rope), kv_dtype,
                                          B, Q, H, _p(prefix), _p(bits), float(scale),
                                          _p(rows_p), n, _p(out), _p(lse), _p(psum))
    if rc != REF_OK:
        raise ValueError(f"oracle verify_attn failed with code {rc}")
    return (out, lse, psum) if want_psum else (out, lse)


def row_probs(q_abs, q_rope, ckv, k_rope, kv_dtype, prefix, bits, scale, row):
    q_abs = _c(q_abs, np.float32)
    q_rope = _c(q_rope, np.float32)
    B, Q, H, _ = q_abs.shape
    prefix = _c(prefix, np.int32)
    b = row // (Q * H)
    probs = np.zeros(int(prefix[b]) + Q, dtype=np.float64)
    rc = _load().ddtvref_row_probs(_p(q_abs), _p(q_rope), _p(_kv(ckv, kv_dtype)),
                                   _p(_kv(k_rope, kv_dtype)), kv_dtype, B, Q, H, _p(prefix),
                                   _p(_c(bits, np.uint32)), float(scale), int(row), _p(probs))
    if rc != REF_OK:
        raise ValueError(f"oracle row_probs failed with code {rc}")
    return probs


def partial(qa, qr, ckv, k_rope, kv_dtype, idx, scale):
    """Unnormalised partial (m, l, o[512]) of one query vector over cache rows ``idx``."""
    qa = _c(qa, np.float32).reshape(D_LATENT)
    qr = _c(qr, np.float32).reshape(D_ROPE)
    idx = _c(idx, np.int64).reshape(-1)
    m = ctypes.c_double()
    l = ctypes.c_double()
    o = np.zeros(D_LATENT, dtype=np.float64)
    rc = _load().ddtvref_partial(_p(qa), _p(qr), _p(_kv(ckv, kv_dtype)), _p(_kv(k_rope, kv_dtype)),
                                 kv_dtype, _p(idx), idx.shape[0], float(scale),
                                 ctypes.byref(m), ctypes.byref(l), _p(o))
    if rc != REF_OK:
        raise ValueError(f"oracle partial failed with code {rc}")
    return m.value, l.value, o


def merge(m, l, o):
    """Log-sum-exp merge of S partials -> (out [512], lse)."""
    m = _c(m, np.float64).reshape(-1)
    l = _c(l, np.float64).reshape(-1)
    o = _c(o, np.float64).reshape(-1, D_LATENT)
    out = np.zeros(D_LATENT, dtype=np.float64)
    lse = ctypes.c_double()
    _load().ddtvref_merge(m.shape[0], _p(m), _p(l), _p(o), _p(out), ctypes.byref(lse))
    return out, lse.value


def attend_workload(w, rows=None, bits=None):
    """Convenience: oracle bits (unless given) + attention for a workloads.Workload."""
    if bits is None:
        bits, _, _ = build_visibility(w.parent)
    return verify_attn(w.q_abs, w.q_rope, w.ckv, w.k_rope, w.kv_dtype, w.prefix, bits,
                       w.scale, rows=rows)


def tree_capacity(D: int, K: int, cap: int = 1 << 40) -> int:
    """Nodes of the full K-ary tree of depth D (saturated at cap)."""
    return int(_load().ddtvref_tree_capacity(D, K, cap))


def build_tree(logp: np.ndarray, Q: int, tokens: np.ndarray | None = None):
    """Best-first draft trees of Q nodes from per-depth top-K log-probs.

    logp: float32 [B][D][K] (each [b][d] sorted descending); tokens: int32 [B][D][K] or None.
    Returns (rc, dict of int32/float32 [B][Q] arrays: parent, depth, rank, token, score)."""
    lib = _load()
    logp = _c(logp, np.float32)
    B, D, K = logp.shape
    tok = None if tokens is None else _c(tokens, np.int32)
    out = {k: np.zeros((B, Q), np.int32) for k in ("parent", "depth", "rank", "token")}
    out["score"] = np.zeros((B, Q), np.float32)
    for b in range(B):
        rc = lib.ddtvref_build_tree_row(_p(logp[b]), _p(None if tok is None else tok[b]), D, K, Q,
                                        _p(out["parent"][b]), _p(out["depth"][b]), _p(out["rank"][b]),
                                        _p(out["token"][b]), _p(out["score"][b]))
        if rc != REF_OK:
            return rc, None
    return REF_OK, out


def tree_accept(logits: np.ndarray, parent: np.ndarray, token: np.ndarray):
    """Greedy acceptance of B verified trees.

    logits: float32 [B][Q][V] (the target's logits after each node); parent, token: int32 [B][Q].
    Returns (rc, dict: pred, path, out_tokens int32 [B][Q]; accept_len int32 [B])."""
    lib = _load()
    logits = _c(logits, np.float32)
    parent = _c(parent, np.int32)
    token = _c(token, np.int32)
    B, Q, V = logits.shape
    out = {k: np.zeros((B, Q), np.int32) for k in ("pred", "path", "out_tokens")}
    out["accept_len"] = np.zeros(B, np.int32)
    for b in range(B):
        k = ctypes.c_int32()
        rc = lib.ddtvref_tree_accept_row(_p(logits[b]), V, _p(parent[b]), _p(token[b]), Q, _p(out["pred"][b]),
                                         _p(out["path"][b]), _p(out["out_tokens"][b]), ctypes.byref(k))
        if rc != REF_OK:
            return rc, None
        out["accept_len"][b] = k.value
    return REF_OK, out


def compact_rows(rows: np.ndarray, prefix: int, path: np.ndarray, k: int) -> np.ndarray:
    """One batch row's cache rows after acceptance (a new array): row prefix + j
    takes row prefix + path[j] for j = 1..k.  rows: [n_rows][...] any dtype."""
    src = np.ascontiguousarray(rows)
    dst = np.empty_like(src)
    n = src.shape[0]
    row_bytes = src.nbytes // max(n, 1)
    _load().ddtvref_compact_rows(_p(src.view(np.uint8)), _p(dst.view(np.uint8)), n, row_bytes, prefix,
                                 _p(_c(path, np.int32)), k)
    return dst


def rope_neox(x: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """NeoX rotation of one 64-wide float32 vector at position ``pos`` (float64 out)."""
    x = _c(x, np.float32).reshape(D_ROPE)
    y = np.zeros(D_ROPE, dtype=np.float64)
    _load().ddtvref_rope_neox(_p(x), int(pos), float(theta), _p(y))
    return y


def tree_positions(parent: np.ndarray, prefix: np.ndarray) -> np.ndarray:
    """Position of every tree node: prefix[b] + depth (int32 [B][Q])."""
    parent = _c(parent, np.int32)
    B, Q = parent.shape
    pos = np.zeros((B, Q), dtype=np.int32)
    rc = _load().ddtvref_tree_positions(_p(parent), _p(_c(prefix, np.int32)), B, Q, _p(pos))
    if rc != REF_OK:
        raise ValueError(f"oracle tree_positions failed with code {rc}")
    return pos


def prepare_query(q: np.ndarray, pos: np.ndarray, theta: float, w_kc: np.ndarray):
    """q float32 [..., H, d_nope + 64] (leading dims = tokens), pos int32 [tokens],
    w_kc float32 [H][d_nope][512] -> (q_abs float64 [..., H, 512], q_rope float64 [..., H, 64])."""
    q = _c(q, np.float32)
    lead = q.shape[:-2]
    H, row = q.shape[-2], q.shape[-1]
    d_nope = row - D_ROPE
    M = int(np.prod(lead)) if lead else 1
    w_kc = _c(w_kc, np.float32)
    assert w_kc.shape == (H, d_nope, D_LATENT)
    pos = _c(pos, np.int32).reshape(-1)
    assert pos.shape[0] == M
    q_abs = np.zeros(lead + (H, D_LATENT), dtype=np.float64)
    q_rope = np.zeros(lead + (H, D_ROPE), dtype=np.float64)
    rc = _load().ddtvref_prepare_query(_p(q), M, H, d_nope, _p(pos), float(theta), _p(w_kc),
                                       _p(q_abs), _p(q_rope))
    if rc != REF_OK:
        raise ValueError(f"oracle prepare_query failed with code {rc}")
    return q_abs, q_rope


def value_proj(o: np.ndarray, w_vc: np.ndarray) -> np.ndarray:
    """o float32 [..., H, 512], w_vc float32 [H][d_v][512] -> v float64 [..., H, d_v]."""
    o = _c(o, np.float32)
    lead = o.shape[:-2]
    H = o.shape[-2]
    M = int(np.prod(lead)) if lead else 1
    w_vc = _c(w_vc, np.float32)
    assert w_vc.shape[0] == H and w_vc.shape[2] == D_LATENT
    d_v = w_vc.shape[1]
    v = np.zeros(lead + (H, d_v), dtype=np.float64)
    rc = _load().ddtvref_value_proj(_p(o), M, H, d_v, _p(w_vc), _p(v))
    if rc != REF_OK:
        raise ValueError(f"oracle value_proj failed with code {rc}")
    return v


def append_kv(latent, k_pe, pos, prefix, theta, ckv, k_rope):
    """Write B trees' new cache rows into float64 copies of ckv [total][512] and
    k_rope [total][64]; latent float32 [B][Q][512], k_pe float32 [B][Q][64],
    pos int32 [B][Q].  Returns the two new arrays."""
    latent = _c(latent, np.float32)
    k_pe = _c(k_pe, np.float32)
    B, Q, _ = latent.shape
    ckv = np.array(ckv, dtype=np.float64, copy=True, order="C")
    k_rope = np.array(k_rope, dtype=np.float64, copy=True, order="C")
    rc = _load().ddtvref_append_kv(_p(latent), _p(k_pe), _p(_c(pos, np.int32)), _p(_c(prefix, np.int32)),
                                   B, Q, float(theta), _p(ckv), _p(k_rope))
    if rc != REF_OK:
        raise ValueError(f"oracle append_kv failed with code {rc}")
    return ckv, k_rope
