"""Helpers for GPU-vs-oracle parity tests (imported by the gpu tests only).

The bar depends on the arithmetic that produced the output, not on the cache's
element type:

- "f32": fp32 arithmetic on values widened exactly (fp32, FP8 E4M3 and bf16
  caches on the VALU and fp32 matrix-core kernels, row-half mode, the sparse
  tail route):  |gpu - ref| <= 1e-4 + 1e-4 |ref| for every element, and lse
  the same way.
- "bf16": the bf16 matrix-core kernel, which rounds the query and the
  probabilities to bf16 before its products.  The stated 2e-2 relative bar is
  read per query row, since single elements of a weighted mean can sit near
  zero:  ||gpu_row - ref_row||_2 <= 2e-2 ||ref_row||_2 for every row.  Each
  element's error is a sum of many small independent rounding errors, roughly
  Gaussian with a spread of (row relative L2) x rms(ref_row), so the largest of
  millions sits several spreads out: every element within 5e-2 rms(ref_row) +
  2e-2 |ref| (the row's own scale sets the absolute part).  lse within 2e-2
  absolute (a 2e-2 relative bar on the softmax normaliser).

Every check prints the errors it saw: max abs, max relative over |ref| > 1e-3,
the largest and median per-row relative L2, and the largest element error over
its row's rms.
"""
from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle

F32, BF16 = "f32", "bf16"
_F32_TOL = (1e-4, 1e-4)
_BF16_ROW_REL_L2 = 2e-2
_BF16_ELEM = (5e-2, 2e-2)   # x rms(ref row), x |ref|
_BF16_LSE_ABS = 2e-2

_WORKERS = max(1, min(16, os.cpu_count() or 1))


def arithmetic(kv_dtype: int, plan_path: int) -> str:
    """The arithmetic of a verify call: bf16 on the bf16 matrix-core kernel (path 2
    on a bf16 cache), fp32 everywhere else."""
    return BF16 if (kv_dtype == 1 and plan_path == 2) else F32


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_rows(w, bits, rows=None, chunk=64):
    """Oracle attention of the given rows (all when None), rows spread over threads
    (the oracle itself is single-threaded; independent rows run side by side)."""
    total = w.B * w.Q * w.H
    rows = np.arange(total, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    parts = [rows[i:i + chunk] for i in range(0, len(rows), chunk)]

    def one(r):
        return oracle.verify_attn(w.q_abs, w.q_rope, w.ckv, w.k_rope, w.kv_dtype, w.prefix, bits, w.scale,
                                  rows=r)

    with ThreadPoolExecutor(_WORKERS) as ex:
        res = list(ex.map(one, parts))
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])


def error_report(got, ref) -> dict:
    """max abs error, max relative error over |ref| > 1e-3, per-row relative L2
    (rows = last axis) and the largest element error over its row's rms."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    big = np.abs(ref) > 1e-3
    er = err.reshape(-1, err.shape[-1])
    rr = ref.reshape(-1, ref.shape[-1])
    rows_err = np.sqrt((er ** 2).sum(-1))
    rows_ref = np.sqrt((rr ** 2).sum(-1))
    nz = rows_ref > 0
    rel_l2 = np.where(nz, rows_err / np.where(nz, rows_ref, 1.0), np.where(rows_err > 0, np.inf, 0.0))
    rms = rows_ref / np.sqrt(rr.shape[-1])
    over_rms = er / np.where(rms > 0, rms, 1.0)[:, None]
    return {"max_abs": float(err.max()) if err.size else 0.0,
            "max_rel": float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0,
            "max_row_rel_l2": float(rel_l2.max()) if rel_l2.size else 0.0,
            "median_row_rel_l2": float(np.median(rel_l2)) if rel_l2.size else 0.0,
            "max_err_over_row_rms": float(over_rms.max()) if over_rms.size else 0.0}


def _arith(a) -> str:
    # 0 / 2 (fp32 / FP8 cache codes) name fp32 arithmetic; bf16 must be named explicitly
    if a in (F32, BF16):
        return a
    if a in (0, 2):
        return F32
    raise ValueError(f"parity bar: name the arithmetic (parity.F32 or parity.BF16), got {a!r}")


def assert_close(got, ref, arith, what=""):
    """Check got against the oracle's ref under the bar of `arith` (see the module
    docstring); return the error report (also printed)."""
    arith = _arith(arith)
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    rep = error_report(got, ref)
    say(f"  [{what}] {arith} bar: max abs {rep['max_abs']:.2e}, max rel (|ref|>1e-3) {rep['max_rel']:.2e}, "
        f"row rel-L2 max {rep['max_row_rel_l2']:.2e} median {rep['median_row_rel_l2']:.2e}, "
        f"max err / row rms {rep['max_err_over_row_rms']:.2e}")
    err = np.abs(got - ref)
    if arith == F32:
        atol, rtol = _F32_TOL
        bound = atol + rtol * np.abs(ref)
    else:
        rows_ref = ref.reshape(-1, ref.shape[-1])
        rms = np.sqrt((rows_ref ** 2).mean(-1, keepdims=True))
        bound = (_BF16_ELEM[0] * rms + _BF16_ELEM[1] * np.abs(rows_ref)).reshape(ref.shape)
        worst = rep["max_row_rel_l2"]
        assert worst <= _BF16_ROW_REL_L2, (f"{what}: a row's relative L2 error {worst:.3e} exceeds "
                                          f"{_BF16_ROW_REL_L2}")
    bad = err > bound
    if bad.any():
        idx = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements outside the {arith} bar; worst at "
                             f"{idx}: got {got[idx]!r} ref {ref[idx]!r} (max abs err {err.max():.3e})")
    return rep["max_abs"]


def assert_lse_close(got, ref, arith, what=""):
    arith = _arith(arith)
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    inf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inf), f"{what}: -inf pattern differs"
    g, r = got[~inf], ref[~inf]
    assert np.isfinite(g).all(), f"{what}: non-finite lse"
    err = np.abs(g - r)
    bound = (_F32_TOL[0] + _F32_TOL[1] * np.abs(r)) if arith == F32 else np.full_like(r, _BF16_LSE_ABS)
    bad = err > bound
    assert not bad.any(), (f"{what} lse: {bad.sum()} of {bad.size} outside the {arith} bar "
                           f"(max abs err {err.max():.3e})")
    e = float(err.max()) if err.size else 0.0
    say(f"  [{what}] lse {arith} bar: max abs {e:.2e}")
    return e
