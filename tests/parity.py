"""Helpers for GPU-vs-oracle parity tests (imported by the gpu tests only)."""
from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle

# Elementwise bar |gpu - ref| <= ATOL + RTOL * |ref|: 1e-4 / 1e-4 for float32 caches,
# 2e-2 / 2e-2 for bf16 caches (the bf16 inputs themselves are exact, so this is the
# budget for bf16 arithmetic inside the kernel), 1e-4 / 1e-4 for FP8 caches (widened
# exactly and computed in fp32).
TOL = {0: (1e-4, 1e-4), 1: (2e-2, 2e-2), 2: (1e-4, 1e-4)}

_WORKERS = max(1, min(16, os.cpu_count() or 1))


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


def assert_close(got, ref, kv_dtype, what=""):
    atol, rtol = TOL[kv_dtype]
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    bad = err > bound
    if bad.any():
        idx = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements outside {atol}+{rtol}|ref|; "
                             f"worst at {idx}: got {got[idx]!r} ref {ref[idx]!r} (max abs err {err.max():.3e})")
    return float(err.max())


def assert_lse_close(got, ref, kv_dtype, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    inf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inf), f"{what}: -inf pattern differs"
    return assert_close(got[~inf], ref[~inf], kv_dtype, what + " lse")
