#!/usr/bin/env python3
"""Benchmark: DDTree tree-verify MLA-absorb attention on one MI355X.

One step = one verify pass of the whole hot path over one batch: the visibility
build (parent arrays -> packed ancestor masks), the masked absorbed-MLA attention
and, when the cache is split, the log-sum-exp merge.  Inputs are seeded and
synthetic and already resident in HBM when the timed region starts.

Prints ONE JSON line.  The default workload is B=8, H=16, prefix 32768,
q_len 128, best-first trees, fp32 cache (``--config c4``).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import re
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tree-verify attn: achieved HBM GB/s (% of peak) and tree-query tokens/sec"
HBM_PEAK_GBPS = 8000.0
# fp32 MFMA: 256 CU x 4 SIMD x 256 flop/clk/CU-equivalent at 2.4 GHz (published 157.3 TFLOP/s).
# VALU without packed fp32: 256 CU x 64 lanes x 2 flop (FMA) x 2.4 GHz = 78.6 TFLOP/s.
PEAK_TFLOPS = {"f32-mfma": 157.3, "bf16-mfma": 2500.0, "f32-valu": 78.6}
# sources of each kernel whose PMC traffic may be quoted (the hash ties counters to code)
KERNEL_SOURCES = {
    "attn_mfma_kernel": ["attn_mfma.hip", "ddtv_internal.hpp"],
    "attn_mfma_bf16_kernel": ["attn_mfma_bf16.hip", "ddtv_internal.hpp"],
    "attn_valu_kernel": ["attn_valu.hip", "ddtv_internal.hpp"],
}


def roofline_bound(valu, flops, nbytes, kernel_ms, peak_tflops):
    """The roofline that binds the attention kernel: the larger of its compute
    floor (flops at the matrix or vector peak) and its memory floor (algorithmic
    bytes at the HBM peak).  The tree workloads are compute-bound; decode-shaped
    rows (q_len 1) carry ~15 flops per byte and are HBM-bound."""
    t = kernel_ms / 1e3
    if nbytes / (HBM_PEAK_GBPS * 1e9) > flops / (peak_tflops * 1e12):
        gbps = nbytes / t / 1e9
        return {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(gbps / HBM_PEAK_GBPS, 4)}
    tflops = flops / t / 1e12
    return {"bound": "alu" if valu else "mfma", "achieved": round(tflops, 3), "peak": peak_tflops,
            "unit": "TFLOP/s", "frac": round(tflops / peak_tflops, 4)}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


CALIB_LIB = os.path.join(ROOT, "tree_masked_mla_amd", "libddtv_calib.so")
# The other workloads of the line (`configs`) warm up for at least this long, so
# that their short launches are timed at the steady-state shader clock.
CONFIG_MIN_WARM_MS = 60.0


CEILING_BYTES = 512 << 20   # well past every cache level (MI355X: 4 MiB L2 per XCD, 256 MiB MALL)


def read_ceiling(hip, stream, dev, workgroups, nbytes=CEILING_BYTES, reps=10, warmup=2):
    """What a bare read stream reaches on this GPU over a zeroed `nbytes` device
    buffer (read once per launch, whole units per workgroup): the calibration
    library's LDS stream (72 KiB tiles by global_load_lds, the attention kernel's
    way of streaming its cache, without the math) and its register stream, one
    512-thread workgroup per CU.  A property of the GPU, not of the workload, so it
    is measured on its own buffer.  Context for memory-bound lines: the roofline's
    peak stays the published 8 TB/s."""
    import torch
    if not os.path.exists(CALIB_LIB):
        raise FileNotFoundError(f"{CALIB_LIB} not found; build it with `python -m tree_masked_mla_amd.build`")
    lib = ctypes.CDLL(CALIB_LIB)   # torch is loaded already: one HIP runtime in the process
    f = lib.ddtv_calib_stream_read
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                  ctypes.POINTER(ctypes.c_int64)]
    f.restype = ctypes.c_int
    buf = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.empty(workgroups * 512, dtype=torch.float32, device=dev)
    out = {"kind": f"bare read stream of a {nbytes >> 20} MiB buffer, one 512-thread workgroup per CU over a "
                   "contiguous share", "workgroups": workgroups}
    for mode, name in ((0, "lds_dma_72KiB_tiles"), (1, "vgpr_16B_loads")):
        nread = ctypes.c_int64()

        def launch():
            rc = f(buf.data_ptr(), nbytes, mode, sink.data_ptr(), workgroups, stream, ctypes.byref(nread))
            assert rc == 0, f"ddtv_calib_stream_read returned {rc}"
        for _ in range(warmup):
            launch()
        e0, e1 = hip.event(), hip.event()
        hip.record(e0, stream)
        for _ in range(reps):
            launch()
        hip.record(e1, stream)
        ms = hip.elapsed_ms(e0, e1) / reps
        out[name] = {"gbps": round(nread.value / (ms / 1e3) / 1e9, 1), "us": round(ms * 1e3, 2),
                     "bytes_read": nread.value}
    out["gbps"] = max(out["lds_dma_72KiB_tiles"]["gbps"], out["vgpr_16B_loads"]["gbps"])
    out["pct_of_peak"] = round(100.0 * out["gbps"] / HBM_PEAK_GBPS, 2)
    del buf, sink
    torch.cuda.empty_cache()
    return out


def with_ceiling(roof, ceiling):
    """A memory-bound roofline also states its fraction of the measured read ceiling."""
    roof = dict(roof)
    if roof["bound"] == "hbm" and ceiling and ceiling["gbps"] > 0:
        roof["read_ceiling_gbps"] = ceiling["gbps"]
        roof["frac_of_read_ceiling"] = round(roof["achieved"] / ceiling["gbps"], 4)
    return roof


# ----------------------------------------------------------------------------- HIP events (ctypes)
# hipEventDisableSystemFence: the events here only time work.  A default event's
# record ends with a system-scope release and acquire, which writes back and
# invalidates the GPU caches; with the per-step events around the attention
# kernel that would sit inside every timed step (c3: 100.7 against 96.5 us per
# step, the attention events 85.9 against 83.9 us).  Reading an event still
# waits for it to complete (hipEventSynchronize).
EVENT_TIMING_ONLY = 0x20000000


class Hip:
    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreateWithFlags(ctypes.byref(e), EVENT_TIMING_ONLY) == 0
        return e.value

    def record(self, e, stream):
        assert self.lib.hipEventRecord(e, stream) == 0

    def elapsed_ms(self, a, b):
        self.lib.hipEventSynchronize(b)
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value


# ----------------------------------------------------------------------------- algorithmic counts
def algorithmic(w):
    """Bytes every step must move at least once and flops of the visible pairs.

    bytes: q_abs + q_rope + each cache row once (latent + rope) + out + lse + parents +
           masks + prefix lengths.
    flops: 2 * (512 + 64) for the score plus 2 * 512 for the weighted sum, per visible
           (query row, cache position) pair.
    """
    import workloads as wl
    esz = 2 if w.kv_dtype == wl.BF16 else 4
    rows = w.B * w.Q * w.H
    W = (w.Q + 31) // 32
    nbytes = (rows * 576 * 4 + w.total_kv * 576 * esz + rows * 512 * 4 + rows * 4
              + w.B * w.Q * 4 + w.B * w.Q * W * 4 + w.B * 4)
    vis_pairs = 0
    for b in range(w.B):
        depth = wl.tree_depths(w.parent[b])
        vis_pairs += w.H * int((int(w.prefix[b]) + depth + 1).sum())
    flops = vis_pairs * 2 * (576 + 512)
    return nbytes, flops, vis_pairs


_COMMENTS = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def kernel_source_hash(kernel):
    """First 16 hex digits of a sha256 over the kernel's sources with comments, blank
    lines and trailing blanks removed: the recorded traffic depends on the code only."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "tree_masked_mla_amd", "csrc", f)) as fh:
            code = _COMMENTS.sub("", fh.read())
        h.update("\n".join(l.rstrip() for l in code.splitlines() if l.strip()).encode())
    return h.hexdigest()[:16]


def load_traffic(config_name, kernel_hash):
    """HBM bytes per launch of the attention kernel from committed rocprofv3 PMC
    summaries (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel calibration),
    or None when absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_attn_{config_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_hash:
        return None
    return t.get("bytes_per_launch")


def load_counters(config_name, kernel_hash):
    """The attention kernel's committed rocprofv3 counter summary: matrix-pipe busy
    fraction per SIMD (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE) and executed
    matrix flops per launch (SQ_INSTS_VALU_MFMA_MOPS_* x 512), or None when absent
    or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"counters_attn_{config_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_hash:
        return None
    return t


# ----------------------------------------------------------------------------- CPU baseline (oracle)
def time_tree_builder(dd, hip, stream, dev, B, Q, D=12, K=4, steps=20, warmup=3):
    """The draft-tree builder (ddtv_build_tree) on B trees of Q nodes from synthetic
    drafter top-K log-probs: average launch time from HIP events on the launch stream."""
    import torch
    import workloads as wl
    lp, tok = wl.drafter_topk(7000 + B + Q, B, D, K)
    lp_d = torch.from_numpy(lp).to(dev)
    tok_d = torch.from_numpy(tok).to(dev)
    outs = [torch.empty((B, Q), dtype=torch.int32, device=dev) for _ in range(4)]
    score = torch.empty((B, Q), dtype=torch.float32, device=dev)

    def launch():
        rc = dd.ddtv_build_tree(lp_d, Q, outs[0], tokens=tok_d, depth=outs[1], rank=outs[2], token=outs[3],
                                score=score, stream=stream)
        assert rc == dd.DDTV_OK, rc
    for _ in range(warmup):
        launch()
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    for _ in range(steps):
        launch()
    hip.record(e1, stream)
    us = hip.elapsed_ms(e0, e1) * 1e3 / steps
    return {"workload": f"B={B} trees of Q={Q} nodes, depth <= {D}, top-{K} per depth (synthetic drafter)",
            "us_per_launch": round(us, 2), "ns_per_node": round(us * 1e3 / Q, 1), "launches": steps,
            "note": "one workgroup per tree: depth-by-depth selection of the Q-1 best lattice nodes (one node per step on ties or positive log-probs)"}


def time_tree_accept(dd, hip, stream, r, V=32768, steps=20, warmup=3):
    """The accept step (ddtv_tree_accept) on the benchmarked trees: target argmax over
    V synthetic logits per node, the greedy walk and in-place compaction of the
    accepted rows of the resident caches; average launch time from HIP events."""
    import torch
    import workloads as wl
    B, Q = r.B, r.Q
    dev = r.device
    logits = torch.from_numpy(wl.target_logits(7100 + B + Q, B, Q, V)).to(dev)
    tok = torch.from_numpy(np.ascontiguousarray(r.w.parent % 997, dtype=np.int32)).to(dev)   # any draft tokens
    o = [torch.empty((B, Q), dtype=torch.int32, device=dev) for _ in range(3)]
    alen = torch.empty(B, dtype=torch.int32, device=dev)

    def launch():
        rc = dd.ddtv_tree_accept(logits, r.parent, tok, r.vis, o[0], o[1], o[2], alen, ckv=r.ckv, k_rope=r.k_rope,
                                 kv_dtype=r.kv_dtype, stream=stream)
        assert rc == dd.DDTV_OK, rc
    for _ in range(warmup):
        launch()
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    for _ in range(steps):
        launch()
    hip.record(e1, stream)
    us = hip.elapsed_ms(e0, e1) * 1e3 / steps
    logit_bytes = B * Q * V * 4
    return {"workload": f"B={B} trees of Q={Q} nodes, V={V} synthetic target logits per node, compaction on",
            "us_per_launch": round(us, 2), "logit_bytes": logit_bytes,
            "logits_gbps": round(logit_bytes / (us * 1e-6) / 1e9, 1), "launches": steps}


def time_tail_mode(dd, hip, stream, r, steps=20, warmup=3):
    """External-prefix mode on the benchmarked workload: the tree rows only, merged
    with a prefix result supplied by the caller (here any normalised rows and
    finite lse: timing only); average call time from HIP events, for the default
    tree-sparse route and for the dense route (forced matrix-core path)."""
    import torch
    w = r.w
    po = torch.zeros_like(r.out)
    pl = torch.zeros((w.B, w.Q, w.H), dtype=torch.float32, device=r.device)
    need = dd.ddtv_tail_workspace_bytes(r.vis, w.H, w.kv_dtype)
    dense = dd.make_opts(path=dd.DDTV_PATH_MFMA)
    need = max(need, dd.ddtv_tail_workspace_bytes(r.vis, w.H, w.kv_dtype, dense))
    ws = torch.empty(need, dtype=torch.uint8, device=r.device)

    def timed(opts):
        def launch():
            rc = dd.ddtv_verify_attn_tail(r.q_abs, r.q_rope, r.ckv, r.k_rope, w.kv_dtype, w.H, r.vis, w.scale, po,
                                          pl, r.out, r.lse, ws, stream=stream, opts=opts)
            assert rc == dd.DDTV_OK, rc
        for _ in range(warmup):
            launch()
        e0, e1 = hip.event(), hip.event()
        hip.record(e0, stream)
        for _ in range(steps):
            launch()
        hip.record(e1, stream)
        return hip.elapsed_ms(e0, e1) * 1e3 / steps

    us = timed(None)
    us_dense = timed(dense)
    nbytes = 4 * w.B * w.Q * w.H * (512 + 64 + 512 + 1 + 512 + 1)   # q, prefix result in, out + lse
    return {"workload": f"the same trees, tree rows only ({w.Q} per batch row) + merge with a caller's prefix result",
            "us_per_call": round(us, 2), "route": "tree-sparse (each node visits its ancestors-or-self)",
            "streamed_bytes": nbytes, "gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "dense_route_us_per_call": round(us_dense, 2), "calls": steps}


def time_iteration(dd, hip, stream, r, V=32768, D=12, K=4, steps=10, warmup=2, grow=False):
    """One whole tree-verify iteration on the device at the benchmarked batch, tree
    size and cache: draft-tree builder -> visibility -> the tree's cache rows ->
    query preparation -> attention (S2..S7) -> value projection -> greedy
    acceptance with compaction.  Synthetic drafter top-K, projections, weights and
    target logits; the resident cache; average iteration time from HIP events.
    The attention goes through the no-allocation entry point, so no workspace is
    sized per plan.

    grow=True: every iteration's prefixes are the last ones plus an accepted
    length + 1 (accepted lengths drawn from a seeded sequence on the host, as a
    decode loop that tracks the cache end would see them), so the batch rows'
    cache offsets and the split plan are recomputed every iteration.  The caches
    get room for the growth (the rows past the benchmarked cache hold zeros)."""
    import torch
    import workloads as wl
    w = r.w
    B, Q, H, dev = w.B, w.Q, w.H, r.device
    lp, tok = wl.drafter_topk(7400 + B + Q, B, D, K)
    lp_d, tok_d = torch.from_numpy(lp).to(dev), torch.from_numpy(tok).to(dev)
    nb = wl.neighbour_inputs(7500 + B + Q, B, Q, H)
    q, w_kc, w_vc = (torch.from_numpy(x).to(dev) for x in (nb.q, nb.w_kc, nb.w_vc))
    lat, k_pe = torch.from_numpy(nb.latent).to(dev), torch.from_numpy(nb.k_pe).to(dev)
    logits = torch.from_numpy(wl.target_logits(7600 + B + Q, B, Q, V)).to(dev)
    i32 = lambda *shape: torch.empty(shape, dtype=torch.int32, device=dev)
    parent, token, pred, path, out_tok, alen = i32(B, Q), i32(B, Q), i32(B, Q), i32(B, Q), i32(B, Q), i32(B)
    q_abs = torch.empty((B, Q, H, 512), dtype=torch.float32, device=dev)
    q_rope = torch.empty((B, Q, H, 64), dtype=torch.float32, device=dev)
    v = torch.empty((B, Q, H, 128), dtype=torch.float32, device=dev)
    vis_buf = torch.empty(dd.ddtv_vis_bytes(B, Q), dtype=torch.uint8, device=dev)
    n_iter = warmup + steps
    prefixes = [np.ascontiguousarray(w.prefix, dtype=np.int32)]
    if grow:
        acc = np.random.default_rng(7700 + B + Q).integers(0, min(D, Q - 1) + 1, size=(n_iter, B))
        for i in range(n_iter - 1):
            prefixes.append((prefixes[-1] + acc[i] + 1).astype(np.int32))
        extra = int((prefixes[-1].astype(np.int64) - prefixes[0]).sum())
        ckv = torch.zeros((r.ckv.shape[0] + extra,) + tuple(r.ckv.shape[1:]), dtype=r.ckv.dtype, device=dev)
        krope = torch.zeros((r.k_rope.shape[0] + extra,) + tuple(r.k_rope.shape[1:]), dtype=r.k_rope.dtype,
                            device=dev)
        ckv[: r.ckv.shape[0]].copy_(r.ckv)
        krope[: r.k_rope.shape[0]].copy_(r.k_rope)
    else:
        prefixes *= n_iter
        ckv, krope = r.ckv, r.k_rope
    keep = []

    def iteration(i):
        ok = dd.DDTV_OK
        assert dd.ddtv_build_tree(lp_d, Q, parent, tokens=tok_d, token=token, stream=stream) == ok
        rc, vis = dd.ddtv_build_visibility(parent, prefixes[i], B, Q, vis_buf, stream=stream)
        assert rc == ok
        assert dd.ddtv_append_kv(lat, k_pe, vis, ckv, krope, w.kv_dtype, nb.theta, stream=stream) == ok
        assert dd.ddtv_prepare_query(q, w_kc, vis, q_abs, q_rope, nb.theta, stream=stream) == ok
        # the split partials go to the library's scratch: no workspace to size per plan
        assert dd.ddtv_verify_attn_noalloc(q_abs, q_rope, ckv, krope, w.kv_dtype, H, vis, w.scale, r.out, r.lse,
                                           stream=stream) == ok
        assert dd.ddtv_value_proj(r.out, w_vc, v, stream=stream) == ok
        assert dd.ddtv_tree_accept(logits, parent, token, vis, pred, path, out_tok, alen, ckv=ckv,
                                   k_rope=krope, kv_dtype=w.kv_dtype, stream=stream) == ok
        keep.append(vis)   # the struct's borrowed arrays stay alive until the stream drains
    for i in range(warmup):
        iteration(i)
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    t0 = time.perf_counter()
    for i in range(warmup, n_iter):
        iteration(i)
    host_us = (time.perf_counter() - t0) * 1e6 / steps
    hip.record(e1, stream)
    us = hip.elapsed_ms(e0, e1) * 1e3 / steps
    res = {"workload": f"builder (top-{K} per depth, depth {D}) -> visibility -> cache append -> query prep "
                       f"(d_nope 128) -> attention -> value projection (d_v 128) -> acceptance over {V} logits "
                       "per node with compaction, on the benchmarked batch and cache",
           "us_per_iteration": round(us, 2), "tree_tokens_per_s": round(B * Q / (us * 1e-6), 1),
           "host_enqueue_us_per_iteration": round(host_us, 2), "iterations": steps}
    if grow:
        res["workload"] += "; prefixes grow by a seeded accepted length + 1 every iteration (plans recomputed)"
        res["prefix_growth"] = int((prefixes[-1].astype(np.int64) - prefixes[0]).sum())
    return res


def time_fp8_cache(dd, hip, stream, r, flops, steps=10, warmup=2):
    """The same verify call on an FP8 E4M3 copy of the benchmarked cache (a quarter
    of the fp32 bytes; widened exactly in the kernel): average call time from HIP
    events and the fp32 matrix-core fraction it reaches."""
    import torch
    import workloads as wl
    from tree_masked_mla_amd.runner import to_device_kv
    w = r.w
    if w.kv_dtype != 0:
        return None
    ckv8 = to_device_kv(wl.round_fp8_bits(w.ckv), wl.FP8, r.device)
    kr8 = to_device_kv(wl.round_fp8_bits(w.k_rope), wl.FP8, r.device)
    need = dd.ddtv_workspace_bytes(r.vis, w.H, wl.FP8)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=r.device)

    def launch():
        rc = dd.ddtv_verify_attn(r.q_abs, r.q_rope, ckv8, kr8, wl.FP8, w.H, r.vis, w.scale, r.out, r.lse, ws, need,
                                 stream=stream)
        assert rc == dd.DDTV_OK, rc
    for _ in range(warmup):
        launch()
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    for _ in range(steps):
        launch()
    hip.record(e1, stream)
    us = hip.elapsed_ms(e0, e1) * 1e3 / steps
    tf = flops / (us * 1e-6) / 1e12
    return {"workload": "the same trees and queries over an FP8 E4M3 copy of the cache (widened to fp32 in the kernel)",
            "cache_bytes": int(ckv8.numel() + kr8.numel()), "us_per_call": round(us, 2),
            "tflops": round(tf, 2), "frac_of_fp32_mfma_peak": round(tf / PEAK_TFLOPS["f32-mfma"], 4),
            "tokens_per_s": round(w.B * w.Q / (us * 1e-6), 1), "calls": steps}


def time_neighbour(dd, hip, stream, r, d_nope=128, d_v=128, steps=20, warmup=3):
    """The steps around the attention at the benchmarked tree and head counts:
    query preparation (split, rotation, w_kc absorb), the w_vc value projection of
    the attention output, and the tree's appended cache rows; synthetic weights
    and projections; average launch times from HIP events."""
    import torch
    import workloads as wl
    w = r.w
    B, Q, H = w.B, w.Q, w.H
    M = B * Q
    dev = r.device
    nb = wl.neighbour_inputs(7300 + B + Q, B, Q, H, d_nope=d_nope, d_v=d_v)
    q = torch.from_numpy(nb.q).to(dev)
    w_kc = torch.from_numpy(nb.w_kc).to(dev)
    w_vc = torch.from_numpy(nb.w_vc).to(dev)
    lat = torch.from_numpy(nb.latent).to(dev)
    k_pe = torch.from_numpy(nb.k_pe).to(dev)
    q_abs = torch.empty((B, Q, H, 512), dtype=torch.float32, device=dev)
    q_rope = torch.empty((B, Q, H, 64), dtype=torch.float32, device=dev)
    v = torch.empty((B, Q, H, d_v), dtype=torch.float32, device=dev)

    def timed(launch):
        for _ in range(warmup):
            launch()
        e0, e1 = hip.event(), hip.event()
        hip.record(e0, stream)
        for _ in range(steps):
            launch()
        hip.record(e1, stream)
        return hip.elapsed_ms(e0, e1) * 1e3 / steps

    def prep():
        assert dd.ddtv_prepare_query(q, w_kc, r.vis, q_abs, q_rope, nb.theta, stream=stream) == dd.DDTV_OK

    def vproj():
        assert dd.ddtv_value_proj(r.out, w_vc, v, stream=stream) == dd.DDTV_OK

    def append():
        assert dd.ddtv_append_kv(lat, k_pe, r.vis, r.ckv, r.k_rope, w.kv_dtype, nb.theta, stream=stream) == dd.DDTV_OK

    elem = 2 if w.kv_dtype == 1 else 4
    res = {"workload": f"B*Q={M} tree nodes x H={H} heads, d_nope={d_nope}, d_v={d_v}, rope theta {nb.theta:g} "
                       "(synthetic weights and projections)"}
    for name, fn, flops, nbytes in (
            ("prepare_query", prep, 2 * M * H * d_nope * 512, 4 * (M * H * (d_nope + 64) + H * d_nope * 512
                                                                   + M * H * (512 + 64))),
            ("value_proj", vproj, 2 * M * H * 512 * d_v, 4 * (M * H * 512 + H * d_v * 512 + M * H * d_v)),
            ("append_kv", append, 0, 4 * M * (512 + 64) + elem * M * (512 + 64))):
        us = timed(fn)
        item = {"us_per_launch": round(us, 2), "algorithmic_bytes": nbytes,
                "gbps": round(nbytes / (us * 1e-6) / 1e9, 1)}
        if flops:
            item["flops"] = flops
            item["tflops"] = round(flops / (us * 1e-6) / 1e12, 2)
            item["frac_of_fp32_mfma_peak"] = round(flops / (us * 1e-6) / 1e12 / PEAK_TFLOPS["f32-mfma"], 4)
        res[name] = item
    res["launches"] = steps
    return res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(w, budget_s=15.0, max_rows=4096):
    """The oracle (single-threaded fp64 C) on a seeded sample of query rows of the
    same workload, for about budget_s seconds, pinned to one host core.  Reported
    as tree-query tokens/s (rows/s divided by H: one token is one tree node across
    all heads)."""
    import oracle
    import workloads as wl
    bits, _, _ = oracle.build_visibility(w.parent)
    rows = wl.sample_rows(w, max_rows, seed=11)
    pinned = None
    if hasattr(os, "sched_setaffinity"):
        pinned = min(os.sched_getaffinity(0))
        os.sched_setaffinity(0, {pinned})
    done = 0
    t0 = time.perf_counter()
    while done < len(rows) and time.perf_counter() - t0 < budget_s:
        k = min(8, len(rows) - done)
        oracle.verify_attn(w.q_abs, w.q_rope, w.ckv, w.k_rope, w.kv_dtype, w.prefix, bits, w.scale,
                           rows=rows[done:done + k])
        done += k
    dt = time.perf_counter() - t0
    return {"value": round(done / dt / w.H, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(), "pinned_cpu": pinned,
            "sample": f"{done} seeded (b,q,h) query rows of the same workload (all batch rows), "
                      f"{dt:.1f} s on 1 host core pinned by affinity; tokens/s = rows/s / H"}


def measure(dd, hip, stream, w, K, warmup, path=0, split_len=0, wg_order=0, dev=None, traffic_name=None,
            min_warm_ms=0.0):
    """Time K verify steps (S1..S7) of workload w after `warmup` untimed ones (and,
    with min_warm_ms, more until that much wall time has passed): the step from
    events around all K, the attention kernel from events the library records
    around it on the same stream.  Returns the run and a result dict."""
    import workloads as wl
    from tree_masked_mla_amd.runner import DeviceRun
    r = DeviceRun(w, device=dev, path=path, split_len=split_len, want_lse=True, wg_order=wg_order)
    rc, ppath, psplit, pn, pwgs, porder = r.plan()
    log(f"{w.name}: plan path={ppath} split_len={psplit} n_split={pn} workgroups={pwgs} wg_order={porder}")
    ev_attn = [(hip.event(), hip.event()) for _ in range(K)]
    ev0, ev1 = hip.event(), hip.event()
    for _ in range(warmup):
        r.step(stream)
    import torch
    torch.cuda.synchronize()
    # Short steps (~0.1 ms) reach the GPU's steady-state shader clock only after
    # tens of milliseconds of work (c3: 95.9 -> 89.3 us per attention launch).
    n_warm = warmup
    t_w0 = time.perf_counter()
    while (time.perf_counter() - t_w0) * 1e3 < min_warm_ms:
        r.step(stream)
        n_warm += 1
        if n_warm % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    t_host0 = time.perf_counter()
    hip.record(ev0, stream)
    for k in range(K):
        r.step(stream, dd.make_opts(path, split_len, ev_attn[k][0], ev_attn[k][1], wg_order))
    hip.record(ev1, stream)
    torch.cuda.synchronize()
    t_host1 = time.perf_counter()
    ms_step = hip.elapsed_ms(ev0, ev1) / K
    attn_all = [hip.elapsed_ms(a, b) for a, b in ev_attn]
    attn_ms = float(np.mean(attn_all))
    attn_med_ms = float(np.median(attn_all))
    nbytes, flops, vis_pairs = algorithmic(w)
    bf16_mma = ppath == dd.DDTV_PATH_MFMA and w.kv_dtype == wl.BF16
    valu = ppath == dd.DDTV_PATH_VALU
    peak_key = "bf16-mfma" if bf16_mma else ("f32-valu" if valu else "f32-mfma")
    kernel = "attn_mfma_bf16_kernel" if bf16_mma else ("attn_valu_kernel" if valu else "attn_mfma_kernel")
    khash = kernel_source_hash(kernel)
    # With splits the merge kernel writes the output and lse; the attention
    # kernel's roofline then leaves those bytes out.
    merged = pn > 1
    attn_nbytes = nbytes - (w.B * w.Q * w.H * (512 + 1) * 4 if merged else 0)
    roof = roofline_bound(valu, flops, attn_nbytes, attn_ms, PEAK_TFLOPS[peak_key])
    roof["bytes_per_launch"] = attn_nbytes
    res = {
        "warmup_steps": n_warm, "ms_per_step": ms_step, "attn_ms": attn_ms, "attn_median_ms": attn_med_ms, "host_ms_per_step": (t_host1 - t_host0) * 1e3 / K,
        "tokens_per_s": w.B * w.Q / (ms_step / 1e3), "hbm_gbps": nbytes / (ms_step / 1e3) / 1e9,
        "dtype": "bf16" if bf16_mma else "f32", "kernel": kernel, "kernel_source_hash": khash,
        "flops": flops, "nbytes": nbytes, "vis_pairs": vis_pairs, "roofline": roof,
        "traffic": load_traffic(traffic_name, khash) if traffic_name else None,
        "counters": load_counters(traffic_name, khash) if traffic_name else None,
        "plan": {"path": ppath, "split_len": psplit, "n_split": pn, "workgroups": pwgs,
                 "wg_order": {1: "xcd-local", 2: "spread"}.get(porder, porder)},
    }
    ctr = res.pop("counters")
    res["mfma_busy"] = ctr.get("mfma_busy_per_simd") if ctr else None
    ex = ctr.get("executed_flops_per_launch") if ctr else None
    # executed matrix flops (counters) over the same events' kernel time: the
    # algorithmic figure plus products spent on masked positions and padding
    res["mfma_executed"] = ({"flops_per_launch": ex, "tflops": round(ex / (attn_ms / 1e3) / 1e12, 3),
                             "over_algorithmic": ctr.get("executed_over_algorithmic_flops")} if ex else None)
    return r, res


def config_entry(name, w, desc, res, steps):
    """One entry of the line's `configs` object."""
    roof = dict(res["roofline"])
    roof["traffic"] = res["traffic"]
    return {"workload": f"{name}: {desc}", "dtype": res["dtype"],
            "arithmetic": ("bf16 MFMA, fp32 accumulation: query and probabilities rounded to bf16"
                           if res["dtype"] == "bf16" else "fp32 (cache values widened exactly)"),
            "kernel": res["kernel"], "kernel_us": round(res["attn_ms"] * 1e3, 2),
            "kernel_us_median": round(res["attn_median_ms"] * 1e3, 2),
            "step_us": round(res["ms_per_step"] * 1e3, 2), "tokens_per_s": round(res["tokens_per_s"], 1),
            "hbm_gbps": round(res["hbm_gbps"], 2), "roofline": roof, "mfma_busy": res["mfma_busy"],
            "mfma_executed": res["mfma_executed"],
            "kernel_source_hash": res["kernel_source_hash"], "flops_per_launch": res["flops"],
            "algorithmic_bytes_per_step": res["nbytes"], "plan": res["plan"], "steps": steps,
            "warmup_steps": res["warmup_steps"]}


# ----------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c4", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--path", type=int, default=0, help="0 auto, 1 VALU, 2 MFMA (cache precision), 3 fp32 MFMA")
    ap.add_argument("--split-len", type=int, default=0)
    ap.add_argument("--wg-order", type=int, default=0, help="0 auto, 1 XCD-local, 2 spread")
    ap.add_argument("--q-len", type=int, default=0,
                    help="override the workload's tree size (probe runs, e.g. q_len 1 = decode); "
                         "not the benchmarked configuration")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-baseline leg")
    ap.add_argument("--no-configs", dest="configs", action="store_false",
                    help="skip the other workloads (c3, c5, the q_len-1 probe) after the c4 headline")
    ap.add_argument("--attn-only", action="store_true",
                    help="time the verify step only (no builder, tail, acceptance, projection, FP8, iteration "
                         "or other-workload sections): for profiler and counter runs")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--read-calibration", type=int, default=0,
                    help="instead of the bench, run N launches of each read-stream calibration kernel over a "
                         "512 MiB buffer (known bytes read, for scaling rocprofv3 FETCH_SIZE)")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="instead of the bench, run N launches of a plain copy of the cache bytes "
                         "(for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as wl
    import tree_masked_mla_amd as dd
    from tree_masked_mla_amd.runner import DeviceRun

    dd.load()   # fails loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.read_calibration:
        hip = Hip()
        stream = torch.cuda.current_stream(dev).cuda_stream
        c = read_ceiling(hip, stream, dev, torch.cuda.get_device_properties(dev).multi_processor_count,
                         reps=args.read_calibration, warmup=0)
        torch.cuda.synchronize()
        print(json.dumps({"read_calibration": c, "launches_per_kernel": args.read_calibration}))
        return

    desc = wl.DESCRIPTIONS[args.config]
    if args.q_len:
        desc += f" [probe: q_len overridden to {args.q_len}]"
    log(f"generating {args.config}: {desc}")
    w = wl.config(args.config, Q=args.q_len) if args.q_len else wl.config(args.config)

    if args.copy_calibration:
        nbytes = w.ckv.nbytes
        src = torch.from_numpy(np.ascontiguousarray(w.ckv).view(np.uint8)).to(dev).view(torch.float32)
        dst = torch.empty_like(src)
        for _ in range(args.copy_calibration):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": nbytes, "bytes_written": nbytes,
                          "launches": args.copy_calibration}))
        return

    hip = Hip()
    stream = torch.cuda.current_stream(dev).cuda_stream
    K = args.steps
    traffic_name = None if args.q_len else args.config
    r, res = measure(dd, hip, stream, w, K, args.warmup, args.path, args.split_len, args.wg_order, dev,
                     traffic_name)
    ceiling = read_ceiling(hip, stream, dev, torch.cuda.get_device_properties(dev).multi_processor_count)
    res["roofline"] = with_ceiling(res["roofline"], ceiling)
    ms_step, attn_avg_ms = res["ms_per_step"], res["attn_ms"]
    tokens = w.B * w.Q
    value = tokens / (ms_step / 1e3)
    hbm_gbps = res["hbm_gbps"]
    plan = res["plan"]

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": res["dtype"],
        "data": "synthetic",
        "config": {"workload": f"{args.config}: {desc}", "B": w.B, "H": w.H,
                   "q_len": w.Q, "prefix": "ragged" if args.config == "c5" else int(w.prefix[0]),
                   "total_kv_rows": w.total_kv, "scale": w.scale, "path": plan["path"],
                   "split_len": plan["split_len"], "n_split": plan["n_split"], "workgroups": plan["workgroups"],
                   "wg_order": plan["wg_order"]},
        "hbm_gbps": round(hbm_gbps, 2),
        "hbm_pct_of_peak": round(100.0 * hbm_gbps / HBM_PEAK_GBPS, 3),
        "attn_kernel_us": round(attn_avg_ms * 1e3, 2),
        "attn_kernel_us_median": round(res["attn_median_ms"] * 1e3, 2),
        "step_us": round(ms_step * 1e3, 2),
        "host_wall_ms_per_step": round(res["host_ms_per_step"], 4),
        "hbm_read_ceiling": ceiling,
        "roofline": {
            **res["roofline"],
            "traffic": res["traffic"],
            "mfma_busy": res["mfma_busy"],
            "mfma_executed": res["mfma_executed"],
            "kernel": res["kernel"],
            "flops_per_launch": res["flops"],
            "algorithmic_bytes_per_step": res["nbytes"],
            "visible_pairs": res["vis_pairs"],
            "kernel_source_hash": res["kernel_source_hash"],
        },
    }
    if not args.attn_only:
        out["tree_build"] = time_tree_builder(dd, hip, stream, dev, w.B, w.Q)
        out["tail_mode"] = time_tail_mode(dd, hip, stream, r)
        out["tree_accept"] = time_tree_accept(dd, hip, stream, r)
        out["neighbour"] = time_neighbour(dd, hip, stream, r)
        out["fp8_cache"] = time_fp8_cache(dd, hip, stream, r, res["flops"])
        out["iteration"] = time_iteration(dd, hip, stream, r)
        out["iteration_growing_prefix"] = time_iteration(dd, hip, stream, r, grow=True)
    if args.configs and not args.attn_only and args.config == "c4" and not args.q_len:
        # the other workloads, each in its own timed region (the headline above stays c4)
        out["configs"] = {}
        del r
        torch.cuda.empty_cache()
        for name, q_len, steps in (("c3", 0, max(K, 50)), ("c4_q_len_1", 1, K), ("c5", 0, K)):
            base = "c4" if q_len else name
            d = wl.DESCRIPTIONS[base] + (f" [decode probe: q_len {q_len}]" if q_len else "")
            log(f"generating {name}: {d}")
            wc = wl.config(base, Q=q_len) if q_len else wl.config(base)
            rc_, res_c = measure(dd, hip, stream, wc, steps, args.warmup, dev=dev, traffic_name=name,
                                 min_warm_ms=CONFIG_MIN_WARM_MS)
            res_c["roofline"] = with_ceiling(res_c["roofline"], ceiling)
            out["configs"][name] = config_entry(name, wc, d, res_c, steps)
            del rc_
            torch.cuda.empty_cache()
    if not args.no_cpu:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(w, budget_s=args.cpu_budget)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
