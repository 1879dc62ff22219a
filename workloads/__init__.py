"""Seeded synthetic inputs for tree-verify MLA-absorb attention.

This module only draws inputs: tree shapes, prefix lengths and the query / latent
KV tensors. It holds none of the attention arithmetic and none of the visibility
logic, so both the CPU oracle and the HIP path can consume what it produces
without sharing any of the computation.

Shapes follow the pages' description of the verify step (absorbed 512-d query
plus a 64-d rope query per (token, head); one 512-d latent plus one 64-d rope key
per cached position, shared by all heads) -- "The Verify-Attn Kernel: A Single
File Write ...", section "The Design Journey: From Concept to CUDA", and the
latent/rope sizes in its section "Assumptions and the Path Forward".

Recipe (for every workload):
  * numpy PCG64 ``default_rng(seed)``;
  * draw order: trees, prefixes, q_abs, q_rope, ckv, k_rope;
  * float32 tensors are ``standard_normal(dtype=float32) * sigma``;
  * bf16 tensors are the float32 draw rounded to nearest-even on the bit pattern;
  * FP8 E4M3 tensors are the float32 draw converted by torch's float8_e4m3fn cast
    (round to nearest even; the draws stay far inside the format's +-448 range).
"""
from __future__ import annotations

import heapq
import math
from dataclasses import dataclass, field

import numpy as np

D_LATENT = 512
D_ROPE = 64
SCALE_192 = 1.0 / math.sqrt(192.0)

F32 = 0
BF16 = 1
FP8 = 2      # FP8 E4M3 ("fn": bias 7, no infinities), one byte per value


# --------------------------------------------------------------------------- trees
def uniform_tree(rng: np.random.Generator, q: int) -> np.ndarray:
    """Random recursive tree: parent[0] = -1, parent[i] uniform in [0, i)."""
    p = np.empty(q, dtype=np.int32)
    p[0] = -1
    for i in range(1, q):
        p[i] = rng.integers(0, i)
    return p


def chain_tree(q: int) -> np.ndarray:
    """Linear chain: parent[i] = i - 1 (the prefill / causal shape)."""
    p = np.arange(-1, q - 1, dtype=np.int32)
    return p


def best_first_tree(rng: np.random.Generator, q: int, depth_cap: int,
                    vocab: int = 32, topk: int = 4, logit_sigma: float = 2.0) -> np.ndarray:
    """Tree shaped like a best-first draft expansion.

    The root has score 0.  Whenever a node at depth < depth_cap is added, ``vocab``
    logits ~ N(0, logit_sigma^2) are drawn, and the ``topk`` best log-softmax
    entries become candidate children with score parent_score + log p.  Candidates
    are popped from a max-heap (ties by push order) until ``q`` nodes exist, so
    parents always precede children, every internal node has 1..topk children and
    the depth (in edges, root = 0) never exceeds ``depth_cap``.
    """
    parent = np.empty(q, dtype=np.int32)
    parent[0] = -1
    depth = [0]
    score = [0.0]
    heap: list[tuple[float, int, int]] = []
    pushes = 0

    def expand(node: int) -> None:
        nonlocal pushes
        if depth[node] >= depth_cap:
            return
        logits = rng.standard_normal(vocab) * logit_sigma
        mx = logits.max()
        logp = logits - (mx + math.log(np.exp(logits - mx).sum()))
        top = np.argsort(-logp, kind="stable")[:topk]
        for t in top:
            heapq.heappush(heap, (-(score[node] + float(logp[t])), pushes, node))
            pushes += 1

    expand(0)
    n = 1
    while n < q:
        if not heap:
            raise RuntimeError("best-first expansion ran out of candidates")
        neg, _, par = heapq.heappop(heap)
        parent[n] = par
        depth.append(depth[par] + 1)
        score.append(-neg)
        expand(n)
        n += 1
    return parent


def tree_depths(parent: np.ndarray) -> np.ndarray:
    """Depth in edges of each node of a topologically ordered tree (input helper)."""
    d = np.zeros(len(parent), dtype=np.int32)
    for i in range(1, len(parent)):
        d[i] = d[parent[i]] + 1
    return d


# --------------------------------------------------------------------------- tensors
def round_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.
    (Finite inputs only: the sum below cannot wrap for them.)"""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (r >> np.uint32(16)).astype(np.uint16)


def round_fp8_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> FP8 E4M3 bytes (uint8) by torch's float8_e4m3fn conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def fp8_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """FP8 E4M3 bytes -> float32 by torch's conversion (exact)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float32).numpy()


def _normal_rows(rng: np.random.Generator, rows: int, cols: int, sigma: float, bf16,
                 chunk_rows: int = 1 << 16) -> np.ndarray:
    """rows x cols draws of N(0, sigma^2) as float32 (or bf16 bits, or FP8 bytes when
    bf16 == FP8), drawn in row chunks: the stream of draws is the same as one big
    call, but a narrow result never holds the whole float32 array in memory."""
    if not isinstance(bf16, bool) and bf16 == FP8:
        out8 = np.empty((rows, cols), dtype=np.uint8)
        for r0 in range(0, rows, chunk_rows):
            r1 = min(rows, r0 + chunk_rows)
            a = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
            if sigma != 1.0:
                a *= np.float32(sigma)
            out8[r0:r1] = round_fp8_bits(a)
        return out8
    if not bf16:
        a = rng.standard_normal((rows, cols), dtype=np.float32)
        if sigma != 1.0:
            a *= np.float32(sigma)
        return a
    out = np.empty((rows, cols), dtype=np.uint16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        a = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        if sigma != 1.0:
            a *= np.float32(sigma)
        out[r0:r1] = round_bf16_bits(a)
    return out


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (h.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Workload:
    name: str
    B: int
    H: int
    Q: int
    prefix: np.ndarray            # int32 [B]
    parent: np.ndarray            # int32 [B][Q]
    q_abs: np.ndarray             # float32 [B][Q][H][512]
    q_rope: np.ndarray            # float32 [B][Q][H][64]
    ckv: np.ndarray               # float32, uint16 (bf16 bits) or uint8 (FP8 bytes) [sum KV][512]
    k_rope: np.ndarray            # same dtype [sum KV][64]
    kv_dtype: int                 # F32 or BF16
    scale: float
    meta: dict = field(default_factory=dict)

    @property
    def kv_len(self) -> np.ndarray:
        return self.prefix.astype(np.int64) + self.Q

    @property
    def kv_off(self) -> np.ndarray:
        """Row offset of each batch row in the packed cache (rows back to back)."""
        off = np.zeros(self.B + 1, dtype=np.int64)
        off[1:] = np.cumsum(self.kv_len)
        return off

    @property
    def total_kv(self) -> int:
        return int(self.kv_len.sum())

    def with_parent(self, parent: np.ndarray, name: str | None = None) -> "Workload":
        w = Workload(**{**self.__dict__})
        w.parent = np.ascontiguousarray(parent, dtype=np.int32).reshape(self.B, self.Q)
        w.name = name or self.name
        return w


def _draw_trees(rng: np.random.Generator, B: int, Q: int, prefix, tree: str, depth_cap: int):
    # 1. trees
    if tree == "uniform":
        parent = np.stack([uniform_tree(rng, Q) for _ in range(B)])
    elif tree == "chain":
        parent = np.stack([chain_tree(Q) for _ in range(B)])
    elif tree == "best_first":
        parent = np.stack([best_first_tree(rng, Q, depth_cap) for _ in range(B)])
    else:
        raise ValueError(tree)
    # 2. prefixes
    if isinstance(prefix, tuple) and prefix and prefix[0] == "uniform":
        pre = rng.integers(prefix[1], prefix[2] + 1, size=B).astype(np.int32)
    elif np.isscalar(prefix):
        pre = np.full(B, int(prefix), dtype=np.int32)
    else:
        pre = np.asarray(prefix, dtype=np.int32).reshape(B)
    return parent.astype(np.int32), pre


def make_workload(name: str, seed: int, B: int, H: int, Q: int, prefix,
                  tree: str = "uniform", depth_cap: int = 0,
                  q_sigma: float = 1.0, kv_sigma: float = 1.0,
                  kv_dtype: int = F32, scale: float = SCALE_192) -> Workload:
    """Draw one workload.  ``prefix`` is an int, a sequence of B ints, or a
    (lo, hi) range given as ``("uniform", lo, hi)`` (inclusive)."""
    rng = np.random.default_rng(seed)
    parent, pre = _draw_trees(rng, B, Q, prefix, tree, depth_cap)
    total_kv = int((pre.astype(np.int64) + Q).sum())
    # 3. tensors
    q_abs = rng.standard_normal((B, Q, H, D_LATENT), dtype=np.float32)
    if q_sigma != 1.0:
        q_abs *= np.float32(q_sigma)
    q_rope = rng.standard_normal((B, Q, H, D_ROPE), dtype=np.float32)
    if q_sigma != 1.0:
        q_rope *= np.float32(q_sigma)
    narrow = FP8 if kv_dtype == FP8 else kv_dtype == BF16
    ckv = _normal_rows(rng, total_kv, D_LATENT, kv_sigma, narrow)
    k_rope = _normal_rows(rng, total_kv, D_ROPE, kv_sigma, narrow)
    return Workload(name=name, B=B, H=H, Q=Q, prefix=pre, parent=parent.astype(np.int32),
                    q_abs=q_abs, q_rope=q_rope, ckv=ckv, k_rope=k_rope,
                    kv_dtype=kv_dtype, scale=float(scale),
                    meta=dict(seed=seed, tree=tree, depth_cap=depth_cap,
                              q_sigma=q_sigma, kv_sigma=kv_sigma))


# --------------------------------------------------------------------------- the five workloads
# c1..c5: the five verify-attention workloads (sizes as named).  Seeds are 1000 + index.
CONFIGS = {
    "c1": dict(B=1, H=8, Q=9, prefix=0, tree="uniform"),
    "c2": dict(B=3, H=8, Q=9, prefix=37, tree="uniform"),
    "c3": dict(B=1, H=16, Q=64, prefix=4096, tree="best_first", depth_cap=8, kv_sigma=0.5),
    "c4": dict(B=8, H=16, Q=128, prefix=32768, tree="best_first", depth_cap=12),
    "c5": dict(B=32, H=64, Q=64, prefix=("uniform", 1024, 131072), tree="uniform", kv_dtype=BF16),
}

DESCRIPTIONS = {
    "c1": "B=1 H=8 prefix=0 q_len=9 uniform tree fp32",
    "c2": "B=3 H=8 prefix=37 q_len=9 uniform trees fp32",
    "c3": "B=1 H=16 prefix=4096 q_len=64 best-first tree (depth<=8) fp32, KV sigma 0.5",
    "c4": "B=8 H=16 prefix=32768 q_len=128 best-first trees (depth<=12) fp32",
    "c5": "B=32 H=64 prefix~U[1024,131072] q_len=64 uniform trees bf16 KV",
}


def config(name: str, seed: int | None = None, **override) -> Workload:
    idx = int(name[1:])
    kw = dict(CONFIGS[name])
    kw.update(override)
    return make_workload(name, 1000 + idx if seed is None else seed, **kw)


def config_trees(name: str, seed: int | None = None):
    """Only the trees and prefixes of a named workload (the first draws of its
    stream), without drawing any tensor."""
    idx = int(name[1:])
    kw = dict(CONFIGS[name])
    rng = np.random.default_rng(1000 + idx if seed is None else seed)
    return _draw_trees(rng, kw["B"], kw["Q"], kw["prefix"], kw["tree"], kw.get("depth_cap", 0))


def c2_chain() -> Workload:
    """c2's tensors with every tree replaced by a chain (must equal causal attention)."""
    w = config("c2")
    return w.with_parent(np.stack([chain_tree(w.Q) for _ in range(w.B)]), name="c2-chain")


def drafter_topk(seed: int, B: int, D: int, K: int, vocab: int = 32, sigma: float = 2.0):
    """Synthetic drafter output for the tree builder: for each batch row and depth,
    logits ~ N(0, sigma^2) over `vocab` tokens, their log-softmax, and the K best
    (log-probability float32 [B][D][K] sorted descending, token id int32 [B][D][K])."""
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((B, D, vocab)) * sigma
    lp = logits - np.log(np.exp(logits - logits.max(-1, keepdims=True)).sum(-1, keepdims=True)) \
        - logits.max(-1, keepdims=True)
    order = np.argsort(-lp, axis=-1, kind="stable")[..., :K]
    return (np.ascontiguousarray(np.take_along_axis(lp, order, -1), dtype=np.float32),
            np.ascontiguousarray(order, dtype=np.int32))


def target_logits(seed: int, B: int, Q: int, V: int) -> np.ndarray:
    """Synthetic target-model logits after each tree node: float32 [B][Q][V], N(0, 1)."""
    return np.random.default_rng(seed).standard_normal((B, Q, V), dtype=np.float32)


def sample_rows(w: Workload, n: int, seed: int = 7) -> np.ndarray:
    """Seeded sample of n flat query-row ids (b*Q + q)*H + h spread over all batch rows."""
    rng = np.random.default_rng(seed)
    total = w.B * w.Q * w.H
    if n >= total:
        return np.arange(total, dtype=np.int64)
    per_b = [n // w.B + (1 if b < n % w.B else 0) for b in range(w.B)]
    rows = []
    for b, k in enumerate(per_b):
        if k == 0:
            continue
        local = rng.choice(w.Q * w.H, size=k, replace=False)
        rows.append(b * w.Q * w.H + np.sort(local))
    return np.concatenate(rows).astype(np.int64)


# --------------------------------------------------------------------------- around the attention
# Rotary base of the synthetic model (a configuration value, as in Kimi K2-style configs).
ROPE_THETA = 50000.0


@dataclass
class NeighbourInputs:
    """Synthetic tensors of the steps around the verify attention for B trees of Q nodes."""
    q: np.ndarray        # float32 [B][Q][H][d_nope + 64]: query projection (nope part, then rope part)
    w_kc: np.ndarray     # float32 [H][d_nope][512]: absorb weights (nope -> latent)
    w_vc: np.ndarray     # float32 [H][d_v][512]: value weights (latent -> value)
    latent: np.ndarray   # float32 [B][Q][512]: the nodes' new latent cache rows
    k_pe: np.ndarray     # float32 [B][Q][64]: the nodes' new rope keys, not yet rotated
    theta: float


def neighbour_inputs(seed: int, B: int, Q: int, H: int, d_nope: int = 128, d_v: int = 128,
                     theta: float = ROPE_THETA) -> NeighbourInputs:
    """Seeded draws, in this order: q ~ N(0,1), w_kc ~ N(0, 1/d_nope), w_vc ~ N(0, 1/512),
    latent ~ N(0,1), k_pe ~ N(0,1).  The weight spreads keep q_abs and v near unit scale."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Q, H, d_nope + D_ROPE), dtype=np.float32)
    w_kc = rng.standard_normal((H, d_nope, D_LATENT), dtype=np.float32) * np.float32(1.0 / math.sqrt(d_nope))
    w_vc = rng.standard_normal((H, d_v, D_LATENT), dtype=np.float32) * np.float32(1.0 / math.sqrt(D_LATENT))
    latent = rng.standard_normal((B, Q, D_LATENT), dtype=np.float32)
    k_pe = rng.standard_normal((B, Q, D_ROPE), dtype=np.float32)
    return NeighbourInputs(q=q, w_kc=w_kc, w_vc=w_vc, latent=latent, k_pe=k_pe, theta=float(theta))
