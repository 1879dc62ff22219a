"""Device-side plumbing around the C ABI: puts a workload's arrays in HBM with
PyTorch, owns the output / visibility / workspace buffers, and runs one verify
step (visibility build + attention + merge) through libddtv.  No arithmetic of
the method happens here."""
from __future__ import annotations

import numpy as np
import torch

from . import (DDTV_BF16, DDTV_FP8_E4M3, DDTV_ORDER_AUTO, DDTV_PATH_AUTO, check, ddtv_build_visibility, ddtv_plan_info, ddtv_vis_bytes,
               ddtv_verify_attn, ddtv_workspace_bytes, load, make_opts)


def to_device_kv(a: np.ndarray, kv_dtype: int, device) -> torch.Tensor:
    """float32 array, bf16 bit patterns (uint16) or FP8 E4M3 bytes (uint8), to a device tensor."""
    if kv_dtype == DDTV_FP8_E4M3:
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(device)
    if kv_dtype == DDTV_BF16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


class DeviceRun:
    """One workload resident on one GPU, ready to run verify steps."""

    def __init__(self, w, device="cuda:0", path: int = DDTV_PATH_AUTO, split_len: int = 0,
                 want_lse: bool = True, parent=None, bits_override: np.ndarray | None = None,
                 wg_order: int = DDTV_ORDER_AUTO):
        load()
        self.w = w
        self.device = torch.device(device)
        self.B, self.Q, self.H = w.B, w.Q, w.H
        self.kv_dtype = w.kv_dtype
        self.scale = w.scale
        self.prefix = np.ascontiguousarray(w.prefix, dtype=np.int32)
        par = w.parent if parent is None else parent
        self.parent = torch.from_numpy(np.ascontiguousarray(par, dtype=np.int32)).to(self.device)
        self.q_abs = torch.from_numpy(np.ascontiguousarray(w.q_abs)).to(self.device)
        self.q_rope = torch.from_numpy(np.ascontiguousarray(w.q_rope)).to(self.device)
        self.ckv = to_device_kv(w.ckv, w.kv_dtype, self.device)
        self.k_rope = to_device_kv(w.k_rope, w.kv_dtype, self.device)
        self.out = torch.empty((w.B, w.Q, w.H, 512), dtype=torch.float32, device=self.device)
        self.lse = torch.empty((w.B, w.Q, w.H), dtype=torch.float32, device=self.device) if want_lse else None
        self.vis_buf = torch.empty(ddtv_vis_bytes(w.B, w.Q), dtype=torch.uint8, device=self.device)
        self.opts = make_opts(path, split_len, wg_order=wg_order)
        self.bits_override = bits_override
        self.vis = self.build_visibility()
        self.ws_bytes = ddtv_workspace_bytes(self.vis, w.H, w.kv_dtype, self.opts)
        self.workspace = (torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
                          if self.ws_bytes else None)

    def build_visibility(self, stream=None):
        rc, vis = ddtv_build_visibility(self.parent, self.prefix, self.B, self.Q, self.vis_buf, stream=stream)
        check(rc, "ddtv_build_visibility")
        if self.bits_override is not None:
            # replace the tree masks with a caller-made mask (same layout)
            n = self.B * self.Q * vis.W
            src = torch.from_numpy(np.ascontiguousarray(self.bits_override, dtype=np.uint32).view(np.int32))
            dst = torch.as_strided(self.vis_buf, (n * 4,), (1,), 0)
            dst.copy_(src.reshape(-1).view(torch.uint8).to(self.device))
        return vis

    def plan(self):
        return ddtv_plan_info(self.vis, self.H, self.kv_dtype, self.opts)

    def verify(self, stream=None, opts=None):
        rc = ddtv_verify_attn(self.q_abs, self.q_rope, self.ckv, self.k_rope, self.kv_dtype, self.H, self.vis,
                              self.scale, self.out, self.lse, self.workspace, self.ws_bytes, stream,
                              opts if opts is not None else self.opts)
        check(rc, "ddtv_verify_attn")

    def step(self, stream=None, opts=None):
        """One full verify step: S1 visibility build, then S2..S7."""
        self.vis = self.build_visibility(stream)
        self.verify(stream, opts)

    def bits(self) -> np.ndarray:
        W = (self.Q + 31) // 32
        n = self.B * self.Q * W
        raw = self.vis_buf[: n * 4].cpu().numpy().view(np.uint32)
        return raw.reshape(self.B, self.Q, W).copy()

    def status(self) -> np.ndarray:
        off = self.vis.status - self.vis_buf.data_ptr()
        return self.vis_buf[off: off + 4 * self.B].cpu().numpy().view(np.int32).copy()

    def results(self):
        torch.cuda.synchronize(self.device)
        out = self.out.cpu().numpy().reshape(-1, 512)
        lse = self.lse.cpu().numpy().reshape(-1) if self.lse is not None else None
        return out, lse
