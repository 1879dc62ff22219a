"""The benchmark's HBM read-stream calibration library (libddtv_calib.so): a
measurement aid outside the verify path.  Host-side argument checks need no
GPU; on the GPU each stream's sink must equal the sums of exactly the data the
kernel claims to have read."""
import ctypes
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CALIB = os.path.join(ROOT, "tree_masked_mla_amd", "libddtv_calib.so")
TILE = 72 * 1024     # mode 0 unit
STEP = 64 * 1024     # mode 1 unit


@pytest.fixture(scope="module")
def fn():
    from tree_masked_mla_amd import share_hip_runtime_with_torch
    share_hip_runtime_with_torch()
    if not os.path.exists(CALIB):
        from tree_masked_mla_amd import build
        build.build()
    f = ctypes.CDLL(CALIB).ddtv_calib_stream_read
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                  ctypes.POINTER(ctypes.c_int64)]
    f.restype = ctypes.c_int
    return f


def test_rejects_bad_arguments_on_the_host(fn):
    n = ctypes.c_int64(-1)
    fake = 1 << 40      # aligned, never dereferenced: every case fails its check first
    assert fn(None, 1 << 20, 0, fake, 4, None, ctypes.byref(n)) == 1
    assert fn(fake, 1 << 20, 0, None, 4, None, ctypes.byref(n)) == 1
    assert fn(fake, 1 << 20, 2, fake, 4, None, ctypes.byref(n)) == 1
    assert fn(fake, 1 << 20, 0, fake, 0, None, ctypes.byref(n)) == 1
    assert fn(fake, 1 << 20, 0, fake, 65536, None, ctypes.byref(n)) == 1
    assert fn(fake + 8, 1 << 20, 0, fake, 4, None, ctypes.byref(n)) == 1
    assert fn(fake, -1, 0, fake, 4, None, ctypes.byref(n)) == 1
    assert fn(fake, 1 << 20, 0, fake, 4, None, None) == 1
    assert n.value == -1


def expected_sink(data, mode, wgs, per_wg):
    """Host model of each thread's sum, in the kernel's order (float32)."""
    v = data[: len(data) // 16 * 16].view(np.float32).reshape(-1, 4)
    out = np.zeros((wgs, 512), dtype=np.float32)
    unit = TILE if mode == 0 else STEP
    for g in range(wgs):
        acc = np.zeros((512, 4), dtype=np.float32)
        base = g * per_wg * unit // 16
        for i in range(per_wg):
            if mode == 0:        # the first 8 KiB of tile i, one 16-byte chunk per thread
                acc += v[base + i * (TILE // 16): base + i * (TILE // 16) + 512]
            else:                # 8 chunks 8 KiB apart per step
                for u in range(8):
                    o = base + i * (STEP // 16) + u * 512
                    acc += v[o: o + 512]
        out[g] = (acc[:, 0] + acc[:, 1]) + (acc[:, 2] + acc[:, 3])
    return out


@pytest.mark.gpu
@pytest.mark.parametrize("mode", [0, 1])
def test_stream_reads_what_it_counts(fn, mode):
    import torch
    rng = np.random.default_rng(5 + mode)
    wgs = 6
    unit = TILE if mode == 0 else STEP
    nbytes = wgs * 5 * unit + 12345                   # a ragged tail the kernel must leave alone
    host = rng.integers(-8, 8, size=nbytes // 4, dtype=np.int32).astype(np.float32)   # exact sums
    buf = torch.from_numpy(host).cuda()
    sink = torch.full((wgs * 512,), float("nan"), dtype=torch.float32, device="cuda")
    n = ctypes.c_int64(-1)
    assert fn(buf.data_ptr(), host.nbytes, mode, sink.data_ptr(), wgs, None, ctypes.byref(n)) == 0
    torch.cuda.synchronize()
    per_wg = host.nbytes // wgs // unit
    assert n.value == per_wg * unit * wgs
    want = expected_sink(host.view(np.uint8), mode, wgs, per_wg)
    assert np.array_equal(sink.cpu().numpy().reshape(wgs, 512), want)
