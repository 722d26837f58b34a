"""Copy ring (linear_gemv_streamed / linear_gemm_streamed): matrices held in page-locked
host memory, streamed through two device slots, give the same bits as the resident calls."""

import ctypes

import numpy as np
import pytest

import synth
import weight_streaming_linear_amd as wsl
from gpu_common import say

pytestmark = pytest.mark.gpu

SHAPES = [(1000, 512), (257, 2048), (4096, 320), (64, 6144), (3000, 1024), (17, 64), (2048, 2048)]


def _stack(wfmt):
    import torch
    mats, dev = [], []
    for i, (n, k) in enumerate(SHAPES):
        w = synth.device_weight(105, i, n, k)
        d = wsl.nf4_pack(w) if wfmt == wsl.WSL_W_NF4 else w
        dev.append(d)
        mats.append((wsl.to_pinned(d), n, k))
    nbytes = max((wsl.nf4_packed_bytes(n, k) if wfmt == wsl.WSL_W_NF4 else 2 * n * k) for n, k in SHAPES)
    return mats, dev, nbytes


@pytest.mark.parametrize("wfmt", [wsl.WSL_W_NF4, wsl.WSL_W_BF16])
def test_gemv_streamed_matches_resident(wfmt):
    import torch
    say(f"ring gemv wfmt={wfmt}")
    mats, dev, nbytes = _stack(wfmt)
    xs = [synth.device_normal_bf16(105, 100 + i, (k,)) for i, (_, k) in enumerate(SHAPES)]
    want = [wsl.linear_gemv(d, x, wfmt=wfmt, n_out=n, k=k) for d, x, (n, k) in zip(dev, xs, SHAPES)]
    ring = wsl.CopyRing(nbytes)
    for rep in range(3):               # the slots and events carry over between calls
        ys = [torch.full((n,), float("nan"), dtype=torch.float32, device="cuda") for n, _ in SHAPES]
        ring.gemv(mats, xs, ys, wfmt=wfmt)
        torch.cuda.synchronize()
        for i, (y, w) in enumerate(zip(ys, want)):
            assert torch.equal(y, w), f"matrix {i} differs on call {rep}"


def test_gemm_streamed_matches_resident():
    import torch
    say("ring gemm")
    mats, dev, nbytes = _stack(wsl.WSL_W_NF4)
    m = 32
    kmax = max(k for _, k in SHAPES)
    xs = [synth.device_normal_bf16(106, 100 + i, (m, k)) for i, (_, k) in enumerate(SHAPES)]
    # one shared leading dimension: X rows padded to kmax, Y rows to the largest n_out
    nmax = max(n for n, _ in SHAPES)
    xp = [torch.zeros((m, kmax), dtype=torch.bfloat16, device="cuda") for _ in SHAPES]
    for a, b in zip(xp, xs):
        a[:, :b.shape[1]] = b
    ws_bytes = max(wsl.linear_gemm_workspace_bytes(wsl.WSL_W_NF4, n, k, m) for n, k in SHAPES)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    want = [wsl.linear_gemm(d, a[:, :k], wfmt=wsl.WSL_W_NF4, n_out=n, k=k, workspace=ws)
            for d, a, (n, k) in zip(dev, xp, SHAPES)]
    ys = [torch.full((m, nmax), float("nan"), dtype=torch.float32, device="cuda") for _ in SHAPES]
    ring = wsl.CopyRing(nbytes)
    ring.gemm(mats, xp, ys, m, kmax, nmax, workspace=ws)
    torch.cuda.synchronize()
    for i, ((n, k), y, w) in enumerate(zip(SHAPES, ys, want)):
        assert torch.equal(y[:, :n], w), f"matrix {i} differs"


def test_streamed_rejects_pageable_host_memory():
    import torch
    n, k = 64, 128
    w = synth.device_weight(107, 0, n, k)
    p = wsl.nf4_pack(w)
    pageable = np.zeros(wsl.nf4_packed_bytes(n, k), dtype=np.uint8)
    x = synth.device_normal_bf16(107, 1, (k,))
    y = torch.empty(n, dtype=torch.float32, device="cuda")
    ring = wsl.CopyRing(wsl.nf4_packed_bytes(n, k))
    hs = (ctypes.c_void_p * 1)(pageable.ctypes.data)
    with pytest.raises(wsl.WSLError) as e:
        ring_call = wsl.lib().linear_gemv_streamed
        rc = ring_call(wsl.WSL_W_NF4, 1, hs, (ctypes.c_int64 * 1)(n), (ctypes.c_int64 * 1)(k),
                       wsl._ptr_array([x]), wsl._ptr_array([y]), wsl._ptr_array(ring.slots), ring.slot_bytes,
                       ctypes.c_void_p(ring.copy_stream.cuda_stream), wsl._stream(None),
                       wsl._ptr_array([ev.cuda_event for ev in ring.events]))
        wsl._check(rc, "linear_gemv_streamed")
    assert e.value.code == 8
    # the refused call left no pending error behind: a normal call still works
    wsl.linear_gemv(p, x, y=y, wfmt=wsl.WSL_W_NF4, n_out=n, k=k)
    torch.cuda.synchronize()
