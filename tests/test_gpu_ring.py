"""Copy ring (linear_gemv_streamed / linear_gemm_streamed): matrices held in page-locked
host memory, streamed through two device slots.  Every streamed output is checked against
the fp64 oracle (deep-fold README, "Метод" table and Figure 1: the same kernels read the
matrices from the slots), and must also equal the resident call bit for bit."""

import ctypes

import numpy as np
import pytest

import oracle
import synth
import weight_streaming_linear_amd as wsl
from gpu_common import to_dev_bf16, f64, say

pytestmark = pytest.mark.gpu

SHAPES = [(1000, 512), (257, 2048), (4096, 320), (64, 6144), (3000, 1024), (17, 64), (2048, 2048)]


def _stack(wfmt):
    """Seeded host weights (bf16 bits), their device form, pinned host copies, and the slot size."""
    mats, dev, bits = [], [], []
    for i, (n, k) in enumerate(SHAPES):
        wb = synth.weight_bits(105, i, n, k)
        w = to_dev_bf16(wb)
        d = wsl.nf4_pack(w) if wfmt == wsl.WSL_W_NF4 else w
        bits.append(wb)
        dev.append(d)
        mats.append((wsl.to_pinned(d), n, k))
    nbytes = max((wsl.nf4_packed_bytes(n, k) if wfmt == wsl.WSL_W_NF4 else 2 * n * k) for n, k in SHAPES)
    return mats, dev, bits, nbytes


def _gemv_ref(wfmt, wb, xb):
    if wfmt == wsl.WSL_W_NF4:
        codes, scales = oracle.pack_codes(f64(wb))
        return oracle.gemv_ref(oracle.dequant_exact(codes, scales), f64(xb))
    return oracle.gemv_ref(f64(wb), f64(xb))


@pytest.mark.parametrize("pace", [True, False])
@pytest.mark.parametrize("wfmt", [wsl.WSL_W_NF4, wsl.WSL_W_BF16])
def test_gemv_streamed_against_oracle(wfmt, pace):
    import torch
    say(f"ring gemv wfmt={wfmt} pace={pace}")
    mats, dev, bits, nbytes = _stack(wfmt)
    xbs = [synth.act_bits(105, 100 + i, (k,)) for i, (_, k) in enumerate(SHAPES)]
    xs = [to_dev_bf16(b) for b in xbs]
    refs = [_gemv_ref(wfmt, wb, xb) for wb, xb in zip(bits, xbs)]
    want = [wsl.linear_gemv(d, x, wfmt=wfmt, n_out=n, k=k) for d, x, (n, k) in zip(dev, xs, SHAPES)]
    ring = wsl.CopyRing(nbytes)
    for rep in range(3):               # the slots and events carry over between calls
        ys = [torch.full((n,), float("nan"), dtype=torch.float32, device="cuda") for n, _ in SHAPES]
        ring.gemv(mats, xs, ys, wfmt=wfmt, pace=pace)
        torch.cuda.synchronize()
        for i, (y, w, (y_ref, s_ref)) in enumerate(zip(ys, want, refs)):
            ok, worst, r = oracle.check_rows_f32(y.cpu().numpy(), y_ref, s_ref)
            assert ok, f"matrix {i} {SHAPES[i]} call {rep}: row {r} worst ratio {worst}"
            assert torch.equal(y, w), f"matrix {i} differs from the resident call on call {rep}"


@pytest.mark.parametrize("ofmt", [wsl.WSL_OUT_F32, wsl.WSL_OUT_BF16])
def test_gemm_streamed_against_oracle(ofmt):
    import torch
    say(f"ring gemm ofmt={ofmt}")
    mats, dev, bits, nbytes = _stack(wsl.WSL_W_NF4)
    m = 32
    kmax = max(k for _, k in SHAPES)
    xbs = [synth.act_bits(106, 100 + i, (m, k)) for i, (_, k) in enumerate(SHAPES)]
    # one shared leading dimension: X rows padded to kmax, Y rows to the largest n_out
    nmax = max(n for n, _ in SHAPES)
    xp = [torch.zeros((m, kmax), dtype=torch.bfloat16, device="cuda") for _ in SHAPES]
    for a, b in zip(xp, xbs):
        a[:, :b.shape[1]] = to_dev_bf16(b)
    ws_bytes = max(wsl.linear_gemm_workspace_bytes(wsl.WSL_W_NF4, n, k, m) for n, k in SHAPES)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    want = [wsl.linear_gemm(d, a[:, :k], wfmt=wsl.WSL_W_NF4, n_out=n, k=k, ofmt=ofmt, workspace=ws)
            for d, a, (n, k) in zip(dev, xp, SHAPES)]
    ydt = torch.float32 if ofmt == wsl.WSL_OUT_F32 else torch.bfloat16
    ys = [torch.full((m, nmax), float("nan"), dtype=ydt, device="cuda") for _ in SHAPES]
    ring = wsl.CopyRing(nbytes)
    ring.gemm(mats, xp, ys, m, kmax, nmax, ofmt=ofmt, workspace=ws)
    torch.cuda.synchronize()
    for i, ((n, k), y, w, wb, xb) in enumerate(zip(SHAPES, ys, want, bits, xbs)):
        codes, scales = oracle.pack_codes(f64(wb))
        t = oracle.f32_from_bf16_bits(oracle.dequant_tile_bits(codes, scales)).astype(np.float64)
        y_ref, s_ref = oracle.gemm_ref(f64(xb), t)
        if ofmt == wsl.WSL_OUT_F32:
            ok, worst, r = oracle.check_rows_f32(y[:, :n].cpu().numpy(), y_ref, s_ref)
        else:
            yb = y[:, :n].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
            ok, worst, r = oracle.check_bf16(yb, y_ref, s_ref)
        assert ok, f"matrix {i} {(n, k)}: element {r} worst ratio {worst}"
        assert torch.equal(y[:, :n], w), f"matrix {i} differs from the resident call"
    # columns past each matrix's n_out are not written
    for (n, _), y in zip(SHAPES, ys):
        assert bool(torch.isnan(y[:, n:].float()).all())


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
                       wsl._ptr_array([ev.cuda_event for ev in ring.events]), 0)
        wsl._check(rc, "linear_gemv_streamed")
    assert e.value.code == 8
    # the refused call left no pending error behind: a normal call still works
    wsl.linear_gemv(p, x, y=y, wfmt=wsl.WSL_W_NF4, n_out=n, k=k)
    torch.cuda.synchronize()
