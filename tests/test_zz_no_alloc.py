"""linear_gemm_noalloc: linear_gemm with its split partials in the library's per-device
scratch instead of a caller workspace, for callers that cannot allocate (graph capture,
serving loops).  Checked through the C ABI against linear_gemm with a workspace (bit for
bit: same kernels, same splits) and against the fp64 oracle, on consecutive calls whose
second input is smaller, so the second call runs on scratch the first one left behind."""

import gc

import numpy as np
import pytest

import oracle
import synth
import weight_streaming_linear_amd as wsl
from gpu_common import to_dev_bf16, bits_of, f64, say

pytestmark = pytest.mark.gpu


def _nf4_case(tid, m, n_out, k):
    wb = synth.weight_bits(111, tid, n_out, k)
    xb = synth.act_bits(111, 100 + tid, (m, k))
    return wb, xb, wsl.nf4_pack(to_dev_bf16(wb)), to_dev_bf16(xb)


def _with_workspace(w, x, n_out, k, wfmt, ofmt):
    import torch
    nb = wsl.linear_gemm_workspace_bytes(wfmt, n_out, k, x.shape[0])
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
    return wsl.linear_gemm(w, x, wfmt=wfmt, n_out=n_out, k=k, ofmt=ofmt, workspace=ws), nb


def _check_oracle(y, xb, t64, cols, ofmt):
    y_ref, s_ref = oracle.gemm_ref(f64(xb), t64)
    if ofmt == wsl.WSL_OUT_F32:
        ok, worst, i = oracle.check_rows_f32(y.cpu().numpy()[:, cols], y_ref, s_ref)
    else:
        ok, worst, i = oracle.check_bf16(bits_of(y)[:, cols], y_ref, s_ref)
    assert ok, f"element {i}: worst ratio {worst}"


@pytest.mark.parametrize("ofmt", [wsl.WSL_OUT_F32, wsl.WSL_OUT_BF16])
def test_noalloc_nf4_two_calls_second_smaller(ofmt):
    """The 32B-class prefill down projection (6 k splits, 3.9 MB of partials), then a smaller
    split shape on the same scratch."""
    import torch
    dt = torch.float32 if ofmt == wsl.WSL_OUT_F32 else torch.bfloat16
    for tid, (m, n_out, k) in enumerate([(32, 5120, 27648), (16, 640, 4096)]):
        say(f"noalloc nf4 m={m} {n_out}x{k} ofmt={ofmt}")
        wb, xb, packed, x = _nf4_case(tid, m, n_out, k)
        want, nb = _with_workspace(packed, x, n_out, k, wsl.WSL_W_NF4, ofmt)
        assert 0 < nb <= wsl.NOALLOC_SCRATCH_BYTES, "the case must use split partials"
        y = torch.full((m, n_out), float("nan"), dtype=dt, device="cuda")
        wsl.linear_gemm_noalloc(packed, x, y, wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k, ofmt=ofmt)
        torch.cuda.synchronize()
        assert torch.equal(y, want), "differs from linear_gemm with a caller workspace"
        cols = np.unique(np.concatenate([[0, n_out - 1], np.random.default_rng(tid).integers(0, n_out, 96)]))
        codes, scales = oracle.pack_codes(f64(wb[cols]))
        _check_oracle(y, xb, f64(oracle.dequant_tile_bits(codes, scales)), cols, ofmt)


def test_noalloc_bf16_two_calls_second_smaller():
    import torch
    for tid, (m, n_out, k) in enumerate([(32, 1000, 8192), (8, 300, 2048)]):
        say(f"noalloc bf16 m={m} {n_out}x{k}")
        wb = synth.weight_bits(112, tid, n_out, k)
        xb = synth.act_bits(112, 100 + tid, (m, k))
        w, x = to_dev_bf16(wb), to_dev_bf16(xb)
        want, nb = _with_workspace(w, x, n_out, k, wsl.WSL_W_BF16, wsl.WSL_OUT_F32)
        assert 0 < nb <= wsl.NOALLOC_SCRATCH_BYTES
        y = torch.full((m, n_out), float("nan"), dtype=torch.float32, device="cuda")
        wsl.linear_gemm_noalloc(w, x, y)
        torch.cuda.synchronize()
        assert torch.equal(y, want)
        _check_oracle(y, xb, f64(wb), np.arange(n_out), wsl.WSL_OUT_F32)


def test_noalloc_rejects_a_shape_beyond_its_scratch():
    """5120x27648 at 64 positions needs 7.9 MB of partials: refused, nothing launched."""
    import torch
    m, n_out, k = 64, 5120, 27648
    assert wsl.linear_gemm_workspace_bytes(wsl.WSL_W_NF4, n_out, k, m) > wsl.NOALLOC_SCRATCH_BYTES
    _, _, packed, x = _nf4_case(3, m, n_out, k)
    y = torch.full((m, n_out), float("nan"), dtype=torch.float32, device="cuda")
    with pytest.raises(wsl.WSLError) as e:
        wsl.linear_gemm_noalloc(packed, x, y, wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k)
    assert e.value.code == wsl.WSL_E_SCRATCH
    torch.cuda.synchronize()
    assert bool(torch.isnan(y).all())


def test_noalloc_under_graph_capture():
    """Captured with no allocation inside; replays (with eager work and a synchronization
    between them) give the eager result."""
    import torch
    m, n_out, k = 32, 5120, 27648
    _, _, packed, x = _nf4_case(0, m, n_out, k)
    want = torch.empty((m, n_out), dtype=torch.float32, device="cuda")
    wsl.linear_gemm_noalloc(packed, x, want, wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k)
    y = torch.empty_like(want)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        wsl.linear_gemm_noalloc(packed, x, y, wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    gc.collect()
    allocs = lambda: torch.cuda.memory_stats().get("allocation.all.allocated", 0)   # requests so far
    with torch.cuda.graph(g):
        # (beginning a capture allocates torch's own bookkeeping, so count around the call;
        # requests, not bytes: a Python object freed meanwhile must not hide an allocation)
        before = allocs()
        wsl.linear_gemm_noalloc(packed, x, y, wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k)
        requested = allocs() - before
    torch.cuda.synchronize()
    assert requested == 0
    for _ in range(3):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, want)
