"""linear_gemm on the GPU against the fp64 CPU oracle.

NF4: the reference multiplies the restored bf16 tile T = bf16(fp32(c * s)); bf16:
the weight as stored.  fp32 output: |Y - Y_ref| <= 1e-4 * S elementwise; bf16 output:
one more bf16 ulp of |Y_ref|.  The full prefill and batch-verification shapes are checked
on sampled rows and columns, including tile edges.
"""

import numpy as np
import pytest

import oracle
import synth
import weight_streaming_linear_amd as wsl
from gpu_common import to_dev_bf16, bits_of, f64, say

pytestmark = pytest.mark.gpu


def _tile_f64(wb):
    codes, scales = oracle.pack_codes(f64(wb))
    return f64(oracle.dequant_tile_bits(codes, scales))


def _check(y_dev, y_ref, s_ref, ofmt):
    if ofmt == wsl.WSL_OUT_F32:
        return oracle.check_rows_f32(y_dev.cpu().numpy(), y_ref, s_ref)
    return oracle.check_bf16(bits_of(y_dev), y_ref, s_ref)


# k % 256 == 0 with m <= 32 takes the shared-X kernel (ragged row counts, one chunk, many
# splits, m < 32); the others the general kernel.
@pytest.mark.parametrize("m,n_out,k", [(5, 100, 192), (32, 96, 640), (70, 33, 128), (130, 160, 256), (1, 32, 64),
                                       (32, 1000, 5120), (7, 300, 512), (32, 257, 1024), (1, 16, 256),
                                       (19, 4109, 2304), (33, 64, 512)])
@pytest.mark.parametrize("ofmt", [wsl.WSL_OUT_F32, wsl.WSL_OUT_BF16])
@pytest.mark.parametrize("use_ws", [False, True])
def test_gemm_nf4_small(m, n_out, k, ofmt, use_ws):
    import torch
    say(f"gemm nf4 m={m} n={n_out} k={k} ofmt={ofmt} ws={use_ws}")
    wb = synth.weight_bits(97, n_out, n_out, k)
    xb = synth.act_bits(97, 1000 + m, (m, k))
    packed = wsl.nf4_pack(to_dev_bf16(wb))
    ws = None
    if use_ws:
        nb = wsl.linear_gemm_workspace_bytes(wsl.WSL_W_NF4, n_out, k, m)
        ws = torch.full((max(nb, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    y = wsl.linear_gemm(packed, to_dev_bf16(xb), wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k, ofmt=ofmt, workspace=ws)
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.gemm_ref(f64(xb), _tile_f64(wb))
    ok, worst, i = _check(y, y_ref, s_ref, ofmt)
    assert ok, f"elem {i}: worst ratio {worst}"


# At least 192 blocks of 128 rows: the shared-X kernel in its 128-row form (two waves per
# 32-row group, k-steps split between them) without a k split -- a partial last block,
# m < 32, a single 256-k chunk, and both output formats.
@pytest.mark.parametrize("m,n_out,k", [(32, 24576 + 67, 512), (7, 24700, 256), (32, 24576, 768)])
@pytest.mark.parametrize("ofmt", [wsl.WSL_OUT_F32, wsl.WSL_OUT_BF16])
def test_gemm_nf4_tall_m32(m, n_out, k, ofmt):
    import torch
    say(f"gemm nf4 tall m={m} n={n_out} k={k} ofmt={ofmt}")
    assert wsl.linear_gemm_workspace_bytes(wsl.WSL_W_NF4, n_out, k, m) == 0
    wb = synth.weight_bits(98, n_out, n_out, k)
    xb = synth.act_bits(98, 1000 + m, (m, k))
    packed = wsl.nf4_pack(to_dev_bf16(wb))
    y = wsl.linear_gemm(packed, to_dev_bf16(xb), wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k, ofmt=ofmt)
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.gemm_ref(f64(xb), _tile_f64(wb))
    ok, worst, i = _check(y, y_ref, s_ref, ofmt)
    assert ok, f"elem {i}: worst ratio {worst}"


@pytest.mark.parametrize("m,n_out,k", [(5, 100, 192), (130, 200, 320), (128, 128, 64), (257, 129, 576), (1, 8, 64)])
@pytest.mark.parametrize("ofmt", [wsl.WSL_OUT_F32, wsl.WSL_OUT_BF16])
def test_gemm_bf16_small(m, n_out, k, ofmt):
    import torch
    say(f"gemm bf16 m={m} n={n_out} k={k} ofmt={ofmt}")
    wb = synth.weight_bits(98, n_out, n_out, k)
    xb = synth.act_bits(98, 1000 + m, (m, k))
    y = wsl.linear_gemm(to_dev_bf16(wb), to_dev_bf16(xb), ofmt=ofmt)
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.gemm_ref(f64(xb), f64(wb))
    ok, worst, i = _check(y, y_ref, s_ref, ofmt)
    assert ok, f"elem {i}: worst ratio {worst}"


# bf16 with k % 256 == 0 where the shared-X kernel runs (M <= 32, and larger M where the
# launch's time model prefers it to the tiles; weights loaded straight into MFMA B
# fragments) -- m < 32, one and two position groups, ragged row counts, a tall matrix
# without a k split, many k splits with and without a workspace, and several position
# blocks on matrices with few rows (M = 65 to 300).  The last two cases (tall matrices,
# M = 96 and 160) are where the model picks the tiled kernel.
@pytest.mark.parametrize("m,n_out,k", [(1, 16, 256), (7, 4109, 2304), (32, 1000, 512), (48, 300, 768),
                                       (64, 24700, 256), (33, 160, 5120), (65, 257, 1024), (130, 257, 1024),
                                       (200, 333, 2048), (300, 512, 4096), (96, 27648, 256), (160, 17500, 512)])
@pytest.mark.parametrize("ofmt", [wsl.WSL_OUT_F32, wsl.WSL_OUT_BF16])
@pytest.mark.parametrize("use_ws", [False, True])
def test_gemm_bf16_shared_x(m, n_out, k, ofmt, use_ws):
    import torch
    say(f"gemm bf16 shared-x m={m} n={n_out} k={k} ofmt={ofmt} ws={use_ws}")
    wb = synth.weight_bits(96, n_out, n_out, k)
    xb = synth.act_bits(96, 1000 + m, (m, k))
    ws = None
    if use_ws:
        nb = wsl.linear_gemm_workspace_bytes(wsl.WSL_W_BF16, n_out, k, m)
        ws = torch.full((max(nb, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    y = wsl.linear_gemm(to_dev_bf16(wb), to_dev_bf16(xb), wfmt=wsl.WSL_W_BF16, ofmt=ofmt, workspace=ws)
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.gemm_ref(f64(xb), f64(wb))
    ok, worst, i = _check(y, y_ref, s_ref, ofmt)
    assert ok, f"elem {i}: worst ratio {worst}"


@pytest.mark.parametrize("m,k", [(40, 192), (20, 512)])
def test_gemm_strided_x_and_y(m, k):
    """Leading dimensions larger than the logical widths."""
    import torch
    n_out = 72
    wb = synth.weight_bits(99, 0, n_out, k)
    xb = synth.act_bits(99, 1, (m, k + 16))
    x = to_dev_bf16(xb)[:, :k]
    y = torch.full((m, n_out + 8), float("nan"), dtype=torch.float32, device="cuda")
    wsl.linear_gemm(to_dev_bf16(wb), x, y=y[:, :n_out])
    packed = wsl.nf4_pack(to_dev_bf16(wb))
    y2 = torch.full((m, n_out + 8), float("nan"), dtype=torch.float32, device="cuda")
    wsl.linear_gemm(packed, x, y=y2[:, :n_out], wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k)
    torch.cuda.synchronize()
    xf = f64(xb)[:, :k]
    y_ref, s_ref = oracle.gemm_ref(xf, f64(wb))
    assert oracle.check_rows_f32(y[:, :n_out].cpu().numpy(), y_ref, s_ref)[0]
    assert torch.isnan(y[:, n_out:]).all()
    y_ref2, s_ref2 = oracle.gemm_ref(xf, _tile_f64(wb))
    assert oracle.check_rows_f32(y2[:, :n_out].cpu().numpy(), y_ref2, s_ref2)[0]
    assert torch.isnan(y2[:, n_out:]).all()


@pytest.mark.parametrize("j,k", [(0, 192), (31, 192), (32, 192), (63, 192), (191, 192), (0, 512), (127, 512),
                                 (128, 512), (255, 512), (300, 512), (511, 512)])
def test_gemm_one_hot_restores_tile_column(j, k):
    """A one-hot row of X picks column j of the bf16 tile exactly (NF4) / of W (bf16).  k = 512
    runs the shared-X kernel, whose lanes take 128-code runs in a permuted k order."""
    import torch
    m, n_out = 3, 96
    wb = synth.weight_bits(100, 0, n_out, k)
    x = np.zeros((m, k), np.float32)
    x[1, j] = 1.0
    x[2, j] = -2.0
    xb = oracle.bf16_bits_from_f32(x)
    packed = wsl.nf4_pack(to_dev_bf16(wb))
    y = wsl.linear_gemm(packed, to_dev_bf16(xb), wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k)
    yb = wsl.linear_gemm(to_dev_bf16(wb), to_dev_bf16(xb))
    torch.cuda.synchronize()
    t = _tile_f64(wb)
    got = y.cpu().numpy()
    assert np.all(got[0] == 0)
    assert np.array_equal(got[1].astype(np.float64), t[:, j])
    assert np.array_equal(got[2].astype(np.float64), -2.0 * t[:, j])
    assert np.array_equal(yb.cpu().numpy()[1].astype(np.float64), f64(wb)[:, j])


def _sample_idx(n, tile, rng, count):
    edges = [0, n - 1] + [v for t in range(tile, n, tile) for v in (t - 1, t)][:16]
    return np.unique(np.concatenate([np.array(edges), rng.integers(0, n, count)]))


# NF4 prefill GEMM, 32 positions, 32B-class FFN (up 5120 -> 27648, down 27648 -> 5120).
@pytest.mark.parametrize("n_out,k,tid", [(27648, 5120, 0), (5120, 27648, 1)])
def test_gemm_nf4_prefill_m32_full_shape_sampled(n_out, k, tid):
    import torch
    say(f"gemm nf4 prefill m=32 {n_out}x{k}")
    m = 32
    wb = synth.weight_bits(3, tid, n_out, k)
    xb = synth.act_bits(3, 2 + tid, (m, k))
    w_dev = to_dev_bf16(wb)
    packed = wsl.nf4_pack(w_dev)
    del w_dev
    nb = wsl.linear_gemm_workspace_bytes(wsl.WSL_W_NF4, n_out, k, m)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
    y = wsl.linear_gemm(packed, to_dev_bf16(xb), wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k, workspace=ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(41 + tid)
    cols = _sample_idx(n_out, 128, rng, 200)
    # packed bytes of the sampled rows are bit-exact
    cb, sc = oracle.canonical_from_device(packed.cpu().numpy(), n_out, k)
    codes, scales = oracle.pack_codes(f64(wb[cols]))
    assert np.array_equal(cb[cols], oracle.codes_to_bytes(codes))
    assert np.array_equal(sc[cols].view(np.uint16), scales.view(np.uint16))
    t = f64(oracle.dequant_tile_bits(codes, scales))
    y_ref, s_ref = oracle.gemm_ref(f64(xb), t)
    ok, worst, i = oracle.check_rows_f32(y.cpu().numpy()[:, cols], y_ref, s_ref)
    assert ok, f"elem {i}: worst ratio {worst}"


# NF4 prefill chunks of more than 32 positions on the 32B-class up projection (5120 -> 27648):
# M = 64 and 128 take the shared-X kernel (two position groups per workgroup, 1 and 2 position
# blocks), M = 256 the tiled kernel, as the launch's time model decides for this shape.
@pytest.mark.parametrize("m", [64, 128, 256])
def test_gemm_nf4_up_27648x5120_mid_m_sampled(m):
    import torch
    say(f"gemm nf4 up 27648x5120 m={m}")
    n_out, k = 27648, 5120
    wb = synth.weight_bits(3, 700, n_out, k)
    xb = synth.act_bits(3, 40 + m, (m, k))
    w_dev = to_dev_bf16(wb)
    packed = wsl.nf4_pack(w_dev)
    del w_dev
    nb = wsl.linear_gemm_workspace_bytes(wsl.WSL_W_NF4, n_out, k, m)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
    y = wsl.linear_gemm(packed, to_dev_bf16(xb), wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k, workspace=ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(71 + m)
    cols = _sample_idx(n_out, 128, rng, 160)
    y_ref, s_ref = oracle.gemm_ref(f64(xb), _tile_f64(wb[cols]))
    ok, worst, i = oracle.check_rows_f32(y.cpu().numpy()[:, cols], y_ref, s_ref)
    assert ok, f"elem {i}: worst ratio {worst}"


def test_binding_refuses_misread_tensors():
    """The binding refuses what the C ABI would read as something else: a transposed X, an
    fp32 X, a non-contiguous bf16 weight, an output of the wrong type, a short packed buffer."""
    import torch
    n_out, k, m = 64, 256, 8
    w = to_dev_bf16(synth.weight_bits(110, 0, n_out, k))
    packed = wsl.nf4_pack(w)
    x = to_dev_bf16(synth.act_bits(110, 1, (m, k)))
    bad = [
        lambda: wsl.linear_gemm(w, x.t().contiguous().t()),                        # column-major view
        lambda: wsl.linear_gemm(w, x.float()),                                     # fp32 activations
        lambda: wsl.linear_gemm(torch.cat([w, w], 1)[:, ::2], x),                  # strided weight
        lambda: wsl.linear_gemm(w, x, y=torch.empty((m, n_out), dtype=torch.float16, device="cuda")),
        lambda: wsl.linear_gemv(packed[:-1], x[0], wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k),
        lambda: wsl.linear_gemv(w, x[0].float()),
        lambda: wsl.linear_gemv(w, x[:, 0]),                                       # strided vector
        lambda: wsl.nf4_pack(w.t()),
    ]
    for i, f in enumerate(bad):
        with pytest.raises(ValueError):
            f()
    torch.cuda.synchronize()


# The tiled bf16 kernel runs one workgroup per CU; an XCD whose last round would leave at
# least half its 32 CUs idle runs those tiles as two 128-row halves.  264 tiles of 256 x 256
# give each XCD 33: 32 whole tiles and one split; 36 tiles split every one (every output
# element checked).
@pytest.mark.parametrize("m,n_out,k", [(2048, 8448, 64), (1536, 1536, 128), (2000, 8400, 192)])
def test_gemm_bf16_tiled_tail_halves(m, n_out, k):
    import torch
    say(f"gemm bf16 tiled tail m={m} n={n_out} k={k}")
    wb = synth.weight_bits(93, 0, n_out, k)
    xb = synth.act_bits(93, 1, (m, k))
    y = wsl.linear_gemm(to_dev_bf16(wb), to_dev_bf16(xb), ofmt=wsl.WSL_OUT_BF16)
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.gemm_ref(f64(xb), f64(wb))
    ok, worst, i = oracle.check_bf16(bits_of(y), y_ref, s_ref)
    assert ok, f"elem {i}: worst ratio {worst}"


# The tiled NF4 kernel splits the tiles of a short last round the same way (k = 64, 192: not
# multiples of 256, so M > 32 takes the tiled kernel; 2048 x 8448 and 2000 x 8400 mix whole
# tiles with halves, 1536 x 1536 runs halves only).
@pytest.mark.parametrize("m,n_out,k", [(2048, 8448, 64), (1536, 1536, 128), (2000, 8400, 192)])
def test_gemm_nf4_tiled_tail_halves(m, n_out, k):
    import torch
    say(f"gemm nf4 tiled tail m={m} n={n_out} k={k}")
    wb = synth.weight_bits(92, 0, n_out, k)
    xb = synth.act_bits(92, 1, (m, k))
    packed = wsl.nf4_pack(to_dev_bf16(wb))
    y = wsl.linear_gemm(packed, to_dev_bf16(xb), wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k, ofmt=wsl.WSL_OUT_F32)
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.gemm_ref(f64(xb), _tile_f64(wb))
    ok, worst, i = _check(y, y_ref, s_ref, wsl.WSL_OUT_F32)
    assert ok, f"elem {i}: worst ratio {worst}"


# bf16 batch verification, M = 8192 positions, gate (5120 -> 17408) and down (17408 -> 5120).
@pytest.mark.parametrize("n_out,k,tid", [(17408, 5120, 0), (5120, 17408, 1)])
def test_gemm_bf16_verify_m8192_full_shape_sampled(n_out, k, tid):
    import torch
    say(f"gemm bf16 verify m=8192 {n_out}x{k}")
    m = 8192
    wb = synth.weight_bits(4, tid, n_out, k)
    xb = synth.act_bits(4, 2 + tid, (m, k))
    y = wsl.linear_gemm(to_dev_bf16(wb), to_dev_bf16(xb), ofmt=wsl.WSL_OUT_BF16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(43 + tid)
    rows = _sample_idx(m, 128, rng, 48)
    cols = _sample_idx(n_out, 128, rng, 160)
    y_ref, s_ref = oracle.gemm_ref(f64(xb[rows]), f64(wb[cols]))
    got = bits_of(y)[np.ix_(rows, cols)]
    ok, worst, i = oracle.check_bf16(got, y_ref, s_ref)
    assert ok, f"elem {i}: worst ratio {worst}"


# NF4 batch verification (M = 8192) on the gate and down shapes: the tiled NF4 kernel.
@pytest.mark.parametrize("n_out,k,tid", [(17408, 5120, 0), (5120, 17408, 1)])
def test_gemm_nf4_verify_m8192_full_shape_sampled(n_out, k, tid):
    import torch
    say(f"gemm nf4 verify m=8192 {n_out}x{k}")
    m = 8192
    wb = synth.weight_bits(108, tid, n_out, k)
    xb = synth.act_bits(108, 2 + tid, (m, k))
    w_dev = to_dev_bf16(wb)
    packed = wsl.nf4_pack(w_dev)
    del w_dev
    y = wsl.linear_gemm(packed, to_dev_bf16(xb), wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k, ofmt=wsl.WSL_OUT_BF16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(47 + tid)
    rows = _sample_idx(m, 256, rng, 40)
    cols = _sample_idx(n_out, 256, rng, 120)
    y_ref, s_ref = oracle.gemm_ref(f64(xb[rows]), _tile_f64(wb[cols]))
    ok, worst, i = oracle.check_bf16(bits_of(y)[np.ix_(rows, cols)], y_ref, s_ref)
    assert ok, f"elem {i}: worst ratio {worst}"


# M > 32 with k % 256 == 0 where the shared-X kernel is the faster one (the launch compares
# a time model of both kernels): two 32-position groups per workgroup and position blocks
# on grid z -- M not a multiple of 32 or 64, ragged row counts, tall matrices without a k
# split, one to sixteen position blocks (M up to 1000 on matrices with few rows, where the
# 256 x 256 tiles would leave most CUs idle).
@pytest.mark.parametrize("m,n_out,k", [(33, 257, 512), (48, 1000, 768), (130, 4109, 2304), (200, 160, 5120),
                                       (257, 130, 2048), (300, 1000, 1024), (333, 300, 2048), (320, 512, 8192),
                                       (1000, 256, 4096)])
@pytest.mark.parametrize("ofmt", [wsl.WSL_OUT_F32, wsl.WSL_OUT_BF16])
def test_gemm_nf4_mid_m_shared_x(m, n_out, k, ofmt):
    import torch
    say(f"gemm nf4 mid m={m} n={n_out} k={k} ofmt={ofmt}")
    wb = synth.weight_bits(99, n_out, n_out, k)
    xb = synth.act_bits(99, 1000 + m, (m, k))
    packed = wsl.nf4_pack(to_dev_bf16(wb))
    nb = wsl.linear_gemm_workspace_bytes(wsl.WSL_W_NF4, n_out, k, m)
    ws = torch.full((max(nb, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    y = wsl.linear_gemm(packed, to_dev_bf16(xb), wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k, ofmt=ofmt, workspace=ws)
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.gemm_ref(f64(xb), _tile_f64(wb))
    ok, worst, i = _check(y, y_ref, s_ref, ofmt)
    assert ok, f"elem {i}: worst ratio {worst}"


# M > 32 with k % 256 != 0, or where the time model prefers 256 x 256 tiles (many rows and
# positions, short k): the tiled kernel.
@pytest.mark.parametrize("m,n_out,k", [(64, 300, 448), (513, 260, 64), (256, 24700, 256), (1024, 8192, 512)])
@pytest.mark.parametrize("ofmt", [wsl.WSL_OUT_F32, wsl.WSL_OUT_BF16])
def test_gemm_nf4_tiled_mid_m(m, n_out, k, ofmt):
    import torch
    say(f"gemm nf4 tiled m={m} n={n_out} k={k} ofmt={ofmt}")
    wb = synth.weight_bits(109, n_out, n_out, k)
    xb = synth.act_bits(109, 1000 + m, (m, k))
    packed = wsl.nf4_pack(to_dev_bf16(wb))
    y = wsl.linear_gemm(packed, to_dev_bf16(xb), wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k, ofmt=ofmt)
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.gemm_ref(f64(xb), _tile_f64(wb))
    ok, worst, i = _check(y, y_ref, s_ref, ofmt)
    assert ok, f"elem {i}: worst ratio {worst}"


# A k split of the tiled kernels: a launch whose 256 x 256 tiles would leave most CUs idle
# runs one work item per (tile, k range), the fp32 partials summed in split order (the
# workspace size names the split: a multiple of M * N * 4 bytes); with M <= 128 the items
# are 128-row half tiles (M = 65, 100).  Ragged M and N, a last k range shorter than the
# others; the same call without a workspace runs unsplit.  bf16: every element against the
# oracle; NF4: all rows, sampled columns with the tile edges.
@pytest.mark.parametrize("wfmt,m,n_out,k", [(wsl.WSL_W_BF16, 513, 777, 12288), (wsl.WSL_W_BF16, 257, 3000, 7680),
                                            (wsl.WSL_W_BF16, 65, 4100, 6144), (wsl.WSL_W_NF4, 1000, 2100, 8192),
                                            (wsl.WSL_W_NF4, 513, 4100, 12288), (wsl.WSL_W_NF4, 100, 6000, 12288)])
@pytest.mark.parametrize("ofmt", [wsl.WSL_OUT_F32, wsl.WSL_OUT_BF16])
def test_gemm_tiled_k_split(wfmt, m, n_out, k, ofmt):
    import torch
    say(f"gemm tiled k split wfmt={wfmt} m={m} n={n_out} k={k} ofmt={ofmt}")
    nb = wsl.linear_gemm_workspace_bytes(wfmt, n_out, k, m)
    assert nb > 0 and nb % (m * n_out * 4) == 0 and nb // (m * n_out * 4) >= 2, nb
    wb = synth.weight_bits(111, n_out, n_out, k)
    xb = synth.act_bits(111, 1000 + m, (m, k))
    w = wsl.nf4_pack(to_dev_bf16(wb)) if wfmt == wsl.WSL_W_NF4 else to_dev_bf16(wb)
    x = to_dev_bf16(xb)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    y_split = wsl.linear_gemm(w, x, wfmt=wfmt, n_out=n_out, k=k, ofmt=ofmt, workspace=ws)
    y_whole = wsl.linear_gemm(w, x, wfmt=wfmt, n_out=n_out, k=k, ofmt=ofmt)
    torch.cuda.synchronize()
    if wfmt == wsl.WSL_W_BF16:
        cols = np.arange(n_out)
        t = f64(wb)
    else:
        cols = _sample_idx(n_out, 256, np.random.default_rng(113 + m), 160)
        t = _tile_f64(wb[cols])
    y_ref, s_ref = oracle.gemm_ref(f64(xb), t)
    for name, y in (("split", y_split), ("unsplit", y_whole)):
        ok, worst, i = _check(y[:, cols], y_ref, s_ref, ofmt)
        assert ok, f"{name}: elem {i}: worst ratio {worst}"


# linear_gemm_noalloc on a shape whose tiled k split would need more than the library's
# scratch: it runs the tiled kernels unsplit (no WSL_E_SCRATCH), bit for bit what
# linear_gemm computes without a workspace.
def test_gemm_noalloc_tiled_runs_unsplit_beyond_scratch():
    import torch
    m, n_out, k = 1000, 2100, 8192
    say(f"gemm noalloc tiled m={m} n={n_out} k={k}")
    assert wsl.linear_gemm_workspace_bytes(wsl.WSL_W_BF16, n_out, k, m) > wsl.NOALLOC_SCRATCH_BYTES
    wb = synth.weight_bits(112, 0, n_out, k)
    xb = synth.act_bits(112, 1, (m, k))
    w, x = to_dev_bf16(wb), to_dev_bf16(xb)
    y = torch.full((m, n_out), float("nan"), dtype=torch.float32, device="cuda")
    wsl.linear_gemm_noalloc(w, x, y)
    y_whole = wsl.linear_gemm(w, x)
    torch.cuda.synchronize()
    assert torch.equal(y, y_whole)
    cols = _sample_idx(n_out, 256, np.random.default_rng(114), 64)
    y_ref, s_ref = oracle.gemm_ref(f64(xb), f64(wb[cols]))
    ok, worst, i = oracle.check_rows_f32(y.cpu().numpy()[:, cols], y_ref, s_ref)
    assert ok, f"elem {i}: worst ratio {worst}"


def test_gemm_deterministic():
    import torch
    m, n_out, k = 32, 5120, 27648 // 4
    wb = synth.weight_bits(101, 0, n_out, k)
    xb = synth.act_bits(101, 1, (m, k))
    packed = wsl.nf4_pack(to_dev_bf16(wb))
    x = to_dev_bf16(xb)
    nb = wsl.linear_gemm_workspace_bytes(wsl.WSL_W_NF4, n_out, k, m)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
    a = wsl.linear_gemm(packed, x, wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k, workspace=ws)
    b = wsl.linear_gemm(packed, x, wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k, workspace=ws)
    c = wsl.linear_gemm(to_dev_bf16(wb), x)
    d = wsl.linear_gemm(to_dev_bf16(wb), x)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(c, d)


# A captured linear_gemm replays to the eager result: the shared-X kernels with a k split
# (workspace + reduction kernel) and the tiled kernels, unsplit and split.  Each replay follows eager work of
# the program's own and a synchronization, with the output poisoned first.
@pytest.mark.parametrize("wfmt,m,n_out,k", [(wsl.WSL_W_NF4, 32, 640, 16384), (wsl.WSL_W_NF4, 300, 1000, 448),
                                            (wsl.WSL_W_BF16, 200, 700, 1024), (wsl.WSL_W_BF16, 200, 700, 1088),
                                            (wsl.WSL_W_BF16, 513, 777, 12288)])
def test_gemm_graph_replays_match_eager(wfmt, m, n_out, k):
    import torch
    say(f"gemm graph wfmt={wfmt} m={m} n={n_out} k={k}")
    wb = synth.weight_bits(91, n_out, n_out, k)
    xb = synth.act_bits(91, 1000 + m, (m, k))
    w = wsl.nf4_pack(to_dev_bf16(wb)) if wfmt == wsl.WSL_W_NF4 else to_dev_bf16(wb)
    x = to_dev_bf16(xb)
    nb = wsl.linear_gemm_workspace_bytes(wfmt, n_out, k, m)
    ws = torch.zeros((max(nb, 16) // 4,), dtype=torch.float32, device="cuda")
    y_eager = wsl.linear_gemm(w, x, wfmt=wfmt, n_out=n_out, k=k, workspace=ws)
    yg = torch.empty_like(y_eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        wsl.linear_gemm(w, x, y=yg, wfmt=wfmt, n_out=n_out, k=k, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        wsl.linear_gemm(w, x, y=yg, wfmt=wfmt, n_out=n_out, k=k, workspace=ws)
    torch.cuda.synchronize()
    for r in range(3):
        yg.fill_(float("nan"))
        ws.fill_(float("nan"))
        scratch = torch.randn(4096, device="cuda").sum()   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(yg, y_eager), f"replay {r}"
    assert torch.isfinite(scratch)
    y_ref, s_ref = oracle.gemm_ref(f64(xb), _tile_f64(wb) if wfmt == wsl.WSL_W_NF4 else f64(wb))
    ok, worst, i = _check(y_eager, y_ref, s_ref, wsl.WSL_OUT_F32)
    assert ok, f"elem {i}: worst ratio {worst}"
