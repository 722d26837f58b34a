"""linear_gemv on the GPU against the fp64 CPU oracle.

Tolerance (per row): |y - y_ref| <= 1e-4 * sum_j |w_hat_ij x_j|, with w_hat the
exact dequantized weight c * s (NF4) or the bf16 weight.  Exact special cases
(small integers, one-hot x, power-of-two scaling) must match bit for bit.
"""

import numpy as np
import pytest

import oracle
import synth
import weight_streaming_linear_amd as wsl
from gpu_common import to_dev_bf16, to_dev_u8, f64, say

pytestmark = pytest.mark.gpu


def _nf4_case(n_out, k, stream, tid_w, tid_x):
    import torch
    wb = synth.weight_bits(stream, tid_w, n_out, k)
    xb = synth.act_bits(stream, tid_x, (k,))
    packed = wsl.nf4_pack(to_dev_bf16(wb))
    y = wsl.linear_gemv(packed, to_dev_bf16(xb), wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k)
    torch.cuda.synchronize()
    codes, scales = oracle.pack_codes(f64(wb))
    y_ref, s_ref = oracle.gemv_ref(oracle.dequant_exact(codes, scales), f64(xb))
    return y.cpu().numpy(), y_ref, s_ref


@pytest.mark.parametrize("n_out,k", [(4096, 4096), (37, 192), (1, 64), (130, 2112), (257, 6144), (64, 16384),
                                     (9, 4160)])
def test_gemv_nf4_tolerance(n_out, k):
    say(f"gemv nf4 {n_out}x{k}")
    y, y_ref, s_ref = _nf4_case(n_out, k, 0 if (n_out, k) == (4096, 4096) else 94, 0, 1)
    ok, worst, i = oracle.check_rows_f32(y, y_ref, s_ref)
    assert ok, f"row {i}: worst ratio {worst}"


@pytest.mark.parametrize("n_out,k", [(4099, 2112), (37, 32832), (130, 40960), (20, 2048), (16, 64), (3073, 16384),
                                     (1029, 16384)])
def test_gemv_nf4_plan_edges(n_out, k):
    """Row counts that leave a partial 16-row block and row groups outside the pipelined
    loop; k > 32768 (several slices per wave); k = 2048 (one full slice).  3073x16384 and
    1029x16384: every workgroup runs an odd number of pipelined row groups without the
    parking flush, then a leftover round in which one team has no row (its partials must
    not overwrite those wave 0 is still summing)."""
    say(f"gemv nf4 {n_out}x{k}")
    y, y_ref, s_ref = _nf4_case(n_out, k, 97, 0, 1)
    ok, worst, i = oracle.check_rows_f32(y, y_ref, s_ref)
    assert ok, f"row {i}: worst ratio {worst}"


def _sample_rows(n, rng, count):
    edges = [0, 1, 2, 3, n - 4, n - 3, n - 2, n - 1] + [v for t in range(16, n, 16) for v in (t - 1, t)][:24]
    return np.unique(np.clip(np.concatenate([np.array(edges), rng.integers(0, n, count)]), 0, n - 1))


# Decode sweep with hidden size 6144: gate/up 6144 -> 32768, down 16384 -> 6144, qkv 6144 -> 8192,
# o 6144 -> 6144; plus ragged large shapes (odd row count, k not a multiple of 2048).  Matrices
# from 32 Mi weights take the pair-table kernel (from 96 Mi when k <= 4096: 28672x4096 does,
# 20000x2112 takes the 16-entry table).  With rows of at most three 2048-code slices the pair
# kernel refills each buffer before the workgroup barrier, with the last one, two or three
# super-groups of a workgroup written out: 8192x6144 gives each workgroup 4, 6144x6144 3,
# 28672x4096 7 and 32768x6144 16; 5700x6080 (712 super-groups on 256 workgroups, k not a
# multiple of 2048, 4 leftover rows) mixes workgroups of 2 and 3.
@pytest.mark.parametrize("n_out,k,tid", [(32768, 6144, 0), (6144, 16384, 1), (12291, 6208, 4), (8195, 6208, 2),
                                         (20000, 2112, 3), (8192, 6144, 5), (6144, 6144, 6), (28672, 4096, 7),
                                         (5700, 6080, 8)])
def test_gemv_nf4_large_sampled(n_out, k, tid):
    import torch
    say(f"gemv nf4 large {n_out}x{k}")
    wb = synth.weight_bits(98, tid, n_out, k)
    xb = synth.act_bits(98, 10 + tid, (k,))
    w_dev = to_dev_bf16(wb)
    packed = wsl.nf4_pack(w_dev)
    del w_dev
    y = wsl.linear_gemv(packed, to_dev_bf16(xb), wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k)
    torch.cuda.synchronize()
    rows = _sample_rows(n_out, np.random.default_rng(50 + tid), 120)
    codes, scales = oracle.pack_codes(f64(wb[rows]))
    y_ref, s_ref = oracle.gemv_ref(oracle.dequant_exact(codes, scales), f64(xb))
    ok, worst, i = oracle.check_rows_f32(y.cpu().numpy()[rows], y_ref, s_ref)
    assert ok, f"row {rows[i]}: worst ratio {worst}"


def _bf16_case(n_out, k, stream, tid_w, tid_x):
    import torch
    wb = synth.weight_bits(stream, tid_w, n_out, k)
    xb = synth.act_bits(stream, tid_x, (k,))
    y = wsl.linear_gemv(to_dev_bf16(wb), to_dev_bf16(xb))
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.gemv_ref(f64(wb), f64(xb))
    return y.cpu().numpy(), y_ref, s_ref


# One dense decoder layer with hidden size 5120: k/v 1024 rows, gate/up 17408 rows, down k = 17408;
# fused q/k/v 7168 rows and fused gate/up 34816 rows (every row of every shape is checked).
@pytest.mark.parametrize("n_out,k,tid", [(5120, 5120, 0), (1024, 5120, 1), (17408, 5120, 4), (5120, 17408, 6),
                                         (7168, 5120, 10), (34816, 5120, 15), (3, 8, 11), (5, 520, 12),
                                         (1, 4104, 13), (333, 1000, 14)])
def test_gemv_bf16_tolerance(n_out, k, tid):
    say(f"gemv bf16 {n_out}x{k}")
    y, y_ref, s_ref = _bf16_case(n_out, k, 1, tid, 100 + tid)
    ok, worst, i = oracle.check_rows_f32(y, y_ref, s_ref)
    assert ok, f"row {i}: worst ratio {worst}"


# Several bf16 GEMVs in one launch (linear_gemv_multi): a layer's q, k and v kept as separate
# matrices; ragged row counts with the most matrices one launch takes; a single matrix.  Each
# output against the oracle, and bit for bit what separate linear_gemv calls give.
@pytest.mark.parametrize("shapes", [[(5120, 5120), (1024, 5120), (1024, 5120)],
                                    [(17, 1032), (300, 1032), (1, 1032), (4099, 1032), (2, 1032), (64, 1032),
                                     (777, 1032), (5, 1032)],
                                    [(333, 17408)]])
def test_gemv_bf16_multi(shapes):
    import torch
    say(f"gemv bf16 multi {shapes}")
    wbs = [synth.weight_bits(117, i, n, k) for i, (n, k) in enumerate(shapes)]
    xbs = [synth.act_bits(117, 100 + i, (k,)) for i, (n, k) in enumerate(shapes)]
    ws_ = [to_dev_bf16(wb) for wb in wbs]
    xs = [to_dev_bf16(xb) for xb in xbs]
    ys = [torch.full((n,), float("nan"), dtype=torch.float32, device="cuda") for n, _ in shapes]
    wsl.linear_gemv_multi(list(zip(ws_, xs, ys)))
    single = [wsl.linear_gemv(w, x) for w, x in zip(ws_, xs)]
    torch.cuda.synchronize()
    for i, (y, y1, wb, xb) in enumerate(zip(ys, single, wbs, xbs)):
        y_ref, s_ref = oracle.gemv_ref(f64(wb), f64(xb))
        ok, worst, r = oracle.check_rows_f32(y.cpu().numpy(), y_ref, s_ref)
        assert ok, f"matrix {i} {shapes[i]}: row {r} worst ratio {worst}"
        assert torch.equal(y, y1), f"matrix {i} differs from its own launch"


def test_gemv_nf4_exact_cases():
    """Codes in {0, 7, 15} (levels -1, 0, +1), power-of-two scales, small integer x: every
    partial sum is an exact integer multiple of the scale, so y must equal the exact result."""
    import torch
    rng = np.random.default_rng(31)
    n_out, k = 70, 4160
    lv = rng.integers(-1, 2, size=(n_out, k)).astype(np.float64)
    e = rng.integers(-3, 4, size=(n_out, k // 64))
    s = np.repeat(np.exp2(e), 64, axis=1)
    lv[:, ::64] = 1.0                                        # every group holds +s: scale is exactly s
    w = lv * s
    wb = oracle.bf16_bits_from_f32(w.astype(np.float32))
    x = rng.integers(-4, 5, size=k).astype(np.float64)
    xb = oracle.bf16_bits_from_f32(x.astype(np.float32))
    packed = wsl.nf4_pack(to_dev_bf16(wb))
    y = wsl.linear_gemv(packed, to_dev_bf16(xb), wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k)
    # x scaled by 2^5 must scale y by exactly 2^5
    x2b = oracle.bf16_bits_from_f32((x * 32).astype(np.float32))
    y2 = wsl.linear_gemv(packed, to_dev_bf16(x2b), wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k)
    torch.cuda.synchronize()
    codes, scales = oracle.pack_codes(f64(wb))
    assert set(np.unique(codes).tolist()) <= {0, 7, 15}
    y_ref, _ = oracle.gemv_ref(oracle.dequant_exact(codes, scales), x)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), y_ref)
    assert np.array_equal(y2.cpu().numpy(), y.cpu().numpy() * np.float32(32))


@pytest.mark.parametrize("j", [0, 63, 64, 2047, 2048, 4159])
def test_gemv_nf4_one_hot(j):
    """x = e_j gives y = fp32(c * s) of column j (one fp32 rounding of the exact product)."""
    import torch
    n_out, k = 50, 4160
    wb = synth.weight_bits(95, 0, n_out, k)
    x = np.zeros(k, np.float32)
    x[j] = 1.0
    packed = wsl.nf4_pack(to_dev_bf16(wb))
    y = wsl.linear_gemv(packed, to_dev_bf16(oracle.bf16_bits_from_f32(x)), wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k)
    torch.cuda.synchronize()
    codes, scales = oracle.pack_codes(f64(wb))
    want = oracle.dequant_exact(codes, scales)[:, j].astype(np.float32)
    assert np.array_equal(y.cpu().numpy(), want)


def test_gemv_bf16_exact_integers():
    import torch
    rng = np.random.default_rng(37)
    n_out, k = 301, 5120
    w = rng.integers(-16, 17, size=(n_out, k)).astype(np.float32)
    x = rng.integers(-16, 17, size=k).astype(np.float32)
    y = wsl.linear_gemv(to_dev_bf16(oracle.bf16_bits_from_f32(w)), to_dev_bf16(oracle.bf16_bits_from_f32(x)))
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.float64), w.astype(np.float64) @ x.astype(np.float64))


def test_gemv_zero_weights_give_zero():
    import torch
    n_out, k = 40, 640
    wb = np.zeros((n_out, k), np.uint16)
    xb = synth.act_bits(96, 0, (k,))
    packed = wsl.nf4_pack(to_dev_bf16(wb))
    y = wsl.linear_gemv(packed, to_dev_bf16(xb), wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k)
    y2 = wsl.linear_gemv(to_dev_bf16(wb), to_dev_bf16(xb))
    torch.cuda.synchronize()
    assert np.all(y.cpu().numpy() == 0) and np.all(y2.cpu().numpy() == 0)


def test_gemv_deterministic_and_graph_capturable():
    """Same bits on repeated calls; a captured graph replays to the eager result (the call
    neither synchronizes nor allocates, or capture would fail)."""
    import torch
    n_out, k = 4096, 4096
    wb = synth.weight_bits(0, 0, n_out, k)
    xb = synth.act_bits(0, 1, (k,))
    packed = wsl.nf4_pack(to_dev_bf16(wb))
    x = to_dev_bf16(xb)
    y1 = wsl.linear_gemv(packed, x, wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k)
    y2 = wsl.linear_gemv(packed, x, wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k)
    yg = torch.empty(n_out, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        wsl.linear_gemv(packed, x, y=yg, wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        wsl.linear_gemv(packed, x, y=yg, wfmt=wsl.WSL_W_NF4, n_out=n_out, k=k)
    torch.cuda.synchronize()
    for _ in range(3):
        yg.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(yg, y1)
    assert torch.equal(y1, y2)
