"""nf4_pack and nf4_dequant_tile on the GPU: bit-exact against the CPU oracle."""

import numpy as np
import pytest

import oracle
import synth
import weight_streaming_linear_amd as wsl
from gpu_common import to_dev_bf16, to_dev_u8, bits_of, f64, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_out,k,stream,tid", [(4096, 4096, 0, 0), (17, 192, 90, 1), (1, 64, 90, 2),
                                             (33, 320, 90, 3), (16, 128, 90, 4), (100, 2112, 90, 5)])
def test_pack_bit_exact(n_out, k, stream, tid):
    import torch
    say(f"pack {n_out}x{k}")
    wb = synth.weight_bits(stream, tid, n_out, k)
    packed = wsl.nf4_pack(to_dev_bf16(wb))
    torch.cuda.synchronize()
    ref = oracle.pack_device(f64(wb))
    got = packed.cpu().numpy()
    assert got.size == ref.size == oracle.packed_bytes(n_out, k)
    assert np.array_equal(got, ref)


def test_pack_special_groups_and_status():
    import torch
    n_out, k = 6, 256
    w = synth.host_normal_f32(91, 0, (n_out, k), 0.02)
    w[0, 0:64] = 0.0                        # all-zero group
    w[1, 64:128] = 1e-9                     # underflows fp16: s = +0
    w[2, 128:192] = -0.0                    # negative zeros
    w[3, 5] = 60000.0                       # large but finite in fp16
    w[4, 70] = 70000.0                      # fp16 overflow -> status bit, group as zeros
    w[5, 200] = np.nan                      # non-finite -> status bit, group as zeros
    wb = synth._bf16_bits_torch(w)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    packed = wsl.nf4_pack(to_dev_bf16(wb), status=status)
    torch.cuda.synchronize()
    st = int(status.item())
    assert st == wsl.WSL_STATUS_NONFINITE | wsl.WSL_STATUS_OVERFLOW
    # the oracle refuses those two groups; everywhere else the bytes must agree,
    # and the refused groups must come out as s = +0 with every code 7
    wf = f64(wb)
    clean = wf.copy()
    clean[4, 64:128] = 0.0
    clean[5, 192:256] = 0.0
    ref = oracle.pack_device(clean)
    assert np.array_equal(packed.cpu().numpy(), ref)
    with pytest.raises(oracle.PackError):
        oracle.pack_codes(wf[4:5])
    with pytest.raises(oracle.PackError):
        oracle.pack_codes(wf[5:6])


def test_fp16_scale_every_bf16_absmax():
    """Every positive finite bf16 value as a group's absmax: the stored fp16 scale (and all
    codes) must equal the oracle's (covers fp16 subnormal, normal and the top binade)."""
    import torch
    bits = np.arange(0x0001, 0x7F80, dtype=np.uint16)
    vals = oracle.f32_from_bf16_bits(bits).astype(np.float64)
    keep = vals < 65520.0                    # above this the scale overflows (status path)
    bits = bits[keep]
    n_out = bits.size
    wb = np.zeros((n_out, 64), dtype=np.uint16)
    wb[:, 0] = bits
    wb[:, 1] = bits ^ 0x8000                 # a negative copy: -a
    wb[:, 2] = (bits >> 1)                   # some smaller value
    packed = wsl.nf4_pack(to_dev_bf16(wb))
    torch.cuda.synchronize()
    ref = oracle.pack_device(f64(wb))
    assert np.array_equal(packed.cpu().numpy(), ref)


def test_dequant_tile_every_scale_and_code():
    """16 codes x every non-negative finite fp16 scale: restored bf16 == oracle, bitwise."""
    import torch
    sc = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).reshape(-1, 1)
    n_out = sc.shape[0]
    codes = np.tile(np.repeat(np.arange(16, dtype=np.uint8), 4), (n_out, 1))
    buf = oracle.device_from_canonical(oracle.codes_to_bytes(codes), sc)
    tile = wsl.nf4_dequant_tile(to_dev_u8(buf), n_out, 64, 0, 0, n_out, 64)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(tile), oracle.dequant_tile_bits(codes, sc))


@pytest.mark.parametrize("row0,k0,rows,cols", [(0, 0, 1, 1), (13, 37, 20, 91), (39, 320, 1, 64), (0, 0, 40, 384),
                                               (31, 383, 9, 1)])
def test_dequant_tile_offsets(row0, k0, rows, cols):
    import torch
    n_out, k = 40, 384
    wb = synth.weight_bits(92, 0, n_out, k)
    packed = wsl.nf4_pack(to_dev_bf16(wb))
    ld = cols + 3
    out = torch.full((rows, ld), float("nan"), dtype=torch.bfloat16, device="cuda")
    wsl.nf4_dequant_tile(packed, n_out, k, row0, k0, rows, cols, tile=out, ld_tile=ld)
    torch.cuda.synchronize()
    codes, scales = oracle.pack_codes(f64(wb))
    ref = oracle.dequant_tile_bits(codes, scales)[row0:row0 + rows, k0:k0 + cols]
    got = bits_of(out)
    assert np.array_equal(got[:, :cols], ref)
    assert np.all(got[:, cols:] == bits_of(torch.full((1,), float("nan"), dtype=torch.bfloat16))[0])


def test_pack_invariants_on_device():
    """Absmax element restores to +-s exactly (bf16(+-s) in the tile); exact zero restores to +0."""
    import torch
    n_out, k = 8, 128
    wb = synth.weight_bits(93, 0, n_out, k)
    wb[2, 9] = 0
    packed = wsl.nf4_pack(to_dev_bf16(wb))
    tile = bits_of(wsl.nf4_dequant_tile(packed, n_out, k, 0, 0, n_out, k))
    torch.cuda.synchronize()
    wf = f64(wb)
    _, scales = oracle.pack_codes(wf)
    for r in range(n_out):
        for g in range(k // 64):
            seg = np.abs(wf[r, g * 64:(g + 1) * 64])
            j = g * 64 + int(np.argmax(seg))
            s = float(scales[r, g])
            want = oracle.bf16_bits_from_f32(np.array([np.sign(wf[r, j]) * s], np.float32))[0]
            assert tile[r, j] == want
    assert tile[2, 9] == 0
