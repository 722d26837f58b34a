"""nf4_embed_rows on the GPU against the CPU oracle: bit-exact restored rows."""

import numpy as np
import pytest

import oracle
import synth
import weight_streaming_linear_amd as wsl
from gpu_common import to_dev_bf16, bits_of, f64, say

pytestmark = pytest.mark.gpu


def _table(n_rows, k, stream):
    wb = synth.weight_bits(stream, 0, n_rows, k)
    codes, scales = oracle.pack_codes(f64(wb))
    return wb, codes, scales


@pytest.mark.parametrize("n_rows,k", [(1000, 320), (37, 64), (4099, 2048)])
def test_embed_rows_bit_exact(n_rows, k):
    """Requested rows (repeats, first and last, ragged 16-row blocks) equal the oracle's
    restored tile rows (bf16) and fp32(c * s) (fp32) bit for bit; ld_out > k leaves the
    padding untouched."""
    import torch
    say(f"embed {n_rows}x{k}")
    wb, codes, scales = _table(n_rows, k, 102)
    packed = wsl.nf4_pack(to_dev_bf16(wb))
    rng = np.random.default_rng(7)
    ids = np.concatenate([[0, n_rows - 1, 5 % n_rows, 5 % n_rows], rng.integers(0, n_rows, 61)]).astype(np.int64)
    d_ids = torch.from_numpy(ids).cuda()
    ld = k + 8
    outb = torch.full((len(ids), ld), -1.0, dtype=torch.bfloat16, device="cuda")
    outf = torch.full((len(ids), ld), float("nan"), dtype=torch.float32, device="cuda")
    wsl.nf4_embed_rows(packed, n_rows, k, d_ids, out=outb[:, :k], ofmt=wsl.WSL_OUT_BF16)
    wsl.nf4_embed_rows(packed, n_rows, k, d_ids, out=outf[:, :k], ofmt=wsl.WSL_OUT_F32)
    torch.cuda.synchronize()
    tile = oracle.dequant_tile_bits(codes[ids], scales[ids])
    assert np.array_equal(bits_of(outb)[:, :k], tile)
    assert np.all(bits_of(outb)[:, k:] == bits_of(torch.tensor([-1.0], dtype=torch.bfloat16))[0])
    exact32 = oracle.dequant_exact(codes[ids], scales[ids]).astype(np.float32)
    assert np.array_equal(outf[:, :k].cpu().numpy(), exact32)
    assert torch.isnan(outf[:, k:]).all()


def test_embed_rows_bad_index_gives_zero_row_and_status():
    import torch
    n_rows, k = 50, 128
    wb, codes, scales = _table(n_rows, k, 103)
    packed = wsl.nf4_pack(to_dev_bf16(wb))
    ids = np.array([3, -1, 50, 49, 1 << 40], dtype=np.int64)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = wsl.nf4_embed_rows(packed, n_rows, k, torch.from_numpy(ids).cuda(), ofmt=wsl.WSL_OUT_F32, status=status)
    clean = torch.zeros(1, dtype=torch.int32, device="cuda")
    wsl.nf4_embed_rows(packed, n_rows, k, torch.from_numpy(ids[[0, 3]]).cuda(), ofmt=wsl.WSL_OUT_F32, status=clean)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(got[[1, 2, 4]] == 0)
    ok = ids[[0, 3]]
    assert np.array_equal(got[[0, 3]], oracle.dequant_exact(codes[ok], scales[ok]).astype(np.float32))
    assert int(status.item()) == 4
    assert int(clean.item()) == 0


def test_embed_rows_empty_and_graph_replay():
    """count = 0 launches nothing; a captured gather replays to the eager result with new
    ids written into the same device buffer (no host copy of the ids)."""
    import torch
    n_rows, k = 300, 256
    wb, codes, scales = _table(n_rows, k, 104)
    packed = wsl.nf4_pack(to_dev_bf16(wb))
    empty = torch.empty(0, dtype=torch.int64, device="cuda")
    assert wsl.nf4_embed_rows(packed, n_rows, k, empty).shape == (0, k)
    ids = torch.tensor([7, 8], dtype=torch.int64, device="cuda")
    out = torch.empty((2, k), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        wsl.nf4_embed_rows(packed, n_rows, k, ids, out=out)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        wsl.nf4_embed_rows(packed, n_rows, k, ids, out=out)
    torch.cuda.synchronize()
    for pair in ([1, 2], [299, 0], [17, 17]):
        ids.copy_(torch.tensor(pair, dtype=torch.int64))
        g.replay()
        torch.cuda.synchronize()
        want = oracle.dequant_tile_bits(codes[pair], scales[pair])
        assert np.array_equal(bits_of(out), want)
