"""The 48-layer NF4 decode sweep (hidden 6144) as the bench times it: 192 linear_gemv launches
in decoder order (qkv 8192x6144, o 6144x6144, gate_up 32768x6144, down 6144x16384 per layer),
captured as one HIP graph per token and replayed.  Sampled rows of every stage of layers 0, 23
and 47 are checked against the fp64 oracle after each replay (deep-fold README, "Метод" table:
decode is an N=1 NF4 GEMV inside a graph of the whole step; IPE page, "How it is checked")."""

import numpy as np
import pytest

import oracle
import synth
import weight_streaming_linear_amd as wsl
from gpu_common import bits_of, f64, say

pytestmark = pytest.mark.gpu

SWEEP_6144 = [("qkv", 8192, 6144), ("o", 6144, 6144), ("gate_up", 32768, 6144), ("down", 6144, 16384)]
LAYERS = 48
CHECKED = (0, 23, 47)


def _rows(n, seed):
    rng = np.random.default_rng(seed)
    edges = [0, 1, n - 2, n - 1, 15, 16, n - 17, n - 16]
    return np.unique(np.concatenate([edges, rng.integers(0, n, 40)]))


def build_sweep():
    """Packed weights of the 48 layers (drawn on the device with the bench's seeds), the stage
    inputs, one output buffer per (layer, stage), and the host bits of the sampled rows of the
    checked layers."""
    import torch
    xs = [synth.device_normal_bf16(2, 1000 + j, (k,)) for j, (_, n, k) in enumerate(SWEEP_6144)]
    packs, ys, sampled = [], [], {}
    for l in range(LAYERS):
        for j, (name, n, k) in enumerate(SWEEP_6144):
            w = synth.device_weight(2, 16 * l + j, n, k)
            if l in CHECKED:
                rows = _rows(n, 100 * l + j)
                sampled[(l, j)] = (rows, bits_of(w[torch.as_tensor(rows, device="cuda")]))
            packs.append((wsl.nf4_pack(w), n, k, j))
            ys.append(torch.empty(n, dtype=torch.float32, device="cuda"))
            del w
    torch.cuda.synchronize()
    return xs, packs, ys, sampled


def check_sweep(xs, ys, sampled, what):
    xbits = [bits_of(x) for x in xs]
    for (l, j), (rows, wb) in sampled.items():
        codes, scales = oracle.pack_codes(f64(wb))
        y_ref, s_ref = oracle.gemv_ref(oracle.dequant_exact(codes, scales), f64(xbits[j]))
        got = ys[4 * l + j].cpu().numpy()[rows]
        ok, worst, i = oracle.check_rows_f32(got, y_ref, s_ref)
        assert ok, f"{what}: layer {l} {SWEEP_6144[j][0]} row {rows[i]} worst ratio {worst}"


def test_decode_sweep_graph_against_oracle():
    import torch
    say("decode sweep: 48 layers, 192 launches in one graph")
    xs, packs, ys, sampled = build_sweep()

    def sweep():
        for (p, n, k, j), y in zip(packs, ys):
            wsl.linear_gemv(p, xs[j], y=y, wfmt=wsl.WSL_W_NF4, n_out=n, k=k)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sweep()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sweep()
    torch.cuda.synchronize()
    for rep in range(2):
        for y in ys:
            y.fill_(float("nan"))                     # eager work of the program between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check_sweep(xs, ys, sampled, f"graph replay {rep}")
