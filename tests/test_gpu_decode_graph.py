"""A decode step captured as one HIP graph: the packed-embedding gather for a device-resident
token id, then NF4 linear stages, with the id advanced on the device by the graph itself.
Replays must reproduce the eager results for every position, read nothing back to the host and
grow no allocation (IPE page, "What is built" / "How it is checked")."""

import numpy as np
import pytest

import oracle
import synth
import weight_streaming_linear_amd as wsl
from gpu_common import to_dev_bf16, f64, say

pytestmark = pytest.mark.gpu

VOCAB, HIDDEN = 1000, 1024
STAGES = [(3072, 1024), (1024, 1024), (4096, 1024)]   # all consume the hidden state


def test_decode_step_graph_device_resident_position():
    import torch
    say("decode step graph")
    emb_bits = synth.weight_bits(110, 0, VOCAB, HIDDEN)
    emb = wsl.nf4_pack(to_dev_bf16(emb_bits))
    ws_bits = [synth.weight_bits(110, 1 + j, n, k) for j, (n, k) in enumerate(STAGES)]
    packs = [wsl.nf4_pack(to_dev_bf16(b)) for b in ws_bits]
    tok = torch.tensor([5], dtype=torch.int64, device="cuda")
    h = torch.empty((1, HIDDEN), dtype=torch.bfloat16, device="cuda")
    ys = [torch.empty(n, dtype=torch.float32, device="cuda") for n, _ in STAGES]

    def step():
        wsl.nf4_embed_rows(emb, VOCAB, HIDDEN, tok, out=h)
        for p, y, (n, k) in zip(packs, ys, STAGES):
            wsl.linear_gemv(p, h[0], y=y, wfmt=wsl.WSL_W_NF4, n_out=n, k=k)
        tok.add_(7)                                       # next position, on the device
        tok.remainder_(VOCAB)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    tok.fill_(5)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    tok.fill_(5)
    before = torch.cuda.memory_allocated()
    outs = []
    for _ in range(4):
        g.replay()
        outs.append([y.clone() for y in ys])        # device-side copies: no host read between replays
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() - before == sum(y.numel() * 4 for y in ys) * 4   # only the clones
    assert int(tok.item()) == (5 + 4 * 7) % VOCAB
    codes_e, scales_e = oracle.pack_codes(f64(emb_bits))
    refs = [oracle.pack_codes(f64(b)) for b in ws_bits]
    for r, got in enumerate(outs):
        t = (5 + 7 * r) % VOCAB
        x = f64(oracle.dequant_tile_bits(codes_e[[t]], scales_e[[t]]))[0]   # the bf16 hidden state
        for (c, sc), y in zip(refs, got):
            y_ref, s_ref = oracle.gemv_ref(oracle.dequant_exact(c, sc), x)
            ok, worst, i = oracle.check_rows_f32(y.cpu().numpy(), y_ref, s_ref)
            assert ok, f"replay {r}: row {i} worst ratio {worst}"
