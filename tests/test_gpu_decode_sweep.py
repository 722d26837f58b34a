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


def _sweep_ws_clear(sw):
    import torch
    return bool((sw.ws == 0).all())


def test_decode_sweep_kernel_against_oracle_and_launches():
    """linear_gemv_sweep over the same 192 stages: sampled rows of layers 0, 23 and 47 against
    the oracle, and every row of every stage equal bit for bit to the stage's own linear_gemv
    launch (same teams, rows and reduction order).  Two calls; the workspace is back to zero
    after each and the status word clear."""
    import torch
    say("decode sweep: one linear_gemv_sweep launch per token")
    xs, packs, ys, sampled = build_sweep()
    sw = wsl.GemvSweep([(p, xs[j], y, n, k) for (p, n, k, j), y in zip(packs, ys)])
    ref = [torch.empty_like(y) for y in ys]
    for (p, n, k, j), y in zip(packs, ref):
        wsl.linear_gemv(p, xs[j], y=y, wfmt=wsl.WSL_W_NF4, n_out=n, k=k)
    for rep in range(2):
        for y in ys:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        sw()
        torch.cuda.synchronize()
        assert sw.status() == 0 and _sweep_ws_clear(sw), f"call {rep}: status {sw.status()}"
        check_sweep(xs, ys, sampled, f"sweep call {rep}")
        for i, (a, b) in enumerate(zip(ys, ref)):
            assert torch.equal(a, b), f"call {rep}: stage {i} differs from its linear_gemv launch"


# Ragged stages reaching every path of the team code inside one sweep: one to sixteen
# slices per row (S = 1 .. 16; 15 slices leave one wave idle, 3 slices four), row counts
# that leave a partial 16-row block or an odd row, workgroups with no super-group, several
# super-groups per workgroup (parked sums), and leftover row groups.
RAGGED = [(1, 64), (37, 192), (130, 2112), (257, 6144), (64, 16384), (9, 4160), (3073, 16384), (1029, 6208),
          (40, 32768), (100, 30720), (4099, 2112), (16, 64), (5000, 4096), (20000, 2048), (1, 32768)]


def test_decode_sweep_kernel_ragged_stages_every_row():
    import torch
    from gpu_common import to_dev_bf16
    say("decode sweep: ragged stages")
    stages, refs = [], []
    for i, (n, k) in enumerate(RAGGED):
        wb = synth.weight_bits(113, i, n, k)
        xb = synth.act_bits(113, 100 + i, (k,))
        codes, scales = oracle.pack_codes(f64(wb))
        refs.append(oracle.gemv_ref(oracle.dequant_exact(codes, scales), f64(xb)))
        stages.append((wsl.nf4_pack(to_dev_bf16(wb)), to_dev_bf16(xb),
                       torch.full((n,), float("nan"), dtype=torch.float32, device="cuda"), n, k))
    sw = wsl.GemvSweep(stages)
    first = None
    for rep in range(3):
        for st in stages:
            st[2].fill_(float("nan"))
        torch.cuda.synchronize()
        sw()
        torch.cuda.synchronize()
        assert sw.status() == 0 and _sweep_ws_clear(sw)
        got = [st[2].clone() for st in stages]
        if first is None:
            first = got
            for i, (y, (y_ref, s_ref)) in enumerate(zip(got, refs)):
                ok, worst, r = oracle.check_rows_f32(y.cpu().numpy(), y_ref, s_ref)
                assert ok, f"stage {i} {RAGGED[i]}: row {r} worst ratio {worst}"
        else:
            assert all(torch.equal(a, b) for a, b in zip(first, got)), f"call {rep} differs from call 0"


def test_decode_sweep_kernel_skips_an_invalid_device_descriptor():
    """A device descriptor that differs from the host one and is invalid (k = 65) is skipped
    with WSL_STATUS_DESCRIPTOR; the other stages are still computed."""
    import torch
    from gpu_common import to_dev_bf16
    shapes = [(300, 1024), (200, 2048), (100, 512)]
    stages, refs = [], []
    for i, (n, k) in enumerate(shapes):
        wb = synth.weight_bits(114, i, n, k)
        xb = synth.act_bits(114, 100 + i, (k,))
        codes, scales = oracle.pack_codes(f64(wb))
        refs.append(oracle.gemv_ref(oracle.dequant_exact(codes, scales), f64(xb)))
        stages.append((wsl.nf4_pack(to_dev_bf16(wb)), to_dev_bf16(xb),
                       torch.full((n,), float("nan"), dtype=torch.float32, device="cuda"), n, k))
    sw = wsl.GemvSweep(stages)
    size = __import__("ctypes").sizeof(wsl.WslGemvStage)
    bad = torch.tensor([65], dtype=torch.int64).view(torch.uint8).to("cuda")
    sw.d[size + 32:size + 40] = bad                 # stage 1's k on the device only
    sw()
    torch.cuda.synchronize()
    assert sw.status() & wsl.WSL_STATUS_DESCRIPTOR
    assert bool(torch.isnan(stages[1][2]).all())
    for i in (0, 2):
        ok, worst, r = oracle.check_rows_f32(stages[i][2].cpu().numpy(), *refs[i])
        assert ok, f"stage {i}: row {r} worst ratio {worst}"
    sw.ws.zero_()


def test_decode_sweep_kernel_graph_replays():
    """The sweep launch captured in a graph replays to the eager result (eager work and a
    synchronization between replays)."""
    import torch
    from gpu_common import to_dev_bf16
    shapes = [(2048, 6144), (6144, 2048), (1000, 16384)]
    stages = []
    for i, (n, k) in enumerate(shapes):
        stages.append((wsl.nf4_pack(to_dev_bf16(synth.weight_bits(115, i, n, k))),
                       to_dev_bf16(synth.act_bits(115, 100 + i, (k,))),
                       torch.empty(n, dtype=torch.float32, device="cuda"), n, k))
    sw = wsl.GemvSweep(stages)
    sw()
    want = [st[2].clone() for st in stages]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sw()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sw()
    torch.cuda.synchronize()
    for _ in range(3):
        for st in stages:
            st[2].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(st[2], w) for st, w in zip(stages, want))
        assert sw.status() == 0 and _sweep_ws_clear(sw)


def test_decode_sweep_kernel_many_stages():
    """A sweep longer than the stage plans the kernel keeps in LDS at once (512: two chunks
    of 256), so later chunks are planned at stage boundaries: 1100 small stages of mixed
    shapes, every stage equal bit for bit to its own linear_gemv launch, a sample of stages
    against the oracle, and one device descriptor in a late chunk made invalid (skipped with
    WSL_STATUS_DESCRIPTOR)."""
    import ctypes
    import torch
    from gpu_common import to_dev_bf16
    say("decode sweep: 1100 stages")
    shapes = [(16, 64), (33, 128), (100, 2048), (64, 6144), (17, 16384), (48, 4096), (250, 1024)]
    stages, bits = [], []
    for i in range(1100):
        n, k = shapes[i % len(shapes)]
        wb = synth.weight_bits(116, i % 61, n, k)
        xb = synth.act_bits(116, 200 + i % 13, (k,))
        bits.append((wb, xb))
        stages.append((wsl.nf4_pack(to_dev_bf16(wb)), to_dev_bf16(xb),
                       torch.full((n,), float("nan"), dtype=torch.float32, device="cuda"), n, k))
    ref = [torch.empty_like(st[2]) for st in stages]
    for st, y in zip(stages, ref):
        wsl.linear_gemv(st[0], st[1], y=y, wfmt=wsl.WSL_W_NF4, n_out=st[3], k=st[4])
    sw = wsl.GemvSweep(stages)
    sw()
    torch.cuda.synchronize()
    assert sw.status() == 0 and _sweep_ws_clear(sw)
    for i, (st, y) in enumerate(zip(stages, ref)):
        assert torch.equal(st[2], y), f"stage {i} {st[3]}x{st[4]} differs from its linear_gemv launch"
    for i in (0, 255, 256, 511, 512, 767, 768, 1023, 1024, 1099):
        wb, xb = bits[i]
        codes, scales = oracle.pack_codes(f64(wb))
        ok, worst, r = oracle.check_rows_f32(stages[i][2].cpu().numpy(),
                                             *oracle.gemv_ref(oracle.dequant_exact(codes, scales), f64(xb)))
        assert ok, f"stage {i}: row {r} worst ratio {worst}"
    bad_stage = 800
    size = ctypes.sizeof(wsl.WslGemvStage)
    for st in stages:
        st[2].fill_(float("nan"))
    sw.d[bad_stage * size + 32:bad_stage * size + 40] = torch.tensor([65], dtype=torch.int64).view(torch.uint8).to("cuda")
    sw()
    torch.cuda.synchronize()
    assert sw.status() & wsl.WSL_STATUS_DESCRIPTOR
    assert bool(torch.isnan(stages[bad_stage][2]).all())
    for i, (st, y) in enumerate(zip(stages, ref)):
        if i != bad_stage:
            assert torch.equal(st[2], y), f"stage {i} differs after the invalid descriptor"
    sw.ws.zero_()
