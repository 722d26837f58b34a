#!/usr/bin/env python3
"""Benchmark of the weight-streaming linear layers on one MI355X.

Headline workload (``value``): the batch-1 NF4 decode sweep over a 48-layer stack of
hidden size 6144 (20B class): per layer qkv 8192x6144, o 6144x6144, gate_up 32768x6144
and down 6144x16384, packed NF4 (group 64, fp16 scales), the 192 GEMVs of a token in
decoder order in one linear_gemv_sweep launch, with a device-wide barrier between stages
so that no stage starts before the one it follows has finished (deep-fold README, "Метод"
table: decode is an N=1 NF4 GEMV per matrix).  A "step" is one token: the W warm-up
tokens and then exactly K timed tokens are launched between
HIP events; ``value`` = packed weight bytes per token (9,946,791,936 B, every byte read
once) / wall time per token, in GB/s (1e9 B/s), every input resident in HBM before the
timed region starts.  The 9.9 GB stack is 39x the 256 MB last-level cache, so no
rotation copies are needed.

``roofline`` describes the dominant kernel, the sweep kernel itself (one launch per token):
its algorithmic bytes per launch (the token's packed bytes) divided by its average launch
duration between HIP events on the launch stream.  ``traffic`` is the HBM bytes
per launch from rocprofv3 FETCH_SIZE/WRITE_SIZE counter runs of ``--traffic-probe``,
scaled by what the same counters read for a plain copy of known size; null when the
kernel source changed since the counters were taken.

``headline_detail`` holds the same 192 GEMVs as separate launches captured in one graph
per token, each stage's launch time in that form, and the decode-step graph.  ``paths``
holds the other workloads of the hot path measured in the same run: the bf16 decode layer of hidden 5120 (fused
q/k/v and gate/up: 4 launches; unfused: 7), the NF4 GEMV 4096x4096, the NF4 prefill GEMM
at 32 positions, the NF4 GEMM at 64/128/256 positions, the bf16 and NF4 verification
GEMMs at 8192 positions, the packed-embedding gather and the copy ring.

Protocol (IPE page, "How it is benchmarked"): a failed sanity gate stops the run before
timing; warm-up and graph capture are outside every timer; by default the whole run is
repeated in three fresh processes, one after another -- the line is the first run's with
the headline value and ms_per_step replaced by the medians, ``repeats`` holds every run's
figures with median, interquartile range and A/A spread, and the SHA-256 of every
workload's outputs must agree across the processes (``determinism``).
"""

import argparse
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, 2.5 PFLOP/s
METRIC = "GEMV effective weight GB/s (% of HBM peak); GEMM TFLOP/s (% of MFMA peak)"
GEMV_SRC = os.path.join(ROOT, "weight_streaming_linear_amd", "csrc", "gemv.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_nf4_sweep_48x6144.json")
DOMINANT = "nf4_gemv_gate_up"   # the largest per-stage launch of the 192-launch form
DOMINANT_KERNEL = "gemv_nf4_sweep_kernel<12> (48-layer hidden-6144 decode sweep, one launch per token)"
SWEEP_KERNEL_MATCH = "gemv_nf4_sweep_kernel"
TEAM_KERNEL_MATCH = "gemv_nf4_team_kernel"
CALIB_BYTES = 1 << 30            # plain copy used to calibrate the byte counters


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- timing helpers
class Launch:
    """One kernel launch of a step: a closure plus its algorithmic work."""

    def __init__(self, fn, nbytes=0, flops=0, name="", dispatches=1):
        self.fn, self.nbytes, self.flops, self.name, self.dispatches = fn, nbytes, flops, name, dispatches


_SPIN = {}


def spin_cycles_per_ms():
    """Rate of torch's spin kernel (torch.cuda._sleep), measured once with HIP events."""
    import torch
    if "rate" not in _SPIN:
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        a.record()
        torch.cuda._sleep(4_000_000)
        b.record()
        torch.cuda.synchronize()
        _SPIN["rate"] = 4_000_000 / max(a.elapsed_time(b), 1e-3)
    return _SPIN["rate"]


# Every timed block, in order: (label, launches timed, dispatches per launch).  With
# --block-log the list is written to a file, so that a rocprofv3 kernel trace of the same
# command can be cut into these blocks (each follows one spin kernel) and summarized per
# workload and shape (--trace-summarize).
BLOCK_LOG = []


def time_block(launches, reps, warmup, label=None, dispatches=1):
    """Average duration of one launch: `warmup` untimed launches, then `reps` launches back to
    back (cycling through `launches`) between one pair of HIP events on the current stream,
    the one the launches use.  A spin kernel queued first keeps the GPU busy while the host
    enqueues the block, so the span holds the kernels and nothing of the host.  (An event
    pair around every single launch would add about 2 us of command-processor overhead to
    each measured launch on this platform.)  The spin lasts twice the host's enqueue time for
    the block, measured on a few launches enqueued without waiting: a much longer spin lets
    the clock settle low, and the launches that follow it run slower until it recovers.
    Returns microseconds per launch."""
    import torch
    for i in range(warmup):
        launches[i % len(launches)].fn()
    torch.cuda.synchronize()
    probe = min(8, max(1, reps))
    t0 = time.perf_counter()
    for i in range(probe):
        launches[i % len(launches)].fn()
    host_ms = 1e3 * (time.perf_counter() - t0) / probe
    torch.cuda.synchronize()
    torch.cuda._sleep(int((2.0 * host_ms * reps + 0.5) * spin_cycles_per_ms()))
    BLOCK_LOG.append((label or launches[0].name or "block", reps, dispatches))
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(reps):
        launches[(warmup + i) % len(launches)].fn()
    b.record()
    torch.cuda.synchronize()
    return 1e3 * a.elapsed_time(b) / reps


def time_step_launches(steps, k_steps, warmup):
    """Per-kernel average durations for a step made of several kinds of launch: launches of
    the same name (one per step copy) are timed together as one block of k_steps launches.
    Returns {name: (avg_us, launch)}."""
    kinds = {}
    for st in steps:
        for l in st:
            kinds.setdefault(l.name, []).append(l)
    return {name: (time_block(ls, k_steps, warmup, label=name, dispatches=ls[0].dispatches), ls[0])
            for name, ls in kinds.items()}


def capture(launches):
    """One HIP graph replaying `launches` in order (captured on a side stream after one
    eager run on it, as torch requires)."""
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for l in launches:
            l.fn()
    torch.cuda.current_stream().wait_stream(s)
    with torch.cuda.graph(g):
        for l in launches:
            l.fn()
    torch.cuda.synchronize()
    return g


READ_CEILING = {}


def measure_read_ceiling(reps=10, nbytes=2 << 30):
    """A reference streaming read on the same GPU: wsl_stream_read (16-byte loads that
    bypass the caches, 1 KB per wave instruction, three in flight per wave, one 8-wave
    workgroup per CU) over a 2 GiB
    buffer, 8x the MALL, timed as one block of launches between HIP events.  A plain read
    kernel, not a bound: a kernel with a better access pattern can exceed it."""
    import torch
    import weight_streaming_linear_amd as wsl
    if "gbs" not in READ_CEILING:
        buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        us = time_block([Launch(lambda: wsl.stream_read(buf, sink))], reps, 3, label="stream_read_probe_2GiB")
        READ_CEILING.update({"gbs": round(nbytes / 1e3 / us, 1), "buffer_bytes": nbytes, "avg_launch_us": round(us, 2),
                             "frac_hbm": round(nbytes / 1e3 / us / HBM_PEAK_GBS, 4),
                             "what": "wsl_stream_read over a 2 GiB buffer (read-only streaming kernel)"})
        del buf
        torch.cuda.empty_cache()
    return READ_CEILING


LAUNCH_FLOOR = {}


def measure_launch_floor(reps=200):
    """t0: the block-timed duration of a launch that does almost nothing (wsl_stream_read of
    16 bytes: one workgroup), the fixed cost every kernel of the path pays on this machine."""
    import torch
    import weight_streaming_linear_amd as wsl
    if "us" not in LAUNCH_FLOOR:
        buf = torch.zeros(16, dtype=torch.uint8, device="cuda")
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        LAUNCH_FLOOR["us"] = round(time_block([Launch(lambda: wsl.stream_read(buf, sink))], reps, 10,
                                              label="launch_floor_t0"), 3)
        LAUNCH_FLOOR["what"] = "block-timed wsl_stream_read of 16 bytes (one workgroup)"
    return LAUNCH_FLOOR


def time_graphs(graphs, k_steps, warmup):
    """Replay graphs[i % len] for `warmup` untimed and k_steps timed steps; wall ms."""
    import torch
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(k_steps):
        graphs[(warmup + i) % len(graphs)].replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b)


def summarize(per_kind, counts=None):
    """Step totals from {name: (avg_us, launch)}; counts[name] = launches of that name per
    step (default 1)."""
    counts = counts or {}
    us = sum(t * counts.get(n, 1) for n, (t, _) in per_kind.items())
    nbytes = sum(l.nbytes * counts.get(n, 1) for n, (_, l) in per_kind.items())
    flops = sum(l.flops * counts.get(n, 1) for n, (_, l) in per_kind.items())
    launches = {}
    for name, (t, l) in per_kind.items():
        e = {"avg_us": round(t, 3), "gbs": round(l.nbytes / 1e3 / t, 1)}
        if l.flops and l.nbytes and l.flops / l.nbytes > 10:
            e["tflops"] = round(l.flops / 1e6 / t, 1)
        launches[name] = e
    return {
        "kernel_ms_per_step": us / 1e3,
        "launches_per_step": sum(counts.get(n, 1) for n in per_kind),
        "bytes_per_step": nbytes,
        "flops_per_step": flops,
        "kernel_gbs": nbytes / 1e3 / us if us > 0 else 0.0,
        "kernel_tflops": flops / 1e6 / us if us > 0 else 0.0,
        "launches": launches,
    }


# ---------------------------------------------------------------- sanity gates
# Parity with the CPU oracle is proven by the test suite.  Before timing, the bench only
# checks sampled outputs against torch fp32 products on the GPU (for NF4, of the tiles the
# library restores with nf4_dequant_tile), and refuses to time anything that fails.
def refuse(name, worst):
    raise SystemExit(f"sanity check failed for {name}: worst ratio {worst}; refusing to time")


def sample_rows(n, count, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, count)]))


def check_close(name, got, ref, scale, rel, ulp_rel=0.0):
    """|got - ref| <= rel * scale + ulp_rel * |ref| elementwise (torch tensors, any device)."""
    import torch
    got = got.double()
    ref = ref.double()
    bound = rel * scale.double() + ulp_rel * ref.abs()
    if not bool(torch.isfinite(got).all()):
        refuse(name, float("inf"))
    ratio = ((got - ref).abs() / bound.clamp_min(1e-300)).max().item()
    if ratio > 1.0:
        refuse(name, ratio)
    return ratio


def nf4_rows_f32(packed, n_out, k, rows):
    """fp32(level * s) of the given rows of a packed matrix, restored by the library's row
    gather (nf4_embed_rows): within 2^-24 relative of the exact level * s."""
    import torch
    import weight_streaming_linear_amd as wsl
    ids = torch.as_tensor(np.asarray(rows), dtype=torch.int64, device="cuda")
    return wsl.nf4_embed_rows(packed, n_out, k, ids, ofmt=wsl.WSL_OUT_F32)


def gate_gemv_nf4(name, y, packed, n_out, k, rows, x):
    """NF4 GEMV rows against fp64 sums of fp32(level * s) * x, at the 1e-4 * sum|w x| bound
    (the restored fp32 weights differ from level * s by at most 2^-24 relative)."""
    import torch
    w = nf4_rows_f32(packed, n_out, k, rows).double()
    xf = x.double()
    return check_close(name, y[torch.as_tensor(np.asarray(rows), device="cuda")], w @ xf, w.abs() @ xf.abs(), 1e-4)


def sha256_of(tensors):
    """SHA-256 of the bytes of device tensors, in order (the determinism record)."""
    h = hashlib.sha256()
    for t in tensors:
        h.update(t.detach().contiguous().view(-1).view(__import__("torch").uint8).cpu().numpy().tobytes())
    return h.hexdigest()


OUTPUT_SHA = {}


def nf4_rows_tile(packed, n_out, k, rows):
    """bf16 tiles of the given rows, restored by the library (one nf4_dequant_tile per row)."""
    import torch
    import weight_streaming_linear_amd as wsl
    t = torch.empty((len(rows), k), dtype=torch.bfloat16, device="cuda")
    for i, r in enumerate(rows):
        wsl.nf4_dequant_tile(packed, n_out, k, int(r), 0, 1, k, tile=t[i:i + 1], ld_tile=k)
    return t


def gate_gemv(name, y, w_rows, x, rel):
    """y[rows] against w_rows (bf16 [r][k]) times x in fp32."""
    wf = w_rows.float()
    xf = x.float()
    return check_close(name, y, wf @ xf, wf.abs() @ xf.abs(), rel)


# ---------------------------------------------------------------- headline: NF4 decode sweep
SWEEP_6144 = [("qkv", 8192, 6144), ("o", 6144, 6144), ("gate_up", 32768, 6144), ("down", 6144, 16384)]
SWEEP_LAYERS = 48


def setup_sweep(layers=SWEEP_LAYERS):
    """The 48-layer stack, packed on the device (seeded weights drawn on the device, stage j
    of layer l with tensor id 16 l + j); one x per stage kind; one y per (layer, stage)."""
    import torch
    import synth
    import weight_streaming_linear_amd as wsl
    xs = [synth.device_normal_bf16(2, 1000 + j, (k,)) for j, (_, n, k) in enumerate(SWEEP_6144)]
    packs, ys = [], []
    t0 = time.time()
    for l in range(layers):
        for j, (name, n, k) in enumerate(SWEEP_6144):
            w = synth.device_weight(2, 16 * l + j, n, k)
            packs.append((wsl.nf4_pack(w), n, k, j))
            ys.append(torch.empty(n, dtype=torch.float32, device="cuda"))
            del w
    torch.cuda.synchronize()
    log(f"nf4 decode sweep: packed {layers} layers in {time.time() - t0:.1f}s")
    return xs, packs, ys


def gate_sweep(name, xs, packs, ys, layers):
    worst = 0.0
    for l in layers:
        for j, (st, n, k) in enumerate(SWEEP_6144):
            p = packs[4 * l + j][0]
            worst = max(worst, gate_gemv_nf4(f"{name} layer {l} {st}", ys[4 * l + j], p, n, k,
                                             sample_rows(n, 24, 100 * l + j), xs[j]))
    return worst


def measure_headline(k_steps, warmup):
    """The decode sweep as one linear_gemv_sweep launch per token (the headline): W untimed
    then exactly K timed launches between HIP events on the stream they run on.  Also the
    same 192 GEMVs as separate launches captured in one graph per token, the per-stage kernel
    blocks of that form (gate_up the largest), and the decode-step graph with the
    packed-embedding gather of a device-resident token."""
    import torch
    import synth
    import weight_streaming_linear_amd as wsl
    xs, packs, ys = setup_sweep()
    token_bytes = sum(wsl.nf4_packed_bytes(n, k) for _, n, k, _ in packs)
    launches = [Launch(lambda p=p, n=n, k=k, j=j, y=y: wsl.linear_gemv(p, xs[j], y=y, wfmt=wsl.WSL_W_NF4, n_out=n,
                                                                       k=k),
                       nbytes=wsl.nf4_packed_bytes(n, k), flops=2 * n * k, name=f"nf4_gemv_{SWEEP_6144[j][0]}")
                for (p, n, k, j), y in zip(packs, ys)]
    for l in launches[:4]:
        l.fn()
    worst = gate_sweep("nf4 decode sweep", xs, packs, ys, [0])
    g = capture(launches)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    for y in ys:
        y.fill_(float("nan"))
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(k_steps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / k_steps
    worst = max(worst, gate_sweep("nf4 decode sweep (graph replay)", xs, packs, ys, [0, 23, 47]))
    OUTPUT_SHA["nf4_decode_sweep_48x6144"] = sha256_of(ys)
    log(f"nf4 decode sweep: {ms:.3f} ms/token (graph), {token_bytes / 1e6 / ms:.0f} GB/s, gate worst {worst:.3g}")

    # one block of launches per stage kind over the 48 layers (the dominant: gate_up)
    per_kind = time_step_launches([launches], 2 * SWEEP_LAYERS, 4)
    kern = summarize(per_kind, {f"nf4_gemv_{st[0]}": SWEEP_LAYERS for st in SWEEP_6144})

    # the headline: the sweep as one launch per token (linear_gemv_sweep)
    sw = wsl.GemvSweep([(p, xs[j], y, n, k) for (p, n, k, j), y in zip(packs, ys)])
    for y in ys:
        y.fill_(float("nan"))
    sw()
    torch.cuda.synchronize()
    if sw.status() != 0:
        refuse("linear_gemv_sweep status", float(sw.status()))
    sw_worst = gate_sweep("nf4 decode sweep (one launch)", xs, packs, ys, [0, 23, 47])
    if sha256_of(ys) != OUTPUT_SHA["nf4_decode_sweep_48x6144"]:
        refuse("linear_gemv_sweep differs from the per-stage launches", float("inf"))
    sw_us = time_block([Launch(sw, nbytes=token_bytes, name="nf4_decode_sweep_kernel")], k_steps, warmup,
                       label="nf4_decode_sweep_kernel_48x6144")
    sw_ms = sw_us / 1e3
    if sw.status() != 0:
        refuse("linear_gemv_sweep status after the timed launches", float(sw.status()))
    log(f"nf4 decode sweep: {sw_ms:.3f} ms/token (one launch), {token_bytes / 1e6 / sw_ms:.0f} GB/s")

    # decode-step graph: embedding gather of a device-resident token id + the sweep + id advance
    emb_n = 128000
    wemb = synth.device_weight(2, 999, emb_n, 6144)
    emb = wsl.nf4_pack(wemb)
    del wemb
    tok = torch.zeros(1, dtype=torch.int64, device="cuda")
    hid = torch.empty((1, 6144), dtype=torch.bfloat16, device="cuda")
    step_launches = [Launch(lambda: wsl.nf4_embed_rows(emb, emb_n, 6144, tok, out=hid))] + launches + \
        [Launch(lambda: tok.add_(1))]
    g2 = capture(step_launches)
    before = torch.cuda.memory_allocated()
    step_ms = time_graphs([g2], k_steps, warmup) / k_steps
    grew = torch.cuda.memory_allocated() - before
    t0 = measure_launch_floor()["us"]
    out = {
        "ms_per_token": sw_ms, "sweep_us": sw_us, "token_bytes": token_bytes,
        "sanity_worst_ratio": max(worst, sw_worst), "kernels": kern,
        "gate_up_avg_us": per_kind[DOMINANT][0], "gate_up_bytes": per_kind[DOMINANT][1].nbytes,
        "graph_192_launches": {"ms_per_token": round(ms, 4), "gbs": round(token_bytes / 1e6 / ms, 1),
                               "frac_hbm": round(token_bytes / 1e6 / ms / HBM_PEAK_GBS, 4),
                               "what": "the same 192 GEMVs as separate linear_gemv launches captured in one "
                                       "graph per token (stream order between stages); outputs bit-identical "
                                       "to the one-launch sweep"},
        "decode_step_graph": {"ms_per_token": round(step_ms, 4), "tokens_per_s": round(1e3 / step_ms, 2),
                              "what": "embedding gather (device-resident token id) + 192 GEMVs + id advance, "
                                      "one graph", "allocator_growth_bytes": grew},
        "launch_floor": {"t0_us": t0, "launches_per_token": len(launches),
                         "t0_ms_per_token": round(len(launches) * t0 / 1e3, 4),
                         "bytes_ms_at_8tbs": round(token_bytes / 8e9, 4)},
    }
    del g, g2, sw, packs, launches, step_launches, emb
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- bf16 decode layer (hidden 5120)
LAYER_5120 = [("qkv", 7168, 5120), ("o", 5120, 5120), ("gate_up", 34816, 5120), ("down", 5120, 17408)]
LAYER_5120_UNFUSED = [("q", 5120, 5120), ("k", 1024, 5120), ("v", 1024, 5120), ("o", 5120, 5120),
                      ("gate", 17408, 5120), ("up", 17408, 5120), ("down", 5120, 17408)]


def setup_layer_5120(mats, copies=2, tid0=0):
    """One dense decoder layer (hidden 5120) in bf16, `copies` distinct copies."""
    import torch
    import synth
    import weight_streaming_linear_amd as wsl
    layers = [[synth.device_weight(1, tid0 + 10 * c + j, n, k) for j, (_, n, k) in enumerate(mats)]
              for c in range(copies)]
    xs = [synth.device_normal_bf16(1, 100 + j, (k,)) for j, (_, n, k) in enumerate(mats)]
    ys = [torch.empty(n, dtype=torch.float32, device="cuda") for (_, n, _) in mats]
    steps = [[Launch(lambda w=ws_[j], x=xs[j], y=ys[j]: wsl.linear_gemv(w, x, y=y), nbytes=2 * n * k,
                     flops=2 * n * k, name=name) for j, (name, n, k) in enumerate(mats)] for ws_ in layers]
    return layers, xs, ys, steps


def run_bf16_decode_layer(k_steps, warmup):
    """bf16 decode GEMV over one dense decoder layer of hidden 5120, batch 1: q/k/v and gate/up
    fused (4 launches per step), as stored (7 launches) and as stored with q/k/v and gate/up
    each in one multi-matrix launch (4 launches), two layer copies alternating (the 1.32 GB
    exceed the 256 MB last-level cache); one graph per step, K steps."""
    import torch
    import weight_streaming_linear_amd as wsl
    out = {}
    for label, mats, tid0 in (("fused", LAYER_5120, 0), ("unfused", LAYER_5120_UNFUSED, 200)):
        layers, xs, ys, steps = setup_layer_5120(mats, tid0=tid0)
        worst = 0.0
        for c, ws_ in enumerate(layers):
            for j, (name, n, k) in enumerate(mats):
                wsl.linear_gemv(ws_[j], xs[j], y=ys[j])
                rows = torch.as_tensor(sample_rows(n, 48, 7 + j + 10 * c), device="cuda")
                worst = max(worst, gate_gemv(f"bf16 layer {label} copy {c} {name}", ys[j][rows], ws_[j][rows],
                                             xs[j], 1e-4))
        OUTPUT_SHA[f"bf16_decode_layer_5120_{label}"] = sha256_of(ys)
        variants = [(label, steps)]
        if label == "unfused":
            # the same separate matrices, q/k/v and gate/up each in one linear_gemv_multi launch
            groups = [("q_k_v", [0, 1, 2]), ("o", [3]), ("gate_up_multi", [4, 5]), ("down", [6])]
            grouped = [[Launch(lambda ws_=ws_, g=g: wsl.linear_gemv_multi([(ws_[j], xs[j], ys[j]) for j in g]),
                               nbytes=sum(2 * mats[j][1] * mats[j][2] for j in g),
                               flops=sum(2 * mats[j][1] * mats[j][2] for j in g), name=name)
                        for name, g in groups] for ws_ in layers]
            for launch in grouped[-1]:
                launch.fn()
            torch.cuda.synchronize()
            if sha256_of(ys) != OUTPUT_SHA[f"bf16_decode_layer_5120_{label}"]:
                refuse("bf16 layer grouped launches differ from the separate launches", float("inf"))
            variants.append(("unfused_grouped", grouped))
        for vlabel, vsteps in variants:
            graphs = [capture(st) for st in vsteps]
            ms = time_graphs(graphs, k_steps, warmup) / k_steps
            per_kind = time_step_launches(vsteps, k_steps, warmup)
            kern = summarize(per_kind)
            nbytes = kern["bytes_per_step"]
            out[vlabel] = {"launches_per_step": len(vsteps[0]), "ms_per_step": round(ms, 5),
                           "gbs": round(nbytes / 1e6 / ms, 1), "frac_hbm": round(nbytes / 1e6 / ms / HBM_PEAK_GBS, 4),
                           "weight_bytes_per_step": nbytes, "kernel_ms_per_step": round(kern["kernel_ms_per_step"], 5),
                           "launches": kern["launches"], "sanity_worst_ratio": worst}
            del graphs
        del steps, layers, variants
        torch.cuda.empty_cache()
    out["workload"] = ("bf16 decode GEMV, batch 1, one dense decoder layer, hidden 5120: fused qkv 7168x5120, o "
                       "5120x5120, gate_up 34816x5120, down 5120x17408; unfused q, k, v, o, gate, up, down as 7 "
                       "launches; unfused_grouped the same matrices as 4 launches (q/k/v and gate/up each one "
                       "linear_gemv_multi)")
    return out


# ---------------------------------------------------------------- other workloads
def run_nf4_gemv_4096(k_steps, warmup, copies=128):
    """NF4 GEMV 4096x4096, 128 packed copies (1.14 GB) in rotation."""
    import torch
    import synth
    import weight_streaming_linear_amd as wsl
    n, k = 4096, 4096
    x = synth.device_normal_bf16(0, 1, (k,))
    y = torch.empty(n, dtype=torch.float32, device="cuda")
    packs = []
    for c in range(copies):
        w = synth.device_weight(0, 1000 + c, n, k)
        packs.append(wsl.nf4_pack(w))
        del w
    wsl.linear_gemv(packs[0], x, y=y, wfmt=wsl.WSL_W_NF4, n_out=n, k=k)
    worst = gate_gemv_nf4("nf4 gemv 4096", y, packs[0], n, k, sample_rows(n, 64, 3), x)
    OUTPUT_SHA["nf4_gemv_4096"] = sha256_of([y])
    nb = wsl.nf4_packed_bytes(n, k)
    steps = [[Launch(lambda p=p: wsl.linear_gemv(p, x, y=y, wfmt=wsl.WSL_W_NF4, n_out=n, k=k), nbytes=nb,
                     flops=2 * n * k, name="nf4_gemv_4096")] for p in packs]
    out = summarize(time_step_launches(steps, k_steps, warmup))
    t0 = measure_launch_floor()["us"]
    us = out["launches"]["nf4_gemv_4096"]["avg_us"]
    out["launch_floor"] = {"t0_us": t0, "ideal_us_at_8tbs": round(nb / 8e12 * 1e6, 3),
                           "us_above_t0": round(us - t0, 3),
                           "gbs_above_t0": round(nb / 1e3 / (us - t0), 1) if us > t0 else None,
                           "bytes_for_75pct_at_this_t0": round(3 * t0 * 1e-6 * HBM_PEAK_GBS * 1e9)}
    out.update({"workload": "NF4 GEMV 4096x4096, fp32 out", "rotation_copies": copies, "sanity_worst_ratio": worst,
                "frac_hbm": out["kernel_gbs"] / HBM_PEAK_GBS,
                "frac_stream_read_probe": out["kernel_gbs"] / measure_read_ceiling()["gbs"]})
    del packs
    torch.cuda.empty_cache()
    return out


def run_nf4_prefill_gemm(k_steps, warmup, copies=16):
    """NF4 prefill GEMM, 32 positions, 32B-class FFN: up 27648x5120 and down 5120x27648."""
    import torch
    import synth
    import weight_streaming_linear_amd as wsl
    m = 32
    mats = [("up", 27648, 5120), ("down", 5120, 27648)]
    xs = [synth.device_normal_bf16(3, 2 + j, (m, k)) for j, (_, n, k) in enumerate(mats)]
    ys = [torch.empty((m, n), dtype=torch.float32, device="cuda") for (_, n, _) in mats]
    wss = [torch.empty(max(16, wsl.linear_gemm_workspace_bytes(wsl.WSL_W_NF4, n, k, m)), dtype=torch.uint8,
                       device="cuda") for (_, n, k) in mats]
    packs = []
    worst = 0.0
    for c in range(copies):
        pc = []
        for j, (name, n, k) in enumerate(mats):
            w = synth.device_weight(3, 100 * c + j, n, k)
            p = wsl.nf4_pack(w)
            if c == 0:
                wsl.linear_gemm(p, xs[j], y=ys[j], wfmt=wsl.WSL_W_NF4, n_out=n, k=k, workspace=wss[j])
                OUTPUT_SHA[f"nf4_prefill_gemm_m32_{name}"] = sha256_of([ys[j]])
                cols = sample_rows(n, 48, 21 + j)
                t = nf4_rows_tile(p, n, k, cols).float()
                xf = xs[j].float()
                worst = max(worst, check_close(f"nf4 prefill gemm {name}", ys[j][:, torch.as_tensor(cols, device="cuda")],
                                               xf @ t.t().contiguous(), xf.abs() @ t.abs().t().contiguous(), 1e-4))
            pc.append(p)
            del w
        packs.append(pc)
    steps = [[Launch(lambda p=pc[j], j=j, n=n, k=k: wsl.linear_gemm(p, xs[j], y=ys[j], wfmt=wsl.WSL_W_NF4, n_out=n,
                                                                      k=k, workspace=wss[j]),
                     nbytes=wsl.nf4_packed_bytes(n, k), flops=2 * m * n * k, name=f"nf4_gemm_{name}",
                     dispatches=2 if wsl.linear_gemm_workspace_bytes(wsl.WSL_W_NF4, n, k, m) > 0 else 1)
              for j, (name, n, k) in enumerate(mats)] for pc in packs]
    out = summarize(time_step_launches(steps, k_steps, warmup))
    ai = out["flops_per_step"] / out["bytes_per_step"]
    roof = min(MFMA_BF16_PEAK_TFLOPS, ai * HBM_PEAK_GBS / 1e3)
    out.update({"workload": "NF4 GEMM M=32: up 27648x5120 and down 5120x27648, fp32 out", "rotation_copies": copies,
                "sanity_worst_ratio": worst, "frac_mfma": out["kernel_tflops"] / MFMA_BF16_PEAK_TFLOPS,
                "roofline_tflops": roof, "frac_roofline": out["kernel_tflops"] / roof,
                "frac_hbm": out["kernel_gbs"] / HBM_PEAK_GBS})
    del packs
    torch.cuda.empty_cache()
    return out


def run_bf16_verify_gemm(k_steps, warmup, copies=2):
    """bf16 batch-verification GEMM, 8192 positions: gate 17408x5120 and down 5120x17408, bf16 out."""
    import torch
    import synth
    import weight_streaming_linear_amd as wsl
    m = 8192
    mats = [("gate", 17408, 5120), ("down", 5120, 17408)]
    xs = [synth.device_normal_bf16(4, 2 + j, (m, k)) for j, (_, n, k) in enumerate(mats)]
    ys = [torch.empty((m, n), dtype=torch.bfloat16, device="cuda") for (_, n, _) in mats]
    ws = [[synth.device_weight(4, 10 * c + j, n, k) for j, (_, n, k) in enumerate(mats)] for c in range(copies)]
    worst = 0.0
    for j, (name, n, k) in enumerate(mats):
        wsl.linear_gemm(ws[0][j], xs[j], y=ys[j], ofmt=wsl.WSL_OUT_BF16)
        rows = torch.as_tensor(sample_rows(m, 24, 31 + j), device="cuda")
        cols = torch.as_tensor(sample_rows(n, 48, 41 + j), device="cuda")
        xf = xs[j][rows].float()
        wf = ws[0][j][cols].float()
        got = ys[j][rows][:, cols]
        worst = max(worst, check_close(f"bf16 verify gemm {name}", got, xf @ wf.t().contiguous(),
                                       xf.abs() @ wf.abs().t().contiguous(), 1e-4, ulp_rel=2.0 ** -8))
        OUTPUT_SHA[f"bf16_verify_gemm_m8192_{name}"] = sha256_of([ys[j]])
    steps = [[Launch(lambda w=wc[j], j=j: wsl.linear_gemm(w, xs[j], y=ys[j], ofmt=wsl.WSL_OUT_BF16),
                     nbytes=2 * n * k, flops=2 * m * n * k, name=f"bf16_gemm_{name}")
              for j, (name, n, k) in enumerate(mats)] for wc in ws]
    out = summarize(time_step_launches(steps, k_steps, warmup))
    out.update({"workload": "bf16 GEMM M=8192: gate 17408x5120 and down 5120x17408, bf16 out",
                "sanity_worst_ratio": worst, "frac_mfma": out["kernel_tflops"] / MFMA_BF16_PEAK_TFLOPS})
    # Context, not a target: the vendor library (torch.matmul, hipBLASLt) on the same shapes
    # and inputs, W^T made contiguous first, bf16 out; timed with events, 10 calls after 3.
    vendor = {}
    for j, (name, n, k) in enumerate(mats):
        wt = ws[0][j].t().contiguous()
        for _ in range(3):
            torch.matmul(xs[j], wt, out=ys[j])
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(10):
            torch.matmul(xs[j], wt, out=ys[j])
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 100.0
        vendor[name] = {"avg_us": round(us, 1), "tflops": round(2 * m * n * k / us / 1e6, 1)}
        del wt
    out["vendor_blas_reference"] = {"what": "torch.matmul (hipBLASLt) on the same shapes, W^T contiguous, bf16 out",
                                    **vendor}
    del ws, xs, ys
    torch.cuda.empty_cache()
    return out


def run_nf4_embed_rows(k_steps, warmup):
    """Packed embedding rows: restore 1 row (a decode step) and 2048 rows (a prefill) of a
    packed NF4 [128000][5120] table to bf16; ids are random and change every launch."""
    import torch
    import synth
    import weight_streaming_linear_amd as wsl
    n_rows, k = 128000, 5120
    w = synth.device_weight(5, 0, n_rows, k)
    packed = wsl.nf4_pack(w)
    del w
    out = {}
    for count in (1, 2048):
        idss = [torch.randint(0, n_rows, (count,), dtype=torch.int64, device="cuda",
                              generator=torch.Generator(device="cuda").manual_seed(c)) for c in range(8)]
        ys = torch.empty((count, k), dtype=torch.bfloat16, device="cuda")
        wsl.nf4_embed_rows(packed, n_rows, k, idss[0], out=ys)
        t = nf4_rows_tile(packed, n_rows, k, idss[0].cpu().numpy()[:4])
        if not torch.equal(ys[:4], t):
            refuse(f"nf4 embed rows count {count}", float("inf"))
        OUTPUT_SHA[f"nf4_embed_rows_{count}"] = sha256_of([ys])
        nbytes = count * (k // 2 + (k // 64) * 2) + count * k * 2      # packed rows read + bf16 rows written
        launches = [Launch(lambda ids=ids: wsl.nf4_embed_rows(packed, n_rows, k, ids, out=ys), nbytes=nbytes,
                           name=f"rows_{count}") for ids in idss]
        us = time_block(launches, k_steps, warmup, label=f"nf4_embed_rows_{count}")
        out[f"rows_{count}"] = {"avg_us": round(us, 3), "gbs": round(nbytes / 1e3 / us, 1)}
    out["workload"] = "NF4 embedding row gather, table 128000x5120 (348 MB packed), bf16 out"
    del packed
    torch.cuda.empty_cache()
    return out


def run_copyring_decode_sweep(k_steps, warmup, layers=48, resident_layers=29):
    """The 48-layer NF4 decode sweep with the packed matrices in page-locked host memory,
    streamed through two device slots (linear_gemv_streamed, paced): every layer from the host, and
    a split with the first `resident_layers` layers on the device (about 6/10 of the weight
    bytes, like a model that overflows the device budget).  Tokens are timed between events on
    the compute stream; the host-to-device rate of a plain 1 GiB pinned copy is the reference."""
    import torch
    import synth
    import weight_streaming_linear_amd as wsl
    xs = [synth.device_normal_bf16(2, 1000 + j, (k,)) for j, (_, n, k) in enumerate(SWEEP_6144)]
    ys = [torch.empty(n, dtype=torch.float32, device="cuda") for (_, n, _) in SWEEP_6144]
    t0 = time.time()
    host, dev = [], []
    for l in range(layers):
        for j, (name, n, k) in enumerate(SWEEP_6144):
            w = synth.device_weight(2, 16 * l + j, n, k)
            p = wsl.nf4_pack(w)
            del w
            host.append((wsl.to_pinned(p), n, k))
            dev.append(p if l < resident_layers else None)
    torch.cuda.synchronize()
    log(f"copy ring: {layers} layers packed and pinned in {time.time() - t0:.1f}s")
    # reference: plain pinned host -> device copy of 1 GiB
    hbuf = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
    dbuf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    for _ in range(2):
        dbuf.copy_(hbuf, non_blocking=True)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(4):
        dbuf.copy_(hbuf, non_blocking=True)
    b.record()
    torch.cuda.synchronize()
    h2d_gbs = 4 * (1 << 30) / 1e6 / a.elapsed_time(b)
    del hbuf, dbuf
    slot = max(wsl.nf4_packed_bytes(n, k) for _, n, k in SWEEP_6144)
    ring = wsl.CopyRing(slot)
    token_bytes = sum(wsl.nf4_packed_bytes(n, k) for _, n, k in host)
    stream_xs = [xs[i % 4] for i in range(len(host))]
    stream_ys = [ys[i % 4] for i in range(len(host))]

    # sanity: one streamed layer equals the resident result
    ring.gemv(host[:4], xs, ys)
    got = [y.clone() for y in ys]
    for j, (_, n, k) in enumerate(SWEEP_6144):
        wsl.linear_gemv(dev[j], xs[j], y=ys[j], wfmt=wsl.WSL_W_NF4, n_out=n, k=k)
    torch.cuda.synchronize()
    if not all(torch.equal(g, y) for g, y in zip(got, ys)):
        refuse("copy ring decode sweep", float("inf"))
    OUTPUT_SHA["copyring_layer0"] = sha256_of(got)

    def all_streamed():
        ring.gemv(host, stream_xs, stream_ys)

    nres = 4 * resident_layers

    def split():
        for i in range(nres):
            _, n, k = host[i]
            wsl.linear_gemv(dev[i], xs[i % 4], y=ys[i % 4], wfmt=wsl.WSL_W_NF4, n_out=n, k=k)
        ring.gemv(host[nres:], stream_xs[nres:], stream_ys[nres:])

    out = {"workload": "NF4 decode sweep, 48 layers of hidden 6144, packed weights in page-locked host memory, "
                       "two device slots, host paced two matrices ahead (WSL_RING_PACE)",
           "h2d_copy_gbs": round(h2d_gbs, 1), "token_bytes": token_bytes}
    for name, fn, host_bytes in (("all_streamed", all_streamed, token_bytes),
                                 ("split", split, sum(wsl.nf4_packed_bytes(n, k) for _, n, k in host[nres:]))):
        for _ in range(max(1, warmup // 2)):
            fn()
        torch.cuda.synchronize()
        steps = max(2, k_steps // 4)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        out[name] = {"ms_per_token": round(ms, 3), "tokens_per_s": round(1e3 / ms, 2),
                     "host_bytes_per_token": host_bytes, "host_gbs": round(host_bytes / 1e6 / ms, 1),
                     "frac_of_h2d_copy": round(host_bytes / 1e6 / ms / h2d_gbs, 3)}
    del host, dev, ring
    torch.cuda.empty_cache()
    return out


def run_nf4_verify_gemm(k_steps, warmup, copies=2):
    """NF4 batch-verification GEMM, 8192 positions: gate 17408x5120 and down 5120x17408 held as
    packed NF4, bf16 out (the restored tiles go straight into MFMA fragments)."""
    import torch
    import synth
    import weight_streaming_linear_amd as wsl
    m = 8192
    mats = [("gate", 17408, 5120), ("down", 5120, 17408)]
    xs = [synth.device_normal_bf16(4, 2 + j, (m, k)) for j, (_, n, k) in enumerate(mats)]
    ys = [torch.empty((m, n), dtype=torch.bfloat16, device="cuda") for (_, n, _) in mats]
    packs = []
    for c in range(copies):
        pc = []
        for j, (_, n, k) in enumerate(mats):
            w = synth.device_weight(4, 10 * c + j, n, k)
            pc.append(wsl.nf4_pack(w))
            del w
        packs.append(pc)
    worst = 0.0
    for j, (name, n, k) in enumerate(mats):
        wsl.linear_gemm(packs[0][j], xs[j], y=ys[j], wfmt=wsl.WSL_W_NF4, n_out=n, k=k, ofmt=wsl.WSL_OUT_BF16)
        rows = torch.as_tensor(sample_rows(m, 24, 51 + j), device="cuda")
        cols = sample_rows(n, 48, 61 + j)
        t = nf4_rows_tile(packs[0][j], n, k, cols).float()
        xf = xs[j][rows].float()
        got = ys[j][rows][:, torch.as_tensor(cols, device="cuda")]
        worst = max(worst, check_close(f"nf4 verify gemm {name}", got, xf @ t.t().contiguous(),
                                       xf.abs() @ t.abs().t().contiguous(), 1e-4, ulp_rel=2.0 ** -8))
        OUTPUT_SHA[f"nf4_verify_gemm_m8192_{name}"] = sha256_of([ys[j]])
    steps = [[Launch(lambda p=pc[j], j=j, n=n, k=k: wsl.linear_gemm(p, xs[j], y=ys[j], wfmt=wsl.WSL_W_NF4, n_out=n,
                                                                      k=k, ofmt=wsl.WSL_OUT_BF16),
                     nbytes=wsl.nf4_packed_bytes(n, k), flops=2 * m * n * k, name=f"nf4_gemm_{name}")
              for j, (name, n, k) in enumerate(mats)] for pc in packs]
    out = summarize(time_step_launches(steps, max(2, k_steps // 4), 2))
    out.update({"workload": "NF4 GEMM M=8192: gate 17408x5120 and down 5120x17408, bf16 out",
                "sanity_worst_ratio": worst, "frac_mfma": out["kernel_tflops"] / MFMA_BF16_PEAK_TFLOPS})
    del packs, xs, ys
    torch.cuda.empty_cache()
    return out


def run_nf4_gemm_mid_m(k_steps, warmup, n=27648, k=5120, seed=700, copies=8):
    """NF4 GEMM between the prefill and verification sizes: the 32B-class up (27648x5120) or
    down (5120x27648) projection at M = 64, 128, 256 (prefill chunks of more than 32
    positions), fp32 out, with the workspace the library asks for (a k split where it
    pays)."""
    import torch
    import synth
    import weight_streaming_linear_amd as wsl
    ms = [64, 128, 256]
    xs = [synth.device_normal_bf16(3, 40 + j, (m, k)) for j, m in enumerate(ms)]
    ys = [torch.empty((m, n), dtype=torch.float32, device="cuda") for m in ms]
    wss = [torch.empty(max(16, wsl.linear_gemm_workspace_bytes(wsl.WSL_W_NF4, n, k, m)), dtype=torch.uint8,
                       device="cuda") for m in ms]
    packs = []
    worst = 0.0
    for c in range(copies):
        w = synth.device_weight(3, seed + c, n, k)
        p = wsl.nf4_pack(w)
        del w
        if c == 0:
            cols = sample_rows(n, 48, 27)
            t = nf4_rows_tile(p, n, k, cols).float()
            for j, m in enumerate(ms):
                wsl.linear_gemm(p, xs[j], y=ys[j], wfmt=wsl.WSL_W_NF4, n_out=n, k=k, workspace=wss[j])
                xf = xs[j].float()
                worst = max(worst, check_close(f"nf4 gemm m={m}", ys[j][:, torch.as_tensor(cols, device="cuda")],
                                               xf @ t.t().contiguous(), xf.abs() @ t.abs().t().contiguous(), 1e-4))
                OUTPUT_SHA[f"nf4_gemm_{n}x{k}_m{m}"] = sha256_of([ys[j]])
        packs.append(p)
    steps = [[Launch(lambda p=p, j=j, m=m: wsl.linear_gemm(p, xs[j], y=ys[j], wfmt=wsl.WSL_W_NF4, n_out=n, k=k,
                                                           workspace=wss[j]),
                     nbytes=wsl.nf4_packed_bytes(n, k), flops=2 * m * n * k, name=f"nf4_gemm_m{m}",
                     dispatches=2 if wsl.linear_gemm_workspace_bytes(wsl.WSL_W_NF4, n, k, m) > 0 else 1)
              for j, m in enumerate(ms)] for p in packs]
    out = summarize(time_step_launches(steps, k_steps, warmup))
    for j, m in enumerate(ms):
        l = out["launches"][f"nf4_gemm_m{m}"]
        ai = 2 * m * n * k / wsl.nf4_packed_bytes(n, k)
        l["frac_roofline"] = l["tflops"] / min(MFMA_BF16_PEAK_TFLOPS, ai * HBM_PEAK_GBS / 1e3)
    out.update({"workload": f"NF4 GEMM {n}x{k} at M = 64, 128, 256, fp32 out", "rotation_copies": copies,
                "sanity_worst_ratio": worst,
                "k_splits": {str(m): wsl.linear_gemm_workspace_bytes(wsl.WSL_W_NF4, n, k, m) // (m * n * 4)
                             for m in ms}})
    del packs
    torch.cuda.empty_cache()
    return out


PATHS = [("bf16_decode_layer_5120", run_bf16_decode_layer), ("nf4_gemv_4096", run_nf4_gemv_4096),
         ("nf4_prefill_gemm_m32", run_nf4_prefill_gemm), ("nf4_gemm_mid_m_27648x5120", run_nf4_gemm_mid_m),
         ("nf4_gemm_mid_m_5120x27648", lambda ks, w: run_nf4_gemm_mid_m(ks, w, n=5120, k=27648, seed=800)),
         ("bf16_verify_gemm_m8192", run_bf16_verify_gemm),
         ("nf4_verify_gemm_m8192", run_nf4_verify_gemm), ("nf4_embed_rows_128000x5120", run_nf4_embed_rows),
         ("copyring_nf4_decode_sweep_48x6144", run_copyring_decode_sweep)]


# ---------------------------------------------------------------- CPU baseline (oracle)
def cpu_baseline(budget_s=15.0):
    """The oracle's decode GEMV on the headline workload, timed on this host's cores: one
    layer of the 48-layer stack (the same seeded weights as layer 0, drawn on the device and
    copied to the host as bf16 bits), encoded once with oracle.pack_codes (untimed: the
    encoding is offline), then passes over the layer's four matrices through
    oracle.dequant_exact + oracle.gemv_ref (fp64 levels * scales, fp64 BLAS matvec) until
    about budget_s.  Reported as packed weight GB/s, like the GPU figure, and as the token
    time it implies for the 48 layers."""
    import torch
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    mats = []
    t_pack = time.perf_counter()
    for j, (_, n, k) in enumerate(SWEEP_6144):
        w = synth.device_weight(2, j, n, k)
        bits = w.view(torch.int16).cpu().numpy().view(np.uint16)
        del w
        codes, scales = oracle.pack_codes(oracle.f32_from_bf16_bits(bits))
        x = synth.device_normal_bf16(2, 1000 + j, (k,)).view(torch.int16).cpu().numpy().view(np.uint16)
        mats.append((codes, scales, oracle.f32_from_bf16_bits(x).astype(np.float64), oracle.packed_bytes(n, k)))
    t_pack = time.perf_counter() - t_pack
    torch.cuda.empty_cache()
    done_bytes, passes = 0, 0
    t0 = time.perf_counter()
    while True:
        for codes, scales, x, nb in mats:
            oracle.gemv_ref(oracle.dequant_exact(codes, scales), x)
            done_bytes += nb
        passes += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    layer_s = dt / passes
    return {"value": done_bytes / 1e9 / dt, "unit": "GB/s", "cores": blas_threads or cores, "kind": "oracle",
            "ms_per_token_48_layers": round(1e3 * layer_s * SWEEP_LAYERS, 1),
            "sample": f"{passes} pass(es) over one layer of the headline stack (qkv 8192x6144, o 6144x6144, gate_up "
                      f"32768x6144, down 6144x16384: {sum(m[3] for m in mats)} packed bytes) through "
                      f"oracle.dequant_exact + oracle.gemv_ref (fp64), {dt:.1f} s timed; the encoding "
                      f"(oracle.pack_codes, {t_pack:.1f} s) untimed; the 48-layer token time is 48x the layer "
                      f"time; host has {cores} cores, BLAS threads {blas_threads}"}


def provenance():
    """What the line was measured with: commit (when the tree is a git checkout), a digest of
    the sources, ROCm / HIP / torch versions, the device and the host CPU."""
    import subprocess
    import torch
    info = {}
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], stdout=subprocess.PIPE, stderr=subprocess.DEVNULL,
                           text=True, timeout=10)
        info["commit"] = r.stdout.strip() or None
    except Exception:
        info["commit"] = None
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "weight_streaming_linear_amd", "csrc", "*")) +
                   glob.glob(os.path.join(ROOT, "include", "*.h")) + [os.path.abspath(__file__)])
    for f in files:
        h.update(open(f, "rb").read())
    info["source_sha256"] = h.hexdigest()
    try:
        info["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except Exception:
        info["rocm"] = None
    info["hip_runtime"] = torch.version.hip
    info["torch"] = torch.__version__
    p = torch.cuda.get_device_properties(0)
    info["device"] = {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
                      "memory_gib": round(p.total_memory / 2 ** 30, 1)}
    try:
        r = subprocess.run(["rocm-smi", "--showproductname", "--showclocks"], stdout=subprocess.PIPE,
                           stderr=subprocess.DEVNULL, text=True, timeout=20)
        keep = [l.strip() for l in r.stdout.splitlines() if any(t in l for t in ("Card SKU", "Card Series", "sclk",
                                                                                  "mclk", "fclk"))]
        info["rocm_smi"] = keep[:12]
    except Exception:
        info["rocm_smi"] = None
    try:
        info["host_cpu"] = next(l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name"))
    except Exception:
        info["host_cpu"] = None
    return info


# ---------------------------------------------------------------- HBM traffic from rocprofv3 counters
def source_sha():
    return hashlib.sha256(open(GEMV_SRC, "rb").read()).hexdigest()


def traffic_probe():
    """The launches that a counter run of this script sees: 3 elementwise copies of CALIB_BYTES
    (torch.neg into a second buffer: a kernel that reads and writes exactly CALIB_BYTES), then
    2 launches of the headline's kernel, the one-launch decode sweep over the 48-layer stack,
    and 4 launches of the largest per-stage GEMV of the 192-launch form (gate_up 32768x6144)
    on 4 of the stack's gate_up matrices.  No timing, no oracle."""
    import torch
    import weight_streaming_linear_amd as wsl
    src = torch.empty(CALIB_BYTES // 2, dtype=torch.bfloat16, device="cuda").normal_()
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    xs, packs, ys = setup_sweep()
    sw = wsl.GemvSweep([(p, xs[j], y, n, k) for (p, n, k, j), y in zip(packs, ys)])
    for _ in range(2):
        sw()
    torch.cuda.synchronize()
    if sw.status() != 0:
        raise SystemExit(f"sweep status {sw.status()}")
    for l in range(4):
        p, n, k, j = packs[4 * l + 2]
        wsl.linear_gemv(p, xs[j], y=ys[4 * l + 2], wfmt=wsl.WSL_W_NF4, n_out=n, k=k)
    torch.cuda.synchronize()
    print("traffic probe done", flush=True)


def _counter_rows(run_dir, counter):
    """(kernel name, dispatch id, value) for every dispatch in a rocprofv3 counter CSV."""
    import csv
    rows = []
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == counter:
                    rows.append((r.get("Kernel_Name", ""), r.get("Dispatch_Id", ""), float(r["Counter_Value"])))
    return rows


def _per_dispatch(rows, match):
    acc = {}
    for name, disp, v in rows:
        if match(name):
            acc[disp] = acc.get(disp, 0.0) + v
    return list(acc.values())


def traffic_summarize(fetch_dir, write_dir, commands):
    """Per-launch HBM bytes from two counter runs of --traffic-probe: the headline's sweep
    kernel (the figure the benchmark line carries) and the gate_up launch of the 192-launch
    form."""
    # calibration: the elementwise negation of CALIB_BYTES (reads and writes CALIB_BYTES)
    is_calib = lambda n: "neg_kernel" in n
    token = SWEEP_LAYERS * sum(n * k // 2 + n * (k // 64) * 2 for _, n, k in SWEEP_6144)
    gate_up = 32768 * 6144 // 2 + 32768 * (6144 // 64) * 2
    kinds = {"sweep": (lambda n: SWEEP_KERNEL_MATCH in n, token),
             "gate_up_launch": (lambda n: TEAM_KERNEL_MATCH in n, gate_up)}
    res = {"kernel": DOMINANT_KERNEL, "kernel_source_sha256": source_sha(), "commands": commands}
    for kind, (match, algo) in kinds.items():
        out = {}
        for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
            rows = _counter_rows(d, counter)
            calib = _per_dispatch(rows, is_calib)
            dom = _per_dispatch(rows, match)
            if not calib or not dom:
                raise SystemExit(f"{counter}: no calibration copy ({len(calib)}) or {kind} ({len(dom)}) rows")
            factor = (np.mean(calib) * 1024) / CALIB_BYTES
            out[counter] = {"kib_per_dispatch_raw": float(np.mean(dom)), "dispatches": len(dom),
                            "calibration_copy_kib": float(np.mean(calib)), "factor": float(factor),
                            "bytes_per_launch": float(np.mean(dom) * 1024 / factor)}
        total = out["FETCH_SIZE"]["bytes_per_launch"] + out["WRITE_SIZE"]["bytes_per_launch"]
        res[kind] = {"algorithmic_bytes_per_launch": algo, "counters": out, "bytes_per_launch": total,
                     "ratio_to_algorithmic": total / algo}
    res["bytes_per_launch"] = res["sweep"]["bytes_per_launch"]
    res["algorithmic_bytes_per_launch"] = token
    res["ratio_to_algorithmic"] = res["sweep"]["ratio_to_algorithmic"]
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))


def traffic_from_file():
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        t = json.load(open(TRAFFIC_FILE))
        return t["bytes_per_launch"] if t.get("kernel_source_sha256") == source_sha() else None
    except Exception:
        return None


# ---------------------------------------------------------------- issue/wait counters of the GEMV
def gemv_counter_summarize(run_dirs, command):
    """Markdown summary of SQ counter runs of --traffic-probe (several passes, one directory
    each): for the sweep kernel's dispatches and for the gate_up launches, the mean of every
    counter per dispatch and the ratios that say where a wave's time goes (issuing VALU /
    LDS / VMEM instructions, waiting on anything / on LDS), instructions per weight, and the
    clock.  SQ cycle counters are summed over the GPU; ratios between them need no unit."""
    import csv
    token_weights = SWEEP_LAYERS * sum(n * k for _, n, k in SWEEP_6144)
    kinds = [("sweep", SWEEP_KERNEL_MATCH, token_weights,
              "`gemv_nf4_sweep_kernel<12>`, the 48-layer decode sweep in one launch (2 launches)"),
             ("gate_up", TEAM_KERNEL_MATCH, 32768 * 6144,
              "`gemv_nf4_team_kernel<2,1,true>`, one gate_up 32768x6144 launch of the 192-launch form (4 launches)")]
    per = {kind: {} for kind, *_ in kinds}
    xccs = 8
    for d in run_dirs:
        for path in glob.glob(os.path.join(d, "**", "*agent_info.csv"), recursive=True):
            with open(path) as f:
                for a in csv.DictReader(f):
                    if a.get("Name", "").startswith("gfx"):
                        xccs = int(a["Num_Xcc"])
        disp = {kind: {} for kind, *_ in kinds}
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    for kind, match, _, _ in kinds:
                        if match not in r.get("Kernel_Name", ""):
                            continue
                        e = disp[kind].setdefault(r["Dispatch_Id"],
                                                  {"t": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
                        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        for kind in disp:
            for e in disp[kind].values():
                for c, v in e.items():
                    per[kind].setdefault(c, []).append(v)
    lines = ["# Issue and wait counters of the NF4 decode GEMV (48-layer hidden-6144 sweep; gate_up launch)", "",
             "Commands (run from the repository root on one MI355X, ROCm 7.2, rocprofv3), one pass per counter set:",
             "", "```", command, "```", "",
             f"Means per dispatch, counters summed over the GPU's {xccs} XCDs.  Summary written by "
             "`python bench.py --gemv-counter-summarize <dirs...> <command>`.", ""]
    for kind, _, weights, what in kinds:
        m = {c: float(np.mean(v)) for c, v in per[kind].items()}
        g = lambda c: m.get(c)
        lines += [f"## {what}", "", "| counter | per dispatch |", "|---|---:|"]
        for c in sorted(k for k in m if k != "t"):
            lines.append(f"| {c} | {m[c]:.4g} |")
        lines += ["", "| derived | value |", "|---|---:|"]
        if g("GRBM_GUI_ACTIVE") and g("t"):
            lines.append(f"| GRBM_GUI_ACTIVE / {xccs} / dispatch duration (counts dispatch overhead too: over-reads "
                         f"the clock on a short launch) | {g('GRBM_GUI_ACTIVE') / xccs / g('t'):.3f} GHz |")
        wc = g("SQ_WAVE_CYCLES")
        for c, w in (("SQ_ACTIVE_INST_VALU", "issuing VALU"), ("SQ_ACTIVE_INST_LDS", "issuing LDS"),
                     ("SQ_ACTIVE_INST_VMEM", "issuing VMEM"), ("SQ_ACTIVE_INST_ANY", "issuing anything"),
                     ("SQ_WAIT_ANY", "waiting on a counter (any)"), ("SQ_WAIT_INST_ANY", "waiting to issue (any)"),
                     ("SQ_WAIT_INST_LDS", "waiting to issue LDS")):
            if wc and g(c) is not None:
                lines.append(f"| share of wave time {w} ({c} / SQ_WAVE_CYCLES) | {g(c) / wc:.3f} |")
        for c in ("SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_VMEM_RD", "SQ_INSTS_SALU"):
            if g(c) is not None:
                lines.append(f"| {c} x 64 lanes per weight | {g(c) * 64 / weights:.3f} |")
        if g("SQ_LDS_BANK_CONFLICT") is not None and g("SQ_LDS_IDX_ACTIVE"):
            lines.append(f"| LDS bank conflicts / LDS active | "
                         f"{g('SQ_LDS_BANK_CONFLICT') / g('SQ_LDS_IDX_ACTIVE'):.4f} |")
        lines.append("")
    print("\n".join(lines))


# ---------------------------------------------------------------- MFMA work from rocprofv3 counters
MFMA_CASES = [("bf16", 8192, 17408, 5120), ("bf16", 8192, 5120, 17408), ("nf4", 8192, 17408, 5120),
              ("nf4", 8192, 5120, 17408), ("nf4", 32, 27648, 5120), ("nf4", 32, 5120, 27648)]


def mfma_probe():
    """The launches that an MFMA counter run of this script sees: for each GEMM case, in
    order, two launches of linear_gemm (bf16 out for M = 8192, fp32 for M = 32; the
    workspace the library asks for).  No timing, no oracle."""
    import torch
    import synth
    import weight_streaming_linear_amd as wsl
    for i, (fmt, m, n, k) in enumerate(MFMA_CASES):
        w = synth.device_weight(4, 50 + i, n, k)
        if fmt == "nf4":
            w = wsl.nf4_pack(w)
        wfmt = wsl.WSL_W_NF4 if fmt == "nf4" else wsl.WSL_W_BF16
        ofmt = wsl.WSL_OUT_BF16 if m > 32 else wsl.WSL_OUT_F32
        x = synth.device_normal_bf16(4, 60 + i, (m, k))
        nb = wsl.linear_gemm_workspace_bytes(wfmt, n, k, m)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
        for _ in range(2):
            wsl.linear_gemm(w, x, wfmt=wfmt, n_out=n, k=k, ofmt=ofmt, workspace=ws)
        torch.cuda.synchronize()
        del w, x, ws
        torch.cuda.empty_cache()
    print("mfma probe done", flush=True)


def mfma_summarize(run_dir, command):
    """Markdown summary of a counter run of --mfma-probe: per GEMM case, the MFMA flops the
    hardware counted (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512) against 2 M N K, and the matrix
    pipes' busy cycles against the GPU-active cycles.  rocprofv3 writes one value per
    counter and dispatch, summed over the XCDs (GRBM_GUI_ACTIVE too, so it is divided by
    the agent's XCD count)."""
    import csv
    simds, xccs = 1024, 8
    for path in glob.glob(os.path.join(run_dir, "**", "*agent_info.csv"), recursive=True):
        with open(path) as f:
            for a in csv.DictReader(f):
                if a.get("Name", "").startswith("gfx"):
                    simds, xccs = int(a["Simd_Count"]), int(a["Num_Xcc"])
    disp = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                name = r.get("Kernel_Name", "")
                if "wsl::gemm_" not in name and "wsl::split_reduce" not in name:
                    continue
                d = disp.setdefault(r["Dispatch_Id"], {"name": name.split("(")[0].replace("void ", ""),
                                                       "t": (int(r["Start_Timestamp"]), int(r["End_Timestamp"])),
                                                       "vals": {}})
                d["vals"][r["Counter_Name"]] = d["vals"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    # the probe's GEMM launches in order, two per case; a split reduction (no MFMA work) is
    # listed with the case whose launch it follows
    cases, idx = [], -1
    for key in sorted(disp, key=int):
        d = disp[key]
        if "split_reduce" in d["name"]:
            if cases:
                cases[-1]["reduce"] = True
            continue
        idx += 1
        if idx // 2 >= len(MFMA_CASES):
            break
        if idx % 2 == 0:
            cases.append({"case": MFMA_CASES[idx // 2], "kernel": d["name"], "launches": [], "reduce": False})
        cases[-1]["launches"].append(d)
    lines = ["# MFMA work of the GEMM kernels from hardware counters", "",
             "Command (run from the repository root on one MI355X, ROCm 7.2, rocprofv3):", "", "```", command, "```", "",
             "Per launch: counted = SQ_INSTS_VALU_MFMA_MOPS_BF16 × 512 (the counter's own flop unit), "
             f"against 2·M·N·K; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES (all {simds} SIMDs) over {simds} × the "
             f"GPU-active cycles of one XCD (GRBM_GUI_ACTIVE / {xccs}); clock = those cycles over the launch's "
             "duration in the counter run; TFLOP/s = counted flops over that duration (launches under a "
             "counter run are serialized, so these run slightly slower than in the benchmark; for launches "
             "of a few tens of µs the active-cycle count also takes in dispatch overhead, so the clock "
             "column over-reads there).  Summary "
             "written by `python bench.py --mfma-summarize <run dir> <command>`.", "",
             "| case (M × N × K) | kernel | launches | counted MFMA flop / launch | 2·M·N·K | ratio | MFMA busy | clock (GHz) | TFLOP/s |",
             "|---|---|---:|---:|---:|---:|---:|---:|---:|"]
    for c in cases:
        fmt, m, n, k = c["case"]
        algo = 2.0 * m * n * k
        ls = c["launches"]
        flops = [d["vals"].get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512 for d in ls]
        cyc = [d["vals"].get("GRBM_GUI_ACTIVE", 0.0) / xccs for d in ls]
        busy = [d["vals"].get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (simds * max(g, 1.0)) for d, g in zip(ls, cyc)]
        dur = [max(d["t"][1] - d["t"][0], 1) * 1e-9 for d in ls]
        kern = c["kernel"] + (" (+ split_reduce_kernel)" if c["reduce"] else "")
        lines.append(f"| {fmt} {m} × {n} × {k} | `{kern}` | {len(ls)} | {np.mean(flops):.4e} | {algo:.4e} | "
                     f"{np.mean(flops) / algo:.4f} | {100 * np.mean(busy):.1f} % | "
                     f"{np.mean([g / t / 1e9 for g, t in zip(cyc, dur)]):.2f} | "
                     f"{np.mean([f / t / 1e12 for f, t in zip(flops, dur)]):.0f} |")
    print("\n".join(lines))


def _trace_rows(run_dir):
    """Every dispatch of a rocprofv3 --kernel-trace --output-format csv run, in start order:
    (short kernel name, grid, workgroup, microseconds)."""
    import csv
    rows = []
    for path in glob.glob(os.path.join(run_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                name = r.get("Kernel_Name", "")
                short = "spin_kernel" if "spin_kernel" in name else name.split("(")[0].replace("void ", "")
                dims = lambda pre: "x".join(r.get(f"{pre}_{a}", "1") for a in "XYZ").replace("x1x1", "").replace(
                    "x1", "") if f"{pre}_X" in r else r.get(pre, "?")
                rows.append((int(r["Start_Timestamp"]), short, dims("Grid_Size"), dims("Workgroup_Size"),
                             (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    rows.sort()
    return [r[1:] for r in rows]


def trace_summarize(run_dir, title, command, block_log=None):
    """Markdown summary of a rocprofv3 --kernel-trace --output-format csv run of this script.
    With the block log the run wrote (--block-log), the dispatches of every timed block --
    the ones that follow its spin kernel -- are attributed to the block's workload and shape;
    the library's dispatches are also grouped by kernel and grid size.  Durations in
    microseconds."""
    rows = _trace_rows(run_dir)
    lines = [f"# {title}", "", "Command (run from the repository root on one MI355X, ROCm 7.2, rocprofv3):", "",
             "```", command, "```", ""]
    if block_log:
        blocks = json.load(open(block_log))
        # torch's spin kernel: two calibration launches come first, then one per block
        spins = [i for i, r in enumerate(rows) if r[0] == "spin_kernel"][-len(blocks):]
        lines += ["## Timed blocks", "",
                  "Each block timed by the benchmark, cut from the trace: the dispatches after the block's spin "
                  "kernel (launches x dispatches per launch).  Summary written by "
                  "`python bench.py --trace-summarize <run dir> <title> <command> <block log>`.", "",
                  "| block (workload / shape) | kernel | grid | dispatches | average (us) | min (us) | max (us) |",
                  "|---|---|---:|---:|---:|---:|---:|"]
        if len(spins) < len(blocks):
            lines.append(f"| (trace has {len(spins)} spin kernels for {len(blocks)} blocks: not attributed) |||||||")
        else:
            for (label, reps, per), si in zip(blocks, spins):
                seg = [r for r in rows[si + 1: si + 1 + reps * per] if "wsl::" in r[0]]
                kinds = {}
                for r in seg:
                    kinds.setdefault((r[0], r[1]), []).append(r[3])
                for (kname, grid), v in kinds.items():
                    lines.append(f"| {label} | `{kname}` | {grid} | {len(v)} | {np.mean(v):.3f} | {min(v):.3f} | "
                                 f"{max(v):.3f} |")
        lines.append("")
    groups = {}
    for short, grid, wg, us in rows:
        if "wsl::" in short:
            groups.setdefault((short, grid, wg), []).append(us)
    total = sum(sum(v) for v in groups.values())
    lines += ["## All library dispatches", "",
              "Grouped by kernel and grid size (one template instance serves several shapes).", "",
              "| kernel | grid | workgroup | calls | total (us) | average (us) | min (us) | max (us) | % of library time |",
              "|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for (short, grid, wg), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{short}` | {grid} | {wg} | {len(v)} | {sum(v):.1f} | {np.mean(v):.3f} | {min(v):.3f} | "
                     f"{max(v):.3f} | {100 * sum(v) / total:.2f} |")
    print("\n".join(lines))


# ---------------------------------------------------------------- main
# Figures summarised across repeats: (label, path of keys into the JSON line).
REPEAT_FIGURES = [
    ("value_gbs", ("value",)),
    ("ms_per_step", ("ms_per_step",)),
    ("dominant_kernel_gbs", ("roofline", "achieved")),
    ("stream_read_probe_gbs", ("stream_read_probe", "gbs")),
    ("graph_192_launches_ms_per_token", ("headline_detail", "graph_192_launches", "ms_per_token")),
    ("bf16_layer_fused_gbs", ("paths", "bf16_decode_layer_5120", "fused", "gbs")),
    ("nf4_gemv_4096_us", ("paths", "nf4_gemv_4096", "launches", "nf4_gemv_4096", "avg_us")),
    ("nf4_gemm_m32_tflops", ("paths", "nf4_prefill_gemm_m32", "kernel_tflops")),
    ("bf16_gemm_m8192_tflops", ("paths", "bf16_verify_gemm_m8192", "kernel_tflops")),
    ("nf4_gemm_m8192_tflops", ("paths", "nf4_verify_gemm_m8192", "kernel_tflops")),
]


def _dig(d, keys):
    for k in keys:
        if not isinstance(d, dict) or k not in d:
            return None
        d = d[k]
    return d if isinstance(d, (int, float)) else None


def run_repeats(args):
    """The same run in args.repeats fresh processes, one at a time (this process never
    touches the GPU).  The printed line is the first run's, with value and ms_per_step
    replaced by the medians over the runs, plus a `repeats` record: for the headline and
    the main path figures every run's value, the median, the interquartile range and the
    A/A spread (max - min over the median: the runs are identical, so this is the noise
    floor the differences between versions have to exceed).  Only the first run times the
    CPU oracle."""
    import subprocess
    lines = []
    for r in range(args.repeats):
        cmd = [sys.executable, os.path.abspath(__file__), "--repeats", "1", "--steps", str(args.steps),
               "--warmup", str(args.warmup)]
        if args.no_paths:
            cmd.append("--no-paths")
        if args.only:
            cmd += ["--only", args.only]
        if args.no_cpu_baseline or r > 0:
            cmd.append("--no-cpu-baseline")
        if args.block_log and r == 0:
            cmd += ["--block-log", args.block_log]
        log(f"repeat {r + 1}/{args.repeats} in a fresh process")
        p = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
        if p.returncode != 0:
            log(f"repeat {r + 1} ended with status {p.returncode}")
            return p.returncode
        lines.append(json.loads(p.stdout.strip().splitlines()[-1]))
    rec = {"processes": len(lines), "figures": {}}
    for label, keys in REPEAT_FIGURES:
        vals = [_dig(l, keys) for l in lines]
        if any(v is None for v in vals):
            continue
        med = float(np.median(vals))
        q75, q25 = np.percentile(vals, [75, 25])
        rec["figures"][label] = {"runs": vals, "median": med, "iqr": float(q75 - q25),
                                 "aa_spread": float((max(vals) - min(vals)) / med) if med else None}
    out = lines[0]
    out["value"] = round(rec["figures"]["value_gbs"]["median"], 2)
    out["ms_per_step"] = round(rec["figures"]["ms_per_step"]["median"], 6)
    out["repeats"] = rec
    # determinism: every workload's outputs hash the same in every process
    shas = [l.get("output_sha256", {}) for l in lines]
    keys = sorted(set().union(*shas))
    differ = [k for k in keys if len({s.get(k) for s in shas}) != 1]
    out["determinism"] = {"processes": len(lines), "workloads": len(keys), "identical": not differ,
                          "what": "SHA-256 of every workload's outputs, compared across the fresh processes"}
    if differ:
        log(f"outputs differ between processes for {differ}: refusing")
        print(json.dumps({"error": "nondeterministic outputs", "workloads": differ}), flush=True)
        return 3
    print(json.dumps(out), flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-paths", action="store_true", help="only the headline workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--repeats", type=int, default=3,
                    help="fresh processes to run (one after another); the line reports medians, IQR and the "
                         "A/A spread over them (1: a single run in this process)")
    ap.add_argument("--only", default="", help="comma list of paths: " + ",".join(n for n, _ in PATHS))
    ap.add_argument("--traffic-probe", action="store_true", help="launch sequence for rocprofv3 counter runs")
    ap.add_argument("--traffic-summarize", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--mfma-probe", action="store_true", help="GEMM launch sequence for rocprofv3 MFMA counter runs")
    ap.add_argument("--mfma-summarize", nargs=2, metavar=("RUN_DIR", "COMMAND"))
    ap.add_argument("--traffic-commands", default="", help="the counter commands, recorded with the summary")
    ap.add_argument("--trace-summarize", nargs="+", metavar="ARG",
                    help="RUN_DIR TITLE COMMAND [BLOCK_LOG]: markdown summary of a rocprofv3 kernel-trace CSV run")
    ap.add_argument("--gemv-counter-summarize", nargs="+", metavar="ARG",
                    help="RUN_DIR... COMMAND: issue/wait counter summary of the dominant GEMV")
    ap.add_argument("--block-log", default="", help="write the timed blocks (label, launches, dispatches per "
                                                     "launch) to this file, for --trace-summarize")
    args = ap.parse_args()
    if args.trace_summarize:
        trace_summarize(*args.trace_summarize)
        return
    if args.gemv_counter_summarize:
        gemv_counter_summarize(args.gemv_counter_summarize[:-1], args.gemv_counter_summarize[-1])
        return
    if args.traffic_summarize:
        traffic_summarize(*args.traffic_summarize, args.traffic_commands)
        return
    if args.mfma_summarize:
        mfma_summarize(*args.mfma_summarize)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): it measures the kernels on a "
              "single MI355X and has no multi-GPU path. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.repeats > 1 and not args.traffic_probe and not args.mfma_probe:
        sys.exit(run_repeats(args))

    import torch
    import weight_streaming_linear_amd as wsl
    wsl.lib()
    if args.traffic_probe:
        traffic_probe()
        return
    if args.mfma_probe:
        mfma_probe()
        return
    props = torch.cuda.get_device_properties(0)
    log(f"device {props.name} ({getattr(props, 'gcnArchName', '?')}), {props.multi_processor_count} CUs")

    head = measure_headline(args.steps, args.warmup)
    value = head["token_bytes"] / 1e9 / (head["ms_per_token"] / 1e3)
    achieved = head["token_bytes"] / 1e3 / head["sweep_us"]   # one sweep launch per token
    gate_up = head["gate_up_bytes"] / 1e3 / head["gate_up_avg_us"]
    log(f"nf4 decode sweep: {head['ms_per_token']:.3f} ms/token (one launch), {value:.0f} GB/s; 192-launch graph "
        f"{head['graph_192_launches']['ms_per_token']:.3f} ms/token; gate_up launch "
        f"{head['gate_up_avg_us']:.2f} us = {gate_up:.0f} GB/s")

    probe = measure_read_ceiling()
    log(f"stream-read probe: {probe['gbs']:.0f} GB/s")

    paths = {}
    if not args.no_paths:
        only = set(filter(None, args.only.split(",")))
        for name, fn in PATHS:
            if only and name not in only:
                continue
            log(f"{name} ...")
            paths[name] = fn(20, 5)
            log(f"{name}: {json.dumps({k: v for k, v in paths[name].items() if isinstance(v, float)})}")

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_token"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,0.02) weights packed to NF4 on the device, N(0,1) bf16 activations; "
                "drawn on the device)",
        "config": {
            "workload": "NF4 decode GEMV sweep, batch 1, 48-layer stack of hidden 6144: qkv 8192x6144, o 6144x6144, "
                        "gate_up 32768x6144, down 6144x16384 per layer; 192 GEMVs per token in decoder order, "
                        "one linear_gemv_sweep launch per token (a device-wide barrier between stages)",
            "weight_format": "NF4: 4-bit codes, groups of 64 along k, one fp16 scale per group (17/32 B per weight)",
            "activations": "bf16, fp32 accumulation, fp32 outputs",
            "weight_bytes_per_token": head["token_bytes"],
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_from_file(),
            "kernel": DOMINANT_KERNEL,
            "bytes_per_launch": head["token_bytes"],
            "avg_launch_us": round(head["sweep_us"], 3),
        },
        "stream_read_probe": probe,
        "headline_detail": {
            "frac_hbm": round(value / HBM_PEAK_GBS, 4),
            "tokens_per_s": round(1e3 / head["ms_per_token"], 2),
            "frac_stream_read_probe": round(value / probe["gbs"], 4),
            "sanity_worst_ratio": head["sanity_worst_ratio"],
            "graph_form_kernel_ms_per_token": round(head["kernels"]["kernel_ms_per_step"], 5),
            "graph_form_kernels": head["kernels"]["launches"],
            "gate_up_launch_gbs": round(gate_up, 1),
            "graph_192_launches": head["graph_192_launches"],
            "decode_step_graph": head["decode_step_graph"],
            "launch_floor": head["launch_floor"],
        },
        "paths": paths,
    }
    out["provenance"] = provenance()
    out["output_sha256"] = dict(OUTPUT_SHA)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline()
    if args.block_log:
        with open(args.block_log, "w") as f:
            json.dump(BLOCK_LOG, f)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
