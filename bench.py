#!/usr/bin/env python3
"""Benchmark of the weight-streaming linear layers on one MI355X.

Headline workload (``value``): batch-1 bf16 decode GEMV over one dense decoder
layer with hidden size 5120 -- q/k/v fused into one 7168x5120 matrix, o
5120x5120, gate/up fused into one 34816x5120 matrix, down 5120x17408 -- four
launches per step in decoder order.  The W warm-up steps and then the K timed
steps are each captured as one HIP graph, the way a decode step's graph holds
every layer of a model (the time with one graph launch per step is reported
beside it).  ``value`` is the effective weight stream: weight bytes read per
step / wall time per step (GB/s, 1e9 B/s), every input resident in HBM before
the timed region starts.  Steps alternate between two distinct copies of the
layer (1.32 GB) so that the 256 MB last-level cache cannot serve the weights.

``roofline`` describes the dominant kernel, the gate/up GEMV (34816x5120, the
largest matrix of the step): its algorithmic bytes per launch divided by its
average launch duration, measured as a block of K back-to-back launches
(alternating the two copies) between one pair of HIP events on the launch
stream.  ``traffic`` is the
HBM bytes per launch read from rocprofv3 FETCH_SIZE/WRITE_SIZE counter runs of
this script (``--traffic-probe``), scaled by what the same counters read for a
plain copy of known size; it is null when the kernel source changed since the
counters were taken.

The same run measures the other workloads of the hot path (under ``paths``):
the NF4 GEMV 4096x4096, the 48-layer NF4 decode sweep (hidden 6144), the NF4
prefill GEMM at 32 positions (5120 <-> 27648) and the bf16 batch-verification
GEMM at 8192 positions (5120 <-> 17408).

GEMV figures are also given against ``read_ceiling``, the rate of a read-only
streaming kernel (``wsl_stream_read``) over 2 GiB on the same box.

Protocol (IPE page, "How it is benchmarked"; deep-fold README, lab-plate
rules): a failed correctness check stops the run before timing; warm-up and
graph capture are outside every timer.  By default the whole run is repeated in
three fresh processes, one after another: the line is the first run's with the
headline value and ms_per_step replaced by the medians, and ``repeats`` holds
every run's figures with their median, interquartile range and A/A spread.
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_bf16_gate_up_34816x5120.json")
DOMINANT = "gate_up"
CALIB_BYTES = 1 << 30            # plain copy used to calibrate the byte counters


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- timing helpers
class Launch:
    """One kernel launch of a step: a closure plus its algorithmic work."""

    def __init__(self, fn, nbytes=0, flops=0, name=""):
        self.fn, self.nbytes, self.flops, self.name = fn, nbytes, flops, name


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


def time_block(launches, reps, warmup):
    """Average duration of one launch: `warmup` untimed launches, then `reps` launches back to
    back (cycling through `launches`) between one pair of HIP events on the current stream,
    the one the launches use.  A spin kernel queued first keeps the GPU busy while the host
    enqueues the block, so the span holds the kernels and nothing of the host.  (An event
    pair around every single launch would add about 2 us of command-processor overhead to
    each measured launch on this platform.)  Returns microseconds per launch."""
    import torch
    for i in range(warmup):
        launches[i % len(launches)].fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    launches[0].fn()
    torch.cuda.synchronize()
    host_ms = 1e3 * (time.perf_counter() - t0)
    torch.cuda._sleep(int((2.0 * host_ms * reps + 2.0) * spin_cycles_per_ms()))
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
    return {name: (time_block(ls, k_steps, warmup), ls[0]) for name, ls in kinds.items()}


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
    """Streaming-read ceiling of the GPU: wsl_stream_read (16-byte loads that bypass the
    caches, 4 KB of consecutive bytes per wave and iteration) over a 2 GiB buffer, 8x the
    MALL, timed as one block of launches between HIP events."""
    import torch
    import weight_streaming_linear_amd as wsl
    if "gbs" not in READ_CEILING:
        buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        us = time_block([Launch(lambda: wsl.stream_read(buf, sink))], reps, 3)
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
        LAUNCH_FLOOR["us"] = round(time_block([Launch(lambda: wsl.stream_read(buf, sink))], reps, 10), 3)
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


# ---------------------------------------------------------------- headline: bf16 decode layer
LAYER_5120 = [("qkv", 7168, 5120), ("o", 5120, 5120), ("gate_up", 34816, 5120), ("down", 5120, 17408)]


def setup_layer_5120(copies=2):
    """One dense decoder layer (hidden 5120) in bf16, `copies` distinct copies."""
    import torch
    import synth
    import weight_streaming_linear_amd as wsl
    layers = [[synth.device_weight(1, 10 * c + j, n, k) for j, (_, n, k) in enumerate(LAYER_5120)]
              for c in range(copies)]
    xs = [synth.device_normal_bf16(1, 100 + j, (k,)) for j, (_, n, k) in enumerate(LAYER_5120)]
    ys = [torch.empty(n, dtype=torch.float32, device="cuda") for (_, n, _) in LAYER_5120]
    steps = [[Launch(lambda w=mats[j], x=xs[j], y=ys[j]: wsl.linear_gemv(w, x, y=y), nbytes=2 * n * k,
                     flops=2 * n * k, name=name) for j, (name, n, k) in enumerate(LAYER_5120)] for mats in layers]
    return layers, xs, ys, steps


def gate_layer_5120(layers, xs, ys):
    import torch
    import weight_streaming_linear_amd as wsl
    worst = 0.0
    for c, mats in enumerate(layers):
        for j, (name, n, k) in enumerate(LAYER_5120):
            wsl.linear_gemv(mats[j], xs[j], y=ys[j])
            rows = torch.as_tensor(sample_rows(n, 48, 7 + j + 10 * c), device="cuda")
            worst = max(worst, gate_gemv(f"bf16 decode layer copy {c} {name}", ys[j][rows], mats[j][rows], xs[j],
                                         1e-4))
    torch.cuda.synchronize()
    return worst


def measure_headline(k_steps, warmup):
    """The W warm-up steps and then exactly K timed steps, each step one pass over the layer's
    four matrices (alternating the two copies), the K steps captured as one graph -- as a
    decode step's graph holds every layer of the model, so no graph launch sits between
    layers.  Also: the same steps with one graph per step (a graph launch per layer), and
    block-timed kernel durations."""
    import torch
    layers, xs, ys, steps = setup_layer_5120(copies=2)
    worst = gate_layer_5120(layers, xs, ys)
    log(f"bf16 decode layer parity ok (worst ratio {worst:.3g})")
    seq = lambda n, start: [l for i in range(n) for l in steps[(start + i) % len(steps)]]
    warm = capture(seq(max(warmup, 1), 0))
    timed = capture(seq(k_steps, max(warmup, 1)))
    warm.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    timed.replay()
    b.record()
    torch.cuda.synchronize()
    gwall = a.elapsed_time(b)
    del warm, timed
    graphs = [capture(st) for st in steps]
    gwall1 = time_graphs(graphs, k_steps, warmup)
    per_kind = time_step_launches(steps, k_steps, warmup)
    per_launch = summarize(per_kind)
    out = {"ms_per_step": gwall / k_steps, "ms_per_step_one_graph_per_step": gwall1 / k_steps,
           "sanity_worst_ratio": worst, "per_launch": per_launch,
           "dominant_avg_us": per_kind[DOMINANT][0], "dominant_bytes": per_kind[DOMINANT][1].nbytes}
    del graphs, steps, layers
    torch.cuda.empty_cache()
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
    rows = sample_rows(n, 64, 3)
    # the GEMV multiplies the exact c*s, the tile is bf16(c*s): 2^-8 relative per weight at most
    worst = gate_gemv("nf4 gemv 4096", y[torch.as_tensor(rows, device="cuda")], nf4_rows_tile(packs[0], n, k, rows),
                      x, 4e-3)
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
                "frac_read_ceiling": out["kernel_gbs"] / measure_read_ceiling()["gbs"]})
    del packs
    torch.cuda.empty_cache()
    return out


SWEEP_6144 = [("qkv", 8192, 6144), ("o", 6144, 6144), ("gate_up", 32768, 6144), ("down", 6144, 16384)]


def run_nf4_decode_sweep(k_steps, warmup, layers=48):
    """48-layer NF4 decode sweep, hidden 6144: 192 launches per token, replayed as one captured
    graph per token; per-stage kernel durations from blocks of launches."""
    import torch
    import synth
    import weight_streaming_linear_amd as wsl
    xs = [synth.device_normal_bf16(2, 1000 + j, (k,)) for j, (_, n, k) in enumerate(SWEEP_6144)]
    ys = [torch.empty(n, dtype=torch.float32, device="cuda") for (_, n, _) in SWEEP_6144]
    packs = []
    t_setup = time.time()
    for l in range(layers):
        for j, (name, n, k) in enumerate(SWEEP_6144):
            w = synth.device_weight(2, 16 * l + j, n, k)
            packs.append((wsl.nf4_pack(w), n, k, j))
            del w
    torch.cuda.synchronize()
    log(f"nf4 decode sweep: packed {layers} layers in {time.time() - t_setup:.1f}s")
    worst = 0.0
    for j, (name, n, k) in enumerate(SWEEP_6144):
        wsl.linear_gemv(packs[j][0], xs[j], y=ys[j], wfmt=wsl.WSL_W_NF4, n_out=n, k=k)
        rows = sample_rows(n, 32, 11 + j)
        worst = max(worst, gate_gemv(f"nf4 decode sweep {name}", ys[j][torch.as_tensor(rows, device="cuda")],
                                     nf4_rows_tile(packs[j][0], n, k, rows), xs[j], 4e-3))
    launches = [Launch(lambda p=p, n=n, k=k, j=j: wsl.linear_gemv(p, xs[j], y=ys[j], wfmt=wsl.WSL_W_NF4, n_out=n, k=k),
                       nbytes=wsl.nf4_packed_bytes(n, k), flops=2 * n * k, name=f"nf4_gemv_{SWEEP_6144[j][0]}")
                for (p, n, k, j) in packs]
    g = capture(launches)
    graph_ms = time_graphs([g], k_steps, warmup) / k_steps
    # the same token step preceded by the packed-embedding gather of a device-resident token id
    # (hidden 6144 table of 128000 rows), the id advanced on the device inside the graph
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
    # per stage: one block of launches over the 48 layers' matrices of that stage
    out = summarize(time_step_launches([launches], 2 * layers, 4), {f"nf4_gemv_{st[0]}": layers for st in SWEEP_6144})
    out.update({
        "workload": "NF4 decode sweep, 48 layers x (qkv 8192x6144, o 6144x6144, gate_up 32768x6144, down 6144x16384)",
        "sanity_worst_ratio": worst, "frac_hbm_kernels": out["kernel_gbs"] / HBM_PEAK_GBS,
        "graph_ms_per_token": graph_ms, "graph_tokens_per_s": 1e3 / graph_ms,
        "graph_gbs": out["bytes_per_step"] / 1e9 / (graph_ms / 1e3),
        "frac_hbm_graph": out["bytes_per_step"] / 1e9 / (graph_ms / 1e3) / HBM_PEAK_GBS,
        "frac_read_ceiling_graph": out["bytes_per_step"] / 1e9 / (graph_ms / 1e3) / measure_read_ceiling()["gbs"],
        "launch_floor_ms_per_token": round(out["launches_per_step"] * measure_launch_floor()["us"] / 1e3, 4),
        "launch_gap_us_per_launch": 1e3 * (graph_ms - out["kernel_ms_per_step"]) / out["launches_per_step"],
        "decode_step_graph": {"ms_per_token": step_ms, "tokens_per_s": 1e3 / step_ms,
                              "what": "embedding gather (device-resident token id) + 192 GEMVs + id advance, one graph",
                              "allocator_growth_bytes": grew},
    })
    del g, g2, packs, launches, step_launches, emb
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
                     nbytes=wsl.nf4_packed_bytes(n, k), flops=2 * m * n * k, name=f"nf4_gemm_{name}")
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
    steps = [[Launch(lambda w=wc[j], j=j: wsl.linear_gemm(w, xs[j], y=ys[j], ofmt=wsl.WSL_OUT_BF16),
                     nbytes=2 * n * k, flops=2 * m * n * k, name=f"bf16_gemm_{name}")
              for j, (name, n, k) in enumerate(mats)] for wc in ws]
    out = summarize(time_step_launches(steps, k_steps, warmup))
    out.update({"workload": "bf16 GEMM M=8192: gate 17408x5120 and down 5120x17408, bf16 out",
                "sanity_worst_ratio": worst, "frac_mfma": out["kernel_tflops"] / MFMA_BF16_PEAK_TFLOPS})
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
        nbytes = count * (k // 2 + (k // 64) * 2) + count * k * 2      # packed rows read + bf16 rows written
        launches = [Launch(lambda ids=ids: wsl.nf4_embed_rows(packed, n_rows, k, ids, out=ys), nbytes=nbytes,
                           name=f"rows_{count}") for ids in idss]
        us = time_block(launches, k_steps, warmup)
        out[f"rows_{count}"] = {"avg_us": round(us, 3), "gbs": round(nbytes / 1e3 / us, 1)}
    out["workload"] = "NF4 embedding row gather, table 128000x5120 (348 MB packed), bf16 out"
    del packed
    torch.cuda.empty_cache()
    return out


def run_copyring_decode_sweep(k_steps, warmup, layers=48, resident_layers=29):
    """The 48-layer NF4 decode sweep with the packed matrices in page-locked host memory,
    streamed through two device slots (linear_gemv_streamed): every layer from the host, and
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

    def all_streamed():
        ring.gemv(host, stream_xs, stream_ys)

    nres = 4 * resident_layers

    def split():
        for i in range(nres):
            _, n, k = host[i]
            wsl.linear_gemv(dev[i], xs[i % 4], y=ys[i % 4], wfmt=wsl.WSL_W_NF4, n_out=n, k=k)
        ring.gemv(host[nres:], stream_xs[nres:], stream_ys[nres:])

    out = {"workload": "NF4 decode sweep, 48 layers of hidden 6144, packed weights in page-locked host memory, "
                       "two device slots", "h2d_copy_gbs": round(h2d_gbs, 1), "token_bytes": token_bytes}
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


def run_nf4_gemm_mid_m(k_steps, warmup, copies=8):
    """NF4 GEMM between the prefill and verification sizes: up 27648x5120 at M = 64, 128, 256
    (prefill chunks of more than 32 positions), fp32 out."""
    import torch
    import synth
    import weight_streaming_linear_amd as wsl
    n, k = 27648, 5120
    ms = [64, 128, 256]
    xs = [synth.device_normal_bf16(3, 40 + j, (m, k)) for j, m in enumerate(ms)]
    ys = [torch.empty((m, n), dtype=torch.float32, device="cuda") for m in ms]
    wss = [torch.empty(max(16, wsl.linear_gemm_workspace_bytes(wsl.WSL_W_NF4, n, k, m)), dtype=torch.uint8,
                       device="cuda") for m in ms]
    packs = []
    worst = 0.0
    for c in range(copies):
        w = synth.device_weight(3, 700 + c, n, k)
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
        packs.append(p)
    steps = [[Launch(lambda p=p, j=j, m=m: wsl.linear_gemm(p, xs[j], y=ys[j], wfmt=wsl.WSL_W_NF4, n_out=n, k=k,
                                                           workspace=wss[j]),
                     nbytes=wsl.nf4_packed_bytes(n, k), flops=2 * m * n * k, name=f"nf4_gemm_m{m}")
              for j, m in enumerate(ms)] for p in packs]
    out = summarize(time_step_launches(steps, k_steps, warmup))
    for j, m in enumerate(ms):
        l = out["launches"][f"nf4_gemm_m{m}"]
        ai = 2 * m * n * k / wsl.nf4_packed_bytes(n, k)
        l["frac_roofline"] = l["tflops"] / min(MFMA_BF16_PEAK_TFLOPS, ai * HBM_PEAK_GBS / 1e3)
    out.update({"workload": "NF4 GEMM up 27648x5120 at M = 64, 128, 256, fp32 out", "rotation_copies": copies,
                "sanity_worst_ratio": worst})
    del packs
    torch.cuda.empty_cache()
    return out


PATHS = [("nf4_gemv_4096", run_nf4_gemv_4096), ("nf4_decode_sweep_48x6144", run_nf4_decode_sweep),
         ("nf4_prefill_gemm_m32", run_nf4_prefill_gemm), ("nf4_gemm_mid_m_27648x5120", run_nf4_gemm_mid_m),
         ("bf16_verify_gemm_m8192", run_bf16_verify_gemm),
         ("nf4_verify_gemm_m8192", run_nf4_verify_gemm), ("nf4_embed_rows_128000x5120", run_nf4_embed_rows),
         ("copyring_nf4_decode_sweep_48x6144", run_copyring_decode_sweep)]


# ---------------------------------------------------------------- CPU baseline (oracle)
def cpu_baseline(budget_s=12.0):
    """The oracle's GEMV (bf16 -> fp64 conversion + fp64 BLAS matvec) on the headline layer,
    timed on this host's cores, repeated over the 4 matrices until about budget_s."""
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    mats = [(synth.weight_bits(1, j, n, k), synth.act_bits(1, 100 + j, (k,))) for j, (_, n, k) in enumerate(LAYER_5120)]
    done_bytes = 0
    t0 = time.perf_counter()
    passes = 0
    while True:
        for wb, xb in mats:
            oracle.gemv_ref(oracle.f32_from_bf16_bits(wb), oracle.f32_from_bf16_bits(xb))
            done_bytes += wb.size * 2
        passes += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done_bytes / 1e9 / dt, "unit": "GB/s", "cores": blas_threads or cores, "kind": "oracle",
            "sample": f"{passes} pass(es) of the headline layer's 4 bf16 matrices (660.6 MB of weights each) "
                      f"through oracle.gemv_ref (bf16->fp64 + fp64 BLAS matvec), {dt:.1f} s; host has {cores} cores"}


# ---------------------------------------------------------------- HBM traffic from rocprofv3 counters
def source_sha():
    return hashlib.sha256(open(GEMV_SRC, "rb").read()).hexdigest()


def traffic_probe():
    """The launches that a counter run of this script sees: 3 elementwise copies of CALIB_BYTES
    (torch.neg into a second buffer: a kernel that reads and writes exactly CALIB_BYTES), then
    4 eager launches of the headline layer's gate_up GEMV (the only GEMV dispatches of the
    run).  No timing, no oracle."""
    import torch
    src = torch.empty(CALIB_BYTES // 2, dtype=torch.bfloat16, device="cuda").normal_()
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    _, _, _, steps = setup_layer_5120(copies=2)
    for i in range(4):
        for l in steps[i % 2]:
            if l.name == "gate_up":
                l.fn()
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
    """Per-launch HBM bytes of the dominant kernel from two counter runs of --traffic-probe."""
    # calibration: the elementwise negation of CALIB_BYTES (reads and writes CALIB_BYTES)
    is_calib = lambda n: "neg_kernel" in n
    is_dom = lambda n: "gemv_bf16_kernel" in n
    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(d, counter)
        calib = _per_dispatch(rows, is_calib)
        dom = _per_dispatch(rows, is_dom)
        if not calib or not dom:
            raise SystemExit(f"{counter}: no calibration copy ({len(calib)}) or dominant kernel ({len(dom)}) rows")
        factor = (np.mean(calib) * 1024) / CALIB_BYTES
        out[counter] = {"kib_per_dispatch_raw": float(np.mean(dom)), "dispatches": len(dom),
                        "calibration_copy_kib": float(np.mean(calib)), "factor": float(factor),
                        "bytes_per_launch": float(np.mean(dom) * 1024 / factor)}
    algo = 2 * 34816 * 5120
    res = {"kernel": "gemv_bf16_kernel<2> (gate_up 34816x5120)", "kernel_source_sha256": source_sha(),
           "algorithmic_bytes_per_launch": algo, "counters": out,
           "bytes_per_launch": out["FETCH_SIZE"]["bytes_per_launch"] + out["WRITE_SIZE"]["bytes_per_launch"],
           "commands": commands}
    res["ratio_to_algorithmic"] = res["bytes_per_launch"] / algo
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


def trace_summarize(run_dir, title, command):
    """Markdown summary of a rocprofv3 --kernel-trace --output-format csv run: the library's
    dispatches grouped by kernel and grid size (one template instance serves several
    matrix shapes, which differ in grid size), durations in microseconds."""
    import csv
    groups = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                name = r.get("Kernel_Name", "")
                if "wsl::" not in name:
                    continue
                short = name.split("(")[0].replace("void ", "")
                us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                dims = lambda pre: "x".join(r.get(f"{pre}_{a}", "1") for a in "XYZ").replace("x1x1", "").replace(
                    "x1", "") if f"{pre}_X" in r else r.get(pre, "?")
                key = (short, dims("Grid_Size"), dims("Workgroup_Size"))
                groups.setdefault(key, []).append(us)
    total = sum(sum(v) for v in groups.values())
    lines = [f"# {title}", "", "Command (run from the repository root on one MI355X, ROCm 7.2, rocprofv3):", "",
             "```", command, "```", "",
             "Library dispatches of the run, grouped by kernel and grid size (work-items); durations "
             "in microseconds from the kernel trace.  Summary written by "
             "`python bench.py --trace-summarize <run dir> <title> <command>`.", "",
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
    ("read_ceiling_gbs", ("read_ceiling", "gbs")),
    ("nf4_sweep_graph_ms_per_token", ("paths", "nf4_decode_sweep_48x6144", "graph_ms_per_token")),
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
    ap.add_argument("--trace-summarize", nargs=3, metavar=("RUN_DIR", "TITLE", "COMMAND"),
                    help="markdown summary of a rocprofv3 kernel-trace CSV run")
    args = ap.parse_args()
    if args.trace_summarize:
        trace_summarize(*args.trace_summarize)
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
    per_launch = head["per_launch"]
    value = per_launch["bytes_per_step"] / 1e9 / (head["ms_per_step"] / 1e3)
    achieved = head["dominant_bytes"] / 1e3 / head["dominant_avg_us"]
    log(f"bf16 decode layer: {head['ms_per_step'] * 1e3:.1f} us/step (graph), {value:.0f} GB/s; "
        f"kernels {per_launch['kernel_ms_per_step'] * 1e3:.1f} us/step; gate_up kernel {achieved:.0f} GB/s")

    ceiling = measure_read_ceiling()
    log(f"streaming-read ceiling: {ceiling['gbs']:.0f} GB/s")

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
        "ms_per_step": round(head["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) activations; drawn on the device)",
        "config": {
            "workload": "bf16 decode GEMV, batch 1, one dense decoder layer, hidden 5120: "
                        "qkv 7168x5120, o 5120x5120, gate_up 34816x5120, down 5120x17408 (4 launches per "
                        "step; the K timed steps replayed as one captured graph, two layer copies alternating)",
            "weight_bytes_per_step": per_launch["bytes_per_step"],
            "rotation_bytes": 2 * per_launch["bytes_per_step"],
            "parallelism": "single GPU",
            "device": props.name,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_from_file(),
            "kernel": "gemv_bf16_kernel<2> (gate_up 34816x5120)",
            "bytes_per_launch": head["dominant_bytes"],
            "avg_launch_us": round(head["dominant_avg_us"], 3),
        },
        "read_ceiling": ceiling,
        "headline_detail": {
            "ms_per_step_one_graph_per_step": round(head["ms_per_step_one_graph_per_step"], 6),
            "gbs_one_graph_per_step": round(per_launch["bytes_per_step"] / 1e9
                                            / (head["ms_per_step_one_graph_per_step"] / 1e3), 2),
            "frac_read_ceiling": round(value / ceiling["gbs"], 4),
            "dominant_frac_read_ceiling": round(achieved / ceiling["gbs"], 4),
            "sanity_worst_ratio": head["sanity_worst_ratio"],
            "kernel_ms_per_step": round(per_launch["kernel_ms_per_step"], 6),
            "launches": per_launch["launches"],
        },
        "paths": paths,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
