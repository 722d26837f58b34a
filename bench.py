#!/usr/bin/env python3
"""Benchmark of the weight-streaming linear layers on one MI355X.

Headline workload (the ``value``): batch-1 bf16 decode GEMV over one dense
decoder layer with hidden size 5120 -- q/k/v fused into one 7168x5120 matrix,
o 5120x5120, gate/up fused into one 34816x5120 matrix, down 5120x17408 --
launched in decoder order (qkv, o, gate_up, down), four launches per step.
``value`` is the effective weight stream: weight bytes read per step / wall
time per step (GB/s, 1e9 B/s), with every input resident in HBM before the
timed region starts.  Weights rotate through two distinct layer copies
(1.32 GB) so the 256 MB last-level cache cannot serve them.

The same run also measures the other workloads of the hot path (reported
under ``paths``): the NF4 GEMV 4096x4096, the 48-layer NF4 decode sweep
(hidden 6144), the NF4 prefill GEMM at 32 positions (5120 <-> 27648) and the
bf16 batch-verification GEMM at 8192 positions (5120 <-> 17408).

Protocol (IPE page, "How it is benchmarked"; deep-fold README, lab-plate
rules): a failed correctness check stops the run before timing; warm-up and
graph capture are outside every timer; per-launch durations come from HIP
events recorded on the stream the kernels run on.
"""

import argparse
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


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- timing helpers
class Launch:
    """One kernel launch of a step: a closure plus its algorithmic work."""

    def __init__(self, fn, nbytes=0, flops=0, name=""):
        self.fn, self.nbytes, self.flops, self.name = fn, nbytes, flops, name


def time_steps(steps_fn, k_steps, warmup, per_launch_events=True):
    """Run warmup steps untimed, then exactly k_steps timed ones.

    steps_fn(i) returns the list of Launch objects of step i.  Returns (wall_ms_total,
    per-launch durations in ms as a list of (launch, ms))."""
    import torch
    for i in range(warmup):
        for l in steps_fn(i):
            l.fn()
    torch.cuda.synchronize()
    recs = []
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(k_steps):
        for l in steps_fn(warmup + i):
            if per_launch_events:
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                l.fn()
                b.record()
                recs.append((l, a, b))
            else:
                l.fn()
    t1.record()
    torch.cuda.synchronize()
    wall = t0.elapsed_time(t1)
    return wall, [(l, a.elapsed_time(b)) for (l, a, b) in recs]


def summarize(wall_ms, recs, k_steps):
    nbytes = sum(l.nbytes for l, _ in recs)
    flops = sum(l.flops for l, _ in recs)
    ksum = sum(ms for _, ms in recs)
    return {
        "ms_per_step": wall_ms / k_steps,
        "kernel_ms_per_step": ksum / k_steps,
        "launches_per_step": len(recs) // k_steps,
        "bytes_per_step": nbytes // k_steps,
        "flops_per_step": flops // k_steps,
        "avg_launch_us": 1e3 * ksum / max(1, len(recs)),
        "kernel_gbs": (nbytes / 1e9) / (ksum / 1e3) if ksum > 0 else 0.0,
        "wall_gbs": (nbytes / 1e9) / (wall_ms / 1e3),
        "kernel_tflops": (flops / 1e12) / (ksum / 1e3) if ksum > 0 else 0.0,
        "wall_tflops": (flops / 1e12) / (wall_ms / 1e3),
    }


# ---------------------------------------------------------------- parity gates
def gate_rows(name, y_dev, w_rows_f64, x_f64, rows):
    import oracle
    y = y_dev.cpu().numpy()[rows]
    y_ref, s_ref = oracle.gemv_ref(w_rows_f64, x_f64)
    ok, worst, _ = oracle.check_rows_f32(y, y_ref, s_ref)
    if not ok:
        raise SystemExit(f"parity check failed for {name}: worst ratio {worst}; refusing to time")
    return worst


def bf16_rows_to_host(t, rows):
    import torch
    return t[torch.as_tensor(rows, device=t.device)].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def sample_rows(n, count, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, count)]))


# ---------------------------------------------------------------- workloads
CFG1_MATS = [("qkv", 7168, 5120), ("o", 5120, 5120), ("gate_up", 34816, 5120), ("down", 5120, 17408)]


def setup_cfg1(copies=2):
    """One dense decoder layer (hidden 5120) in bf16, `copies` distinct copies."""
    import torch
    import synth
    layers = []
    for c in range(copies):
        mats = [synth.device_weight(1, 10 * c + j, n, k) for j, (_, n, k) in enumerate(CFG1_MATS)]
        layers.append(mats)
    xs = [synth.device_normal_bf16(1, 100 + j, (k,)) for j, (_, n, k) in enumerate(CFG1_MATS)]
    ys = [torch.empty(n, dtype=torch.float32, device="cuda") for (_, n, _) in CFG1_MATS]
    return layers, xs, ys


def cfg1_steps(layers, xs, ys):
    import weight_streaming_linear_amd as wsl
    steps = []
    for mats in layers:
        st = []
        for j, (name, n, k) in enumerate(CFG1_MATS):
            st.append(Launch(lambda w=mats[j], x=xs[j], y=ys[j]: wsl.linear_gemv(w, x, y=y),
                             nbytes=2 * n * k, flops=2 * n * k, name=f"bf16_gemv_{name}"))
        steps.append(st)
    return lambda i: steps[i % len(steps)]


def gate_cfg1(layers, xs, ys):
    import torch
    import oracle
    import weight_streaming_linear_amd as wsl
    worst = 0.0
    for j, (name, n, k) in enumerate(CFG1_MATS):
        wsl.linear_gemv(layers[0][j], xs[j], y=ys[j])
        torch.cuda.synchronize()
        rows = sample_rows(n, 48, 7 + j)
        wb = bf16_rows_to_host(layers[0][j], rows)
        xb = xs[j].view(torch.int16).cpu().numpy().view(np.uint16)
        worst = max(worst, gate_rows(f"cfg1/{name}", ys[j], oracle.f32_from_bf16_bits(wb).astype(np.float64),
                                     oracle.f32_from_bf16_bits(xb).astype(np.float64), rows))
    return worst


def nf4_gate_rows(name, w_bf16_rows_bits, packed_rows_y, x_bits):
    import oracle
    wf = oracle.f32_from_bf16_bits(w_bf16_rows_bits).astype(np.float64)
    codes, scales = oracle.pack_codes(wf)
    y_ref, s_ref = oracle.gemv_ref(oracle.dequant_exact(codes, scales),
                                   oracle.f32_from_bf16_bits(x_bits).astype(np.float64))
    ok, worst, _ = oracle.check_rows_f32(packed_rows_y, y_ref, s_ref)
    if not ok:
        raise SystemExit(f"parity check failed for {name}: worst ratio {worst}; refusing to time")
    return worst


def run_cfg0(k_steps, warmup, copies=128):
    """NF4 GEMV 4096x4096 (configs[0]), 128 packed copies (1.14 GB) in rotation."""
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
        if c == 0:
            rows = sample_rows(n, 64, 3)
            wrows = bf16_rows_to_host(w, rows)
        del w
    wsl.linear_gemv(packs[0], x, y=y, wfmt=wsl.WSL_W_NF4, n_out=n, k=k)
    torch.cuda.synchronize()
    xb = x.view(torch.int16).cpu().numpy().view(np.uint16)
    worst = nf4_gate_rows("cfg0", wrows, y.cpu().numpy()[rows], xb)
    nb = wsl.nf4_packed_bytes(n, k)
    steps = [[Launch(lambda p=p: wsl.linear_gemv(p, x, y=y, wfmt=wsl.WSL_W_NF4, n_out=n, k=k), nbytes=nb,
                     flops=2 * n * k, name="nf4_gemv")] for p in packs]
    wall, recs = time_steps(lambda i: steps[i % copies], k_steps, warmup)
    out = summarize(wall, recs, k_steps)
    out.update({"workload": "NF4 GEMV 4096x4096, fp32 out", "rotation_copies": copies, "parity_worst_ratio": worst,
                "frac_hbm": out["kernel_gbs"] / HBM_PEAK_GBS})
    del packs
    torch.cuda.empty_cache()
    return out


CFG2_STAGES = [("qkv", 8192, 6144), ("o", 6144, 6144), ("gate_up", 32768, 6144), ("down", 6144, 16384)]


def run_cfg2(k_steps, warmup, layers=48):
    """48-layer NF4 decode sweep, hidden 6144 (configs[2]): 192 launches per token."""
    import torch
    import synth
    import weight_streaming_linear_amd as wsl
    xs = [synth.device_normal_bf16(2, 1000 + j, (k,)) for j, (_, n, k) in enumerate(CFG2_STAGES)]
    ys = [torch.empty(n, dtype=torch.float32, device="cuda") for (_, n, _) in CFG2_STAGES]
    packs = []
    gate_src = {}
    t_setup = time.time()
    for l in range(layers):
        for j, (name, n, k) in enumerate(CFG2_STAGES):
            w = synth.device_weight(2, 16 * l + j, n, k)
            packs.append((wsl.nf4_pack(w), n, k, j))
            if l == 0:
                rows = sample_rows(n, 32, 11 + j)
                gate_src[j] = (rows, bf16_rows_to_host(w, rows))
            del w
    torch.cuda.synchronize()
    log(f"cfg2: packed {layers} layers in {time.time() - t_setup:.1f}s")
    worst = 0.0
    for j, (name, n, k) in enumerate(CFG2_STAGES):
        p = packs[j][0]
        wsl.linear_gemv(p, xs[j], y=ys[j], wfmt=wsl.WSL_W_NF4, n_out=n, k=k)
        torch.cuda.synchronize()
        rows, wrows = gate_src[j]
        xb = xs[j].view(torch.int16).cpu().numpy().view(np.uint16)
        worst = max(worst, nf4_gate_rows(f"cfg2/{name}", wrows, ys[j].cpu().numpy()[rows], xb))
    launches = [Launch(lambda p=p, n=n, k=k, j=j: wsl.linear_gemv(p, xs[j], y=ys[j], wfmt=wsl.WSL_W_NF4, n_out=n, k=k),
                       nbytes=wsl.nf4_packed_bytes(n, k), flops=2 * n * k, name=f"nf4_gemv_{CFG2_STAGES[j][0]}")
                for (p, n, k, j) in packs]
    wall, recs = time_steps(lambda i: launches, k_steps, warmup)
    out = summarize(wall, recs, k_steps)
    # the same sweep replayed as one captured graph per token
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
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(k_steps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    graph_ms = a.elapsed_time(b) / k_steps
    out.update({
        "workload": "NF4 decode sweep, 48 layers x (qkv 8192x6144, o 6144x6144, gate_up 32768x6144, down 6144x16384)",
        "parity_worst_ratio": worst, "frac_hbm": out["kernel_gbs"] / HBM_PEAK_GBS,
        "graph_ms_per_token": graph_ms, "graph_tokens_per_s": 1e3 / graph_ms,
        "graph_gbs": out["bytes_per_step"] / 1e9 / (graph_ms / 1e3),
        "eager_tokens_per_s": 1e3 / out["ms_per_step"],
        "launch_gap_us_per_launch": 1e3 * (graph_ms - out["kernel_ms_per_step"]) / out["launches_per_step"],
    })
    del g, packs, launches
    torch.cuda.empty_cache()
    return out


def run_cfg3(k_steps, warmup, copies=16):
    """NF4 prefill GEMM, 32 positions, 32B-class FFN (configs[3])."""
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
                import oracle
                wsl.linear_gemm(p, xs[j], y=ys[j], wfmt=wsl.WSL_W_NF4, n_out=n, k=k, workspace=wss[j])
                torch.cuda.synchronize()
                cols = sample_rows(n, 48, 21 + j)
                wf = oracle.f32_from_bf16_bits(bf16_rows_to_host(w, cols)).astype(np.float64)
                codes, scales = oracle.pack_codes(wf)
                t = oracle.f32_from_bf16_bits(oracle.dequant_tile_bits(codes, scales)).astype(np.float64)
                xf = oracle.f32_from_bf16_bits(xs[j].view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
                y_ref, s_ref = oracle.gemm_ref(xf, t)
                ok, wr, _ = oracle.check_rows_f32(ys[j].cpu().numpy()[:, cols], y_ref, s_ref)
                if not ok:
                    raise SystemExit(f"parity check failed for cfg3/{name}: worst {wr}; refusing to time")
                worst = max(worst, wr)
            pc.append(p)
            del w
        packs.append(pc)
    steps = [[Launch(lambda p=pc[j], j=j, n=n, k=k: wsl.linear_gemm(p, xs[j], y=ys[j], wfmt=wsl.WSL_W_NF4, n_out=n,
                                                                      k=k, workspace=wss[j]),
                     nbytes=wsl.nf4_packed_bytes(n, k), flops=2 * m * n * k, name=f"nf4_gemm_{name}")
              for j, (name, n, k) in enumerate(mats)] for pc in packs]
    wall, recs = time_steps(lambda i: steps[i % copies], k_steps, warmup)
    out = summarize(wall, recs, k_steps)
    ai = out["flops_per_step"] / out["bytes_per_step"]
    roof = min(MFMA_BF16_PEAK_TFLOPS, ai * HBM_PEAK_GBS / 1e3)
    out.update({"workload": "NF4 GEMM M=32: up 27648x5120 and down 5120x27648, fp32 out", "rotation_copies": copies,
                "parity_worst_ratio": worst, "frac_mfma": out["kernel_tflops"] / MFMA_BF16_PEAK_TFLOPS,
                "roofline_tflops": roof, "frac_roofline": out["kernel_tflops"] / roof,
                "frac_hbm": out["kernel_gbs"] / HBM_PEAK_GBS})
    del packs
    torch.cuda.empty_cache()
    return out


def run_cfg4(k_steps, warmup, copies=2):
    """bf16 batch-verification GEMM, 8192 positions (configs[4]), bf16 out."""
    import torch
    import synth
    import oracle
    import weight_streaming_linear_amd as wsl
    m = 8192
    mats = [("gate", 17408, 5120), ("down", 5120, 17408)]
    xs = [synth.device_normal_bf16(4, 2 + j, (m, k)) for j, (_, n, k) in enumerate(mats)]
    ys = [torch.empty((m, n), dtype=torch.bfloat16, device="cuda") for (_, n, _) in mats]
    ws = [[synth.device_weight(4, 10 * c + j, n, k) for j, (_, n, k) in enumerate(mats)] for c in range(copies)]
    worst = 0.0
    for j, (name, n, k) in enumerate(mats):
        wsl.linear_gemm(ws[0][j], xs[j], y=ys[j], ofmt=wsl.WSL_OUT_BF16)
        torch.cuda.synchronize()
        rows = sample_rows(m, 24, 31 + j)
        cols = sample_rows(n, 48, 41 + j)
        xf = oracle.f32_from_bf16_bits(bf16_rows_to_host(xs[j], rows)).astype(np.float64)
        wf = oracle.f32_from_bf16_bits(bf16_rows_to_host(ws[0][j], cols)).astype(np.float64)
        y_ref, s_ref = oracle.gemm_ref(xf, wf)
        got = ys[j].view(torch.int16).cpu().numpy().view(np.uint16)[np.ix_(rows, cols)]
        ok, wr, _ = oracle.check_bf16(got, y_ref, s_ref)
        if not ok:
            raise SystemExit(f"parity check failed for cfg4/{name}: worst {wr}; refusing to time")
        worst = max(worst, wr)
    steps = [[Launch(lambda w=wc[j], j=j: wsl.linear_gemm(w, xs[j], y=ys[j], ofmt=wsl.WSL_OUT_BF16),
                     nbytes=2 * n * k, flops=2 * m * n * k, name=f"bf16_gemm_{name}")
              for j, (name, n, k) in enumerate(mats)] for wc in ws]
    wall, recs = time_steps(lambda i: steps[i % copies], k_steps, warmup)
    out = summarize(wall, recs, k_steps)
    out.update({"workload": "bf16 GEMM M=8192: gate 17408x5120 and down 5120x17408, bf16 out",
                "parity_worst_ratio": worst, "frac_mfma": out["kernel_tflops"] / MFMA_BF16_PEAK_TFLOPS})
    del ws, xs, ys
    torch.cuda.empty_cache()
    return out


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
    mats = [(synth.weight_bits(1, j, n, k), synth.act_bits(1, 100 + j, (k,))) for j, (_, n, k) in enumerate(CFG1_MATS)]
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


# ---------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-paths", action="store_true", help="only the headline workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="", help="comma list of paths to run (cfg0,cfg2,cfg3,cfg4)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the weight-streaming kernels run on a single MI355X; "
              "multi-GPU sharding is described in DESIGN.md but not built. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import weight_streaming_linear_amd as wsl
    wsl.lib()
    props = torch.cuda.get_device_properties(0)
    log(f"device {props.name} ({getattr(props, 'gcnArchName', '?')}), {props.multi_processor_count} CUs")

    # headline: configs[1]
    layers, xs, ys = setup_cfg1(copies=2)
    worst = gate_cfg1(layers, xs, ys)
    log(f"cfg1 parity ok (worst ratio {worst:.3g})")
    steps_fn = cfg1_steps(layers, xs, ys)
    wall, recs = time_steps(steps_fn, args.steps, args.warmup)
    head = summarize(wall, recs, args.steps)
    value = head["bytes_per_step"] / 1e9 / (head["ms_per_step"] / 1e3)
    avg_launch_s = head["avg_launch_us"] / 1e6
    bytes_per_launch = head["bytes_per_step"] / head["launches_per_step"]
    achieved = bytes_per_launch / 1e9 / avg_launch_s
    log(f"cfg1: {head['ms_per_step'] * 1e3:.1f} us/step, {value:.0f} GB/s wall, {achieved:.0f} GB/s kernel")
    del layers
    torch.cuda.empty_cache()

    paths = {}
    if not args.no_paths:
        only = set(filter(None, args.only.split(",")))
        for name, fn in [("cfg0", run_cfg0), ("cfg2", run_cfg2), ("cfg3", run_cfg3), ("cfg4", run_cfg4)]:
            if only and name not in only:
                continue
            log(f"{name} ...")
            paths[name] = fn(20, 5)
            log(f"{name}: {json.dumps({k: v for k, v in paths[name].items() if isinstance(v, float)})}")

    traffic = None
    tfile = os.path.join(ROOT, "profiles", "traffic_gemv_bf16_cfg1.json")
    if os.path.exists(tfile):
        try:
            t = json.load(open(tfile))
            src_hash = t.get("kernel_source_sha256")
            import hashlib
            cur = hashlib.sha256(open(os.path.join(ROOT, "weight_streaming_linear_amd", "csrc", "gemv.hip"),
                                      "rb").read()).hexdigest()
            if src_hash == cur:
                traffic = t.get("bytes_per_launch")
        except Exception:
            traffic = None

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
                        "qkv 7168x5120, o 5120x5120, gate_up 34816x5120, down 5120x17408 (4 launches/step)",
            "weight_bytes_per_step": head["bytes_per_step"],
            "rotation_bytes": 2 * head["bytes_per_step"],
            "parallelism": "single GPU",
            "device": props.name,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "gemv_bf16_kernel",
            "bytes_per_launch": bytes_per_launch,
            "avg_launch_us": round(head["avg_launch_us"], 3),
        },
        "paths": paths,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
