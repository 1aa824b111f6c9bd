"""Benchmark of the W4A16 hot path on one MI355X.

Headline (``value``): the M = 1 W4A16 linear ``y = x . w_hat^T`` over the
Llama-3-8B-shaped decode layer set (qkv, o, gate_up, down; G = 128), in GB/s
of algorithmic HBM bytes. A step is one pass over the four layers, run back
to back as a decode step runs them (the timed steps are captured in one HIP
graph), with >= 1 GiB of distinct quantized weight copies rotated so that no
cache holds the weights. ``roofline`` is the decode GEMV kernel against the 8 TB/s HBM
peak; ``roofline_prefill`` is the M = 2048 GEMM on the Gemma3-12B-shaped
layer set against the 2.5 PFLOP/s dense bf16 matrix peak (the metric's second
half). ``components`` times every other kernel and workload on its own (the
quantizer, the quantize + linear step, M = 16 decode at G = 32 and 64, the
32768-square layer, the pre-shuffled layout, W4A8, int8 weight-only) next to
a plain read-only streaming kernel at the same sizes (the achievable
ceiling). ``cpu_baseline`` times the CPU oracle on bounded samples of each
workload.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("W4A16 linear: achieved HBM GB/s (M=1) and TFLOP/s (M=2048), "
          "% of roofline")
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
MFMA_INT8_PEAK_TOPS = 5000.0    # MI355X dense int8 matrix peak
ROTATE_BYTES = 1 << 30          # rotate weight copies over >= 1 GiB
CSRC = os.path.join(ROOT, "bit_gemm_quantize_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
# device sources each kernel is compiled from (a change voids its counters;
# the launch header only declares host functions and is left out)
KERNEL_SOURCES = {
    "quantize_kernel": ["quantize.hip", "w4_device.h"],
    "quantize_kernel_fake": ["quantize.hip", "w4_device.h"],
    "quantize_batch_kernel": ["quantize.hip", "w4_device.h"],
    "gemv1_kernel": ["gemv.hip", "w4_device.h"],
    "gemv1_kernel_m2": ["gemv.hip", "w4_device.h"],
    "gemv_split_kernel_g32": ["gemv.hip", "w4_device.h"],
    "gemv_split_kernel_g64": ["gemv.hip", "w4_device.h"],
    "gemm_kernel": ["gemm.hip", "w4_device.h"],
    "gemm_kernel_ps": ["gemm.hip", "w4_device.h"],
    "quantize8_kernel": ["w8a16.hip", "w4_device.h"],
    "w8a16_gemv_rows_kernel": ["w8a16_rows.hip", "w4_rows.h", "w4_device.h"],
    "w8a16_gemm_kernel": ["w8a16.hip", "w4_device.h"],
    "w4a8_gemm_kernel": ["w4a8.hip", "w4_device.h"],
    "w4a8_gemv_rows_kernel": ["w4a8_rows.hip", "w4_rows.h", "w4_device.h"],
    "act_quant_kernel": ["w4a8.hip", "w4_device.h"],
    "read_stream_kernel": ["measure.hip", "w4_device.h"],
}
PARTS = ["all", "decode", "gemm", "step", "quantize", "fake", "gemv2", "gemv16", "square", "ps", "w4a8",
         "w8a16", "stream", "copy"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def quant_bytes(N, K, G):
    """Algorithmic bytes of one quantize pass: read W, write codes, scales, zeros."""
    return 2 * N * K + N * K // 2 + 4 * N * K // G


def linear_bytes(M, N, K, G):
    """Algorithmic bytes of one linear: codes, scales, zeros, x and y once each."""
    return N * K // 2 + 4 * N * K // G + 2 * M * K + 2 * M * N


def kernel_source_hash(kernel):
    """sha256 over the device sources a kernel is compiled from."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this kernel (FETCH_SIZE + WRITE_SIZE, each scaled by the factor the same
    counter gives for a plain elementwise kernel of known size). None when no
    summary exists or the kernel's sources changed since it was taken. The
    summary carries one machine-readable line:
      traffic: kernel=<name> sources_sha256=<hex> fetch_bytes=<B> write_bytes=<B>
    """
    try:
        names = sorted(os.listdir(PROFILES))
    except OSError:
        return None
    want = kernel_source_hash(kernel)
    for n in names:
        if not n.endswith((".md", ".txt")):
            continue
        with open(os.path.join(PROFILES, n)) as fh:
            for line in fh:
                line = line.strip().strip("`")
                if not line.startswith("traffic:"):
                    continue
                kv = dict(t.split("=", 1) for t in line[len("traffic:"):].split() if "=" in t)
                if kv.get("kernel") != kernel:
                    continue
                if kv.get("sources_sha256") != want:
                    return None
                return {"fetch_bytes_per_launch": float(kv["fetch_bytes"]),
                        "write_bytes_per_launch": float(kv["write_bytes"]),
                        "bytes_per_launch": float(kv["fetch_bytes"]) + float(kv["write_bytes"]),
                        "source": f"profiles/{n}"}
    return None


def graph_of(torch, fns):
    """Capture the launches made by fns (in order) into one HIP graph."""
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for fn in fns:
            fn()
    torch.cuda.synchronize()
    return g


def time_graphs(torch, graphs, reps, warmup=2, warm_ms=30.0, passes=3):
    """Replay the graphs round-robin; HIP events on torch's current stream
    (the stream every launch is enqueued on) around the timed replays.
    Untimed replays first: at least ``warmup`` rounds and ``warm_ms`` of the
    same work, so that the clocks have settled on this kernel. Then
    ``passes`` timed passes of ``reps`` replays each. Returns milliseconds
    per replay: the median over the passes of each pass's mean."""
    t0 = time.perf_counter()
    i = 0
    while i < warmup * len(graphs) or (time.perf_counter() - t0) * 1e3 < warm_ms:
        graphs[i % len(graphs)].replay()
        i += 1
        if i % len(graphs) == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    per = []
    for _ in range(max(1, passes)):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            graphs[i % len(graphs)].replay()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / reps)
    return sorted(per)[len(per) // 2]


def time_launches(torch, fns, reps):
    """ms per launch of fns[i % len(fns)]: one graph holding every fn once,
    replayed ceil(reps / len(fns)) times."""
    g = graph_of(torch, fns)
    n = max(2, -(-reps // len(fns)))
    ms = time_graphs(torch, [g], n) / len(fns)
    del g
    return ms


def make_weight(torch, N, K, seed, dev, outlier_cols=None):
    """Seeded synthetic weight on the device: N(0, 0.02) in fp32, cast to bf16
    (round to nearest even); optional outlier columns scaled x20 first."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    W = torch.randn((N, K), generator=g, device=dev, dtype=torch.float32) * 0.02
    if outlier_cols is not None:
        W[:, torch.as_tensor(outlier_cols, device=dev)] *= 20.0
    return W.to(torch.bfloat16)


def make_x(torch, M, K, seed, dev):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return torch.randn((M, K), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)


def rate(b, ms):
    return b / (ms * 1e-3) / 1e9


# ------------------------------------------------------------------ decode
def decode_set(torch, w4, dev, layers, M, G, seed0, reps, ps=False, outliers=False,
               kernel="", want_step=False, steps=0, warmup=0):
    """M-row linear on each layer. Per layer: one graph of >= 64 launches over
    >= 1 GiB of that layer's quantized copies (so no cache holds the weights
    and graph-launch gaps are amortized). The set back to back: a graph of
    exactly ``steps`` decode steps (the four layers, copy i % n on step i)
    after a graph of ``warmup`` steps. Returns (component dict, step timing or
    None)."""
    import workloads
    names = list(layers)
    set_bytes = sum(linear_bytes(M, N, K, G) for N, K in layers.values())

    def make_copy(name, N, K, li, r):
        oc = workloads.outlier_columns(K, seed0 + li) if outliers else None
        W = make_weight(torch, N, K, seed0 + 1000 * r + li, dev, oc)
        c, s_, z = w4.quantize_int4_grouped(W, G)
        del W
        if ps:
            c, s_ = w4.repack_int4_preshuffled(c, s_, z, G)
            z = None
        x = make_x(torch, M, K, seed0 + 500 + 1000 * r + li, dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        return (x, c, s_, z, y)

    def fn(e):
        x, c, s_, z, y = e
        if ps:
            return lambda: w4.w4a16_linear_preshuffled(x, c, s_, G, out=y)
        return lambda: w4.w4a16_linear(x, c, s_, z, G, out=y)

    per = {}
    tot_ms = 0.0
    for li, (name, (N, K)) in enumerate(layers.items()):
        b = linear_bytes(M, N, K, G)
        n_l = max(2, -(-ROTATE_BYTES // b))
        # a few distinct weights, the rest byte copies of them (the bytes a
        # launch reads do not change its time; only that they are not cached)
        base = [make_copy(name, N, K, li, r) for r in range(min(n_l, 4))]
        cps = [tuple(t.clone() if t is not None else None for t in base[r % len(base)])
               for r in range(n_l)]
        del base
        for e in cps:
            fn(e)()
        fns = [fn(e) for e in cps] * max(1, -(-64 // n_l))
        g = graph_of(torch, fns)
        ms = time_graphs(torch, [g], max(2, -(-reps // len(fns)))) / len(fns)
        del g, fns, cps
        per[name] = {"us": round(ms * 1e3, 3), "GBps": round(rate(b, ms), 1), "bytes": b,
                     "rotating_copies": n_l}
        tot_ms += ms
    comp = {
        "kernel": kernel, "bound": "hbm", "M": M, "G": G,
        "layout": "pre-shuffled" if ps else "plain",
        "avg_launch_us": round(tot_ms * 1e3 / len(layers), 3),
        "achieved_GBps": round(rate(set_bytes, tot_ms), 1),
        "frac": round(rate(set_bytes, tot_ms) / HBM_PEAK_GBS, 4),
        "bytes_per_set": set_bytes, "per_layer": per,
    }
    # the four layers back to back, as a decode step runs them
    n_cp = max(2, -(-ROTATE_BYTES // set_bytes))
    log(f"decode M={M} G={G}{' pre-shuffled' if ps else ''}: set back to back over "
        f"{n_cp} rotating copies of {set_bytes / 1e6:.1f} MB")
    copies = [{name: make_copy(name, N, K, li, r) for li, (name, (N, K)) in enumerate(layers.items())}
              for r in range(n_cp)]
    torch.cuda.synchronize()

    def step_fns(n):
        return [fn(copies[i % n_cp][name]) for i in range(n) for name in names]

    for f in step_fns(n_cp):
        f()
    comp["rotating_copies"] = n_cp
    step = None
    n_timed = max(steps, 1) if want_step else max(2 * n_cp, reps)
    g_warm = graph_of(torch, step_fns(max(warmup, 1)))
    g_time = graph_of(torch, step_fns(n_timed))
    if want_step:
        log(f"decode step: warmup {warmup}, timed {n_timed} (one graph of {n_timed} steps)")
    g_warm.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    g_time.replay()
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / n_timed
    set_ms = e0.elapsed_time(e1) / n_timed
    if want_step:
        step = {"ms": set_ms, "wall_ms": wall_ms, "bytes": set_bytes, "copies": n_cp}
    comp["set_back_to_back_us"] = round(set_ms * 1e3, 3)
    comp["set_back_to_back_GBps"] = round(rate(set_bytes, set_ms), 1)
    del g_warm, g_time, copies
    return comp, step


def warm_gpu(torch, w4, dev, seconds=1.0):
    """Sustained streaming reads for about ``seconds`` before anything is
    timed, so that the first measurement does not pay for the clocks and
    memory system coming out of idle."""
    buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    buf.fill_(0x5A)
    sink = torch.empty(64, dtype=torch.int32, device=dev)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(50):
            w4.read_stream(buf, buf.numel(), sink)
        torch.cuda.synchronize()
    del buf


def stream_ceiling(torch, w4, dev, sizes, reps):
    """The plain read-only streaming kernel over each size, rotating through a
    buffer of >= 1 GiB so that every launch reads distinct bytes."""
    def plan(b):
        b16 = b - b % 16
        step = -(-b16 // 4096) * 4096
        n = max(2, -(-ROTATE_BYTES // step) + 1)
        return b16, step, n

    total = max(n * step for _, step, n in (plan(b) for b in sizes.values()))
    buf = torch.empty(total, dtype=torch.uint8, device=dev)
    buf.fill_(0x5A)
    sink = torch.empty(64, dtype=torch.int32, device=dev)
    out = {}
    for label, b in sizes.items():
        b16, step, n = plan(b)
        offs = [i * step for i in range(n)]
        fns = [(lambda o=o: w4.read_stream(buf[o:o + b16], b16, sink)) for o in offs]
        ms = time_launches(torch, fns, max(reps, 2 * n))
        out[label] = {"us": round(ms * 1e3, 3), "GBps": round(rate(b16, ms), 1), "bytes": b16}
    del buf
    return out


# ------------------------------------------------------------------- prefill
def prefill_set(torch, w4, dev, layers, M, G, reps, ps=False, kernel=""):
    log(f"prefill M={M} G={G}{' pre-shuffled' if ps else ''}: Gemma3-12B-shaped layers")
    per = {}
    tot_ms = 0.0
    tot_f = 0
    for i, (name, (N, K)) in enumerate(layers.items()):
        W = make_weight(torch, N, K, 50 + i, dev)
        c, s_, z = w4.quantize_int4_grouped(W, G)
        del W
        if ps:
            c, s_ = w4.repack_int4_preshuffled(c, s_, z, G)
            z = None
        x = make_x(torch, M, K, 550 + i, dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        if ps:
            fn = (lambda x=x, c=c, s_=s_, y=y: w4.w4a16_linear_preshuffled(x, c, s_, G, out=y))
        else:
            fn = (lambda x=x, c=c, s_=s_, z=z, y=y: w4.w4a16_linear(x, c, s_, z, G, out=y))
        fn()
        ms = time_launches(torch, [fn], max(3, reps // 5))
        f = 2 * M * N * K
        per[name] = {"us": round(ms * 1e3, 2), "TFLOPs": round(f / (ms * 1e-3) / 1e12, 1)}
        tot_ms += ms
        tot_f += f
        del x, c, s_, z, y
    tf = tot_f / (tot_ms * 1e-3) / 1e12
    return {"kernel": kernel, "bound": "mfma", "M": M, "G": G,
            "layout": "pre-shuffled" if ps else "plain",
            "avg_launch_us": round(tot_ms * 1e3 / len(layers), 2),
            "achieved_TFLOPs": round(tf, 1), "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "flops_per_set": tot_f, "set_us": round(tot_ms * 1e3, 2), "per_layer": per}


# ------------------------------------------------------------------ oracle
def cpu_baseline(G_dec=128):
    """The CPU oracle (numpy; the quantizer single-threaded, the fp64 matmul
    on all BLAS threads) timed on bounded samples of every workload, on this
    host. The headline figure is the M = 1 linear over the whole decode set in
    GB/s of the same algorithmic bytes as ``value``."""
    import numpy as np

    import oracle
    import workloads

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()
                            if i.get("user_api") == "blas"] or [1])
    except Exception:                                   # pragma: no cover
        blas_threads = 1
    per = {}

    def timed(fn):
        t0 = time.perf_counter()
        r = fn()
        return r, time.perf_counter() - t0

    # config 1: the 512 x 512 layer, G = 32, one input row
    W1 = workloads.weight_bits(1, "linear")
    x1 = workloads.activation_bits(1, 1, 512)
    (c1, s1, z1), tq = timed(lambda: oracle.quantize_ref(W1, 32))
    _, tl = timed(lambda: oracle.linear_ref(x1, c1, s1, z1, 32))
    per["tiny_512_g32"] = {"quantize_ms": round(tq * 1e3, 3), "linear_m1_ms": round(tl * 1e3, 3)}

    # config 2: the decode set, whole layers: quantize once, then the M = 1
    # linear repeated until >= 6 s of work has been timed
    layers = dict(workloads.LLAMA3_8B)
    qs = {}
    tq_tot = 0.0
    for name in layers:
        W = workloads.weight_bits(2, name)
        qs[name], t = timed(lambda W=W: oracle.quantize_ref(W, G_dec))
        tq_tot += t
        del W
    xs = {name: workloads.activation_bits(2, 1, K) for name, (N, K) in layers.items()}
    lin_b = 0
    lin_t = 0.0
    passes = 0
    while lin_t < 6.0 and passes < 10:
        for name, (N, K) in layers.items():
            c, s_, z = qs[name]
            _, t = timed(lambda: oracle.linear_ref(xs[name], c, s_, z, G_dec))
            lin_t += t
            lin_b += linear_bytes(1, N, K, G_dec)
        passes += 1
    qb = sum(quant_bytes(N, K, G_dec) for N, K in layers.values())
    per["llama3_8b_decode_m1_g128"] = {
        "linear_GBps": round(lin_b / lin_t / 1e9, 4), "linear_passes": passes,
        "quantize_GBps": round(qb / tq_tot / 1e9, 4), "quantize_s": round(tq_tot, 2)}
    headline = lin_b / lin_t / 1e9
    del qs

    # config 3: M = 16, G = 32 and 64, outlier columns: the o layer
    N, K = layers["o"]
    for G in (32, 64):
        W = workloads.weight_bits(3, "o")
        x = workloads.activation_bits(3, 16, K)
        (c, s_, z), tq = timed(lambda: oracle.quantize_ref(W, G))
        _, tl = timed(lambda: oracle.linear_ref(x, c, s_, z, G))
        per[f"llama3_8b_m16_g{G}_o"] = {"linear_GBps": round(linear_bytes(16, N, K, G) / tl / 1e9, 4),
                                         "quantize_GBps": round(quant_bytes(N, K, G) / tq / 1e9, 4)}

    # config 4: M = 2048, G = 128: the k layer (2048 x 3840)
    N, K = dict(workloads.GEMMA3_12B)["k"]
    W = workloads.weight_bits(4, "k")
    x = workloads.activation_bits(4, 2048, K)
    c, s_, z = oracle.quantize_ref(W, 128)
    _, tl = timed(lambda: oracle.linear_ref(x, c, s_, z, 128))
    per["gemma3_12b_prefill_m2048_k"] = {"linear_TFLOPs": round(2 * 2048 * N * K / tl / 1e12, 5)}

    # config 5: 32768 x 32768, G = 64, on 1024 seeded weight rows; the full
    # size is extrapolated from the sample (labelled so)
    rows = 1024
    NS = KS = 32768
    W = workloads.weight_bits(5, "square", rows=(0, rows))
    (c, s_, z), tq = timed(lambda: oracle.quantize_ref(W, 64))
    x1 = workloads.activation_bits(5, 1, KS)
    _, tl1 = timed(lambda: oracle.linear_ref(x1, c, s_, z, 64))
    x256 = workloads.activation_bits(5, 256, KS, rows=(0, 256))
    _, tl256 = timed(lambda: oracle.linear_ref(x256, c, s_, z, 64))
    scale_n = NS / rows
    per["square_32768_g64"] = {
        "sample": f"{rows} of {NS} weight rows (quantize, M=1); 256 of 32768 x rows x "
                  f"{rows} weight rows (M=32768); full-size times extrapolated",
        "quantize_s_extrapolated": round(tq * scale_n, 2),
        "quantize_GBps": round(quant_bytes(rows, KS, 64) / tq / 1e9, 4),
        "linear_m1_s_extrapolated": round(tl1 * scale_n, 3),
        "linear_m32768_s_extrapolated": round(tl256 * scale_n * (32768 / 256), 1),
        "linear_m32768_TFLOPs": round(2 * 256 * rows * KS / tl256 / 1e12, 5)}
    del W, c, s_, z

    return {
        "value": round(headline, 4),
        "unit": "GB/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": ("numpy oracle: M=1 fp64 linear (BLAS, "
                   f"{blas_threads} threads) over the four whole decode layers, {passes} passes; "
                   "per_config: the other workloads on bounded samples (quantizer single-threaded)"),
        "per_config": per,
        "host_cpus": os.cpu_count(),
        "host_affinity": len(os.sched_getaffinity(0)),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=PARTS, default="all",
                    help="restrict to one part (for profiling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU part: every box here has one GPU)", file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_gemm_quantize_amd as w4
    import workloads

    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    w4.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    G = 128
    layers = dict(workloads.LLAMA3_8B)
    glayers = dict(workloads.GEMMA3_12B)
    out = {}
    reps = max(args.steps, 1)
    only = args.only

    def want(*parts):
        return only == "all" or only in parts

    if only != "copy":
        warm_gpu(torch, w4, dev)

    # ---- headline: M = 1 linear over the decode set --------------------------
    step = None
    if want("decode"):
        comp, step = decode_set(
            torch, w4, dev, layers, 1, G, 0, reps,
            kernel="gemv1_kernel<128, 4, false, false, 1> (qkv, o, gate_up), "
                   "gemv1_kernel<128, 4, true, false, 1> (down)",
            want_step=True, steps=max(args.steps, 1), warmup=args.warmup)
        out["gemv_m1_g128"] = comp
    if want("decode", "stream"):
        sizes = {n: linear_bytes(1, N, K, G) for n, (N, K) in layers.items()}
        sizes["square_m1"] = linear_bytes(1, 32768, 32768, 64)
        sizes["1GiB"] = 1 << 30
        ceil = stream_ceiling(torch, w4, dev, sizes, reps)
        dec = {k: v for k, v in ceil.items() if k in layers}
        set_b = sum(v["bytes"] for v in dec.values())
        set_us = sum(v["us"] for v in dec.values())
        out["read_stream_ceiling"] = {
            "kernel": "read_stream_kernel (plain read-only stream, 4 KB per wave)",
            "per_size": ceil, "decode_set_GBps": round(set_b / (set_us * 1e-6) / 1e9, 1),
            "decode_set_frac": round(set_b / (set_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}

    # ---- the metric's second half: M = 2048 GEMM -----------------------------
    if want("gemm"):
        out["gemm_m2048_g128"] = prefill_set(torch, w4, dev, glayers, 2048, G, reps,
                                             kernel="gemm_kernel<128, false, true, 128|256> (128 x 256 blocks except k, v)")

    # ---- decode step with the quantizer: quantize the four weights (one
    # batched launch) then the four M = 1 linears on the fresh codes ----------
    if want("step", "quantize"):
        set_qbytes = sum(quant_bytes(N, K, G) for N, K in layers.values())
        n_sets = max(2, -(-ROTATE_BYTES // set_qbytes))
        log(f"quantize: {n_sets} rotating copies of {set_qbytes / 1e6:.1f} MB")
        sets = []
        for r in range(n_sets):
            entry = {}
            for i, (name, (N, K)) in enumerate(layers.items()):
                W = make_weight(torch, N, K, 1000 * r + i, dev)
                entry[name] = (W, make_x(torch, 1, K, 7000 + 1000 * r + i, dev),
                               torch.empty((N, K // 2), dtype=torch.uint8, device=dev),
                               torch.empty((N, K // G), dtype=torch.bfloat16, device=dev),
                               torch.empty((N, K // G), dtype=torch.bfloat16, device=dev),
                               torch.empty((1, N), dtype=torch.bfloat16, device=dev))
            sets.append(entry)
        names = list(layers)

        def qbatch(e):
            return lambda: w4.quantize_int4_grouped_batch(
                [e[n][0] for n in names], G, outs=[(e[n][2], e[n][3], e[n][4]) for n in names])

        def lin(e, n):
            return lambda: w4.w4a16_linear(e[n][1], e[n][2], e[n][3], e[n][4], G, out=e[n][5])

        for e in sets:
            qbatch(e)()
            for n in names:
                lin(e, n)()
        if want("step"):
            g = [graph_of(torch, [qbatch(e)] + [lin(e, n) for n in names]) for e in sets]
            ms = time_graphs(torch, g, max(reps, 2 * n_sets))
            del g
            sb = set_qbytes + sum(linear_bytes(1, N, K, G) for N, K in layers.values())
            out["decode_step_quantize_and_linear"] = {
                "what": "quantize the four bf16 weights (one batched launch), then the four "
                        "M=1 linears on the fresh codes; one graph replay",
                "ms": round(ms, 5), "bytes": sb, "GBps": round(rate(sb, ms), 1)}
        qb_ms = time_launches(torch, [qbatch(e) for e in sets], max(reps, 2 * n_sets))
        out["quantize_batch_g128"] = {
            "kernel": "quantize_batch_kernel<128, 2>", "bound": "hbm",
            "avg_launch_us": round(qb_ms * 1e3, 3), "bytes_per_launch": set_qbytes,
            "achieved_GBps": round(rate(set_qbytes, qb_ms), 1),
            "frac": round(rate(set_qbytes, qb_ms) / HBM_PEAK_GBS, 4)}
        per = {}
        tot_b = 0
        tot_ms = 0.0
        for name, (N, K) in layers.items():
            fns = [(lambda e=e, n=name: w4.quantize_int4_grouped(e[n][0], G, e[n][2], e[n][3],
                                                                 e[n][4])) for e in sets]
            ms = time_launches(torch, fns, max(reps, 2 * n_sets))
            b = quant_bytes(N, K, G)
            per[name] = {"us": round(ms * 1e3, 3), "GBps": round(rate(b, ms), 1)}
            tot_b += b
            tot_ms += ms
        out["quantize_g128"] = {
            "kernel": "quantize_kernel<128, false, 2>", "bound": "hbm",
            "avg_launch_us": round(tot_ms * 1e3 / len(layers), 3),
            "achieved_GBps": round(rate(tot_b, tot_ms), 1),
            "frac": round(rate(tot_b, tot_ms) / HBM_PEAK_GBS, 4),
            "bytes_per_set": tot_b, "per_layer": per}
        del sets

    # ---- fake-quantize round trip (QAT forward weight), G = 32 ---------------
    if want("fake"):
        per = {}
        tot_b = 0
        tot_ms = 0.0
        for i, (name, (N, K)) in enumerate(layers.items()):
            n_cp = max(2, -(-ROTATE_BYTES // (4 * N * K)))
            Ws = [make_weight(torch, N, K, 3000 + 100 * r + i, dev) for r in range(n_cp)]
            wout = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
            fns = [(lambda W=W: w4.fake_quant_int4_grouped(W, 32, out=wout)) for W in Ws]
            for f in fns:
                f()
            ms = time_launches(torch, fns, max(reps, 2 * n_cp))
            b = 4 * N * K
            per[name] = {"us": round(ms * 1e3, 3), "GBps": round(rate(b, ms), 1)}
            tot_b += b
            tot_ms += ms
            del Ws, wout, fns
        out["fake_quant_g32"] = {
            "kernel": "quantize_kernel<32, true, 2>", "bound": "hbm",
            "achieved_GBps": round(rate(tot_b, tot_ms), 1),
            "frac": round(rate(tot_b, tot_ms) / HBM_PEAK_GBS, 4),
            "bytes_per_set": tot_b, "set_us": round(tot_ms * 1e3, 3), "per_layer": per}

    # ---- small-batch decode: M = 2 (vector-ALU kernel, both x rows per lane)
    # and M = 4 (matrix-core split kernel), G = 128 ------------------------------
    if want("gemv2"):
        comp, _ = decode_set(
            torch, w4, dev, layers, 2, G, 3000, reps,
            kernel="gemv1_kernel<128, 4, false, false, 2> (qkv, o, gate_up), "
                   "gemv1_kernel<128, 4, true, false, 2> (down)")
        out["gemv_m2_g128"] = comp
        comp, _ = decode_set(
            torch, w4, dev, layers, 4, G, 3000, reps,
            kernel="gemv_split_kernel<128, 8, false, false>")
        out["gemv_m4_g128"] = comp

    # ---- small-batch decode: M = 16, G = 32 and 64, outlier columns ----------
    if want("gemv16"):
        for Gs in (32, 64):
            comp, _ = decode_set(
                torch, w4, dev, layers, 16, Gs, 7000, reps, outliers=True,
                kernel=f"gemv_split_kernel<{Gs}, 8, true, false> (qkv, o, gate_up), "
                       f"gemv_direct_kernel<{Gs}, 8, false> (down)")
            out[f"gemv_m16_g{Gs}"] = comp

    # ---- the 32768-square layer, G = 64: quantize pass, M = 1, M = 32768 -----
    if want("square"):
        NS = KS = 32768
        Gq = 64
        log("square 32768^2: quantize pass, M=1 linear, M=32768 linear")
        W = make_weight(torch, NS, KS, 5, dev)
        c, s_, z = w4.quantize_int4_grouped(W, Gq)
        torch.cuda.synchronize()
        qfn = (lambda: w4.quantize_int4_grouped(W, Gq, c, s_, z))
        q_ms = time_launches(torch, [qfn], 6)
        qb = quant_bytes(NS, KS, Gq)
        del W
        c2, s2, z2 = w4.quantize_int4_grouped(make_weight(torch, NS, KS, 55, dev), Gq)
        x1 = [make_x(torch, 1, KS, 5005, dev), make_x(torch, 1, KS, 5006, dev)]
        y1 = torch.empty((1, NS), dtype=torch.bfloat16, device=dev)
        fns = [(lambda: w4.w4a16_linear(x1[0], c, s_, z, Gq, out=y1)),
               (lambda: w4.w4a16_linear(x1[1], c2, s2, z2, Gq, out=y1))]
        for f in fns:
            f()
        m1_ms = time_launches(torch, fns, 20)
        m1b = linear_bytes(1, NS, KS, Gq)
        del c2, s2, z2
        xb = make_x(torch, 32768, KS, 5007, dev)
        yb = torch.empty((32768, NS), dtype=torch.bfloat16, device=dev)
        big = (lambda: w4.w4a16_linear(xb, c, s_, z, Gq, out=yb))
        big()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(2):
            big()
        e1.record()
        torch.cuda.synchronize()
        big_ms = e0.elapsed_time(e1) / 2
        f = 2 * 32768 * NS * KS
        out["square_32768_g64"] = {
            "quantize": {"kernel": "quantize_kernel<64, false, 2>", "us": round(q_ms * 1e3, 2),
                         "bytes": qb, "GBps": round(rate(qb, q_ms), 1),
                         "frac": round(rate(qb, q_ms) / HBM_PEAK_GBS, 4)},
            "linear_m1": {"kernel": "gemv1_kernel<64, 4, true, false, 1>", "us": round(m1_ms * 1e3, 2),
                          "bytes": m1b, "GBps": round(rate(m1b, m1_ms), 1),
                          "frac": round(rate(m1b, m1_ms) / HBM_PEAK_GBS, 4)},
            "linear_m32768": {"kernel": "gemm_kernel<64, false, true, 256>", "ms": round(big_ms, 3),
                              "flops": f, "TFLOPs": round(f / (big_ms * 1e-3) / 1e12, 1),
                              "frac": round(f / (big_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}}
        del xb, yb, c, s_, z, x1, y1

    # ---- pre-shuffled layout: decode M = 1 and prefill M = 2048 --------------
    if want("ps"):
        comp, _ = decode_set(torch, w4, dev, layers, 1, G, 0, reps, ps=True,
                             kernel="gemv1_kernel<128, 4, false|true, true, 1>")
        out["gemv_m1_g128_ps"] = comp
        out["gemm_m2048_g128_ps"] = prefill_set(torch, w4, dev, glayers, 2048, G, reps, ps=True,
                                                kernel="gemm_kernel<128, true, true, 128|256> (128 x 256 blocks except k, v)")

    # ---- W4A8: per-token int8 activations + int4 weights on int8 MFMA -------
    if want("w4a8"):
        # decode: M = 1 over the Llama-3-8B-shaped set (vector-ALU row kernel),
        # each layer over >= 1 GiB of rotating copies in one graph
        per = {}
        tot_ms, tot_b = 0.0, 0
        for li, (name, (N, K)) in enumerate(layers.items()):
            b1 = N * K // 2 + 4 * N * K // G + K + 4 + 2 * N
            n_l = max(2, -(-ROTATE_BYTES // b1))
            W = make_weight(torch, N, K, 60 + li, dev)
            c, s_, z = w4.quantize_int4_grouped(W, G)
            del W
            x8, sx = w4.quantize_act_int8(make_x(torch, 1, K, 660 + li, dev))
            cps = [(c.clone(), s_.clone(), z.clone(), torch.empty((1, N), dtype=torch.bfloat16, device=dev))
                   for _ in range(n_l)]
            fns = [(lambda e=e: w4.w4a8_linear(x8, sx, e[0], e[1], e[2], G, out=e[3])) for e in cps]
            for f_ in fns:
                f_()
            fns = fns * max(1, -(-64 // n_l))
            g = graph_of(torch, fns)
            ms = time_graphs(torch, [g], max(2, -(-reps // len(fns)))) / len(fns)
            del g, fns, cps
            per[name] = {"us": round(ms * 1e3, 3), "GBps": round(rate(b1, ms), 1)}
            tot_ms += ms
            tot_b += b1
        out["w4a8_gemv_m1_g128"] = {
            "kernel": "w4a8_gemv_rows_kernel<128, 1>", "bound": "hbm",
            "avg_launch_us": round(tot_ms * 1e3 / len(layers), 3),
            "achieved_GBps": round(rate(tot_b, tot_ms), 1),
            "frac": round(rate(tot_b, tot_ms) / HBM_PEAK_GBS, 4), "per_layer": per}
        M = 2048
        for Gw in (128, 32):
            log(f"w4a8 G={Gw}: Gemma3-12B-shaped layers, M=2048")
            per = {}
            tot_ms = tot_aq_ms = 0.0
            tot_f = tot_aq_b = 0
            for i, (name, (N, K)) in enumerate(glayers.items()):
                W = make_weight(torch, N, K, 50 + i, dev)
                c, s_, z = w4.quantize_int4_grouped(W, Gw)
                del W
                x = make_x(torch, M, K, 550 + i, dev)
                x8, sx = w4.quantize_act_int8(x)
                y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
                fn = (lambda x8=x8, sx=sx, c=c, s_=s_, z=z, y=y, Gw=Gw:
                      w4.w4a8_linear(x8, sx, c, s_, z, Gw, out=y))
                fn()
                ms = time_launches(torch, [fn], max(3, reps // 5))
                ms_aq = None
                if Gw == 128:
                    # the activation quantizer over >= 1 GiB of distinct x copies,
                    # one graph of all of them (a launch of a few us is not
                    # timed alone: the graph launch itself would dominate)
                    n_x = max(2, -(-ROTATE_BYTES // (3 * M * K)))
                    xs = [(x.clone(), torch.empty_like(x8), torch.empty_like(sx)) for _ in range(n_x)]
                    aqs = [(lambda e=e: w4.quantize_act_int8(e[0], x8=e[1], sx=e[2])) for e in xs]
                    for a_ in aqs:
                        a_()
                    ms_aq = time_launches(torch, aqs, max(2 * n_x, 32))
                    del xs, aqs
                f = 2 * M * N * K
                per[name] = {"us": round(ms * 1e3, 2), "TOPs": round(f / (ms * 1e-3) / 1e12, 1)}
                if ms_aq is not None:
                    per[name]["act_quant_us"] = round(ms_aq * 1e3, 2)
                    tot_aq_ms += ms_aq
                    tot_aq_b += 3 * M * K + 4 * M
                tot_ms += ms
                tot_f += f
                del x, x8, sx, c, s_, z, y
            out[f"w4a8_gemm_m2048_g{Gw}"] = {
                "kernel": f"w4a8_gemm_kernel<{Gw}>", "bound": "mfma (int8)",
                "achieved_TOPs": round(tot_f / (tot_ms * 1e-3) / 1e12, 1),
                "frac": round(tot_f / (tot_ms * 1e-3) / 1e12 / MFMA_INT8_PEAK_TOPS, 4),
                "ops_per_set": tot_f, "set_us": round(tot_ms * 1e3, 2), "per_layer": per}
            if tot_aq_ms > 0:
                out[f"w4a8_gemm_m2048_g{Gw}"]["act_quant"] = {
                    "kernel": "act_quant_reg_kernel<2> (K = 3840, 4096), act_quant_reg_kernel<8> (K = 15360)",
                    "bound": "hbm", "achieved_GBps": round(rate(tot_aq_b, tot_aq_ms), 1),
                    "frac": round(rate(tot_aq_b, tot_aq_ms) / HBM_PEAK_GBS, 4),
                    "set_us": round(tot_aq_ms * 1e3, 2),
                    "bytes_per_set": tot_aq_b}

    # ---- int8 weight-only: quantizer, decode (M = 1) and prefill (M = 2048) --
    if want("w8a16"):
        def w8_bytes(M, N, K, Gq):
            return N * K + 2 * N * (K // Gq) + 2 * M * K + 2 * M * N

        gb8 = sum(w8_bytes(1, N, K, G) for N, K in layers.values())
        n8 = max(2, -(-ROTATE_BYTES // gb8))
        log(f"w8a16 decode: {n8} rotating copies of {gb8 / 1e6:.1f} MB")
        per = {}
        tot_ms = tot_q_ms = 0.0
        tot_b = tot_q_b = 0
        for li, (name, (N, K)) in enumerate(layers.items()):
            copies = []
            for r in range(n8):
                W = make_weight(torch, N, K, 1000 * r + li, dev)
                q8, s8 = w4.quantize_int8_grouped(W, G)
                copies.append((W, make_x(torch, 1, K, 9000 + 1000 * r + li, dev), q8, s8,
                               torch.empty((1, N), dtype=torch.bfloat16, device=dev)))
            ms = time_launches(torch, [(lambda e=e: w4.w8a16_linear(e[1], e[2], e[3], G, out=e[4]))
                                       for e in copies], max(reps, 2 * n8))
            ms_q = time_launches(torch, [(lambda e=e: w4.quantize_int8_grouped(e[0], G, e[2], e[3]))
                                         for e in copies], max(reps, 2 * n8))
            b = w8_bytes(1, N, K, G)
            bq = 3 * N * K + 2 * N * (K // G)
            per[name] = {"us": round(ms * 1e3, 3), "GBps": round(rate(b, ms), 1),
                         "quantize_us": round(ms_q * 1e3, 3), "quantize_GBps": round(rate(bq, ms_q), 1)}
            tot_ms += ms
            tot_b += b
            tot_q_ms += ms_q
            tot_q_b += bq
            del copies
        out["w8a16_gemv_m1"] = {
            "kernel": "w8a16_gemv_rows_kernel<128, 1>", "bound": "hbm",
            "avg_launch_us": round(tot_ms * 1e3 / len(layers), 3),
            "achieved_GBps": round(rate(tot_b, tot_ms), 1),
            "frac": round(rate(tot_b, tot_ms) / HBM_PEAK_GBS, 4), "bytes_per_set": tot_b,
            "per_layer": per}
        out["quantize8_g128"] = {
            "kernel": "quantize8_kernel<128>", "bound": "hbm",
            "achieved_GBps": round(rate(tot_q_b, tot_q_ms), 1),
            "frac": round(rate(tot_q_b, tot_q_ms) / HBM_PEAK_GBS, 4), "bytes_per_set": tot_q_b}
        M = 2048
        log("w8a16 prefill: Gemma3-12B-shaped layers, M=2048")
        per = {}
        tot_ms = 0.0
        tot_f = 0
        for i, (name, (N, K)) in enumerate(glayers.items()):
            W = make_weight(torch, N, K, 50 + i, dev)
            q8, s8 = w4.quantize_int8_grouped(W, G)
            del W
            x = make_x(torch, M, K, 550 + i, dev)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            fn = (lambda x=x, q8=q8, s8=s8, y=y: w4.w8a16_linear(x, q8, s8, G, out=y))
            fn()
            ms = time_launches(torch, [fn], max(3, reps // 5))
            f = 2 * M * N * K
            per[name] = {"us": round(ms * 1e3, 2), "TFLOPs": round(f / (ms * 1e-3) / 1e12, 1)}
            tot_ms += ms
            tot_f += f
            del x, q8, s8, y
        out["w8a16_gemm_m2048"] = {
            "kernel": "w8a16_gemm_kernel<128>", "bound": "mfma",
            "achieved_TFLOPs": round(tot_f / (tot_ms * 1e-3) / 1e12, 1),
            "frac": round(tot_f / (tot_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "flops_per_set": tot_f, "set_us": round(tot_ms * 1e3, 2), "per_layer": per}

    # ---- torch's device copy, and the counter calibration kernel ------------
    # An elementwise bitwise_not reads 1 GiB and writes 1 GiB per launch: the
    # known-size kernel the HBM byte counters are scaled by.
    if want("copy"):
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        ms = time_launches(torch, [lambda: b.copy_(a)], 20)
        ms_not = time_launches(torch, [lambda: torch.bitwise_not(a, out=b)], 20)
        out["hbm_reference"] = {"what": "torch device copy of 1 GiB (read + write)",
                                "GBps": round(rate(2 * (1 << 30), ms), 1),
                                "elementwise_GBps": round(rate(2 * (1 << 30), ms_not), 1)}
        del a, b

    # ---- report --------------------------------------------------------------
    for comp, kern in (("gemv_m1_g128", "gemv1_kernel"), ("gemv_m2_g128", "gemv1_kernel_m2"),
                       ("gemm_m2048_g128", "gemm_kernel"),
                       ("quantize_g128", "quantize_kernel"), ("fake_quant_g32", "quantize_kernel_fake"),
                       ("quantize_batch_g128", "quantize_batch_kernel"),
                       ("gemm_m2048_g128_ps", "gemm_kernel_ps"),
                       ("w8a16_gemv_m1", "w8a16_gemv_rows_kernel"), ("quantize8_g128", "quantize8_kernel"),
                       ("w8a16_gemm_m2048", "w8a16_gemm_kernel"),
                       ("w4a8_gemm_m2048_g128", "w4a8_gemm_kernel"),
                       ("w4a8_gemv_m1_g128", "w4a8_gemv_rows_kernel"),
                       ("gemv_m16_g32", "gemv_split_kernel_g32"),
                       ("gemv_m16_g64", "gemv_split_kernel_g64")):
        if comp in out:
            tr = measured_traffic(kern)
            out[comp]["traffic_bytes_per_launch"] = round(tr["bytes_per_launch"]) if tr else None

    value = None
    roofline = None
    if step is not None:
        g = out["gemv_m1_g128"]
        value = rate(step["bytes"], step["ms"])
        tr = measured_traffic("gemv1_kernel")
        roofline = {"bound": "hbm", "achieved": g["achieved_GBps"], "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": g["frac"],
                    "traffic": round(tr["bytes_per_launch"]) if tr else None,
                    "traffic_unit": "HBM bytes per launch, mean over the four layers "
                                    "(rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                    "traffic_detail": tr,
                    "kernel": g["kernel"],
                    "avg_launch_us": g["avg_launch_us"],
                    "bytes_per_launch_avg": g["bytes_per_set"] // len(layers),
                    "achieved_is": "mean algorithmic bytes per launch / mean launch duration "
                                   "(HIP events around a graph of >= 64 launches of each "
                                   "layer over >= 1 GiB of its copies)"}
        if "read_stream_ceiling" in out:
            roofline["read_stream_ceiling_GBps"] = out["read_stream_ceiling"]["decode_set_GBps"]
    roofline_prefill = None
    if "gemm_m2048_g128" in out:
        g = out["gemm_m2048_g128"]
        tr = measured_traffic("gemm_kernel")
        roofline_prefill = {"bound": "mfma", "achieved": g["achieved_TFLOPs"],
                            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": g["frac"],
                            "traffic": round(tr["bytes_per_launch"]) if tr else None,
                            "kernel": g["kernel"], "avg_launch_us": g["avg_launch_us"],
                            "workload": "gemma3_12b_prefill_layer_set_m2048_g128"}

    cpu = None
    if not args.no_cpu_baseline and only == "all":
        log("cpu baseline: oracle on bounded samples")
        cpu = cpu_baseline(G)

    line = {
        "metric": METRIC,
        "value": round(value, 1) if value is not None else None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step["ms"], 6) if step is not None else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "llama3_8b_decode_layer_set_m1_g128",
            "layers": {k: list(v) for k, v in layers.items()},
            "M": 1, "G": G,
            "step": "y = x . w_hat^T for the four layers back to back (M=1); the K timed "
                    "steps are one HIP graph of 4K launches, weights quantized beforehand, "
                    ">= 1 GiB of weight copies rotated",
            "step_bytes": step["bytes"] if step else None,
            "rotating_copies": step["copies"] if step else None,
            "step_wall_ms": round(step["wall_ms"], 6) if step else None,
        },
        "roofline": roofline,
        "roofline_prefill": roofline_prefill,
        "cpu_baseline": cpu,
        "components": out,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
