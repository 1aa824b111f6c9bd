"""Benchmark of the W4A16 hot path on one MI355X.

A step is one pass of the whole path over the Llama-3-8B-shaped decode layer
set (qkv, o, gate_up, down; M = 1, G = 128): quantize each layer's bf16
weight, then run the M = 1 linear on it. ``value`` is the step's algorithmic
HBM bytes divided by its time. The same run also measures each kernel on
its own (decode GEMV over rotating weight copies, the quantizer, and the
M = 2048 prefill GEMM on the Gemma3-12B-shaped layer set) and times the CPU
oracle on a bounded sample of the step's work.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("W4A16 linear: achieved HBM GB/s (M=1) and TFLOP/s (M=2048), "
          "% of roofline")
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
ROTATE_BYTES = 1 << 30          # rotate weight copies over >= 1 GiB


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def quant_bytes(N, K, G):
    return 2 * N * K + N * K // 2 + 4 * N * K // G


def linear_bytes(M, N, K, G):
    return N * K // 2 + 4 * N * K // G + 2 * M * K + 2 * M * N


class Timer:
    """HIP events around each launch, on the stream the kernels run on."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def run(self, name, fn):
        ev0 = self.torch.cuda.Event(enable_timing=True)
        ev1 = self.torch.cuda.Event(enable_timing=True)
        ev0.record()
        fn()
        ev1.record()
        self.pairs.setdefault(name, []).append((ev0, ev1))

    def total_ms(self, name):
        return sum(a.elapsed_time(b) for a, b in self.pairs.get(name, []))

    def count(self, name):
        return len(self.pairs.get(name, []))


def make_layer(torch, N, K, seed, M, dev):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    W = (torch.randn((N, K), generator=g, device=dev, dtype=torch.float32) * 0.02
         ).to(torch.bfloat16)
    x = torch.randn((M, K), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    return W, x


def cpu_baseline(layers, G, budget_s=25.0):
    """Time the CPU oracle (quantize + M = 1 linear) on the first half of the
    output rows of each decode layer, on this host's cores."""
    import numpy as np

    import oracle
    import workloads

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()
                            if i.get("user_api") == "blas"] or [1])
    except Exception:                                   # pragma: no cover
        blas_threads = 1
    total_bytes = 0
    t_total = 0.0
    done = []
    for name, (N, K) in layers.items():
        rows = N // 2
        W = workloads.weight_bits(2, name, rows=(0, rows))
        x = workloads.activation_bits(2, 1, K)
        t0 = time.perf_counter()
        c, s, z = oracle.quantize_ref(W, G)
        oracle.linear_ref(x, c, s, z, G)
        dt = time.perf_counter() - t0
        t_total += dt
        total_bytes += quant_bytes(rows, K, G) + linear_bytes(1, rows, K, G)
        done.append(f"{name}[:{rows}]")
        if t_total > budget_s:
            break
    return {
        "value": round(total_bytes / t_total / 1e9, 4),
        "unit": "GB/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": ("numpy oracle, quantize (single thread) + float64 M=1 linear "
                   f"(BLAS, {blas_threads} threads) on the first half of the output "
                   f"rows of {', '.join(done)}; {total_bytes / 1e6:.1f} MB of "
                   f"algorithmic bytes in {t_total:.2f} s"),
        "host_cpus": os.cpu_count(),
        "host_affinity": len(os.sched_getaffinity(0)),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["all", "step", "gemv", "gemm", "quantize"],
                    default="all", help="restrict to one part (for profiling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU part in this build)", file=sys.stderr)
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
    names = list(layers)
    timer = Timer(torch)
    out = {}

    # ---- inputs of the step: rotating copies of the decode layer set -----
    set_bytes = sum(quant_bytes(N, K, G) for N, K in layers.values())
    n_sets = max(2, -(-ROTATE_BYTES // set_bytes))
    log(f"decode layer set: {n_sets} rotating copies of {set_bytes / 1e6:.1f} MB")
    sets = []
    for r in range(n_sets):
        entry = {}
        for i, (name, (N, K)) in enumerate(layers.items()):
            W, x = make_layer(torch, N, K, 1000 * r + i, 1, dev)
            codes = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
            sc = torch.empty((N, K // G), dtype=torch.bfloat16, device=dev)
            ze = torch.empty((N, K // G), dtype=torch.bfloat16, device=dev)
            y = torch.empty((1, N), dtype=torch.bfloat16, device=dev)
            entry[name] = (W, x, codes, sc, ze, y)
        sets.append(entry)
    torch.cuda.synchronize()

    def step(r, timed):
        e = sets[r % n_sets]
        for name in names:
            W, x, codes, sc, ze, y = e[name]
            fn = (lambda W=W, c=codes, s=sc, z=ze: w4.quantize_int4_grouped(W, G, c, s, z))
            timer.run(f"quantize:{name}", fn) if timed else fn()
        for name in names:
            W, x, codes, sc, ze, y = e[name]
            fn = (lambda x=x, c=codes, s=sc, z=ze, y=y: w4.w4a16_linear(x, c, s, z, G, out=y))
            timer.run(f"gemv:{name}", fn) if timed else fn()

    step_bytes = sum(quant_bytes(N, K, G) + linear_bytes(1, N, K, G)
                     for N, K in layers.values())
    ms_per_step = None
    if args.only in ("all", "step", "quantize"):
        log(f"step: warmup {args.warmup}, timed {args.steps}")
        for i in range(args.warmup):
            step(i, False)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i, True)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms_per_step = (t1 - t0) * 1e3 / args.steps
        log(f"step: {ms_per_step:.4f} ms")

        q_ms = sum(timer.total_ms(f"quantize:{n}") for n in names)
        g_ms = sum(timer.total_ms(f"gemv:{n}") for n in names)
        q_bytes = args.steps * sum(quant_bytes(N, K, G) for N, K in layers.values())
        g_bytes = args.steps * sum(linear_bytes(1, N, K, G) for N, K in layers.values())
        out["quantize"] = {
            "kernel": "quantize_kernel<128>", "bound": "hbm",
            "achieved_GBps": round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
            "frac": round(q_bytes / (q_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "avg_launch_us": round(q_ms * 1e3 / timer.count(f"quantize:{names[0]}") / len(names), 3),
            "per_layer_us": {n: round(timer.total_ms(f"quantize:{n}") * 1e3 / args.steps, 3)
                             for n in names},
        }
        out["gemv_in_step"] = {
            "achieved_GBps": round(g_bytes / (g_ms * 1e-3) / 1e9, 1),
            "note": "codes were just written by the quantizer and may be cache resident",
        }
        out["_step"] = dict(q_ms=q_ms, g_ms=g_ms, q_bytes=q_bytes, g_bytes=g_bytes)

    # ---- decode GEMV on its own over rotating quantized copies ----------
    if args.only in ("all", "gemv"):
        gset_bytes = sum(linear_bytes(1, N, K, G) for N, K in layers.values())
        n_g = max(2, -(-ROTATE_BYTES // gset_bytes))
        log(f"gemv: {n_g} rotating quantized copies of {gset_bytes / 1e6:.1f} MB")
        gsets = []
        for r in range(n_g):
            src = sets[r % n_sets]
            entry = {}
            for name, (N, K) in layers.items():
                W, x = src[name][0], src[name][1]
                c, s, z = w4.quantize_int4_grouped(W, G)
                entry[name] = (x, c, s, z, torch.empty((1, N), dtype=torch.bfloat16, device=dev))
            gsets.append(entry)
        torch.cuda.synchronize()
        gt = Timer(torch)
        for i in range(args.warmup + args.steps):
            e = gsets[i % n_g]
            for name in names:
                x, c, s, z, y = e[name]
                fn = (lambda x=x, c=c, s=s, z=z, y=y: w4.w4a16_linear(x, c, s, z, G, out=y))
                gt.run(name, fn) if i >= args.warmup else fn()
        torch.cuda.synchronize()
        per = {}
        tot_ms = 0.0
        tot_b = 0
        for name, (N, K) in layers.items():
            ms = gt.total_ms(name)
            b = args.steps * linear_bytes(1, N, K, G)
            per[name] = {"us": round(ms * 1e3 / args.steps, 3),
                         "GBps": round(b / (ms * 1e-3) / 1e9, 1)}
            tot_ms += ms
            tot_b += b
        out["gemv_m1"] = {
            "kernel": "gemv_kernel<128,1,4>", "bound": "hbm",
            "achieved_GBps": round(tot_b / (tot_ms * 1e-3) / 1e9, 1),
            "frac": round(tot_b / (tot_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "per_layer": per,
            "set_us": round(tot_ms * 1e3 / args.steps, 3),
        }
        del gsets

    # ---- prefill GEMM, Gemma3-12B-shaped layers, M = 2048 ----------------
    if args.only in ("all", "gemm"):
        M = 2048
        glayers = dict(workloads.GEMMA3_12B)
        log("gemm: Gemma3-12B-shaped layers, M=2048")
        pre = {}
        for i, (name, (N, K)) in enumerate(glayers.items()):
            W, x = make_layer(torch, N, K, 50 + i, M, dev)
            c, s, z = w4.quantize_int4_grouped(W, G)
            pre[name] = (x, c, s, z, torch.empty((M, N), dtype=torch.bfloat16, device=dev))
            del W
        torch.cuda.synchronize()
        gt = Timer(torch)
        steps = max(5, args.steps // 2)
        for i in range(args.warmup + steps):
            for name in glayers:
                x, c, s, z, y = pre[name]
                fn = (lambda x=x, c=c, s=s, z=z, y=y: w4.w4a16_linear(x, c, s, z, G, out=y))
                gt.run(name, fn) if i >= args.warmup else fn()
        torch.cuda.synchronize()
        per = {}
        tot_ms = 0.0
        tot_f = 0
        for name, (N, K) in glayers.items():
            ms = gt.total_ms(name)
            f = steps * 2 * M * N * K
            per[name] = {"us": round(ms * 1e3 / steps, 2),
                         "TFLOPs": round(f / (ms * 1e-3) / 1e12, 1)}
            tot_ms += ms
            tot_f += f
        out["gemm_m2048"] = {
            "kernel": "gemm_kernel<128>", "bound": "mfma",
            "achieved_TFLOPs": round(tot_f / (tot_ms * 1e-3) / 1e12, 1),
            "frac": round(tot_f / (tot_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "per_layer": per,
            "set_us": round(tot_ms * 1e3 / steps, 2),
        }
        del pre

    # ---- report ------------------------------------------------------------
    st = out.pop("_step", None)
    roofline = None
    value = None
    if st is not None:
        value = step_bytes / (ms_per_step * 1e-3) / 1e9
        # dominant kernel of the step: the one with the larger share of time
        if st["q_ms"] >= st["g_ms"]:
            a = st["q_bytes"] / (st["q_ms"] * 1e-3) / 1e9
            name = "quantize_kernel<128>"
        else:
            a = st["g_bytes"] / (st["g_ms"] * 1e-3) / 1e9
            name = "gemv_kernel<128,1,4>"
        roofline = {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(a / HBM_PEAK_GBS, 4), "traffic": None,
                    "kernel": name}

    cpu = None
    if not args.no_cpu_baseline and args.only == "all":
        log("cpu baseline: oracle on a bounded sample")
        cpu = cpu_baseline(layers, G)

    line = {
        "metric": METRIC,
        "value": round(value, 1) if value is not None else None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5) if ms_per_step is not None else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "llama3_8b_decode_layer_set_m1_g128",
            "layers": {k: list(v) for k, v in layers.items()},
            "M": 1, "G": G,
            "step": "quantize each layer's bf16 weight, then y = x . w_hat^T (M=1)",
            "step_bytes": step_bytes,
            "rotating_copies": n_sets,
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "components": out,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
