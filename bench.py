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
MFMA_INT8_PEAK_TOPS = 5000.0    # MI355X dense int8 matrix peak
ROTATE_BYTES = 1 << 30          # rotate weight copies over >= 1 GiB
CSRC = os.path.join(ROOT, "bit_gemm_quantize_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
# device sources each kernel is built from (a change voids its counters)
# device sources of each kernel (the launch header only declares host
# functions and is left out)
KERNEL_SOURCES = {
    "quantize_kernel": ["quantize.hip", "w4_device.h"],
    "quantize_kernel_fake": ["quantize.hip", "w4_device.h"],
    "quantize_batch_kernel": ["quantize.hip", "w4_device.h"],
    "gemv_split_kernel": ["gemv.hip", "w4_device.h"],
    "gemm_kernel": ["gemm.hip", "w4_device.h"],
    "gemm_kernel_ps": ["gemm.hip", "w4_device.h"],
    "quantize8_kernel": ["w8a16.hip", "w4_device.h"],
    "w8a16_gemv_kernel": ["w8a16.hip", "w4_device.h"],
    "w8a16_gemm_kernel": ["w8a16.hip", "w4_device.h"],
    "w4a8_gemm_kernel": ["w4a8.hip", "w4_device.h"],
    "act_quant_kernel": ["w4a8.hip", "w4_device.h"],
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def quant_bytes(N, K, G):
    return 2 * N * K + N * K // 2 + 4 * N * K // G


def linear_bytes(M, N, K, G):
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
    counter gives for a plain device copy of known size). Returns None when
    no summary exists or the kernel's sources changed since it was taken.
    The summary carries one machine-readable line:
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


def time_graphs(torch, graphs, reps, warmup=2):
    """Replay the graphs round-robin; HIP events around the timed replays on
    the current stream. Returns milliseconds per replay."""
    for i in range(warmup * len(graphs)):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        graphs[i % len(graphs)].replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def make_layer(torch, N, K, seed, M, dev):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    W = (torch.randn((N, K), generator=g, device=dev, dtype=torch.float32) * 0.02
         ).to(torch.bfloat16)
    x = torch.randn((M, K), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    return W, x


def cpu_baseline(layers, G, min_s=10.0, max_s=30.0):
    """Time the CPU oracle (quantize + M = 1 linear) on the decode layer set,
    on this host's cores: whole layers, cycling through the set until at
    least min_s of work has been timed (stopping early past max_s)."""
    import oracle
    import workloads

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()
                            if i.get("user_api") == "blas"] or [1])
    except Exception:                                   # pragma: no cover
        blas_threads = 1
    inputs = {name: (workloads.weight_bits(2, name), workloads.activation_bits(2, 1, K))
              for name, (N, K) in layers.items()}
    total_bytes = 0
    t_total = 0.0
    done = []
    while t_total < min_s:
        for name, (N, K) in layers.items():
            W, x = inputs[name]
            t0 = time.perf_counter()
            c, s, z = oracle.quantize_ref(W, G)
            oracle.linear_ref(x, c, s, z, G)
            t_total += time.perf_counter() - t0
            total_bytes += quant_bytes(N, K, G) + linear_bytes(1, N, K, G)
            done.append(name)
            if t_total > max_s:
                break
        if t_total > max_s:
            break
    return {
        "value": round(total_bytes / t_total / 1e9, 4),
        "unit": "GB/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": ("numpy oracle, quantize (single thread) + float64 M=1 linear "
                   f"(BLAS, {blas_threads} threads) over whole decode layers "
                   f"({len(done)} layer passes: {', '.join(done)}); "
                   f"{total_bytes / 1e6:.1f} MB of algorithmic bytes in {t_total:.2f} s"),
        "host_cpus": os.cpu_count(),
        "host_affinity": len(os.sched_getaffinity(0)),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["all", "step", "gemv", "gemv16", "gemm", "quantize", "fake", "ps", "w4a8",
                                       "w8a16", "copy"],
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
    out = {}
    reps = max(args.steps, 1)

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

    def q_fn(e, name):
        W, x, codes, sc, ze, y = e[name]
        return lambda: w4.quantize_int4_grouped(W, G, codes, sc, ze)

    def l_fn(e, name):
        W, x, codes, sc, ze, y = e[name]
        return lambda: w4.w4a16_linear(x, codes, sc, ze, G, out=y)

    step_bytes = sum(quant_bytes(N, K, G) + linear_bytes(1, N, K, G)
                     for N, K in layers.values())
    ms_per_step = None
    step_per_layer_ms = None
    qb_ms = None
    q_ms_launch = {}
    if args.only in ("all", "step", "quantize"):
        # one graph per rotating copy: quantize the four layers, then the
        # four M = 1 linears on the fresh codes
        for e in sets:                      # eager warm-up of every launch
            for name in names:
                q_fn(e, name)()
                l_fn(e, name)()
        # one quantize launch per layer (reported for comparison), then the
        # step proper: the four weights quantized in one launch
        per_layer = [graph_of(torch, [q_fn(e, n) for n in names] + [l_fn(e, n) for n in names])
                     for e in sets]
        step_per_layer_ms = time_graphs(torch, per_layer, max(args.steps, 2))
        del per_layer

        def qbatch(e):
            return lambda: w4.quantize_int4_grouped_batch(
                [e[n][0] for n in names], G, outs=[(e[n][2], e[n][3], e[n][4]) for n in names])

        step_graphs = [graph_of(torch, [qbatch(e)] + [l_fn(e, n) for n in names]) for e in sets]
        log(f"step: warmup {args.warmup}, timed {args.steps} (graph replays)")
        for i in range(args.warmup):
            step_graphs[i % n_sets].replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for i in range(args.steps):
            step_graphs[i % n_sets].replay()
        e1.record()
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        ms_per_step = e0.elapsed_time(e1) / args.steps
        log(f"step: {ms_per_step:.4f} ms (events), {wall_ms:.4f} ms (host clock)")
        del step_graphs

        # the batched quantizer alone: one graph of n_sets launches
        g = graph_of(torch, [qbatch(e) for e in sets])
        qb_ms = time_graphs(torch, [g], max(2, reps // n_sets)) / n_sets
        del g
        qb_bytes = sum(quant_bytes(N, K, G) for N, K in layers.values())
        out["quantize_batch"] = {
            "kernel": "quantize_batch_kernel<128>", "bound": "hbm",
            "launches_per_step": 1, "avg_launch_us": round(qb_ms * 1e3, 3),
            "achieved_GBps": round(qb_bytes / (qb_ms * 1e-3) / 1e9, 1),
            "frac": round(qb_bytes / (qb_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes_per_launch": qb_bytes,
        }

        # the quantizer alone, per layer: one graph of n_sets launches
        per = {}
        tot_b = 0
        tot_ms = 0.0
        for name, (N, K) in layers.items():
            g = graph_of(torch, [q_fn(e, name) for e in sets])
            ms = time_graphs(torch, [g], max(2, reps // n_sets)) / n_sets
            q_ms_launch[name] = ms
            b = quant_bytes(N, K, G)
            per[name] = {"us": round(ms * 1e3, 3), "GBps": round(b / (ms * 1e-3) / 1e9, 1)}
            tot_b += b
            tot_ms += ms
            del g
        out["quantize"] = {
            "kernel": "quantize_kernel<128, false>", "bound": "hbm",
            "avg_launch_us": round(tot_ms * 1e3 / len(layers), 3),
            "achieved_GBps": round(tot_b / (tot_ms * 1e-3) / 1e9, 1),
            "frac": round(tot_b / (tot_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes_per_set": tot_b, "set_us": round(tot_ms * 1e3, 3),
            "per_layer": per,
        }

    # ---- fake-quantize round trip (QAT forward weight), G = 32 ------------
    if args.only in ("all", "fake"):
        GF = 32
        per = {}
        tot_b = 0
        tot_ms = 0.0
        for name, (N, K) in layers.items():
            wout = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
            fns = [(lambda e=e, n=name, o=wout: w4.fake_quant_int4_grouped(e[n][0], GF, out=o))
                   for e in sets]
            for f in fns:
                f()
            g = graph_of(torch, fns)
            ms = time_graphs(torch, [g], max(2, reps // n_sets)) / n_sets
            b = 4 * N * K                   # read W, write W_hat (bf16 each)
            per[name] = {"us": round(ms * 1e3, 3), "GBps": round(b / (ms * 1e-3) / 1e9, 1)}
            tot_b += b
            tot_ms += ms
            del g, wout, fns
        out["fake_quant_g32"] = {
            "kernel": "quantize_kernel<32, true>", "bound": "hbm",
            "achieved_GBps": round(tot_b / (tot_ms * 1e-3) / 1e9, 1),
            "frac": round(tot_b / (tot_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes_per_set": tot_b, "set_us": round(tot_ms * 1e3, 3), "per_layer": per,
        }

    # ---- decode GEMV on its own over rotating quantized copies ----------
    g_ms_launch = {}

    def prep(c, s_, z, Gx, ps):
        """Weights in the plain layout, or repacked to the pre-shuffled one."""
        if not ps:
            return c, s_, z
        cp, sz = w4.repack_int4_preshuffled(c, s_, z, Gx)
        return cp, sz, None

    def lin(x, c, s_, z, Gx, y, ps):
        if ps:
            return lambda: w4.w4a16_linear_preshuffled(x, c, s_, Gx, out=y)
        return lambda: w4.w4a16_linear(x, c, s_, z, Gx, out=y)

    layouts = [False] if args.only in ("step", "gemv", "gemv16", "gemm") else \
        [True] if args.only == "ps" else [False, True]
    for ps in layouts:
        sfx = "_ps" if ps else ""
        if args.only not in ("all", "step", "gemv", "ps"):
            break
        if ps and args.only == "step":
            break
        gset_bytes = sum(linear_bytes(1, N, K, G) for N, K in layers.values())
        n_g = max(2, -(-ROTATE_BYTES // gset_bytes))
        log(f"gemv{sfx}: {n_g} rotating quantized copies of {gset_bytes / 1e6:.1f} MB")
        gsets = []
        for r in range(n_g):
            src = sets[r % n_sets]
            entry = {}
            for name, (N, K) in layers.items():
                W, x = src[name][0], src[name][1]
                c, s_, z = prep(*w4.quantize_int4_grouped(W, G), G, ps)
                entry[name] = (x, c, s_, z, torch.empty((1, N), dtype=torch.bfloat16, device=dev))
            gsets.append(entry)
        torch.cuda.synchronize()

        def g_fn(e, name):
            x, c, s_, z, y = e[name]
            return lin(x, c, s_, z, G, y, ps)

        per = {}
        tot_ms = 0.0
        tot_b = 0
        for name, (N, K) in layers.items():
            g = graph_of(torch, [g_fn(e, name) for e in gsets])
            ms = time_graphs(torch, [g], max(2, reps // 2)) / n_g
            if not ps:
                g_ms_launch[name] = ms
            b = linear_bytes(1, N, K, G)
            per[name] = {"us": round(ms * 1e3, 3), "GBps": round(b / (ms * 1e-3) / 1e9, 1)}
            tot_ms += ms
            tot_b += b
            del g
        # the four layers back to back, as a decode step runs them
        g = graph_of(torch, [g_fn(e, n) for e in gsets for n in names])
        set_ms = time_graphs(torch, [g], max(2, reps // 2)) / n_g
        del g
        out["gemv_m1" + sfx] = {
            "kernel": f"gemv_split_kernel<128, 8, false, {'true' if ps else 'false'}>", "bound": "hbm",
            "layout": "pre-shuffled" if ps else "plain",
            "avg_launch_us": round(tot_ms * 1e3 / len(layers), 3),
            "achieved_GBps": round(tot_b / (tot_ms * 1e-3) / 1e9, 1),
            "frac": round(tot_b / (tot_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes_per_set": tot_b,
            "per_layer": per,
            "set_back_to_back_us": round(set_ms * 1e3, 3),
            "set_back_to_back_GBps": round(tot_b / (set_ms * 1e-3) / 1e9, 1),
        }
        del gsets

    # ---- small-batch decode GEMV, M = 16, G = 32 (same layer shapes) ------
    for ps in layouts:
        sfx = "_ps" if ps else ""
        if args.only not in ("all", "gemv16", "ps"):
            break
        M16, G16 = 16, 32
        gb16 = sum(linear_bytes(M16, N, K, G16) for N, K in layers.values())
        n16 = max(2, -(-ROTATE_BYTES // gb16))
        log(f"gemv M=16{sfx}: {n16} rotating quantized copies of {gb16 / 1e6:.1f} MB")
        per = {}
        tot_ms = 0.0
        tot_b = 0
        for li, (name, (N, K)) in enumerate(layers.items()):
            copies = []
            for r in range(n16):
                W, x = make_layer(torch, N, K, 7000 + 100 * r + li, M16, dev)
                c, s_, z = prep(*w4.quantize_int4_grouped(W, G16), G16, ps)
                del W
                copies.append((x, c, s_, z, torch.empty((M16, N), dtype=torch.bfloat16, device=dev)))
            fns = [lin(e[0], e[1], e[2], e[3], G16, e[4], ps) for e in copies]
            g = graph_of(torch, fns)
            ms = time_graphs(torch, [g], max(2, reps // 2)) / n16
            b = linear_bytes(M16, N, K, G16)
            per[name] = {"us": round(ms * 1e3, 3), "GBps": round(b / (ms * 1e-3) / 1e9, 1)}
            tot_ms += ms
            tot_b += b
            del g, copies, fns
        t = "true" if ps else "false"
        out["gemv_m16_g32" + sfx] = {
            "kernel": f"gemv_split_kernel<32, 8, true, {t}> (qkv, o, gate_up), "
                      f"gemv_direct_kernel<32, 8, {t}> (down)", "bound": "hbm",
            "layout": "pre-shuffled" if ps else "plain",
            "achieved_GBps": round(tot_b / (tot_ms * 1e-3) / 1e9, 1),
            "frac": round(tot_b / (tot_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes_per_set": tot_b, "per_layer": per,
        }

    # ---- prefill GEMM, Gemma3-12B-shaped layers, M = 2048 ----------------
    for ps in layouts:
        sfx = "_ps" if ps else ""
        if args.only not in ("all", "gemm", "ps"):
            break
        M = 2048
        glayers = dict(workloads.GEMMA3_12B)
        log(f"gemm{sfx}: Gemma3-12B-shaped layers, M=2048")
        per = {}
        tot_ms = 0.0
        tot_f = 0
        for i, (name, (N, K)) in enumerate(glayers.items()):
            W, x = make_layer(torch, N, K, 50 + i, M, dev)
            c, s_, z = prep(*w4.quantize_int4_grouped(W, G), G, ps)
            del W
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            fn = lin(x, c, s_, z, G, y, ps)
            fn()
            g = graph_of(torch, [fn])
            ms = time_graphs(torch, [g], max(3, reps // 5))
            f = 2 * M * N * K
            per[name] = {"us": round(ms * 1e3, 2), "TFLOPs": round(f / (ms * 1e-3) / 1e12, 1)}
            tot_ms += ms
            tot_f += f
            del g, x, c, s_, z, y
        out["gemm_m2048" + sfx] = {
            "kernel": f"gemm_kernel<128, {'true' if ps else 'false'}>", "bound": "mfma",
            "layout": "pre-shuffled" if ps else "plain",
            "avg_launch_us": round(tot_ms * 1e3 / len(glayers), 2),
            "achieved_TFLOPs": round(tot_f / (tot_ms * 1e-3) / 1e12, 1),
            "frac": round(tot_f / (tot_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "flops_per_set": tot_f,
            "per_layer": per,
            "set_us": round(tot_ms * 1e3, 2),
        }

    # ---- W4A8: per-token int8 activations + int4 weights on int8 MFMA -----
    if args.only in ("all", "w4a8"):
        M = 2048
        glayers = dict(workloads.GEMMA3_12B)
        for Gw in (128, 32):
            log(f"w4a8 G={Gw}: Gemma3-12B-shaped layers, M=2048")
            per = {}
            tot_ms = tot_aq_ms = 0.0
            tot_f = tot_aq_b = 0
            for i, (name, (N, K)) in enumerate(glayers.items()):
                W, x = make_layer(torch, N, K, 50 + i, M, dev)
                c, s_, z = w4.quantize_int4_grouped(W, Gw)
                del W
                x8, sx = w4.quantize_act_int8(x)
                y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
                fn = (lambda x8=x8, sx=sx, c=c, s_=s_, z=z, y=y, Gw=Gw:
                      w4.w4a8_linear(x8, sx, c, s_, z, Gw, out=y))
                fn()
                g = graph_of(torch, [fn])
                ms = time_graphs(torch, [g], max(3, reps // 5))
                del g
                aq = (lambda x=x, x8=x8, sx=sx: w4.quantize_act_int8(x, x8=x8, sx=sx))
                g = graph_of(torch, [aq])
                ms_aq = time_graphs(torch, [g], max(3, reps // 5))
                del g
                f = 2 * M * N * K
                per[name] = {"us": round(ms * 1e3, 2), "TOPs": round(f / (ms * 1e-3) / 1e12, 1),
                             "act_quant_us": round(ms_aq * 1e3, 2)}
                tot_ms += ms
                tot_f += f
                tot_aq_ms += ms_aq
                tot_aq_b += 3 * M * K + 4 * M
                del x, x8, sx, c, s_, z, y
            out[f"w4a8_gemm_m2048_g{Gw}"] = {
                "kernel": f"w4a8_gemm_kernel<{Gw}>", "bound": "mfma (int8)",
                "achieved_TOPs": round(tot_f / (tot_ms * 1e-3) / 1e12, 1),
                "frac": round(tot_f / (tot_ms * 1e-3) / 1e12 / MFMA_INT8_PEAK_TOPS, 4),
                "ops_per_set": tot_f, "set_us": round(tot_ms * 1e3, 2), "per_layer": per,
                "act_quant": {"kernel": "act_quant_kernel", "bound": "hbm",
                              "achieved_GBps": round(tot_aq_b / (tot_aq_ms * 1e-3) / 1e9, 1),
                              "set_us": round(tot_aq_ms * 1e3, 2)},
            }

    # ---- int8 weight-only: quantizer, decode (M = 1) and prefill (M = 2048) --
    if args.only in ("all", "w8a16"):
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
                src = sets[r % n_sets][name]
                q8, s8 = w4.quantize_int8_grouped(src[0], G)
                copies.append((src[0], src[1], q8, s8,
                               torch.empty((1, N), dtype=torch.bfloat16, device=dev)))
            g = graph_of(torch, [(lambda e=e: w4.w8a16_linear(e[1], e[2], e[3], G, out=e[4]))
                                 for e in copies])
            ms = time_graphs(torch, [g], max(2, reps // 2)) / n8
            del g
            g = graph_of(torch, [(lambda e=e: w4.quantize_int8_grouped(e[0], G, e[2], e[3]))
                                 for e in copies])
            ms_q = time_graphs(torch, [g], max(2, reps // 2)) / n8
            del g
            b = w8_bytes(1, N, K, G)
            bq = 3 * N * K + 2 * N * (K // G)
            per[name] = {"us": round(ms * 1e3, 3), "GBps": round(b / (ms * 1e-3) / 1e9, 1),
                         "quantize_us": round(ms_q * 1e3, 3),
                         "quantize_GBps": round(bq / (ms_q * 1e-3) / 1e9, 1)}
            tot_ms += ms
            tot_b += b
            tot_q_ms += ms_q
            tot_q_b += bq
            del copies
        out["w8a16_gemv_m1"] = {
            "kernel": "w8a16_gemv_kernel<128>", "bound": "hbm",
            "avg_launch_us": round(tot_ms * 1e3 / len(layers), 3),
            "achieved_GBps": round(tot_b / (tot_ms * 1e-3) / 1e9, 1),
            "frac": round(tot_b / (tot_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes_per_set": tot_b, "per_layer": per,
        }
        out["quantize8_g128"] = {
            "kernel": "quantize8_kernel<128>", "bound": "hbm",
            "achieved_GBps": round(tot_q_b / (tot_q_ms * 1e-3) / 1e9, 1),
            "frac": round(tot_q_b / (tot_q_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes_per_set": tot_q_b,
        }
        M = 2048
        glayers = dict(workloads.GEMMA3_12B)
        log("w8a16 prefill: Gemma3-12B-shaped layers, M=2048")
        per = {}
        tot_ms = 0.0
        tot_f = 0
        for i, (name, (N, K)) in enumerate(glayers.items()):
            W, x = make_layer(torch, N, K, 50 + i, M, dev)
            q8, s8 = w4.quantize_int8_grouped(W, G)
            del W
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            fn = (lambda x=x, q8=q8, s8=s8, y=y: w4.w8a16_linear(x, q8, s8, G, out=y))
            fn()
            g = graph_of(torch, [fn])
            ms = time_graphs(torch, [g], max(3, reps // 5))
            del g
            f = 2 * M * N * K
            per[name] = {"us": round(ms * 1e3, 2), "TFLOPs": round(f / (ms * 1e-3) / 1e12, 1)}
            tot_ms += ms
            tot_f += f
            del x, q8, s8, y
        out["w8a16_gemm_m2048"] = {
            "kernel": "w8a16_gemm_kernel<128>", "bound": "mfma",
            "achieved_TFLOPs": round(tot_f / (tot_ms * 1e-3) / 1e12, 1),
            "frac": round(tot_f / (tot_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "flops_per_set": tot_f, "set_us": round(tot_ms * 1e3, 2), "per_layer": per,
        }

    # ---- achievable-bandwidth reference: torch's own device copy ----------
    # The same buffers calibrate the HBM byte counters: an elementwise
    # bitwise_not is a plain kernel that reads 1 GiB and writes 1 GiB per
    # launch (the device copy above may run as a runtime blit).
    if args.only in ("all", "copy"):
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        g = graph_of(torch, [lambda: b.copy_(a)])
        ms = time_graphs(torch, [g], 20)
        del g
        g = graph_of(torch, [lambda: torch.bitwise_not(a, out=b)])
        ms_not = time_graphs(torch, [g], 20)
        # read-only stream: a reduction over the same 1 GiB, timed eagerly
        # (a multi-block reduction clears memory and stays out of graphs)
        a32 = a.view(torch.float32)
        for _ in range(3):
            torch.sum(a32)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            torch.sum(a32)
        e1.record()
        torch.cuda.synchronize()
        ms_rd = e0.elapsed_time(e1) / 10
        out["hbm_reference"] = {"what": "torch device copy of 1 GiB (read + write)",
                                "GBps": round(2 * (1 << 30) / (ms * 1e-3) / 1e9, 1),
                                "elementwise_GBps": round(2 * (1 << 30) / (ms_not * 1e-3) / 1e9, 1),
                                "read_only_GBps": round((1 << 30) / (ms_rd * 1e-3) / 1e9, 1)}
        del a, b, g

    # ---- report ------------------------------------------------------------
    roofline = None
    value = None
    if ms_per_step is not None:
        value = step_bytes / (ms_per_step * 1e-3) / 1e9
        # dominant kernel of the step: the one with the larger share of time
        # (the step quantizes the four weights in one batched launch)
        q_ms = qb_ms
        g_ms = sum(g_ms_launch.values()) if g_ms_launch else 0.0
        if q_ms >= g_ms:
            b = sum(quant_bytes(N, K, G) for N, K in layers.values())
            a_gbs = b / (q_ms * 1e-3) / 1e9
            kname, klabel = "quantize_batch_kernel", "quantize_batch_kernel<128>"
            nl = 1
        else:
            b = sum(linear_bytes(1, N, K, G) for N, K in layers.values())
            a_gbs = b / (g_ms * 1e-3) / 1e9
            kname, klabel = "gemv_split_kernel", "gemv_split_kernel<128, 8, false, false>"
            nl = len(g_ms_launch)
        tr = measured_traffic(kname)
        roofline = {"bound": "hbm", "achieved": round(a_gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(a_gbs / HBM_PEAK_GBS, 4),
                    "traffic": round(tr["bytes_per_launch"]) if tr else None,
                    "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                    "copy-calibrated)",
                    "traffic_detail": tr,
                    "kernel": klabel,
                    "avg_launch_us": round((q_ms if q_ms >= g_ms else g_ms) * 1e3 / nl, 3),
                    "bytes_per_launch_avg": b // nl}

    for comp, kern in (("quantize", "quantize_kernel"), ("fake_quant_g32", "quantize_kernel_fake"),
                       ("quantize_batch", "quantize_batch_kernel"),
                       ("gemv_m1", "gemv_split_kernel"), ("gemm_m2048", "gemm_kernel"),
                       ("gemm_m2048_ps", "gemm_kernel_ps"), ("w8a16_gemv_m1", "w8a16_gemv_kernel"),
                       ("quantize8_g128", "quantize8_kernel"), ("w8a16_gemm_m2048", "w8a16_gemm_kernel"),
                       ("w4a8_gemm_m2048_g128", "w4a8_gemm_kernel")):
        if comp in out:
            tr = measured_traffic(kern)
            out[comp]["traffic_bytes_per_launch"] = round(tr["bytes_per_launch"]) if tr else None

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
            "step": "quantize the four bf16 weights (one batched launch), then "
                    "y = x . w_hat^T per layer (M=1); one HIP graph replay per step",
            "ms_per_step_one_quantize_launch_per_layer":
                round(step_per_layer_ms, 5) if step_per_layer_ms is not None else None,
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
