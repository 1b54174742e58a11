"""W4A16 benchmark on one MI355X: decode GEMV effective HBM GB/s (M = 1) and
prefill GEMM TFLOP/s (M = 2048), each as a fraction of its roofline.

A step is one decode pass over the seven linear layers of a Llama-7B-shaped
decoder layer (q/k/v/o 4096x4096, gate/up 11008x4096, down 4096x11008; INT4,
group 128, zero-points) at M = 1 through awq_gemm. Weights rotate over enough
copies (> 1 GB) that the 256 MB last-level cache cannot hold them, so every
step streams its weights from HBM. The same run also times the prefill GEMM
(x[2048, K] times the two MLP shapes), the quantize kernel and one full scale
search (W[11008, 4096], X[65536, 4096], 20 alphas), and the CPU oracle on a
bounded sample for the baseline.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "W4A16 GEMV eff. HBM GB/s (M=1) + GEMM TFLOP/s (M=2048), % of roofline"
HBM_PEAK_GBS = 8000.0
F16_MFMA_PEAK_TFLOPS = 2500.0
G = 128


def gemv_bytes(M, N, K, g=G):
    """Algorithmic bytes of one W4A16 product: packed codes, fp16 scale and
    zero per group, fp16 x in, fp16 y out."""
    return N * K // 2 + N * (K // g) * 4 + M * K * 2 + M * N * 2


def quantize_bytes(N, K, g=G):
    """fp16 W in; packed codes and fp16 scales/zeros out."""
    return N * K * 2 + N * K // 2 + N * (K // g) * 4


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class StreamTimer:
    """HIP events on the stream the library's kernels are enqueued on."""

    def __init__(self, torch):
        self.torch = torch
        self.stream = torch.cuda.current_stream()

    def time(self, fn, reps):
        t = self.torch
        start = t.cuda.Event(enable_timing=True)
        stop = t.cuda.Event(enable_timing=True)
        t.cuda.synchronize()
        start.record(self.stream)
        for i in range(reps):
            fn(i)
        stop.record(self.stream)
        stop.synchronize()
        return start.elapsed_time(stop) / 1e3   # seconds


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=240)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-search", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the library has no multi-GPU "
                                   "path (--gpus must be 1)"}))
        sys.exit(2)

    import torch
    import weight_only_int4_quantize_amd as awq

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = "cuda:0"
    timer = StreamTimer(torch)

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # ---------------------------------------------------------------- decode layer
    log("setup decode layer")
    shapes = {}
    for (N, K) in synth.DECODE_SHAPES:
        lay = synth.decode_layer(N, K, 1)
        qw, sc, zr = awq.awq_quantize(d(lay["w"]), G)
        shapes[(N, K)] = (qw, sc, zr, d(lay["x"]))
    linears = [(name, N, K) for (name, N, K) in synth.LLAMA7B_LAYER]
    step_bytes = sum(gemv_bytes(1, N, K) for (_, N, K) in linears)
    n_copies = max(2, int(np.ceil(1.2e9 / step_bytes)))
    copies = []
    for c in range(n_copies):
        layer = []
        for (name, N, K) in linears:
            qw, sc, zr, x = shapes[(N, K)]
            layer.append((qw.clone(), sc.clone(), zr.clone(), x, torch.empty((1, N), dtype=torch.float16, device=dev),
                          N, K))
        copies.append(layer)
    torch.cuda.synchronize()

    def step(i):
        for (qw, sc, zr, x, y, N, K) in copies[i % n_copies]:
            awq.awq_gemm(x, qw, sc, zr, G, out=y)

    for i in range(max(args.warmup, 1)):
        step(i)
    torch.cuda.synchronize()

    def capture(fn, count):
        """HIP graph of `count` calls fn(0..count-1); replays have no host
        launch cost between kernels."""
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for i in range(count):
                    fn(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        return g

    # one graph per full rotation over the weight copies, one for the rest,
    # so that exactly args.steps steps are timed
    g_full = capture(step, n_copies)
    rem = args.steps % n_copies
    g_rem = capture(step, rem) if rem else None
    n_full = args.steps // n_copies

    def timed_steps(_):
        for _r in range(n_full):
            g_full.replay()
        if g_rem is not None:
            g_rem.replay()

    g_full.replay()
    t_steps = timer.time(timed_steps, 1)
    ms_per_step = t_steps / args.steps * 1e3
    value = step_bytes * args.steps / t_steps / 1e9
    log(f"decode layer: {ms_per_step * 1e3:.1f} us/step, {value:.0f} GB/s")

    # per-shape GEMV launch durations (graph of back-to-back launches over the
    # rotated copies)
    per_shape = {}
    for (N, K) in synth.DECODE_SHAPES:
        idx = [j for j, (_, n, k) in enumerate(linears) if (n, k) == (N, K)][0]
        bufs = [copies[c][idx] for c in range(n_copies)]

        def one(i, bufs=bufs):
            qw, sc, zr, x, y, _, _ = bufs[i % len(bufs)]
            awq.awq_gemm(x, qw, sc, zr, G, out=y)

        reps = 8 * n_copies
        g1 = capture(one, reps)
        g1.replay()
        t = timer.time(lambda _: g1.replay(), 4) / (4 * reps)
        b = gemv_bytes(1, N, K)
        per_shape[f"{N}x{K}"] = {"us": round(t * 1e6, 3), "GB/s": round(b / t / 1e9, 1), "bytes": b}
        log(f"gemv {N}x{K}: {t * 1e6:.2f} us, {b / t / 1e9:.0f} GB/s")
        del g1
    big = per_shape[f"{11008}x{4096}"]

    # ---------------------------------------------------------------- prefill GEMM
    log("setup prefill")
    gemm = {}
    tot_flop, tot_t = 0.0, 0.0
    for (N, K) in synth.PREFILL_SHAPES:
        lay = synth.prefill_layer(N, K)
        qw, sc, zr = awq.awq_quantize(d(lay["w"]), G)
        x = d(lay["x"])
        y = torch.empty((synth.PREFILL_M, N), dtype=torch.float16, device=dev)

        def g(i, x=x, qw=qw, sc=sc, zr=zr, y=y):
            awq.awq_gemm(x, qw, sc, zr, G, out=y)

        for i in range(5):
            g(i)
        reps = 50
        t = timer.time(g, reps) / reps
        flop = 2.0 * synth.PREFILL_M * N * K
        tot_flop += flop
        tot_t += t
        gemm[f"{synth.PREFILL_M}x{N}x{K}"] = {"us": round(t * 1e6, 2), "TFLOP/s": round(flop / t / 1e12, 1)}
        log(f"gemm M={synth.PREFILL_M} {N}x{K}: {t * 1e6:.1f} us, {flop / t / 1e12:.0f} TFLOP/s")
    gemm_tflops = tot_flop / tot_t / 1e12

    # ---------------------------------------------------------------- quantize
    N, K = 11008, 4096
    w16 = d(synth.decode_layer(N, K, 0)["w"])
    outs = awq.awq_quantize(w16, G)

    def q(i):
        awq.awq_quantize(w16, G, out=outs)

    for i in range(5):
        q(i)
    tq = timer.time(q, 50) / 50
    quant = {"shape": f"{N}x{K}", "us": round(tq * 1e6, 2),
             "GB/s": round(quantize_bytes(N, K) / tq / 1e9, 1)}
    log(f"quantize {N}x{K}: {tq * 1e6:.1f} us, {quant['GB/s']} GB/s")

    # ---------------------------------------------------------------- scale search
    search = None
    if not args.no_search:
        log("setup scale search")
        lay = synth.search_layer()
        ws, xs = d(lay["w"]), d(lay["x"])
        del lay
        nb = awq.scale_search_workspace_bytes(ws.shape[0], ws.shape[1], xs.shape[0], G, 20)
        wsp = torch.empty(nb, dtype=torch.uint8, device=dev)
        awq.awq_scale_search(ws, xs, G, workspace=wsp)   # warm-up
        t0 = time.perf_counter()
        losses, best, _ = awq.awq_scale_search(ws, xs, G, workspace=wsp)
        ts = time.perf_counter() - t0
        flop = 21 * 2.0 * xs.shape[0] * ws.shape[0] * ws.shape[1]
        search = {"ms": round(ts * 1e3, 2), "best_alpha": best / 20, "TFLOP/s": round(flop / ts / 1e12, 1),
                  "frac_of_f16_peak": round(flop / ts / 1e12 / F16_MFMA_PEAK_TFLOPS, 4)}
        log(f"scale search: {ts * 1e3:.1f} ms, alpha* = {best / 20}")

    # ---------------------------------------------------------------- CPU oracle
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        cores = len(os.sched_getaffinity(0))
        t_cpu, b_cpu, n = 0.0, 0, 0
        lay_cache = {}
        t_start = time.perf_counter()
        while time.perf_counter() - t_start < 12.0:
            for (name, N, K) in linears:
                if (N, K) not in lay_cache:
                    lay = synth.decode_layer(N, K, 1)
                    lay_cache[(N, K)] = (oracle.quantize(lay["w"], G), lay["x"])
                (qw, sc, zr), x = lay_cache[(N, K)]
                t0 = time.perf_counter()
                oracle.linear_ref(x, qw, sc, zr, G)
                t_cpu += time.perf_counter() - t0
                b_cpu += gemv_bytes(1, N, K)
                n += 1
        cpu = {"value": round(b_cpu / t_cpu / 1e9, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
               "sample": f"{n} M=1 products over the 7 Llama-7B linear shapes (oracle dequantize + fp64 "
                         f"matmul), {t_cpu:.1f} s"}

    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "llama7b_decoder_layer_decode_m1_int4_g128", "M": 1, "group_size": G,
                   "linears": [f"{n}:{N}x{K}" for (n, N, K) in linears], "weight_copies": n_copies},
        "roofline": {"bound": "hbm", "achieved": big["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(big["GB/s"] / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "gemv 11008x4096 M=1", "bytes_per_launch": big["bytes"],
                     "launch_us": big["us"]},
        "step_frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "gemv_per_shape": per_shape,
        "gemm": {"M": synth.PREFILL_M, "TFLOP/s": round(gemm_tflops, 1),
                 "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": F16_MFMA_PEAK_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(gemm_tflops / F16_MFMA_PEAK_TFLOPS, 4)},
                 "per_shape": gemm},
        "quantize": quant,
        "scale_search": search,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
