"""W4A16 benchmark on one MI355X: decode GEMV effective HBM GB/s (M = 1) and
prefill GEMM TFLOP/s (M = 2048), each against its roofline.

A step is one decode pass over the seven linear layers of a Llama-7B-shaped
decoder layer (q/k/v/o 4096x4096, gate/up 11008x4096, down 4096x11008; INT4,
group 128, zero-points) at M = 1 through awq_gemm. The weights rotate over
enough copies (> 1.2 GB) that the 256 MB last-level cache cannot hold them,
so every step streams its weights from HBM; the steps are replayed from HIP
graphs, so host launch cost is outside the timed kernels. `value` is the
step's algorithmic bytes over its time.

The same run also times, each in its own section:
  * the roofline kernel: the gate/up GEMV (11008x4096, the largest launch of
    the step) back to back over the rotated copies;
  * the same layer with fused q/k/v (12288x4096) and gate/up (22016x4096)
    projections, four launches per step;
  * the per-node floor of a graph of tiny kernels (launch cost context);
  * batched decode rows on the skinny MFMA kernel (M = 16 on the decode
    shapes, M = 32 on the 13B/70B sweep shapes);
  * the roofline GEMV at group sizes 32, 64, 128, 256 and 512;
  * the W8A16 form (8-bit weights): the roofline GEMV and the prefill GEMM;
  * the prefill GEMM, x[2048, K] times the two MLP shapes;
  * the quantize kernel on 11008x4096;
  * one full scale search (W[11008, 4096], X[65536, 4096], 20 alphas), the
    clip search after it, and the fp16-salient-channel ablation (output loss
    of plain RTN, the searched scales and the mixed-precision layer);
  * an HBM copy of 1 GiB (context for the achievable bandwidth, and the
    calibration of the FETCH_SIZE / WRITE_SIZE counters);
  * the CPU oracle on a bounded sample (the CPU baseline).

    python bench.py [--gpus 1] [--steps 2400] [--warmup 20] [--only SECTION]
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
ROOFLINE_SHAPE = (11008, 4096)     # gate/up projection, the step's largest launch
COPY_BYTES = 1 << 30
CLIP_BENCH_FRACTION = 0.01                                # the clip of xxmr.cn §1.5
CLIP_GRID = [0.0, 0.001, 0.002, 0.005, 0.01, 0.02]       # clip-search fractions


def gemv_bytes(M, N, K, g=G):
    """Algorithmic bytes of one W4A16 product: packed codes, fp16 scale and
    zero per group, fp16 x in, fp16 y out."""
    return N * K // 2 + N * (K // g) * 4 + M * K * 2 + M * N * 2


def quantize_bytes(N, K, g=G):
    """fp16 W in; packed codes and fp16 scales/zeros out."""
    return N * K * 2 + N * K // 2 + N * (K // g) * 4


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic():
    """HBM bytes per launch of the roofline kernel, from the FETCH_SIZE and
    WRITE_SIZE counter runs recorded under profiles/ (scaled by the same
    counters read on a copy of known size). None once the kernel source has
    changed since the counters were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "gemv_m1_11008x4096_counters.json")
    try:
        with open(path) as f:
            rec = json.load(f)
        with open(os.path.join(ROOT, rec["source"]), "rb") as f:
            current = hashlib.sha256(f.read()).hexdigest()
    except (OSError, KeyError, ValueError):
        return None, None
    if current != rec.get("source_sha256"):
        return None, None
    return int(rec["traffic_bytes_per_launch"]), rec["copy_calibration"]


class Bench:
    def __init__(self, args):
        import torch
        import weight_only_int4_quantize_amd as awq

        self.torch, self.awq, self.args = torch, awq, args
        if not torch.cuda.is_available():
            raise SystemExit("bench.py needs a GPU")
        self.dev = "cuda:0"
        # HIP events recorded on the stream the library's kernels are enqueued
        # on (the binding passes torch's current stream)
        self.stream = torch.cuda.current_stream()

    def d(self, a):
        return self.torch.from_numpy(np.ascontiguousarray(a)).to(self.dev)

    def time(self, fn, reps=1):
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

    def warm(self, fn, ms=50.0):
        """Untimed calls of fn until `ms` of GPU time has passed. The clocks
        ramp up over the first ~20 ms of sustained MFMA load: a GEMM timed
        right after a few warm-up launches reads 10-15% slower than in
        steady state."""
        done, i = 0.0, 0
        while done < ms * 1e-3:
            done += self.time(lambda j: fn(i + j), 8)
            i += 8

    def capture(self, fn, count):
        """HIP graph of `count` calls fn(0..count-1)."""
        t = self.torch
        g = t.cuda.CUDAGraph()
        side = t.cuda.Stream()
        side.wait_stream(t.cuda.current_stream())
        with t.cuda.stream(side):
            with t.cuda.graph(g, stream=side):
                for i in range(count):
                    fn(i)
        t.cuda.current_stream().wait_stream(side)
        t.cuda.synchronize()
        return g

    # ------------------------------------------------------------ decode layer
    def setup_decode(self):
        torch, awq = self.torch, self.awq
        log("setup decode layer")
        shapes = {}
        for (N, K) in synth.DECODE_SHAPES:
            lay = synth.decode_layer(N, K, 1)
            qw, sc, zr = awq.awq_quantize(self.d(lay["w"]), G)
            shapes[(N, K)] = (qw, sc, zr, self.d(lay["x"]))
        self.linears = list(synth.LLAMA7B_LAYER)
        self.step_bytes = sum(gemv_bytes(1, N, K) for (_, N, K) in self.linears)
        self.n_copies = max(2, int(np.ceil(1.2e9 / self.step_bytes)))
        self.copies = []
        for _ in range(self.n_copies):
            layer = []
            for (_, N, K) in self.linears:
                qw, sc, zr, x = shapes[(N, K)]
                y = torch.empty((1, N), dtype=torch.float16, device=self.dev)
                layer.append((qw.clone(), sc.clone(), zr.clone(), x, y, N, K))
            self.copies.append(layer)
        torch.cuda.synchronize()

    def decode_step(self, i):
        for (qw, sc, zr, x, y, N, K) in self.copies[i % self.n_copies]:
            self.awq.awq_gemm(x, qw, sc, zr, G, out=y)

    def run_decode(self):
        args = self.args
        for i in range(max(args.warmup, 1)):
            self.decode_step(i)
        self.torch.cuda.synchronize()
        # one graph per full rotation over the copies, one for the rest, so
        # that exactly args.steps steps are timed
        g_full = self.capture(self.decode_step, self.n_copies)
        rem = args.steps % self.n_copies
        g_rem = self.capture(self.decode_step, rem) if rem else None
        n_full = args.steps // self.n_copies

        def steps(_):
            for _r in range(n_full):
                g_full.replay()
            if g_rem is not None:
                g_rem.replay()

        g_full.replay()
        t = self.time(steps)
        ms = t / args.steps * 1e3
        value = self.step_bytes * args.steps / t / 1e9
        log(f"decode layer: {ms * 1e3:.2f} us/step, {value:.0f} GB/s")
        return value, ms

    def run_decode_fused(self):
        """The decoder layer with fused q/k/v and gate/up projections: four
        launches per step instead of seven, same weight bytes."""
        torch, awq, args = self.torch, self.awq, self.args
        log("setup fused decode layer")
        layer = list(synth.LLAMA7B_LAYER_FUSED)
        step_bytes = sum(gemv_bytes(1, N, K) for (_, N, K) in layer)
        n_copies = max(2, int(np.ceil(1.2e9 / step_bytes)))
        base = []
        for (_, N, K) in layer:
            lay = synth.decode_layer(N, K, 1)
            qw, sc, zr = awq.awq_quantize(self.d(lay["w"]), G)
            base.append((qw, sc, zr, self.d(lay["x"]), N, K))
        copies = []
        for _ in range(n_copies):
            copies.append([(qw.clone(), sc.clone(), zr.clone(), x,
                            torch.empty((1, N), dtype=torch.float16, device=self.dev), N, K)
                           for (qw, sc, zr, x, N, K) in base])
        torch.cuda.synchronize()

        def step(i):
            for (qw, sc, zr, x, y, N, K) in copies[i % n_copies]:
                awq.awq_gemm(x, qw, sc, zr, G, out=y)

        for i in range(max(args.warmup, 1)):
            step(i)
        g = self.capture(step, n_copies)
        g.replay()
        reps = max(1, args.steps // n_copies)
        t = self.time(lambda _: [g.replay() for _r in range(reps)])
        n = reps * n_copies
        us = t / n * 1e6
        gbs = step_bytes * n / t / 1e9
        log(f"fused decode layer: {us:.2f} us/step, {gbs:.0f} GB/s")
        per_launch = {}
        for j, (name, N, K) in enumerate(layer):
            def one(i, j=j):
                qw, sc, zr, x, y, _, _ = copies[i % n_copies][j]
                awq.awq_gemm(x, qw, sc, zr, G, out=y)
            gj = self.capture(one, 4 * n_copies)
            gj.replay()
            tj = self.time(lambda _: gj.replay()) / (4 * n_copies)
            per_launch[name] = {"shape": f"{N}x{K}", "us": round(tj * 1e6, 2),
                                "GB/s": round(gemv_bytes(1, N, K) / tj / 1e9, 1)}
        del copies
        torch.cuda.synchronize()
        return {"workload": "llama7b_decoder_layer_fused_qkv_gateup_m1_int4_g128",
                "linears": [f"{n}:{N}x{K}" for (n, N, K) in layer], "step_bytes": step_bytes,
                "weight_copies": n_copies, "us_per_step": round(us, 2), "GB/s": round(gbs, 1),
                "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "per_launch": per_launch}

    def run_decode_model(self, n_layers=32):
        """Every linear layer of a Llama-7B-shaped model at M = 1, layer after
        layer, each layer with weights of its own (32 x 107.7 MB, far past
        every cache), unfused (7 launches per layer) and with fused q/k/v and
        gate/up (4 per layer). One token's pass is one graph; its time bounds
        the decode rate the linear layers allow (attention, norms and
        sampling not included)."""
        torch, awq, args = self.torch, self.awq, self.args
        out = {}
        for label, layer in (("unfused", synth.LLAMA7B_LAYER), ("fused", synth.LLAMA7B_LAYER_FUSED)):
            log(f"setup {n_layers}-layer decode pass ({label})")
            layer = list(layer)
            base = []
            for (_, N, K) in layer:
                lay = synth.decode_layer(N, K, 1)
                qw, sc, zr = awq.awq_quantize(self.d(lay["w"]), G)
                base.append((qw, sc, zr, self.d(lay["x"]), N, K))
            model = [[(qw.clone(), sc.clone(), zr.clone(), x,
                       torch.empty((1, N), dtype=torch.float16, device=self.dev), N, K)
                      for (qw, sc, zr, x, N, K) in base] for _ in range(n_layers)]
            torch.cuda.synchronize()

            def token(_):
                for lin in model:
                    for (qw, sc, zr, x, y, N, K) in lin:
                        awq.awq_gemm(x, qw, sc, zr, G, out=y)

            for i in range(max(args.warmup, 1)):
                token(i)
            g = self.capture(token, 1)
            g.replay()
            reps = 50
            t = self.time(lambda _: [g.replay() for _r in range(reps)])
            us = t / reps * 1e6
            token_bytes = n_layers * sum(gemv_bytes(1, N, K) for (_, N, K) in layer)
            out[label] = {"launches_per_token": n_layers * len(layer), "us_per_token": round(us, 1),
                          "tokens_per_s": round(1e6 / us, 1), "bytes_per_token": token_bytes,
                          "GB/s": round(token_bytes / (us * 1e-6) / 1e9, 1)}
            log(f"{n_layers}-layer decode pass ({label}): {us:.1f} us/token, {1e6 / us:.0f} tok/s")
            del model, base, g
            torch.cuda.synchronize()
        out["workload"] = f"llama7b_{n_layers}_layers_linears_m1_int4_g128"
        out["note"] = ("linear layers only; the pages quote 58 tok/s for a GPTQ-4bit 7B model on an A10G "
                       "(whole model, other hardware): context, not a target")
        return out

    def run_skinny(self):
        """Batched decode rows (awq_gemm_ex with a workspace): M = 4 on the
        decode shapes (the GEMV), M = 16 on the decode shapes and M = 32 on
        the sweep shapes (the skinny MFMA kernel), weights rotated over
        copies like the decode step."""
        torch, awq = self.torch, self.awq
        ws = awq.gemm_workspace(64, 1, 1, self.dev)
        out = {}
        cases = [(4, N, K, 128) for (N, K) in synth.DECODE_SHAPES] + \
                [(16, N, K, 128) for (N, K) in synth.DECODE_SHAPES] + \
                [(32, N, K, 128) for (N, K) in synth.SWEEP_SHAPES]
        for (M, N, K, g) in cases:
            lay = synth.decode_layer(N, K, M) if M <= 16 else synth.sweep_layer(N, K, M, g)
            qw, sc, zr = awq.awq_quantize(self.d(lay["w"]), g)
            x = self.d(lay["x"])
            nbytes = gemv_bytes(M, N, K, g)
            n_copies = max(2, int(np.ceil(1.2e9 / nbytes)))
            cps = [(qw.clone(), sc.clone(), zr.clone()) for _ in range(n_copies)]
            y = torch.empty((M, N), dtype=torch.float16, device=self.dev)

            def one(i, cps=cps, x=x, y=y, g=g):
                q = cps[i % len(cps)]
                awq.awq_gemm(x, q[0], q[1], q[2], g, out=y, workspace=ws)

            gr = self.capture(one, 2 * n_copies)
            gr.replay()
            t = self.time(lambda _: gr.replay()) / (2 * n_copies)
            key = f"M{M}_{N}x{K}"
            out[key] = {"us": round(t * 1e6, 2), "GB/s": round(nbytes / t / 1e9, 1),
                        "frac_of_hbm_peak": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4),
                        "kernel": "gemv" if M <= 4 else "skinny"}
            log(f"batched decode {key}: {t * 1e6:.2f} us, {nbytes / t / 1e9:.0f} GB/s")
            del cps, gr
        torch.cuda.synchronize()
        return out

    def run_group_sizes(self):
        """The roofline GEMV shape (11008x4096, M = 1) at every supported group
        size, weights rotated over copies: the pages weigh group 128 against
        256 (fewer scales, less traffic)."""
        torch, awq = self.torch, self.awq
        N, K = ROOFLINE_SHAPE
        out = {}
        for g in (32, 64, 128, 256, 512):
            lay = synth.decode_layer(N, K, 1, g)
            qw, sc, zr = awq.awq_quantize(self.d(lay["w"]), g)
            x = self.d(lay["x"])
            nbytes = gemv_bytes(1, N, K, g)
            n_copies = max(2, int(np.ceil(1.2e9 / nbytes)))
            cps = [(qw.clone(), sc.clone(), zr.clone()) for _ in range(n_copies)]
            y = torch.empty((1, N), dtype=torch.float16, device=self.dev)

            def one(i, cps=cps, x=x, y=y, g=g):
                q = cps[i % len(cps)]
                awq.awq_gemm(x, q[0], q[1], q[2], g, out=y)

            gr = self.capture(one, 4 * n_copies)
            gr.replay()
            t = self.time(lambda _: gr.replay()) / (4 * n_copies)
            out[f"G{g}"] = {"us": round(t * 1e6, 2), "bytes": nbytes, "GB/s": round(nbytes / t / 1e9, 1)}
            log(f"gemv {N}x{K} G={g}: {t * 1e6:.2f} us, {nbytes / t / 1e9:.0f} GB/s")
            del cps, gr
        torch.cuda.synchronize()
        return out

    def run_w8(self):
        """W8A16 (8-bit weights, fp16 activations): the decode GEMV on the
        roofline shape (weights rotated over copies) and the prefill GEMM."""
        torch, awq = self.torch, self.awq
        N, K = ROOFLINE_SHAPE
        lay = synth.decode_layer(N, K, 1, G)
        qw, sc, zr = awq.awq_quantize_w8(self.d(lay["w"]), G)
        x = self.d(lay["x"])
        nbytes = N * K + N * (K // G) * 4 + K * 2 + N * 2
        n_copies = max(2, int(np.ceil(1.2e9 / nbytes)))
        cps = [(qw.clone(), sc.clone(), zr.clone()) for _ in range(n_copies)]
        y = torch.empty((1, N), dtype=torch.float16, device=self.dev)

        def one(i):
            q = cps[i % len(cps)]
            awq.awq_gemm_w8(x, q[0], q[1], q[2], G, out=y)

        gr = self.capture(one, 4 * n_copies)
        gr.replay()
        t = self.time(lambda _: gr.replay()) / (4 * n_copies)
        log(f"w8 gemv {N}x{K}: {t * 1e6:.2f} us, {nbytes / t / 1e9:.0f} GB/s")
        del cps, gr
        out = {"gemv_m1": {"shape": f"{N}x{K}", "us": round(t * 1e6, 2), "bytes": nbytes,
                           "GB/s": round(nbytes / t / 1e9, 1), "frac_of_hbm_peak": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)}}
        M = synth.PREFILL_M
        lay = synth.prefill_layer(N, K)
        qw, sc, zr = awq.awq_quantize_w8(self.d(lay["w"]), G)
        xm = self.d(lay["x"])
        ym = torch.empty((M, N), dtype=torch.float16, device=self.dev)
        self.warm(lambda i: awq.awq_gemm_w8(xm, qw, sc, zr, G, out=ym))
        t = self.time(lambda i: awq.awq_gemm_w8(xm, qw, sc, zr, G, out=ym), 50) / 50
        flop = 2.0 * M * N * K
        log(f"w8 gemm M={M} {N}x{K}: {t * 1e6:.1f} us, {flop / t / 1e12:.0f} TFLOP/s")
        out["gemm_m2048"] = {"shape": f"{M}x{N}x{K}", "us": round(t * 1e6, 2), "TFLOP/s": round(flop / t / 1e12, 1)}
        return out

    def run_launch_floor(self):
        """Per-node cost of a HIP graph of tiny kernels (a one-element fill):
        the floor under every back-to-back launch timed here."""
        torch = self.torch
        t1 = torch.empty(1, dtype=torch.float32, device=self.dev)
        n = 400
        g = self.capture(lambda i: t1.fill_(float(i)), n)
        g.replay()
        us = min(self.time(lambda _: g.replay()) for _ in range(3)) / n * 1e6
        log(f"graph launch floor: {us:.2f} us per node")
        return round(us, 3)

    def run_gemv_shapes(self, shapes):
        """Back-to-back launches of one shape over the rotated copies."""
        out = {}
        for (N, K) in shapes:
            idx = [j for j, (_, n, k) in enumerate(self.linears) if (n, k) == (N, K)][0]
            bufs = [self.copies[c][idx] for c in range(self.n_copies)]

            def one(i, bufs=bufs):
                qw, sc, zr, x, y, _, _ = bufs[i % len(bufs)]
                self.awq.awq_gemm(x, qw, sc, zr, G, out=y)

            reps = 8 * self.n_copies
            g1 = self.capture(one, reps)
            g1.replay()
            t = self.time(lambda _: g1.replay(), 4) / (4 * reps)
            b = gemv_bytes(1, N, K)
            out[f"{N}x{K}"] = {"us": round(t * 1e6, 3), "GB/s": round(b / t / 1e9, 1), "bytes": b,
                               "launches_timed": 4 * reps}
            log(f"gemv {N}x{K}: {t * 1e6:.2f} us, {b / t / 1e9:.0f} GB/s")
            del g1
        return out

    # ------------------------------------------------------------ prefill GEMM
    def run_gemm(self):
        torch, awq = self.torch, self.awq
        log("setup prefill")
        per_shape, tot_flop, tot_t = {}, 0.0, 0.0
        # one workspace serves both shapes (stream-K split where it pays)
        ws = awq.gemm_workspace(synth.PREFILL_M, max(n for n, _ in synth.PREFILL_SHAPES),
                                max(k for _, k in synth.PREFILL_SHAPES), self.dev)
        for (N, K) in synth.PREFILL_SHAPES:
            lay = synth.prefill_layer(N, K)
            qw, sc, zr = awq.awq_quantize(self.d(lay["w"]), G)
            x = self.d(lay["x"])
            y = torch.empty((synth.PREFILL_M, N), dtype=torch.float16, device=self.dev)

            def g(i, x=x, qw=qw, sc=sc, zr=zr, y=y):
                awq.awq_gemm(x, qw, sc, zr, G, out=y, workspace=ws)

            self.warm(g)
            reps = 50
            t = self.time(g, reps) / reps
            flop = 2.0 * synth.PREFILL_M * N * K
            tot_flop += flop
            tot_t += t
            per_shape[f"{synth.PREFILL_M}x{N}x{K}"] = {"us": round(t * 1e6, 2),
                                                       "TFLOP/s": round(flop / t / 1e12, 1)}
            log(f"gemm M={synth.PREFILL_M} {N}x{K}: {t * 1e6:.1f} us, {flop / t / 1e12:.0f} TFLOP/s")
        tflops = tot_flop / tot_t / 1e12
        # the 13B/70B sweep shapes at M = 512 (not part of the prefill figure)
        sweep = {}
        for (N, K) in synth.SWEEP_SHAPES:
            M = 512
            lay = synth.sweep_layer(N, K, M, G)
            qw, sc, zr = awq.awq_quantize(self.d(lay["w"]), G)
            x = self.d(lay["x"])
            y = torch.empty((M, N), dtype=torch.float16, device=self.dev)

            def g(i, x=x, qw=qw, sc=sc, zr=zr, y=y):
                awq.awq_gemm(x, qw, sc, zr, G, out=y, workspace=ws)

            self.warm(g)
            t = self.time(g, 20) / 20
            flop = 2.0 * M * N * K
            sweep[f"{M}x{N}x{K}"] = {"us": round(t * 1e6, 2), "TFLOP/s": round(flop / t / 1e12, 1)}
            log(f"gemm M={M} {N}x{K}: {t * 1e6:.1f} us, {flop / t / 1e12:.0f} TFLOP/s")
        return {"M": synth.PREFILL_M, "TFLOP/s": round(tflops, 1), "sweep_m512": sweep,
                "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": F16_MFMA_PEAK_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(tflops / F16_MFMA_PEAK_TFLOPS, 4)},
                "per_shape": per_shape}

    # ------------------------------------------------------------ quantize
    def run_quantize(self):
        N, K = 11008, 4096
        w16 = self.d(synth.decode_layer(N, K, 0)["w"])
        outs = self.awq.awq_quantize(w16, G)

        def q(i):
            self.awq.awq_quantize(w16, G, out=outs)

        self.warm(q)
        tq = self.time(q, 50) / 50
        gbs = quantize_bytes(N, K) / tq / 1e9
        log(f"quantize {N}x{K}: {tq * 1e6:.1f} us, {gbs:.0f} GB/s")

        def qc(i):
            self.awq.awq_quantize(w16, G, out=outs, clip_fraction=CLIP_BENCH_FRACTION)

        self.warm(qc)
        tc = self.time(qc, 50) / 50
        log(f"clipped quantize {N}x{K} (p={CLIP_BENCH_FRACTION}): {tc * 1e6:.1f} us")
        return {"shape": f"{N}x{K}", "us": round(tq * 1e6, 2), "GB/s": round(gbs, 1),
                "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                "clipped": {"clip_fraction": CLIP_BENCH_FRACTION, "us": round(tc * 1e6, 2),
                            "GB/s": round(quantize_bytes(N, K) / tc / 1e9, 1)}}

    # ------------------------------------------------------------ scale search
    def run_search(self):
        torch, awq = self.torch, self.awq
        log("setup scale search")
        lay = synth.search_layer()
        ws, xs = self.d(lay["w"]), self.d(lay["x"])
        del lay
        nb = awq.scale_search_workspace_bytes(ws.shape[0], ws.shape[1], xs.shape[0], G, 20)
        wsp = torch.empty(nb, dtype=torch.uint8, device=self.dev)
        awq.awq_scale_search(ws, xs, G, workspace=wsp)   # warm-up
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        losses, best, best_s = awq.awq_scale_search(ws, xs, G, workspace=wsp)
        ts = time.perf_counter() - t0
        flop = 21 * 2.0 * xs.shape[0] * ws.shape[0] * ws.shape[1]
        log(f"scale search: {ts * 1e3:.1f} ms, alpha* = {best / 20}")
        out = {"ms": round(ts * 1e3, 2), "best_alpha": best / 20, "TFLOP/s": round(flop / ts / 1e12, 1),
               "frac_of_f16_peak": round(flop / ts / 1e12 / F16_MFMA_PEAK_TFLOPS, 4),
               "workload": "W[11008,4096], X[65536,4096], 20 alphas, G=128 (21 GEMMs)"}
        del wsp
        out["clip_search"] = self.run_clip_search(ws, xs, best_s)
        out["salient_fp16_ablation"] = self.run_salient(ws, xs, float(losses[0]), float(losses[best]), best / 20)
        return out

    def run_salient(self, ws, xs, loss_alpha0, loss_best, alpha):
        """Mixed precision with the top 1 % channels in fp16 against plain
        RTN and the searched scales, by the same output loss, plus the cost of
        the fp16 side product at decode."""
        torch, awq = self.torch, self.awq
        N, K, T = ws.shape[0], ws.shape[1], xs.shape[0]
        n = int(round(0.01 * K))
        nb = awq.load().awq_salient_loss_workspace_bytes(N, K, T, G, n)
        wsp = torch.empty(nb, dtype=torch.uint8, device=self.dev)
        awq.awq_salient_loss(ws, xs, G, n, workspace=wsp)   # warm-up
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        lr, ls, idx = awq.awq_salient_loss(ws, xs, G, n, workspace=wsp)
        tl = time.perf_counter() - t0
        del wsp
        log(f"salient fp16 ablation: rtn {lr:.4g}, awq alpha={alpha} {loss_best:.4g}, salient {ls:.4g} "
            f"({tl * 1e3:.1f} ms)")
        # decode: side product of the mixed gate/up layer at M = 1
        x1 = xs[:1].contiguous()
        qw, sc, zr, w_sal = awq.awq_quantize_salient(ws, G, idx)
        y = torch.empty((1, N), dtype=torch.float16, device=self.dev)
        for i in range(5):
            awq.awq_salient_apply(x1, idx, w_sal, y)
        reps = 200
        g = self.capture(lambda i: awq.awq_salient_apply(x1, idx, w_sal, y), reps)
        g.replay()
        t_apply = self.time(lambda i: g.replay()) / reps
        log(f"salient side product M=1 {N}x{n}: {t_apply * 1e6:.2f} us")
        return {"n_salient": n, "loss_rtn": lr, "loss_awq_best": loss_best, "awq_best_alpha": alpha,
                "loss_salient_fp16": ls, "rtn_equals_alpha0": abs(lr - loss_alpha0) <= 2e-3 * loss_alpha0,
                "ms": round(tl * 1e3, 2), "side_product_m1_us": round(t_apply * 1e6, 2),
                "side_bytes_m1": n * N * 2 + n * 2 + N * 4,
                "workload": f"W[{N},{K}], X[{T},{K}], G=128, top {n} channels by mean |x| kept in fp16"}

    def run_clip_search(self, ws, xs, s):
        """The clip search after the scale search: W diag(s) at the chosen
        scales s, X / s, one reference GEMM and one quantize + loss GEMM per
        fraction."""
        torch, awq = self.torch, self.awq
        N, K, T = ws.shape[0], ws.shape[1], xs.shape[0]
        n = len(CLIP_GRID)
        nb = awq.load().awq_clip_search_workspace_bytes(N, K, T, G, n, 1)
        wsp = torch.empty(nb, dtype=torch.uint8, device=self.dev)
        awq.awq_clip_search(ws, xs, CLIP_GRID, G, channel_scale=s, workspace=wsp)   # warm-up
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        losses, best = awq.awq_clip_search(ws, xs, CLIP_GRID, G, channel_scale=s, workspace=wsp)
        tc = time.perf_counter() - t0
        flop = (n + 1) * 2.0 * T * N * K
        log(f"clip search: {tc * 1e3:.1f} ms, p* = {CLIP_GRID[best]}")
        return {"ms": round(tc * 1e3, 2), "fractions": CLIP_GRID, "best_fraction": CLIP_GRID[best],
                "loss_ratio_best_to_unclipped": round(float(losses[best] / losses[0]), 6),
                "TFLOP/s": round(flop / tc / 1e12, 1),
                "workload": f"W[{N},{K}] diag(s), X[{T},{K}] / s, {n} fractions, G=128 ({n + 1} GEMMs)"}

    # ------------------------------------------------------------ HBM copy
    def run_copy(self):
        torch = self.torch
        a = torch.empty(COPY_BYTES // 2, dtype=torch.float16, device=self.dev)
        b = torch.empty_like(a)
        a.fill_(1.0)
        for _ in range(3):
            b.copy_(a)
        t = self.time(lambda _: b.copy_(a), 10) / 10
        gbs = 2 * COPY_BYTES / t / 1e9
        log(f"copy 1 GiB: {t * 1e6:.0f} us, {gbs:.0f} GB/s (read + write)")
        return {"bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES, "us": round(t * 1e6, 1),
                "GB/s": round(gbs, 1)}

    # ------------------------------------------------------------ CPU oracle
    def run_cpu_baseline(self):
        import oracle

        try:
            from threadpoolctl import threadpool_info
            blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        except Exception:
            blas_threads = 1
        t_cpu, b_cpu, n = 0.0, 0, 0
        cache = {}
        t_start = time.perf_counter()
        while time.perf_counter() - t_start < 12.0:
            for (_, N, K) in self.linears:
                if (N, K) not in cache:
                    lay = synth.decode_layer(N, K, 1)
                    cache[(N, K)] = (oracle.quantize(lay["w"], G), lay["x"])
                (qw, sc, zr), x = cache[(N, K)]
                t0 = time.perf_counter()
                oracle.linear_ref(x, qw, sc, zr, G)
                t_cpu += time.perf_counter() - t0
                b_cpu += gemv_bytes(1, N, K)
                n += 1
        value = b_cpu / t_cpu / 1e9
        log(f"cpu oracle: {value:.2f} GB/s over {n} products")
        return {"value": round(value, 3), "unit": "GB/s", "cores": int(blas_threads), "kind": "oracle",
                "sample": f"{n} M=1 products over the 7 Llama-7B linear shapes, each the oracle's fp64 "
                          f"dequantize (single-threaded NumPy) + fp64 matrix-vector product "
                          f"({blas_threads} BLAS threads); {t_cpu:.1f} s of CPU work"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-search", action="store_true")
    ap.add_argument("--only", choices=["decode", "decode-fused", "decode-model", "gemv-roofline", "skinny", "gemm", "quantize",
                                       "search", "copy", "w8"],
                    help="run one section (for profiler runs); timings go to stderr")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the library has no multi-GPU "
                                   "path (--gpus must be 1)"}))
        sys.exit(2)

    b = Bench(args)
    if args.only:
        if args.only in ("decode", "gemv-roofline"):
            b.setup_decode()
            if args.only == "decode":
                b.run_decode()
            else:
                b.run_gemv_shapes([ROOFLINE_SHAPE])
        elif args.only == "decode-fused":
            b.run_decode_fused()
        elif args.only == "decode-model":
            b.run_decode_model()
        elif args.only == "skinny":
            b.run_skinny()
        elif args.only == "gemm":
            b.run_gemm()
        elif args.only == "quantize":
            b.run_quantize()
        elif args.only == "search":
            b.run_search()
        elif args.only == "w8":
            b.run_w8()
        else:
            b.run_copy()
        return

    b.setup_decode()
    value, ms_per_step = b.run_decode()
    per_shape = b.run_gemv_shapes(synth.DECODE_SHAPES)
    roof = per_shape[f"{ROOFLINE_SHAPE[0]}x{ROOFLINE_SHAPE[1]}"]
    del b.copies
    fused = b.run_decode_fused()
    model = b.run_decode_model()
    floor_us = b.run_launch_floor()
    skinny = b.run_skinny()
    groups = b.run_group_sizes()
    w8 = b.run_w8()
    copy = b.run_copy()
    gemm = b.run_gemm()
    quant = b.run_quantize()
    search = None if args.no_search else b.run_search()
    cpu = None if args.no_cpu_baseline else b.run_cpu_baseline()

    traffic, calib = measured_traffic()
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
                   "linears": [f"{n}:{N}x{K}" for (n, N, K) in b.linears], "weight_copies": b.n_copies,
                   "step_bytes": b.step_bytes},
        "roofline": {"bound": "hbm", "achieved": roof["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(roof["GB/s"] / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "traffic_unit": "bytes per launch (FETCH_SIZE x fetch_factor + WRITE_SIZE x write_factor)",
                     "traffic_calibration": calib,
                     "kernel": f"gemv M=1 {ROOFLINE_SHAPE[0]}x{ROOFLINE_SHAPE[1]} (gate/up projection)",
                     "bytes_per_launch": roof["bytes"], "launch_us": roof["us"],
                     "frac_of_copy_bandwidth": round(roof["GB/s"] / copy["GB/s"], 4),
                     "graph_launch_floor_us": floor_us},
        "step_frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "hbm_copy_1GiB": copy,
        "gemv_per_shape": per_shape,
        "decode_fused": fused,
        "decode_model": model,
        "skinny_batched_decode": skinny,
        "gemv_group_sizes": groups,
        "w8a16": w8,
        "gemm": gemm,
        "quantize": quant,
        "scale_search": search,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
