"""W4A16 benchmark on one MI355X: decode GEMV effective HBM GB/s (M = 1) and
prefill GEMM TFLOP/s (M = 2048), each against its roofline.

A step is one decode pass over the seven linear layers of a Llama-7B-shaped
decoder layer (q/k/v/o 4096x4096, gate/up 11008x4096, down 4096x11008; INT4,
group 128, zero-points; seven weight tensors) at M = 1, in the order a
decoder layer allows: q/k/v in one awq_gemm_grouped launch (they read the
same x), o, gate/up in one grouped launch, down. The weights rotate over
enough copies (> 1.2 GB) that the 256 MB last-level cache cannot hold them,
so every step streams its weights from HBM; the steps are replayed from HIP
graphs, so host launch cost is outside the timed kernels. `value` is the
step's algorithmic bytes over its time.

The same run also times, each in its own section:
  * the same step as seven awq_gemm launches, one per layer;
  * each GEMV launch of the step on its own, back to back over the rotated
    copies (the per-launch roofline fractions);
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
# The decode step's launches: layers of synth.LLAMA7B_LAYER by index; q/k/v
# and gate/up read the same x and run as one grouped launch each.
DECODE_GROUPS = (("qkv", (0, 1, 2)), ("o_proj", (3,)), ("gate_up", (4, 5)), ("down_proj", (6,)))
COPY_BYTES = 1 << 30
CLIP_BENCH_FRACTION = 0.01                                # the clip of xxmr.cn §1.5
CLIP_GRID = [0.0, 0.001, 0.002, 0.005, 0.01, 0.02]       # clip-search fractions


def gemv_bytes(M, N, K, g=G):
    """Algorithmic bytes of one W4A16 product: packed codes, fp16 scale and
    zero per group, fp16 x in, fp16 y out."""
    return N * K // 2 + N * (K // g) * 4 + M * K * 2 + M * N * 2


def grouped_bytes(M, shapes, g=G):
    """Algorithmic bytes of one grouped launch over layers (N, K) sharing x:
    every layer's codes, scales, zeros and y, and x once."""
    K = shapes[0][1]
    return sum(N * K // 2 + N * (K // g) * 4 + M * N * 2 for (N, _) in shapes) + M * K * 2


def step_launches(linears):
    """(label, layer indices, algorithmic bytes) of each launch of the decode
    step."""
    out = []
    for name, idx in DECODE_GROUPS:
        shapes = [(linears[j][1], linears[j][2]) for j in idx]
        label = f"{len(idx)}x{shapes[0][0]}x{shapes[0][1]}" if len(idx) > 1 else f"{shapes[0][0]}x{shapes[0][1]}"
        out.append((label, idx, grouped_bytes(1, shapes)))
    return out


def quantize_bytes(N, K, g=G):
    """fp16 W in; packed codes and fp16 scales/zeros out."""
    return N * K * 2 + N * K // 2 + N * (K // g) * 4


def log(*a):
    print(*a, file=sys.stderr, flush=True)


COUNTERS_FILE = os.path.join("profiles", "counters_gemv_gemm.json")
GEMV_SOURCE = os.path.join("weight_only_int4_quantize_amd", "csrc", "gemv.hip")


def source_sha256(rel):
    import hashlib

    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(linears):
    """HBM bytes of one decode step, from the FETCH_SIZE and WRITE_SIZE
    counter runs summarized under profiles/ (each scaled by the same counter
    read on a copy of known size), summed over the step's launches. None
    once the GEMV source has changed since the counters were taken."""
    try:
        with open(os.path.join(ROOT, COUNTERS_FILE)) as f:
            rec = json.load(f)
        if source_sha256(GEMV_SOURCE) != rec.get("gemv_source_sha256"):
            return None, None
        by_label = {g["label"]: g for g in rec["groups"] if g["kind"] == "gemv"}
        total = sum(by_label[f"gemv_M1_{label}"]["traffic_bytes"] for (label, _, _) in step_launches(linears))
        calib = next(g for g in rec["groups"] if g["kind"] == "copy")
    except (OSError, KeyError, ValueError, StopIteration):
        return None, None
    return int(total), {"copy_bytes": calib["bytes"], "fetch_factor": calib.get("fetch_factor"),
                        "write_factor": calib.get("write_factor")}


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
        self.launches = step_launches(self.linears)
        self.step_bytes = sum(b for (_, _, b) in self.launches)
        self.step_bytes_seven = sum(gemv_bytes(1, N, K) for (_, N, K) in self.linears)
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

    def launch(self, layer, idx):
        """One launch of the step: the layers idx of a copy (one awq_gemm, or
        one awq_gemm_grouped when they share x)."""
        if len(idx) == 1:
            qw, sc, zr, x, y, _, _ = layer[idx[0]]
            self.awq.awq_gemm(x, qw, sc, zr, G, out=y)
        else:
            self.awq.awq_gemm_grouped(layer[idx[0]][3], [layer[j][:3] for j in idx], G,
                                      outs=[layer[j][4] for j in idx])

    def decode_step(self, i):
        layer = self.copies[i % self.n_copies]
        for (_, idx, _) in self.launches:
            self.launch(layer, idx)

    def decode_step_seven(self, i):
        for (qw, sc, zr, x, y, N, K) in self.copies[i % self.n_copies]:
            self.awq.awq_gemm(x, qw, sc, zr, G, out=y)

    def run_decode(self, step_fn=None, step_bytes=None, label="decode layer"):
        args = self.args
        step_fn = step_fn or self.decode_step
        step_bytes = step_bytes or self.step_bytes
        for i in range(max(args.warmup, 1)):
            step_fn(i)
        self.torch.cuda.synchronize()
        # one graph per full rotation over the copies, one for the rest, so
        # that exactly args.steps steps are timed
        g_full = self.capture(step_fn, self.n_copies)
        rem = args.steps % self.n_copies
        g_rem = self.capture(step_fn, rem) if rem else None
        n_full = args.steps // self.n_copies

        def steps(_):
            for _r in range(n_full):
                g_full.replay()
            if g_rem is not None:
                g_rem.replay()

        g_full.replay()
        t = self.time(steps)
        ms = t / args.steps * 1e3
        value = step_bytes * args.steps / t / 1e9
        log(f"{label}: {ms * 1e3:.2f} us/step, {value:.0f} GB/s")
        return value, ms

    def run_decode_seven(self):
        """The same step as seven awq_gemm launches, one per layer."""
        value, ms = self.run_decode(self.decode_step_seven, self.step_bytes_seven, "decode layer, seven launches")
        return {"launches": 7, "us_per_step": round(ms * 1e3, 2), "step_bytes": self.step_bytes_seven,
                "GB/s": round(value, 1), "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4)}

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

    def run_decode_batched(self):
        """The decode step at a batch of M = 4 and 16 tokens, as a serving
        loop calls it (no workspace): the seven linears as four launches
        (q/k/v and gate/up grouped: one column-tile launch over the stacked
        layers) and as seven awq_gemm calls, weights rotated over the decode
        step's copies. Layers of one launch group share x."""
        torch, awq = self.torch, self.awq
        out = {}
        group_of = {}
        for gi, (_, idx) in enumerate(DECODE_GROUPS):
            for j in idx:
                group_of[j] = gi
        for M in (4, 16):
            xs = [self.d(synth.make_layer(1, self.linears[idx[0]][2], M, seed=[12, M, gi], w_std=0.02)["x"])
                  for gi, (_, idx) in enumerate(DECODE_GROUPS)]
            copies = [[(qw, sc, zr, xs[group_of[j]], torch.empty((M, N), dtype=torch.float16, device=self.dev), N, K)
                       for j, (qw, sc, zr, _, _, N, K) in enumerate(layer)] for layer in self.copies]
            groups = [idx for (_, idx) in DECODE_GROUPS]
            bytes4 = sum(grouped_bytes(M, [(self.linears[j][1], self.linears[j][2]) for j in idx]) for idx in groups)
            bytes7 = sum(gemv_bytes(M, N, K) for (_, N, K) in self.linears)

            def step(i, copies=copies):
                for idx in groups:
                    self.launch(copies[i % len(copies)], idx)

            def step_seven(i, copies=copies):
                for (qw, sc, zr, x, y, _, _) in copies[i % len(copies)]:
                    awq.awq_gemm(x, qw, sc, zr, G, out=y)

            res = {}
            for label, fn, nbytes in (("grouped_4_launches", step, bytes4), ("seven_launches", step_seven, bytes7)):
                for i in range(4):
                    fn(i)
                g = self.capture(fn, len(copies))
                g.replay()
                reps = 10
                t = min(self.time(lambda _: [g.replay() for _r in range(reps)]) for _ in range(3)) / (reps * len(copies))
                del g
                res[label] = {"us_per_step": round(t * 1e6, 2), "GB/s": round(nbytes / t / 1e9, 1),
                              "frac_of_hbm_peak": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)}
                log(f"decode step M={M}, {label}: {t * 1e6:.2f} us, {nbytes / t / 1e9:.0f} GB/s")
            res["kernel"] = awq.gemm_kernel(M, 12288, 4096, G)
            out[f"M{M}"] = res
            del copies
        torch.cuda.synchronize()
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
                        "kernel": awq.gemm_kernel(M, N, K, g, workspace=True)}
            log(f"batched decode {key}: {t * 1e6:.2f} us, {nbytes / t / 1e9:.0f} GB/s")
            del cps, gr
        torch.cuda.synchronize()
        return out

    def rotated_product(self, M, N, K, g, lay, workspace=None, reps_per_copy=2):
        """Back-to-back launches of one W4A16 product with the weights rotated
        over enough copies (> 1.2 GB) that no cache holds them; returns the
        time per launch in seconds."""
        torch, awq = self.torch, self.awq
        qw, sc, zr = awq.awq_quantize(self.d(lay["w"]), g)
        x = self.d(lay["x"])
        nbytes = gemv_bytes(M, N, K, g)
        n_copies = max(2, int(np.ceil(1.2e9 / nbytes)))
        cps = [(qw.clone(), sc.clone(), zr.clone()) for _ in range(n_copies)]
        del qw, sc, zr
        y = torch.empty((M, N), dtype=torch.float16, device=self.dev)

        def one(i):
            q = cps[i % len(cps)]
            awq.awq_gemm(x, q[0], q[1], q[2], g, out=y, workspace=workspace)

        for i in range(4):
            one(i)
        gr = self.capture(one, reps_per_copy * n_copies)
        gr.replay()
        t = min(self.time(lambda _: gr.replay()) for _ in range(3)) / (reps_per_copy * n_copies)
        del cps, gr
        torch.cuda.synchronize()
        return t

    def run_sweep(self):
        """The larger shapes and group sizes of the 13B / 70B sweep: M = 1 (the
        GEMV) and M = 32 (the skinny kernel) at group sizes 64 and 128, in
        effective HBM GB/s with the weights rotated past every cache, and
        M = 512 (the MFMA GEMM) at group size 64 in TFLOP/s (group size 128
        is in the GEMM section)."""
        ws = self.awq.gemm_workspace(512, 1, 1, self.dev)
        out = {}
        for (N, K) in synth.SWEEP_SHAPES:
            for g in synth.SWEEP_G:
                for M in (1, 32):
                    lay = synth.sweep_layer(N, K, M, g)
                    t = self.rotated_product(M, N, K, g, lay, workspace=ws)
                    b = gemv_bytes(M, N, K, g)
                    key = f"M{M}_{N}x{K}_G{g}"
                    out[key] = {"us": round(t * 1e6, 2), "bytes": b, "GB/s": round(b / t / 1e9, 1),
                                "frac_of_hbm_peak": round(b / t / 1e9 / HBM_PEAK_GBS, 4),
                                "kernel": self.awq.gemm_kernel(M, N, K, g, workspace=True)}
                    log(f"sweep {key}: {t * 1e6:.2f} us, {b / t / 1e9:.0f} GB/s")
            M, g = 512, 64
            lay = synth.sweep_layer(N, K, M, g)
            qw, sc, zr = self.awq.awq_quantize(self.d(lay["w"]), g)
            x = self.d(lay["x"])
            y = self.torch.empty((M, N), dtype=self.torch.float16, device=self.dev)

            def gm(i, x=x, qw=qw, sc=sc, zr=zr, y=y, g=g):
                self.awq.awq_gemm(x, qw, sc, zr, g, out=y, workspace=ws)

            self.warm(gm)
            t = self.time(gm, 20) / 20
            flop = 2.0 * M * N * K
            key = f"M{M}_{N}x{K}_G{g}"
            out[key] = {"us": round(t * 1e6, 2), "TFLOP/s": round(flop / t / 1e12, 1),
                        "frac_of_f16_peak": round(flop / t / 1e12 / F16_MFMA_PEAK_TFLOPS, 4), "kernel": "gemm"}
            log(f"sweep {key}: {t * 1e6:.1f} us, {flop / t / 1e12:.0f} TFLOP/s")
        return out

    def run_shard(self):
        """One GPU's share of the decode layer under 8-way column (output)
        parallelism: every projection keeps 1/8 of its rows (q/k/v/o
        512x4096, gate/up 1376x4096, down 512x11008), so each GPU streams
        1/8 of the weights with the same GEMV; the step's four launches
        (q/k/v and gate/up grouped) are timed as in the decode step, and the
        seven single launches beside them. The all-gather of y is not part of
        it (one GPU)."""
        torch, awq = self.torch, self.awq
        layer = [(n, N // 8, K) for (n, N, K) in synth.LLAMA7B_LAYER]
        step_bytes = sum(gemv_bytes(1, N, K) for (_, N, K) in layer)
        n_copies = max(2, int(np.ceil(1.2e9 / step_bytes)))
        base = {}
        for (_, N, K) in layer:
            if (N, K) not in base:
                lay = synth.make_layer(N, K, 1, seed=[8, N, K], w_std=0.02)
                qw, sc, zr = awq.awq_quantize(self.d(lay["w"]), G)
                base[(N, K)] = (qw, sc, zr, self.d(lay["x"]))
        # (qw, sc, zr, x, y, N, K) per linear; layers of one shape share x
        copies = [[(*[t.clone() for t in base[(N, K)][:3]], base[(N, K)][3],
                    torch.empty((1, N), dtype=torch.float16, device=self.dev), N, K) for (_, N, K) in layer]
                  for _ in range(n_copies)]
        groups = [idx for (_, idx) in DECODE_GROUPS]

        def step(i):
            for idx in groups:
                self.launch(copies[i % n_copies], idx)

        def step_seven(i):
            for (qw, sc, zr, x, y, _, _) in copies[i % n_copies]:
                awq.awq_gemm(x, qw, sc, zr, G, out=y)

        def timed(fn):
            for i in range(4):
                fn(i)
            g = self.capture(fn, n_copies)
            g.replay()
            reps = 20
            t = min(self.time(lambda _: [g.replay() for _r in range(reps)]) for _ in range(3)) / (reps * n_copies)
            del g
            return t

        t = timed(step)
        t7 = timed(step_seven)
        del copies
        torch.cuda.synchronize()
        log(f"tp8 shard step: {t * 1e6:.2f} us, {step_bytes / t / 1e9:.0f} GB/s (seven launches {t7 * 1e6:.2f} us)")
        return {"workload": "llama7b_decoder_layer_m1_int4_g128, one GPU's share under 8-way column parallelism",
                "linears": [f"{n}:{N}x{K}" for (n, N, K) in layer], "step_bytes": step_bytes,
                "launches": len(groups), "us_per_step": round(t * 1e6, 2), "GB/s": round(step_bytes / t / 1e9, 1),
                "frac_of_hbm_peak": round(step_bytes / t / 1e9 / HBM_PEAK_GBS, 4),
                "seven_launches_us_per_step": round(t7 * 1e6, 2)}

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

    def run_step_launches(self):
        """Each launch of the decode step on its own, back to back over the
        rotated copies."""
        out = {}
        for (label, idx, b) in self.launches:
            def one(i, idx=idx):
                self.launch(self.copies[i % self.n_copies], idx)

            reps = 8 * self.n_copies
            g1 = self.capture(one, reps)
            g1.replay()
            t = self.time(lambda _: g1.replay(), 4) / (4 * reps)
            out[label] = {"us": round(t * 1e6, 3), "GB/s": round(b / t / 1e9, 1), "bytes": b,
                          "launches_timed": 4 * reps,
                          "layers": [self.linears[j][0] for j in idx]}
            log(f"step launch {label}: {t * 1e6:.2f} us, {b / t / 1e9:.0f} GB/s")
            del g1
        return out

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

    # ------------------------------------------------------------ counter runs
    def run_counters(self, reps=4):
        """Fixed launches in a known order for rocprofv3 --pmc runs (one counter
        pass per run): a 1 GiB copy (the FETCH_SIZE / WRITE_SIZE calibration),
        the decode and fused GEMV shapes at M = 1 (weights rotated over `reps`
        copies, so every launch fetches from HBM), the prefill GEMM shapes at
        M = 2048 and the sweep at M = 512. Prints the manifest (label, work
        and launch count per group, in order) as one JSON line on stdout; the
        summary mode matches it to the counter rows."""
        torch, awq = self.torch, self.awq
        manifest = []
        a = torch.empty(COPY_BYTES // 2, dtype=torch.float16, device=self.dev)
        b = torch.empty_like(a)
        a.fill_(1.0)
        torch.cuda.synchronize()
        for _ in range(2):
            b.copy_(a)
        manifest.append({"label": "copy_1GiB", "kind": "copy", "bytes": COPY_BYTES, "launches": 2})
        del a, b
        torch.cuda.synchronize()
        gemv_shapes = list(synth.DECODE_SHAPES) + [(N, K) for (_, N, K) in synth.LLAMA7B_LAYER_FUSED
                                                    if (N, K) not in synth.DECODE_SHAPES]
        for (N, K) in gemv_shapes:
            lay = synth.decode_layer(N, K, 1)
            qw, sc, zr = awq.awq_quantize(self.d(lay["w"]), G)
            x = self.d(lay["x"])
            cps = [(qw.clone(), sc.clone(), zr.clone()) for _ in range(reps)]
            y = torch.empty((1, N), dtype=torch.float16, device=self.dev)
            torch.cuda.synchronize()
            for i in range(reps):
                awq.awq_gemm(x, *cps[i], G, out=y)
            torch.cuda.synchronize()
            manifest.append({"label": f"gemv_M1_{N}x{K}", "kind": "gemv", "M": 1, "N": N, "K": K,
                             "bytes": gemv_bytes(1, N, K), "launches": reps})
            del cps, qw, sc, zr
        # the decode step's grouped launches (layers of their own weights, one x)
        for (label, idx, nbytes) in step_launches(list(synth.LLAMA7B_LAYER)):
            if len(idx) == 1:
                continue
            shapes = [synth.LLAMA7B_LAYER[j][1:] for j in idx]
            K = shapes[0][1]
            parts = []
            for j, (N, _) in enumerate(shapes):
                lay = synth.decode_layer(N, K, 1)
                qw, sc, zr = awq.awq_quantize(self.d(lay["w"]), G)
                parts.append([(qw.clone(), sc.clone(), zr.clone()) for _ in range(reps)])
                x = self.d(lay["x"])
            ys = [torch.empty((1, N), dtype=torch.float16, device=self.dev) for (N, _) in shapes]
            torch.cuda.synchronize()
            for i in range(reps):
                awq.awq_gemm_grouped(x, [p[i] for p in parts], G, outs=ys)
            torch.cuda.synchronize()
            manifest.append({"label": f"gemv_M1_{label}", "kind": "gemv", "M": 1,
                             "N": sum(N for (N, _) in shapes), "K": K, "layers": len(idx), "bytes": nbytes,
                             "launches": reps})
            del parts
        ws = awq.gemm_workspace(synth.PREFILL_M, 11008, 11008, self.dev)
        gemm_shapes = [(synth.PREFILL_M, N, K) for (N, K) in synth.PREFILL_SHAPES] + \
                      [(512, N, K) for (N, K) in synth.SWEEP_SHAPES]
        for (M, N, K) in gemm_shapes:
            lay = synth.prefill_layer(N, K) if M == synth.PREFILL_M else synth.sweep_layer(N, K, M, G)
            qw, sc, zr = awq.awq_quantize(self.d(lay["w"]), G)
            x = self.d(lay["x"])
            y = torch.empty((M, N), dtype=torch.float16, device=self.dev)
            torch.cuda.synchronize()
            for i in range(reps):
                awq.awq_gemm(x, qw, sc, zr, G, out=y, workspace=ws)
            torch.cuda.synchronize()
            manifest.append({"label": f"gemm_{M}x{N}x{K}", "kind": "gemm", "M": M, "N": N, "K": K,
                             "flop": 2 * M * N * K, "launches": reps})
        print(json.dumps({"manifest": manifest}))

    # ------------------------------------------------------------ CPU oracle
    def run_cpu_baseline(self):
        """The oracle as it stands, timed on this host's cores: its BLAS uses
        as many threads as the process may run on (os.sched_getaffinity);
        the record names that count and the BLAS library."""
        import oracle

        cores = len(os.sched_getaffinity(0))
        blas = "unknown"
        try:
            from threadpoolctl import threadpool_info, threadpool_limits
            threadpool_limits(limits=cores, user_api="blas")
            info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
            blas_threads = max([p.get("num_threads", 1) for p in info] or [1])
            if info:
                blas = f"{info[0].get('internal_api')} {info[0].get('version')} ({info[0].get('threading_layer')})"
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
                "affinity_cores": cores, "blas": blas,
                "sample": f"{n} M=1 products over the 7 Llama-7B linear shapes, each the oracle's fp64 "
                          f"dequantize (NumPy elementwise, one thread) + fp64 matrix-vector product "
                          f"({blas_threads} BLAS threads, {blas}); {t_cpu:.1f} s of CPU work"}


# ---------------------------------------------------------------- profile summaries
# Run on the CSV output of rocprofv3 (--output-format csv -d DIR); they read
# nothing else and touch no GPU.

def _csv_rows(dirs, suffix):
    import csv
    import glob

    rows = []
    for d in dirs:
        for path in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
            with open(path, newline="") as f:
                rows.extend(csv.DictReader(f))
    return rows


def _short(name, n=90):
    return name if len(name) <= n else name[:n - 3] + "..."


def summarize_trace(dirs, out_path, command):
    """Per (kernel, grid) dispatch counts and start-to-end durations of a
    --kernel-trace run, sorted by total time, as markdown."""
    rows = _csv_rows(dirs, "kernel_trace.csv")
    groups = {}
    for r in rows:
        grid = int(r.get("Grid_Size_X", r.get("Grid_Size", 0))) * int(r.get("Grid_Size_Y", 1) or 1) * \
            int(r.get("Grid_Size_Z", 1) or 1)
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        groups.setdefault((r["Kernel_Name"], grid), []).append(dur)
    lines = ["# Kernel trace", "", "Command (from the repository root, on one MI355X):", "", f"    {command}",
             "", "Per (kernel, grid): dispatches and start-to-end durations, sorted by total time.", "",
             "| kernel | grid (threads) | dispatches | avg us | median us | total ms |", "|---|---|---|---|---|---|"]
    for (name, grid), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        d = np.array(d)
        lines.append(f"| `{_short(name)}` | {grid} | {d.size} | {d.mean():.2f} | {np.median(d):.2f} | "
                     f"{d.sum() / 1e3:.2f} |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_counters(dirs, manifest_path, out_path, commands):
    """Counter values per manifest group of a `bench.py --only counters` run:
    the dispatches of each group are the next `launches` dispatches whose
    kernel matches the group's kind, in dispatch order. Writes JSON with the
    per-dispatch averages and the derived figures (HBM bytes from
    FETCH_SIZE / WRITE_SIZE scaled by the copy calibration; MFMA FLOPs from
    SQ_INSTS_MFMA x 32768, checked against 2MNK; MFMA-busy % = 100 x
    SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs))."""
    with open(manifest_path) as f:
        text = f.read()
    manifest = json.loads([ln for ln in text.splitlines() if ln.startswith('{"manifest"')][-1])["manifest"]
    match = {"copy": ("copy", "Copy"), "gemv": ("gemv_kernel", "gemv_grouped_kernel", "gemv_grouped_packed_kernel", "skinny_kernel"),
             "gemm": ("gemm_kernel", "skinny_kernel")}
    out = [dict(g, avg={}) for g in manifest]
    for d in dirs:                     # one counter pass (one run of the same launches) per directory
        per_dispatch = {}
        for r in _csv_rows([d], "counter_collection.csv"):
            key = int(r["Dispatch_Id"])
            e = per_dispatch.setdefault(key, {"kernel": r["Kernel_Name"], "grid": int(r.get("Grid_Size", 0)),
                                              "counters": {}})
            e["counters"][r["Counter_Name"]] = e["counters"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            if r.get("Start_Timestamp") and r.get("End_Timestamp"):
                e["counters"]["duration_us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        order = sorted(per_dispatch)
        pos = 0
        for o in out:
            picked = []
            while pos < len(order) and len(picked) < o["launches"]:
                e = per_dispatch[order[pos]]
                pos += 1
                if any(m in e["kernel"] for m in match[o["kind"]]):
                    picked.append(e)
            if len(picked) < o["launches"]:
                raise SystemExit(f"{d}: counter rows end before group {o['label']}")
            if o.get("grid", picked[0]["grid"]) != picked[0]["grid"]:
                raise SystemExit(f"{d}: group {o['label']} matched another grid")
            o["kernel"], o["grid"] = _short(picked[0]["kernel"], 120), picked[0]["grid"]
            for c in sorted({c for e in picked for c in e["counters"]}):
                o["avg"][c] = float(np.mean([e["counters"].get(c, 0.0) for e in picked]))
    calib = next((o for o in out if o["kind"] == "copy"), None)
    if calib is not None:
        fk, wk = calib["avg"].get("FETCH_SIZE"), calib["avg"].get("WRITE_SIZE")
        fetch_factor = calib["bytes"] / (fk * 1024) if fk else None
        write_factor = calib["bytes"] / (wk * 1024) if wk else None
        for o in out:
            if o["kind"] == "copy":
                continue
            if fetch_factor and "FETCH_SIZE" in o["avg"]:
                o["fetch_bytes"] = round(o["avg"]["FETCH_SIZE"] * 1024 * fetch_factor)
            if write_factor and "WRITE_SIZE" in o["avg"]:
                o["write_bytes"] = round(o["avg"]["WRITE_SIZE"] * 1024 * write_factor)
            if "fetch_bytes" in o and "write_bytes" in o:
                o["traffic_bytes"] = o["fetch_bytes"] + o["write_bytes"]
                if "bytes" in o:
                    o["traffic_over_algorithmic"] = round(o["traffic_bytes"] / o["bytes"], 4)
                elif o["kind"] == "gemm":
                    # x, packed weights, fp16 scale and zero per group (G = 128), y
                    M, N, K = o["M"], o["N"], o["K"]
                    o["algorithmic_bytes"] = M * K * 2 + N * K // 2 + N * (K // G) * 4 + M * N * 2
                    o["traffic_over_algorithmic"] = round(o["traffic_bytes"] / o["algorithmic_bytes"], 4)
        calib["fetch_factor"], calib["write_factor"] = fetch_factor, write_factor
    # The CSV's GRBM_GUI_ACTIVE is the sum over the 8 XCDs' GRBMs (its rate
    # per us of dispatch is 8 x the clock), so one XCD's active cycles, the
    # denominator of a busy percentage, are an eighth of it (rocprofv3's
    # MfmaUtil takes the max over the XCDs, which agrees).
    xcds, simds = 8, 4 * 256
    for o in out:
        c = o["avg"]
        if "SQ_INSTS_MFMA" in c:
            o["mfma_flop"] = c["SQ_INSTS_MFMA"] * 32768
            if "flop" in o:
                o["mfma_flop_equals_2MNK"] = abs(o["mfma_flop"] - o["flop"]) <= 1e-9 * o["flop"]
        active = c.get("GRBM_GUI_ACTIVE", 0.0) / xcds
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c and active:
            o["mfma_busy_pct"] = round(100.0 * c["SQ_VALU_MFMA_BUSY_CYCLES"] / (active * simds), 2)
        if "MfmaUtil" in c:
            o["mfma_util_pct"] = round(c["MfmaUtil"], 2)      # rocprofv3's own derived metric
        if "TA_BUSY_avr" in c and active:
            o["ta_busy_pct"] = round(100.0 * c["TA_BUSY_avr"] / active, 2)
            # TD_TD_BUSY and TA_TA_BUSY are summed over the same CU
            # instances: the texture-data unit's busy share is the address
            # unit's scaled by their ratio
            if c.get("TA_TA_BUSY") and "TD_TD_BUSY" in c:
                o["td_busy_pct"] = round(o["ta_busy_pct"] * c["TD_TD_BUSY"] / c["TA_TA_BUSY"], 2)
        if c.get("SQ_WAVE_CYCLES"):
            # shares of the waves' resident time (both counters in quad-cycles)
            for k, name in (("SQ_WAIT_INST_ANY", "wave_wait_issue_pct"), ("SQ_ACTIVE_INST_VALU", "wave_valu_pct"),
                            ("SQ_ACTIVE_INST_LDS", "wave_lds_pct")):
                if k in c:
                    o[name] = round(100.0 * c[k] / c["SQ_WAVE_CYCLES"], 2)
        if active and c.get("duration_us") and o["kind"] != "gemv":
            # one XCD's active cycles per us of dispatch (long dispatches only:
            # the active count also covers a dispatch's start-up)
            o["clock_mhz"] = round(active / c["duration_us"], 1)
    lines = ["# Counters of the GEMV and GEMM launches", "", "Commands (from the repository root, on one MI355X):", ""]
    lines += [f"    {c}" for c in commands]
    lines += ["", "Per launch (average over the group's dispatches). HBM bytes = FETCH_SIZE x fetch factor + "
              "WRITE_SIZE x write factor (both from the 1 GiB copy); algorithmic bytes as in bench.py. "
              "MFMA FLOPs = SQ_INSTS_MFMA x 32768. MfmaUtil is rocprofv3's derived metric. TA busy = "
              "TA_BUSY_avr over one XCD's active cycles; TD busy = TA busy x TD_TD_BUSY / TA_TA_BUSY (both "
              "summed over the same CUs). Waiting to issue and in VALU: SQ_WAIT_INST_ANY and SQ_ACTIVE_INST_VALU "
              "over SQ_WAVE_CYCLES (shares of the waves' resident time).", "",
              "| launch | grid | HBM bytes | / algorithmic | MFMA FLOPs = 2MNK | MfmaUtil % | TA busy % | TD busy % "
              "| waves waiting to issue % | waves in VALU % | clock MHz |",
              "|---|---|---|---|---|---|---|---|---|---|---|"]
    for o in out:
        if o["kind"] == "copy":
            lines.append(f"| copy 1 GiB (calibration: fetch x{o.get('fetch_factor', 0):.3f}, write "
                         f"x{o.get('write_factor', 0):.3f}) | {o['grid']} | | | | | {o.get('ta_busy_pct', '')} | "
                         f"{o.get('td_busy_pct', '')} | | | {o.get('clock_mhz', '')} |")
            continue
        lines.append(f"| {o['label']} | {o['grid']} | {o.get('traffic_bytes', '')} | {o.get('traffic_over_algorithmic', '')} "
                     f"| {o.get('mfma_flop_equals_2MNK', '')} | {o.get('mfma_util_pct', '')} | {o.get('ta_busy_pct', '')} "
                     f"| {o.get('td_busy_pct', '')} | {o.get('wave_wait_issue_pct', '')} | {o.get('wave_valu_pct', '')} "
                     f"| {o.get('clock_mhz', '')} |")
    with open(os.path.splitext(out_path)[0] + ".md", "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(out_path, "w") as f:
        json.dump({"commands": commands, "gemv_source_sha256": source_sha256(GEMV_SOURCE),
                   "gemm_source_sha256": source_sha256(os.path.join("weight_only_int4_quantize_amd", "csrc",
                                                                    "gemm.hip")),
                   "groups": out}, f, indent=1)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-search", action="store_true")
    ap.add_argument("--only", choices=["decode", "decode-fused", "decode-model", "gemv-roofline", "skinny", "gemm", "quantize",
                                       "search", "copy", "w8", "sweep", "shard", "counters", "decode-batched"],
                    help="run one section (for profiler runs); timings go to stderr")
    ap.add_argument("--summarize-trace", nargs="+", metavar="DIR",
                    help="summarize rocprofv3 kernel-trace CSVs under DIR into --out (no GPU)")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="summarize rocprofv3 counter CSVs under DIR (a --only counters run) into --out")
    ap.add_argument("--manifest", help="stdout of the --only counters run (its manifest line)")
    ap.add_argument("--out", help="summary file to write")
    ap.add_argument("--command", action="append", default=[], help="profiling command(s) to record in the summary")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.out, " ; ".join(args.command))
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.manifest, args.out, args.command)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the library has no multi-GPU "
                                   "path (--gpus must be 1)"}))
        sys.exit(2)

    b = Bench(args)
    if args.only:
        if args.only in ("decode", "gemv-roofline", "decode-batched"):
            b.setup_decode()
            if args.only == "decode":
                b.run_decode()
            elif args.only == "decode-batched":
                b.run_decode_batched()
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
        elif args.only == "sweep":
            b.run_sweep()
        elif args.only == "shard":
            b.run_shard()
        elif args.only == "counters":
            b.run_counters()
        else:
            b.run_copy()
        return

    b.setup_decode()
    value, ms_per_step = b.run_decode()
    seven = b.run_decode_seven()
    per_launch = b.run_step_launches()
    per_shape = b.run_gemv_shapes(synth.DECODE_SHAPES)
    batched = b.run_decode_batched()
    del b.copies
    fused = b.run_decode_fused()
    model = b.run_decode_model()
    floor_us = b.run_launch_floor()
    skinny = b.run_skinny()
    sweep = b.run_sweep()
    shard = b.run_shard()
    groups = b.run_group_sizes()
    w8 = b.run_w8()
    copy = b.run_copy()
    gemm = b.run_gemm()
    quant = b.run_quantize()
    search = None if args.no_search else b.run_search()
    cpu = None if args.no_cpu_baseline else b.run_cpu_baseline()

    traffic, calib = measured_traffic(b.linears)
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
                   "linears": [f"{n}:{N}x{K}" for (n, N, K) in b.linears],
                   "launches": [f"{name}:{label}" for (name, _), (label, _, _) in zip(DECODE_GROUPS, b.launches)],
                   "weight_copies": b.n_copies, "step_bytes": b.step_bytes},
        "roofline": {"bound": "hbm", "achieved": round(value, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "traffic_unit": "HBM bytes per step: FETCH_SIZE x fetch_factor + WRITE_SIZE x "
                                     "write_factor summed over the step's four GEMV launches",
                     "traffic_calibration": calib,
                     "kernel": "gemv, the four M=1 launches of one decode step (q/k/v grouped, o, gate/up "
                               "grouped, down; one graph replay)",
                     "bytes_per_launch": b.step_bytes, "launch_us": round(ms_per_step * 1e3, 3),
                     "per_launch": {k: {**v, "frac": round(v["GB/s"] / HBM_PEAK_GBS, 4)} for k, v in per_launch.items()},
                     "frac_of_copy_bandwidth": round(value / copy["GB/s"], 4),
                     "graph_launch_floor_us": floor_us},
        "step_frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "decode_seven_launches": seven,
        "hbm_copy_1GiB": copy,
        "gemv_per_shape": {k: {**v, "frac": round(v["GB/s"] / HBM_PEAK_GBS, 4)} for k, v in per_shape.items()},
        "decode_fused": fused,
        "decode_model": model,
        "skinny_batched_decode": skinny,
        "sweep_13b_70b": sweep,
        "tp8_shard_1gpu": shard,
        "decode_batched": batched,
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
