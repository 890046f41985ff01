#!/usr/bin/env python3
"""Throughput of the quantized-actor W8A8 linear path on one MI355X.

Workload of one step (the Qwen2.5-1.5B-shaped INT8 W8A8 decoder linears, stacked to the model's 28 layers
so that the weights streamed per pass -- 1.31 GB of INT8 codes, 2.62 GB of bf16 masters -- are far larger
than the 256 MB last-level cache and every read comes from HBM):
  1. publish, once per RL step ("QuRL: Efficient Reinforcement Learning with Quantized Rollout", section 4):
     a1  quantize every bf16 master weight to INT8 codes + one fp32 scale per output channel;
     a5  count the codes (and scales) that changed since the previously published set (section 4.3);
  2. decode, at every batch M in (1, 16, 64) ("QuRL" section 5: token-wise activation scales), for each
     layer and each of qkv 1536->2048, o 1536->1536, gate/up 1536->2x8960, down 8960->1536:
     a2  quantize the layer's bf16 activations per token;
     a3  the W8A8 linear with its dequantization epilogue, bf16 out;
     at M = 1 both run in one launch (qr_w8a8_linear_bf16: each workgroup quantizes the token row into its LDS,
     the same codes and outputs bit for bit), at M = 16 and 64 as two launches.
The step is captured once in a HIP graph (about 680 launches, most of them a few microseconds long) and
replayed; inputs are resident in HBM before the timed region starts.

value = algorithmic HBM bytes of one step (what the method must move: codes, scales, bf16 inputs and
outputs) x steps / elapsed seconds. The JSON line also carries, per step of the path, the average launch
duration from HIP events on the stream the kernels run on, the roofline of the dominant kernel (its measured
HBM traffic when profiles/ holds a FETCH_SIZE / WRITE_SIZE summary taken on the current kernel sources), the CPU
oracle timed on a bounded sample of the same step, and (unless --quick) the FP8 7B-shaped linears at the
MFMA-bound batches and the grouped MoE FFN linears.

Counter runs for the traffic figure (each counter in a run of its own):
  rocprofv3 --pmc FETCH_SIZE -d DIR_F -o t --output-format csv -- python3 bench.py --profile-row ROW
  rocprofv3 --pmc WRITE_SIZE -d DIR_W -o t --output-format csv -- python3 bench.py --profile-row ROW
  python3 bench.py --profile-row ROW --traffic-summary DIR_F DIR_W > profiles/traffic_ROW.md
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W8A8 linear TOPS (MFMA % peak) + HBM GB/s at rollout decode shapes, 1 GPU"
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E, published
MFMA_PEAK_TOPS = 5000.0       # MI355X dense INT8 POP/s and FP8 PFLOP/s, published (x1000)

LAYERS = 28
LINEARS = (("qkv", 2048, 1536), ("o", 1536, 1536), ("gate_up", 17920, 1536), ("down", 1536, 8960))
BATCHES = (1, 16, 64)
FUSED_BATCHES = (1,)          # decode batches whose activation quantization runs inside the linear
M_MAX = max(BATCHES)
WEIGHT_STD = 0.02
W4_GROUP = 128                # input channels per INT4 scale group (W4A16)


def log(msg):
    sys.stderr.write("[bench] %s\n" % msg)
    sys.stderr.flush()


# ----------------------------------------------------------------------------------------------------------
# algorithmic bytes and operations per call
# ----------------------------------------------------------------------------------------------------------
def bytes_quantize(rows, k, in_bytes):
    return rows * k * in_bytes + rows * k + 4 * rows


def bytes_linear(m, n, k, out_bytes=2):
    return n * k + 4 * n + m * k + 4 * m + m * n * out_bytes


def bytes_count(codes, scales):
    return 2 * codes + 2 * 4 * scales


def ops_linear(m, n, k):
    return 2 * m * n * k


# ----------------------------------------------------------------------------------------------------------
# synthetic inputs, generated on the GPU (seeded)
# ----------------------------------------------------------------------------------------------------------
def normal_bf16(gen, shape, std, dev):
    import torch

    return (torch.randn(shape, generator=gen, device=dev, dtype=torch.float32) * std).to(torch.bfloat16)


def activations_bf16(gen, layers, m, k, dev):
    """N(0, 1) per element with 4 outlier input channels x20 per layer."""
    import torch

    x = torch.randn((layers, m, k), generator=gen, device=dev, dtype=torch.float32)
    for l in range(layers):
        cols = torch.randperm(k, generator=gen, device=dev)[:4]
        x[l, :, cols] *= 20.0
    return x.to(torch.bfloat16)


class TimedGraph:
    """A HIP graph of a fixed launch sequence, replayed on the current stream and timed with events."""

    def __init__(self, fn, launches):
        import torch

        self.launches = launches
        fn()  # eager warm-up outside capture (loads code objects)
        torch.cuda.synchronize()
        self.g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g):
            fn()
        torch.cuda.synchronize()

    def replay(self):
        self.g.replay()

    def time_ms(self, reps):
        """Average milliseconds per replay over `reps` back-to-back replays."""
        import torch

        self.g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            self.g.replay()
        b.record()
        b.synchronize()
        return a.elapsed_time(b) / reps


# ----------------------------------------------------------------------------------------------------------
# the main workload
# ----------------------------------------------------------------------------------------------------------
class DecoderStack:
    def __init__(self, dev, seed=0):
        import torch

        import quantized_rollout_amd as qr

        self.qr = qr
        self.dev = dev
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed)
        rows_total = sum(LAYERS * n for _, n, _ in LINEARS)
        codes_total = sum(LAYERS * n * k for _, n, k in LINEARS)
        self.codes_total, self.rows_total = codes_total, rows_total
        # one contiguous code / scale buffer for the whole published set (the changed-code count is one pass)
        self.codes = torch.empty(codes_total, dtype=torch.uint8, device=dev)
        self.scales = torch.empty(rows_total, dtype=torch.float32, device=dev)
        self.prev_codes = torch.empty_like(self.codes)
        self.prev_scales = torch.empty_like(self.scales)
        self.count = torch.zeros(3, dtype=torch.int64, device=dev)
        self.w, self.wc, self.ws, self.pc, self.ps = {}, {}, {}, {}, {}
        self.x, self.xc, self.xs, self.y = {}, {}, {}, {}
        co, so = 0, 0
        for name, n, k in LINEARS:
            self.w[name] = normal_bf16(gen, (LAYERS * n, k), WEIGHT_STD, dev)
            self.wc[name] = self.codes[co:co + LAYERS * n * k].view(LAYERS * n, k)
            self.pc[name] = self.prev_codes[co:co + LAYERS * n * k].view(LAYERS * n, k)
            self.ws[name] = self.scales[so:so + LAYERS * n]
            self.ps[name] = self.prev_scales[so:so + LAYERS * n]
            co += LAYERS * n * k
            so += LAYERS * n
        # the previously published set: the same masters before an update dW ~ N(0, 1e-5)
        for name, n, k in LINEARS:
            w_prev = (self.w[name].float() - torch.randn(self.w[name].shape, generator=gen, device=dev) * 1e-5)
            qr.qr_quantize_weights(w_prev.to(torch.bfloat16), qr.QR_INT8, codes=self.pc[name], scales=self.ps[name])
            del w_prev
        for name, n, k in LINEARS:
            self.x[name] = activations_bf16(gen, LAYERS, M_MAX, k, dev)
            self.xc[name] = torch.empty((LAYERS, M_MAX, k), dtype=torch.uint8, device=dev)
            self.xs[name] = torch.empty((LAYERS, M_MAX), dtype=torch.float32, device=dev)
            self.y[name] = torch.empty((M_MAX, n), dtype=torch.bfloat16, device=dev)
        self.wsp = qr.Workspace()
        need = max(max(qr.qr_workspace_bytes(qr.QR_INT8, m, n, k),
                       qr.qr_w8a8_linear_bf16_workspace_bytes(qr.QR_INT8, m, n, k))
                   for m in BATCHES for _, n, k in LINEARS)
        self.wsp.get(need)
        torch.cuda.synchronize()

    # the pieces of one step -------------------------------------------------------------------------------
    def publish_quantize(self):
        qr = self.qr
        for name, n, k in LINEARS:
            qr.qr_quantize_weights(self.w[name], qr.QR_INT8, codes=self.wc[name], scales=self.ws[name])

    def publish_count(self):
        qr = self.qr
        qr.qr_count_code_changes(self.codes, self.prev_codes, qr.QR_INT8, self.scales, self.prev_scales,
                                 out3=self.count)

    def decode_acts(self, m):
        qr = self.qr
        for l in range(LAYERS):
            for name, n, k in LINEARS:
                qr.qr_quantize_acts(self.x[name][l, :m], qr.QR_INT8, codes=self.xc[name][l, :m],
                                    scales=self.xs[name][l, :m])

    def decode_linears(self, m):
        qr = self.qr
        for l in range(LAYERS):
            for name, n, k in LINEARS:
                qr.qr_w8a8_linear(qr.QR_INT8, self.xc[name][l, :m], self.xs[name][l, :m],
                                  self.wc[name][l * n:(l + 1) * n], self.ws[name][l * n:(l + 1) * n],
                                  y=self.y[name][:m], workspace=self.wsp)

    def decode_separate(self, m):
        """a2 then a3 for every linear: two launches each"""
        qr = self.qr
        for l in range(LAYERS):
            for name, n, k in LINEARS:
                qr.qr_quantize_acts(self.x[name][l, :m], qr.QR_INT8, codes=self.xc[name][l, :m],
                                    scales=self.xs[name][l, :m])
                qr.qr_w8a8_linear(qr.QR_INT8, self.xc[name][l, :m], self.xs[name][l, :m],
                                  self.wc[name][l * n:(l + 1) * n], self.ws[name][l * n:(l + 1) * n],
                                  y=self.y[name][:m], workspace=self.wsp)

    def decode_fused(self, m):
        """a2 inside a3 (qr_w8a8_linear_bf16 on the bfloat16 activations): one launch per linear"""
        qr = self.qr
        for l in range(LAYERS):
            for name, n, k in LINEARS:
                qr.qr_w8a8_linear_bf16(qr.QR_INT8, self.x[name][l, :m], self.wc[name][l * n:(l + 1) * n],
                                       self.ws[name][l * n:(l + 1) * n], y=self.y[name][:m], workspace=self.wsp)

    def decode(self, m):
        # single-token decode runs the activation quantization inside the linear's kernel (the same codes and
        # outputs, bit for bit, one launch instead of two); larger batches quantize first, then run the linear
        if m in FUSED_BATCHES:
            self.decode_fused(m)
        else:
            self.decode_separate(m)

    def step(self):
        self.publish_quantize()
        self.publish_count()
        for m in BATCHES:
            self.decode(m)

    # algorithmic work ---------------------------------------------------------------------------------------
    @staticmethod
    def row_work():
        """{row: (bytes, ops, launches)} of one step."""
        w = {}
        w["a1_quantize_weights"] = (sum(bytes_quantize(LAYERS * n, k, 2) for _, n, k in LINEARS), 0, len(LINEARS))
        codes = sum(LAYERS * n * k for _, n, k in LINEARS)
        rows = sum(LAYERS * n for _, n, _ in LINEARS)
        w["a5_count_changes"] = (bytes_count(codes, rows), 0, 1)
        for m in BATCHES:
            w["a2_quantize_acts_m%d" % m] = (LAYERS * sum(bytes_quantize(m, k, 2) for _, n, k in LINEARS), 0,
                                             LAYERS * len(LINEARS))
            w["a3_linear_m%d" % m] = (LAYERS * sum(bytes_linear(m, n, k) for _, n, k in LINEARS),
                                      LAYERS * sum(ops_linear(m, n, k) for _, n, k in LINEARS),
                                      LAYERS * len(LINEARS))
        return w

    def snapshot(self):
        import torch

        out = [self.codes.clone(), self.scales.clone(), self.count.clone()]
        for name, _, _ in LINEARS:
            out += [self.y[name].clone(), self.xc[name].clone(), self.xs[name].clone()]
        torch.cuda.synchronize()
        return out


# ----------------------------------------------------------------------------------------------------------
# other configurations of the path (side measurements, not part of `value`)
# ----------------------------------------------------------------------------------------------------------
def measure_fp8_7b(dev, reps):
    """7B-shaped FP8 linears (qkv 3584->4608, o 3584->3584, gate/up 3584->2x18944, down 18944->3584), codes
    of 5 distinct layers (1.17 GB) rotated; every batch of the configuration."""
    import torch

    import quantized_rollout_amd as qr

    L = 5
    lins = (("qkv", 4608, 3584), ("o", 3584, 3584), ("gate_up", 37888, 3584), ("down", 3584, 18944))
    batches = (1, 16, 128, 512, 2048)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1)
    wc, ws, xc, xs, y = {}, {}, {}, {}, {}
    for name, n, k in lins:
        w = normal_bf16(gen, (L * n, k), WEIGHT_STD, dev)
        wc[name], ws[name] = qr.qr_quantize_weights(w, qr.QR_FP8_E4M3)
        del w
        x = activations_bf16(gen, 1, max(batches), k, dev)[0]
        xc[name], xs[name] = qr.qr_quantize_acts(x, qr.QR_FP8_E4M3)
        y[name] = torch.empty((max(batches), n), dtype=torch.bfloat16, device=dev)
    wsp = qr.Workspace()
    wsp.get(max(qr.qr_workspace_bytes(qr.QR_FP8_E4M3, m, n, k) for m in batches for _, n, k in lins))
    out = {}
    for m in batches:
        def run(m=m):
            for l in range(L):
                for name, n, k in lins:
                    qr.qr_w8a8_linear(qr.QR_FP8_E4M3, xc[name][:m], xs[name][:m], wc[name][l * n:(l + 1) * n],
                                      ws[name][l * n:(l + 1) * n], y=y[name][:m], workspace=wsp)
        g = TimedGraph(run, L * len(lins))
        ms = g.time_ms(reps)
        nb = L * sum(bytes_linear(m, n, k) for _, n, k in lins)
        no = L * sum(ops_linear(m, n, k) for _, n, k in lins)
        out["m%d" % m] = {"us_per_layer": round(ms * 1e3 / L, 2), "GB/s": round(nb / ms / 1e6, 1),
                          "TFLOP/s": round(no / ms / 1e9, 1), "hbm_frac": round(nb / ms / 1e6 / HBM_PEAK_GBS, 3),
                          "mfma_frac": round(no / ms / 1e9 / MFMA_PEAK_TOPS, 3)}
        del g
    # per-shape at the MFMA-bound batches
    for m in (512, 2048):
        for name, n, k in lins:
            def run1(m=m, name=name, n=n):
                for l in range(L):
                    qr.qr_w8a8_linear(qr.QR_FP8_E4M3, xc[name][:m], xs[name][:m], wc[name][l * n:(l + 1) * n],
                                      ws[name][l * n:(l + 1) * n], y=y[name][:m], workspace=wsp)
            g = TimedGraph(run1, L)
            ms = g.time_ms(reps)
            no = L * ops_linear(m, n, k)
            out["m%d_%s" % (m, name)] = {"us": round(ms * 1e3 / L, 2), "TFLOP/s": round(no / ms / 1e9, 1),
                                         "mfma_frac": round(no / ms / 1e9 / MFMA_PEAK_TOPS, 3)}
            del g
    del wc, ws, xc, xs, y, wsp
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def measure_publish_fused(stack, reps):
    """The publish of the 1.5B stack (112 matrices, bf16 masters -> INT8) as one fused requantize + diff pass per
    weight (codes, scales, per-row change triples and their sums) against the step's separate quantize (a1) and
    changed-code count (a5); both out of place against the same previous publish, so they can be compared."""
    import torch

    qr = stack.qr
    rc = {name: torch.empty((LAYERS * n, 3), dtype=torch.int32, device=stack.dev) for name, n, _ in LINEARS}
    o3 = torch.empty((len(LINEARS), 3), dtype=torch.int64, device=stack.dev)

    def fused():
        for i, (name, n, k) in enumerate(LINEARS):
            qr.qr_requantize_weights(stack.w[name], qr.QR_INT8, stack.pc[name], stack.ps[name],
                                     codes=stack.wc[name], scales=stack.ws[name], row_counts=rc[name], out3=o3[i])

    def separate():
        stack.publish_quantize()
        stack.publish_count()

    gs, gf = TimedGraph(separate, len(LINEARS) + 2), TimedGraph(fused, 2 * len(LINEARS))
    ms_sep, ms_fused = gs.time_ms(reps), gf.time_ms(reps)
    gs.replay()
    torch.cuda.synchronize()
    sep_codes, sep_count = stack.codes.clone(), stack.count.clone()
    gf.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(stack.codes, sep_codes) and torch.equal(o3.sum(dim=0), sep_count))
    codes, rows = stack.codes_total, stack.rows_total
    nb = 2 * codes + codes + codes + 4 * rows + 4 * rows + 12 * rows  # masters, previous codes, new codes, scales
    del gs, gf
    return {"us_fused": round(ms_fused * 1e3, 1), "us_separate": round(ms_sep * 1e3, 1),
            "speedup": round(ms_sep / ms_fused, 3), "GB/s": round(nb / ms_fused / 1e6, 1),
            "hbm_frac": round(nb / ms_fused / 1e6 / HBM_PEAK_GBS, 3), "bytes": int(nb),
            "changed": [int(v) for v in sep_count.tolist()], "matches_separate": same}


def measure_decode_fused(stack, reps):
    """The m = 1 decode of the 1.5B stack (112 linears) on bfloat16 activations with the activation quantization
    inside the linear (qr_w8a8_linear_bf16) against the step's two launches per linear (a2 then a3); both are
    replayed as HIP graphs and their outputs compared bit for bit."""
    import torch

    qr = stack.qr

    def fused():
        for l in range(LAYERS):
            for name, n, k in LINEARS:
                qr.qr_w8a8_linear_bf16(qr.QR_INT8, stack.x[name][l, :1], stack.wc[name][l * n:(l + 1) * n],
                                       stack.ws[name][l * n:(l + 1) * n], y=stack.y[name][:1], workspace=stack.wsp)

    g2, gf = (TimedGraph(lambda: stack.decode_separate(1), 2 * LAYERS * len(LINEARS)),
              TimedGraph(fused, LAYERS * len(LINEARS)))
    ms2, msf = g2.time_ms(reps), gf.time_ms(reps)
    outs = []
    for g in (g2, gf):
        g.replay()
        torch.cuda.synchronize()
        outs.append([stack.y[name][:1].clone() for name, _, _ in LINEARS])
    same = all(torch.equal(a, b) for a, b in zip(*outs))
    del g2, gf
    return {"us_two_launches": round(ms2 * 1e3, 1), "us_fused": round(msf * 1e3, 1),
            "speedup": round(ms2 / msf, 3), "us_per_layer_fused": round(msf * 1e3 / LAYERS, 2),
            "y_matches_two_launches": same}


def bytes_w4a16(m, n, k, out_bytes=2):
    """HBM bytes a W4A16 linear must move: packed codes, group scales, bf16 activations, the output."""
    return n * k // 2 + 4 * n * (k // W4_GROUP) + 2 * m * k + out_bytes * m * n


def measure_w4a16_7b(dev, reps):
    """7B-shaped W4A16 linears (the same four shapes as the FP8 ones), INT4 codes and group scales of 5
    distinct layers (585 MB) rotated; the decode batches m = 1 and 16."""
    import torch

    import quantized_rollout_amd as qr

    L = 5
    lins = (("qkv", 4608, 3584), ("o", 3584, 3584), ("gate_up", 37888, 3584), ("down", 3584, 18944))
    batches = (1, 16)
    gen = torch.Generator(device=dev)
    gen.manual_seed(2)
    wc, ws, x, y = {}, {}, {}, {}
    for name, n, k in lins:
        w = normal_bf16(gen, (L * n, k), WEIGHT_STD, dev)
        wc[name], ws[name] = qr.qr_quantize_weights_w4(w)
        del w
        x[name] = activations_bf16(gen, 1, max(batches), k, dev)[0]
        y[name] = torch.empty((max(batches), n), dtype=torch.bfloat16, device=dev)
    out = {}
    for m in batches:
        def run(m=m):
            for l in range(L):
                for name, n, k in lins:
                    qr.qr_w4a16_linear(x[name][:m], wc[name][l * n:(l + 1) * n], ws[name][l * n:(l + 1) * n],
                                       y=y[name][:m])
        g = TimedGraph(run, L * len(lins))
        ms = g.time_ms(reps)
        nb = L * sum(bytes_w4a16(m, n, k) for _, n, k in lins)
        out["m%d" % m] = {"us_per_layer": round(ms * 1e3 / L, 2), "GB/s": round(nb / ms / 1e6, 1),
                          "hbm_frac": round(nb / ms / 1e6 / HBM_PEAK_GBS, 3)}
        del g
        for name, n, k in lins:
            def run1(m=m, name=name, n=n):
                for l in range(L):
                    qr.qr_w4a16_linear(x[name][:m], wc[name][l * n:(l + 1) * n], ws[name][l * n:(l + 1) * n],
                                       y=y[name][:m])
            g = TimedGraph(run1, L)
            ms = g.time_ms(reps)
            nb = L * bytes_w4a16(m, n, k)
            out["m%d_%s" % (m, name)] = {"us": round(ms * 1e3 / L, 2), "GB/s": round(nb / ms / 1e6, 1),
                                         "hbm_frac": round(nb / ms / 1e6 / HBM_PEAK_GBS, 3)}
            del g
    del wc, ws, x, y
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def measure_moe(dev, reps):
    """Qwen3-30B-A3B-shaped MoE expert linears in FP8: 128 experts, gate/up 2048->2x768, down 768->2048, top-8
    routing of 256 tokens from N(0, 1) logits; two copies of the expert codes (1.2 GB) rotated."""
    import numpy as np
    import torch

    import quantized_rollout_amd as qr
    from quantized_rollout_amd import synth

    C, E, H, I, T, TOPK = 2, 128, 2048, 768, 256, 8
    gen = torch.Generator(device=dev)
    gen.manual_seed(2)
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    off, rows = synth.route_top_k(logits, TOPK)
    R = int(off[-1])
    off_d = torch.from_numpy(off).to(dev)
    rows_d = torch.from_numpy(rows).to(dev)
    wgu_c, wgu_s, wd_c, wd_s = [], [], [], []
    for c in range(C):
        w = normal_bf16(gen, (E * 2 * I, H), WEIGHT_STD, dev)
        a, b = qr.qr_quantize_weights(w, qr.QR_FP8_E4M3)
        wgu_c.append(a.view(E, 2 * I, H))
        wgu_s.append(b.view(E, 2 * I))
        w = normal_bf16(gen, (E * H, I), WEIGHT_STD, dev)
        a, b = qr.qr_quantize_weights(w, qr.QR_FP8_E4M3)
        wd_c.append(a.view(E, H, I))
        wd_s.append(b.view(E, H))
        del w
    x = activations_bf16(gen, 1, T, H, dev)[0]
    h = activations_bf16(gen, 1, R, I, dev)[0]
    xc, xs = qr.qr_quantize_acts(x, qr.QR_FP8_E4M3)
    hc, hs = qr.qr_quantize_acts(h, qr.QR_FP8_E4M3)
    ygu = torch.empty((R, 2 * I), dtype=torch.bfloat16, device=dev)
    yd = torch.empty((R, H), dtype=torch.bfloat16, device=dev)

    def gate_up():
        for c in range(C):
            qr.qr_w8a8_grouped_linear(qr.QR_FP8_E4M3, off_d, rows_d, R, xc, xs, wgu_c[c], wgu_s[c], y=ygu)

    def down():
        for c in range(C):
            qr.qr_w8a8_grouped_linear(qr.QR_FP8_E4M3, off_d, None, R, hc, hs, wd_c[c], wd_s[c], y=yd)

    out = {"routed_rows": R, "experts_hit": int((np.diff(off) > 0).sum())}
    for name, fn, n, k, xrows in (("gate_up", gate_up, 2 * I, H, T), ("down", down, H, I, R)):
        g = TimedGraph(fn, C)
        ms = g.time_ms(reps) / C
        nb = E * n * k + E * n * 4 + xrows * k + 4 * xrows + R * n * 2
        no = 2 * R * n * k
        out[name] = {"us": round(ms * 1e3, 2), "GB/s": round(nb / ms / 1e6, 1),
                     "hbm_frac": round(nb / ms / 1e6 / HBM_PEAK_GBS, 3), "TFLOP/s": round(no / ms / 1e9, 2)}
        del g

    # the whole expert FFN, every step on the GPU: routing of the logits into the token lists, the tokens'
    # activation codes, grouped gate/up, SiLU product fused with its per-row codes, grouped down, weighted
    # combine; and the glue kernels alone
    logits_d = torch.from_numpy(logits).to(dev)
    route = qr.qr_moe_route(logits_d, TOPK)
    xq = (torch.empty((T, H), dtype=torch.uint8, device=dev), torch.empty(T, dtype=torch.float32, device=dev))
    hq = (torch.empty((R, I), dtype=torch.uint8, device=dev), torch.empty(R, dtype=torch.float32, device=dev))
    y_out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)

    def ffn():
        for c in range(C):
            qr.qr_moe_route(logits_d, TOPK, out=route)
            qr.qr_quantize_acts(x, qr.QR_FP8_E4M3, codes=xq[0], scales=xq[1])
            qr.qr_w8a8_grouped_linear(qr.QR_FP8_E4M3, route["expert_offsets"], route["row_ids"], R, xq[0], xq[1],
                                      wgu_c[c], wgu_s[c], y=ygu)
            qr.qr_silu_mul_quantize(ygu, qr.QR_FP8_E4M3, codes=hq[0], scales=hq[1])
            qr.qr_w8a8_grouped_linear(qr.QR_FP8_E4M3, route["expert_offsets"], None, R, hq[0], hq[1], wd_c[c],
                                      wd_s[c], y=yd)
            qr.qr_moe_combine(yd, route["topk_weight"], route["pair_rows"], out=y_out)

    g = TimedGraph(ffn, 6 * C)
    ms = g.time_ms(reps) / C
    torch.cuda.synchronize()
    replayed = y_out.clone()
    ffn()  # eager: the replays must have produced the same bits
    torch.cuda.synchronize()
    same = bool(torch.equal(replayed.view(torch.int16), y_out.view(torch.int16)))
    del g
    nb = T * E * 4 + T * H * 2 + E * (2 * I * H + 2 * I * 4 + H * I + H * 4) + T * H * 2
    ffn_out = {"us": round(ms * 1e3, 2), "GB/s": round(nb / ms / 1e6, 1),
               "hbm_frac": round(nb / ms / 1e6 / HBM_PEAK_GBS, 3), "bytes": nb,
               "steps": "route, activation codes, grouped gate/up, SiLU product + codes, grouped down, combine",
               "graph_replay_equals_eager": same}
    reps_glue = 20
    for name, fn in (("route", lambda: qr.qr_moe_route(logits_d, TOPK, out=route)),
                     ("silu_mul_quantize", lambda: qr.qr_silu_mul_quantize(ygu, qr.QR_FP8_E4M3, codes=hq[0],
                                                                           scales=hq[1])),
                     ("combine", lambda: qr.qr_moe_combine(yd, route["topk_weight"], route["pair_rows"],
                                                           out=y_out))):
        def many(fn=fn):
            for _ in range(reps_glue):
                fn()
        g = TimedGraph(many, reps_glue)
        ffn_out[name + "_us"] = round(g.time_ms(max(2, reps // 4)) / reps_glue * 1e3, 2)
        del g
    out["ffn"] = ffn_out
    del wgu_c, wgu_s, wd_c, wd_s
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same step
# ----------------------------------------------------------------------------------------------------------
def cpu_baseline(stack, budget_s):
    """The oracle (plain C, one thread) runs the step of the main workload layer by layer -- a1 and a5 on
    the layer's four weight matrices, a2 and a3 at M = 1, 16, 64 -- until `budget_s` seconds have passed.
    It also checks the GPU's published codes and scales of each sampled layer bit for bit."""
    import numpy as np
    import torch

    from oracle import core as O

    def bits(t):
        return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    t_total, nbytes, layers, parity = 0.0, 0, 0, True
    while t_total < budget_s and layers < LAYERS:
        l = layers
        host = {}
        for name, n, k in LINEARS:
            host[name] = (bits(stack.w[name][l * n:(l + 1) * n]), bits(stack.x[name][l]),
                          stack.pc[name][l * n:(l + 1) * n].cpu().numpy(), stack.ps[name][l * n:(l + 1) * n].cpu().numpy(),
                          stack.wc[name][l * n:(l + 1) * n].cpu().numpy(), stack.ws[name][l * n:(l + 1) * n].cpu().numpy())
        t0 = time.perf_counter()
        for name, n, k in LINEARS:
            w, x, pc, ps, _, _ = host[name]
            wc, ws = O.quantize_rows(w, O.INT8)
            O.count_code_changes(wc, pc, O.INT8, ws, ps)
            nbytes += bytes_quantize(n, k, 2) + bytes_count(n * k, n)
            for m in BATCHES:
                xc, xs = O.quantize_rows(x[:m], O.INT8, s_mode=O.S_MUL_RECIP)
                O.linear(O.INT8, xc, xs, wc, ws, O.BF16)
                nbytes += bytes_quantize(m, k, 2) + bytes_linear(m, n, k)
            host[name] = host[name] + (wc, ws)
        t_total += time.perf_counter() - t0
        for name, n, k in LINEARS:
            gc, gs, wc, ws = host[name][4], host[name][5], host[name][6], host[name][7]
            parity = parity and np.array_equal(gc, wc) and np.array_equal(gs.view(np.uint32), ws.view(np.uint32))
        layers += 1
    return {"value": round(nbytes / t_total / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "%d of %d layers of the step (a1+a5 on the 4 weight matrices, a2+a3 at M=1,16,64), "
                      "%.1f s of single-thread CPU time; host has %d cores available"
                      % (layers, LAYERS, t_total, len(os.sched_getaffinity(0))),
            "seconds": round(t_total, 2), "publish_codes_match_gpu": bool(parity)}


# ----------------------------------------------------------------------------------------------------------
# ----------------------------------------------------------------------------------------------------------
# measured HBM traffic of a row (rocprofv3 FETCH_SIZE / WRITE_SIZE counters, scaled by a plain copy)
# ----------------------------------------------------------------------------------------------------------
TRAFFIC_COPY_BYTES = 256 << 20  # the scale reference: a device copy of 256 MiB (reads and writes that many)


def row_pieces(stack):
    """{row: function that launches that row's kernels once}, as timed in `rows`."""
    pieces = {"a1_quantize_weights": stack.publish_quantize, "a5_count_changes": stack.publish_count}
    for m in BATCHES:
        pieces["a2_quantize_acts_m%d" % m] = lambda m=m: stack.decode_acts(m)
        pieces["a3_linear_m%d" % m] = lambda m=m: stack.decode_linears(m)
    return pieces


# the library sources each row's kernels are built from (plus the shared device and host headers and the ABI,
# which holds the planners' inputs): a measured traffic figure stays valid while these files are unchanged
ROW_SOURCES = {"a1": ["qr_quantize.hip"], "a2": ["qr_quantize.hip"], "a5": ["qr_grouped.hip"],
               "a3": ["qr_linear.hip", "qr_gemm.hip"]}
SHARED_SOURCES = ["qr_device.hpp", "qr_internal.hpp", "qr_abi.hip"]


def sources_digest(row):
    """sha256 over the library sources of `row`'s kernels: a traffic figure is only reported for the sources it
    was measured on."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_rollout_amd", "csrc")
    for name in sorted(ROW_SOURCES[row.split("_")[0]] + SHARED_SOURCES):
        h.update(name.encode())
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profile_row(stack, name, reps):
    """The launches the counter runs look at: a plain device copy, `reps` eager passes of one row, the copy
    again (the copies bracket the row and give the counters' scale)."""
    import torch

    fn = row_pieces(stack)[name]
    # an elementwise kernel (never a DMA-engine copy): reads and writes TRAFFIC_COPY_BYTES of fp32
    src = torch.ones(TRAFFIC_COPY_BYTES // 4, dtype=torch.float32, device=stack.dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()


def profile_linear(dev, spec, reps):
    """One W8A8 linear shape for counter runs: `spec` = "int8|fp8:M:N:K"; distinct weight-code copies (together
    past the caches) are used in turn for `reps` calls between two elementwise copies (the markers)."""
    import torch

    import quantized_rollout_amd as qr

    qname, m, n, k = spec.split(":")
    q = {"int8": qr.QR_INT8, "fp8": qr.QR_FP8_E4M3}[qname]
    m, n, k = int(m), int(n), int(k)
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    copies = max(2, min(reps, int(1.2e9 // (n * k)) + 1))
    # codes of N(0, 0.02) weights and N(0, 1) activations quantized by the library (every byte a valid code)
    w = [qr.qr_quantize_weights(normal_bf16(gen, (n, k), WEIGHT_STD, dev), q) for _ in range(copies)]
    xc, xs = qr.qr_quantize_acts(activations_bf16(gen, 1, m, k, dev)[0], q)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    wsp = qr.Workspace()
    src = torch.ones(TRAFFIC_COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    for i in range(reps):
        qr.qr_w8a8_linear(q, xc, xs, w[i % copies][0], w[i % copies][1], y=y, workspace=wsp)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log("profiled %d calls of %s" % (reps, spec))


def _counter_dispatches(directory, counter):
    """[(dispatch id, kernel name, value)] of one counter from a rocprofv3 csv output directory."""
    import csv
    import glob

    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % directory)
    per = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                key = int(r["Dispatch_Id"])
                name, v = per.get(key, (r["Kernel_Name"], 0.0))
                per[key] = (name, v + float(r["Counter_Value"]))
    return [(k, per[k][0], per[k][1]) for k in sorted(per)]


def traffic_summary(fetch_dir, write_dir, name, reps, command):
    """Markdown summary of the two counter runs of `profile_row`: per-dispatch FETCH_SIZE / WRITE_SIZE of the
    row's launches between the two copies, each scaled by what the counter reads for the copy."""
    launches = DecoderStack.row_work()[name][2]
    nbytes = DecoderStack.row_work()[name][0]
    out = {}
    for counter, directory in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        ds = _counter_dispatches(directory, counter)
        copies = [i for i, (_, kname, _) in enumerate(ds) if "qr::" not in kname and "neg" in kname]
        if len(copies) < 2:
            raise SystemExit("copy markers not found in %s" % directory)
        a, b = copies[-2], copies[-1]
        row = [d for d in ds[a + 1:b] if "qr::" in d[1]]
        # a launch of the row is one library call; a call may run more than one kernel (a split-K reduction
        # after the linear), so every library dispatch between the copies counts, per call
        if len(row) < reps * launches:
            raise SystemExit("%s: %d row dispatches between the copies, expected at least %d"
                             % (counter, len(row), reps * launches))
        copy_kib = (ds[a][2] + ds[b][2]) / 2
        scale = TRAFFIC_COPY_BYTES / (copy_kib * 1024.0)
        out[counter] = (sum(v for _, _, v in row) / (reps * launches), copy_kib, scale, len(row))
    per_launch = sum(v * 1024.0 * sc for v, _, sc, _ in out.values())
    dispatches = out["FETCH_SIZE"][3]
    lines = [
        "# HBM traffic of `%s` (rocprofv3 FETCH_SIZE / WRITE_SIZE), one MI355X" % name,
        "",
        "Commands (from the repository root):",
        "",
        "```",
        command,
        "```",
        "",
        "The row's %d launches (library calls) are run %d times between two elementwise passes over %d MiB of fp32 "
        "(a plain copy that reads and writes %d MiB): %d kernel dispatches. Each counter's readings (KiB) are "
        "summed per call and scaled by the copy's to bytes." % (
            launches, reps, TRAFFIC_COPY_BYTES >> 20, TRAFFIC_COPY_BYTES >> 20, dispatches),
        "",
        "| counter | mean per row launch (KiB) | copy reading (KiB) | scale to bytes per KiB |",
        "|---|---|---|---|",
    ]
    for counter, (v, ck, sc, _) in out.items():
        lines.append("| %s | %.1f | %.1f | %.4f x 1024 |" % (counter, v, ck, sc))
    lines += [
        "",
        "| | bytes per launch |",
        "|---|---|",
        "| algorithmic (what the method must move) | %d |" % (nbytes // launches),
        "| measured HBM traffic (fetch + write, scaled) | %d |" % int(per_launch),
        "",
        "traffic_row: %s" % name,
        "traffic_bytes_per_launch: %d" % int(per_launch),
        "traffic_sources_sha256: %s" % sources_digest(name),
        "",
    ]
    return "\n".join(lines)


def read_traffic(name):
    """Measured traffic per launch of `name` from profiles/, or None when absent or taken on other sources."""
    import glob

    for f in sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.md"))):
        fields = {}
        with open(f) as fh:
            for line in fh:
                if line.startswith("traffic_") and ":" in line:
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        if fields.get("traffic_row") == name and fields.get("traffic_sources_sha256") == sources_digest(name):
            return int(fields["traffic_bytes_per_launch"])
    return None


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--reps", type=int, default=50, help="replays per per-row timing")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="skip the FP8 7B and MoE side measurements")
    ap.add_argument("--profile-row", metavar="ROW", help="only run ROW between two device copies (for the "
                    "rocprofv3 counter runs) and exit")
    ap.add_argument("--profile-reps", type=int, default=3)
    ap.add_argument("--profile-linear", metavar="Q:M:N:K", help="only run one W8A8 linear shape (int8 or fp8) "
                    "--profile-reps times between two device copies (for the rocprofv3 counter runs) and exit")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the markdown summary of the two counter runs of --profile-row ROW and exit")
    ap.add_argument("--traffic-command", default="", help="the command lines recorded in that summary")
    args = ap.parse_args()

    if args.traffic_summary:
        print(traffic_summary(args.traffic_summary[0], args.traffic_summary[1], args.profile_row,
                              args.profile_reps, args.traffic_command))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the library runs on one GPU only (no collectives or sharding); --gpus %d is not "
              "supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import quantized_rollout_amd as qr

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    qr.lib()  # raises if libqr.so is not built: there is no fallback
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("device %s, libqr %s" % (torch.cuda.get_device_name(dev), qr.qr_version()))

    if args.profile_linear:
        profile_linear(dev, args.profile_linear, args.profile_reps)
        return 0
    stack = DecoderStack(dev)
    if args.profile_row:
        profile_row(stack, args.profile_row, args.profile_reps)
        return 0
    work = stack.row_work()
    step_bytes = sum(v[0] for v in work.values())
    step_ops = sum(v[1] for v in work.values())
    log("inputs resident: %.2f GB of bf16 masters, %.2f GB of codes" %
        (sum(w.numel() * 2 for w in stack.w.values()) / 1e9, stack.codes_total / 1e9))

    # eager reference of one step, then the graph of the whole step
    stack.step()
    ref = stack.snapshot()
    step_graph = TimedGraph(stack.step, None)
    log("step graph captured")

    for _ in range(args.warmup):
        step_graph.replay()
    torch.cuda.synchronize()
    t_a, t_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    t_a.record()
    for _ in range(args.steps):
        step_graph.replay()
    t_b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_total = t_a.elapsed_time(t_b)
    ms_step = ms_total / args.steps
    log("timed %d steps: %.3f ms/step (events), %.3f ms/step (host clock)" % (args.steps, ms_step,
                                                                              wall * 1e3 / args.steps))

    # every replay reproduces the eager step bit for bit (INT8 path: exact integers, fixed epilogue)
    got = stack.snapshot()
    replay_ok = all(torch.equal(a, b) for a, b in zip(ref, got))
    if not replay_ok:
        log("ERROR: graph replay differs from the eager step")

    # per-row launch timing (HIP events on the stream the kernels run on)
    rows = {}
    for name, fn in row_pieces(stack).items():
        nb, no, launches = work[name]
        g = TimedGraph(fn, launches)
        ms = g.time_ms(args.reps)
        rows[name] = {"launches": launches, "us_per_launch": round(ms * 1e3 / launches, 3),
                      "us_total": round(ms * 1e3, 2), "GB/s": round(nb / ms / 1e6, 1),
                      "hbm_frac": round(nb / ms / 1e6 / HBM_PEAK_GBS, 4)}
        if no:
            rows[name]["TOPS"] = round(no / ms / 1e9, 2)
        del g
    dominant = max(rows, key=lambda r: rows[r]["us_total"])
    d = rows[dominant]
    nb = work[dominant][0]
    achieved = nb / (d["us_total"] * 1e3)  # GB/s
    traffic = read_traffic(dominant)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": dominant,
                "bytes_per_launch": int(nb // d["launches"]), "us_per_launch": d["us_per_launch"]}

    extra = {}
    if not args.quick:
        del step_graph
        torch.cuda.synchronize()
        log("FP8 7B-shaped linears")
        extra["fp8_7b_linears"] = measure_fp8_7b(dev, max(5, args.reps // 5))
        log("MoE grouped linears")
        extra["moe_fp8_grouped"] = measure_moe(dev, max(5, args.reps // 5))
        log("W4A16 7B-shaped linears")
        extra["w4a16_7b_linears"] = measure_w4a16_7b(dev, max(5, args.reps // 5))
        log("fused requantize + diff publish")
        extra["publish_fused_requant_diff"] = measure_publish_fused(stack, max(5, args.reps // 5))
        log("decode at m = 1 with the activation quantization fused")
        extra["decode_m1_fused_act_quant"] = measure_decode_fused(stack, max(5, args.reps // 5))

    cpu = None
    if not args.no_cpu_baseline:
        log("CPU oracle baseline (%.0f s budget)" % args.cpu_budget)
        cpu = cpu_baseline(stack, args.cpu_budget)

    value = step_bytes * args.steps / (ms_total / 1e3) / 1e9
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": "qwen2.5-1.5b-shaped INT8 W8A8 decoder linears x %d layers: publish (a1+a5) + "
                               "decode at M=1,16,64 (a2+a3; at M=1 in one launch)" % LAYERS,
                   "layers": LAYERS, "linears": {n: [nn, k] for n, nn, k in LINEARS}, "batches": list(BATCHES),
                   "weights": "bf16 N(0,0.02)", "acts": "bf16 N(0,1), 4 outlier channels x20"},
        "tops": round(step_ops * args.steps / (ms_total / 1e3) / 1e12, 3),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "step_bytes": int(step_bytes), "replay_matches_eager": bool(replay_ok),
        "roofline": roofline, "cpu_baseline": cpu, "rows": rows, "extra": extra,
    }
    print(json.dumps(line), flush=True)
    return 0 if replay_ok else 1


if __name__ == "__main__":
    sys.exit(main())
