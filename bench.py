#!/usr/bin/env python3
"""Throughput of the quantized-actor W8A8 linear on one MI355X, on the 7B-shaped FP8 workload.

Workload of one step: the four linears of a 7B-shaped decoder layer in FP8 E4M3 W8A8 -- qkv 3584->4608,
o 3584->3584, gate/up 3584->2x18944, down 18944->3584 -- at every batch M in (1, 16, 128, 512, 2048): for
each M, each of LAYERS distinct layers and each linear,
  a2  the per-token quantization of the bf16 activations ("QuRL: Efficient Reinforcement Learning with
      Quantized Rollout", section 5: token-wise activation scales), and
  a3  the W8A8 linear with its dequantization epilogue, bf16 out (QuRL section 5; "QaRL: Rollout-Aligned
      Quantization-Aware RL ...", sections 2.2 and 3.1),
through qr_w8a8_linear_bf16 (at M = 1 the activation quantization runs inside the linear's kernel where that
pays; otherwise the two launches run back to back). The layers' FP8 codes (LAYERS x 233 MB) are distinct and
far larger than the 256 MB last-level cache, so every weight read comes from HBM. The codes are published once
by a1 before the timed region (the publish is measured on its own in `extra`). The step is captured once in a
HIP graph and replayed; inputs are resident in HBM before the timed region starts.

value = operations of one step (2 M N K summed over every linear, layer and M) x steps / elapsed seconds, in
TOPS (FP8 operations). The JSON line also carries, per M, the time of one layer and its fraction of the
binding roofline (HBM 8 TB/s for M <= 128, FP8 MFMA 5.0 PFLOP/s for M >= 512); per linear and M, the linear's
own kernel time on codes; the roofline of the dominant kernel (the FP8 gate/up GEMM at M = 2048, its measured
HBM traffic when profiles/ holds a FETCH_SIZE / WRITE_SIZE summary taken on the current kernel sources), the
decode layer's HBM fraction at M <= 16, and the CPU oracle timed on a bounded sample of the same step (one
thread and all host cores). Unless --quick, `extra` holds the other workloads: the publish between RL steps on
the 7B linears (fp32 masters, INT8 and FP8, with and without s; changed-code counts), the grouped MoE FFN, the
1.5B-shaped INT8 linears, W4A16, and the RMSNorm producer that quantizes a linear's input in the normalization's
own pass.

Counter runs for the traffic figure (each counter in a run of its own):
  rocprofv3 --pmc FETCH_SIZE -d DIR_F -o t --output-format csv -- python3 bench.py --profile-kernel NAME
  rocprofv3 --pmc WRITE_SIZE -d DIR_W -o t --output-format csv -- python3 bench.py --profile-kernel NAME
  python3 bench.py --profile-kernel NAME --traffic-summary DIR_F DIR_W > profiles/traffic_NAME.md
"""
import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W8A8 linear TOPS (MFMA % peak) + HBM GB/s at rollout decode shapes, 1 GPU"
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E, published
MFMA_PEAK_TOPS = 5000.0       # MI355X dense FP8 PFLOP/s and INT8 POP/s, published (x1000)

LINEARS_7B = (("qkv", 4608, 3584), ("o", 3584, 3584), ("gate_up", 37888, 3584), ("down", 3584, 18944))
BATCHES_7B = (1, 16, 128, 512, 2048)
MFMA_BOUND_M = 512            # M >= 512: bound by the FP8 MFMA peak; below, by HBM
LAYERS = 5                    # distinct layers of codes in the step (5 x 233 MB)
LINEARS_1P5B = (("qkv", 2048, 1536), ("o", 1536, 1536), ("gate_up", 17920, 1536), ("down", 1536, 8960))
BATCHES_1P5B = (1, 16, 64)
WEIGHT_STD = 0.02
W4_GROUP = 128                # input channels per INT4 scale group (W4A16)
DOMINANT = ("gate_up", 2048)  # the kernel that dominates the step: the FP8 gate/up GEMM at M = 2048

# kernels the counter runs profile: name -> (format, m, n, k) of one W8A8 linear on codes
PROFILE_KERNELS = {
    "a3_fp8_gate_up_m2048": ("fp8", 2048, 37888, 3584),
    "a3_fp8_gate_up_m512": ("fp8", 512, 37888, 3584),
    "a3_fp8_gate_up_m128": ("fp8", 128, 37888, 3584),
    "a3_fp8_qkv_m128": ("fp8", 128, 4608, 3584),
    "a3_fp8_gate_up_m1": ("fp8", 1, 37888, 3584),
    "a3_fp8_gate_up_m16": ("fp8", 16, 37888, 3584),
    "a3_fp8_down_m1": ("fp8", 1, 3584, 18944),
    "a3_fp8_down_m16": ("fp8", 16, 3584, 18944),
    "a3_int8_gate_up_1p5b_m64": ("int8", 64, 17920, 1536),
}


def log(msg):
    sys.stderr.write("[bench] %s\n" % msg)
    sys.stderr.flush()


# ----------------------------------------------------------------------------------------------------------
# algorithmic bytes and operations per call (what the method must move: codes, scales, bf16 in and out)
# ----------------------------------------------------------------------------------------------------------
def bytes_quantize(rows, k, in_bytes):
    return rows * k * in_bytes + rows * k + 4 * rows


def bytes_linear(m, n, k, out_bytes=2):
    return n * k + 4 * n + m * k + 4 * m + m * n * out_bytes


def bytes_linear_bf16(m, n, k, out_bytes=2):
    """the linear on bf16 activations (a2 inside or before a3): bf16 activations in instead of codes"""
    return n * k + 4 * n + 2 * m * k + m * n * out_bytes


def bytes_count(codes, scales):
    return 2 * codes + 2 * 4 * scales


def ops_linear(m, n, k):
    return 2 * m * n * k


def bound_of(m):
    return "mfma" if m >= MFMA_BOUND_M else "hbm"


def frac_of(m, nbytes, ops, ms):
    """fraction of the binding roofline of a call sequence taking ms milliseconds"""
    if bound_of(m) == "mfma":
        return ops / ms / 1e9 / MFMA_PEAK_TOPS
    return nbytes / ms / 1e6 / HBM_PEAK_GBS


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
# the main workload: the 7B-shaped FP8 linears at every batch of the configuration
# ----------------------------------------------------------------------------------------------------------
class Dense7B:
    """LAYERS distinct 7B-shaped layers: bf16 N(0, 0.02) masters published once (a1) to FP8 codes and scales,
    bf16 N(0, 1) activations with 4 outlier channels x20 at the largest batch (smaller batches use row
    prefixes), bf16 outputs."""

    def __init__(self, dev, seed=0):
        import torch

        import quantized_rollout_amd as qr

        self.qr, self.dev = qr, dev
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed)
        self.wc, self.ws, self.x, self.xc, self.xs, self.y = {}, {}, {}, {}, {}, {}
        m_max = max(BATCHES_7B)
        for name, n, k in LINEARS_7B:
            codes = torch.empty((LAYERS * n, k), dtype=torch.uint8, device=dev)
            scales = torch.empty((LAYERS * n,), dtype=torch.float32, device=dev)
            for l in range(LAYERS):
                w = normal_bf16(gen, (n, k), WEIGHT_STD, dev)
                qr.qr_quantize_weights(w, qr.QR_FP8_E4M3, codes=codes[l * n:(l + 1) * n],
                                       scales=scales[l * n:(l + 1) * n])
                del w
            self.wc[name], self.ws[name] = codes, scales
            self.x[name] = activations_bf16(gen, LAYERS, m_max, k, dev)
            # the activations' codes, for the linear's own kernel timed on codes
            self.xc[name] = torch.empty((LAYERS, m_max, k), dtype=torch.uint8, device=dev)
            self.xs[name] = torch.empty((LAYERS, m_max), dtype=torch.float32, device=dev)
            for l in range(LAYERS):
                qr.qr_quantize_acts(self.x[name][l], qr.QR_FP8_E4M3, codes=self.xc[name][l], scales=self.xs[name][l])
            self.y[name] = torch.empty((m_max, n), dtype=torch.bfloat16, device=dev)
        self.wsp = qr.Workspace()
        need = max(max(qr.qr_workspace_bytes(qr.QR_FP8_E4M3, m, n, k),
                       qr.qr_w8a8_linear_bf16_workspace_bytes(qr.QR_FP8_E4M3, m, n, k))
                   for m in BATCHES_7B for _, n, k in LINEARS_7B)
        self.wsp.get(need)
        torch.cuda.synchronize()

    def w(self, name, l):
        n = dict((a, b) for a, b, _ in LINEARS_7B)[name]
        return self.wc[name][l * n:(l + 1) * n], self.ws[name][l * n:(l + 1) * n]

    # pieces of the step -----------------------------------------------------------------------------------
    def linear_bf16(self, name, m, l):
        """a2 + a3 of one linear on bf16 activations (one launch where the quantization runs inside)"""
        qr = self.qr
        wc, ws = self.w(name, l)
        qr.qr_w8a8_linear_bf16(qr.QR_FP8_E4M3, self.x[name][l, :m], wc, ws, y=self.y[name][:m], workspace=self.wsp)

    def linear_codes(self, name, m, l):
        """a3 alone, on the activation codes"""
        qr = self.qr
        wc, ws = self.w(name, l)
        qr.qr_w8a8_linear(qr.QR_FP8_E4M3, self.xc[name][l, :m], self.xs[name][l, :m], wc, ws, y=self.y[name][:m],
                          workspace=self.wsp)

    def acts(self, name, m, l):
        """a2 alone"""
        qr = self.qr
        qr.qr_quantize_acts(self.x[name][l, :m], qr.QR_FP8_E4M3, codes=self.xc[name][l, :m],
                            scales=self.xs[name][l, :m])

    def batch(self, m):
        for l in range(LAYERS):
            for name, _, _ in LINEARS_7B:
                self.linear_bf16(name, m, l)

    def step(self):
        for m in BATCHES_7B:
            self.batch(m)

    @staticmethod
    def step_work():
        """(bytes, ops) of one step"""
        nb = LAYERS * sum(bytes_linear_bf16(m, n, k) for m in BATCHES_7B for _, n, k in LINEARS_7B)
        no = LAYERS * sum(ops_linear(m, n, k) for m in BATCHES_7B for _, n, k in LINEARS_7B)
        return nb, no

    def snapshot(self):
        import torch

        out = [self.y[name].clone() for name, _, _ in LINEARS_7B]
        torch.cuda.synchronize()
        return out


def measure_rows(d, reps):
    """Per batch: one layer's four linears on bf16 activations (a2 + a3, as in the step); per batch and linear:
    the linear's own kernels on codes (a3, `us`), the activation quantization alone (`a2_us`) and the two through
    the bf16 entry point as in the step (`a2_a3_us`). HIP events around graph replays on the stream the kernels
    run on; LAYERS distinct layers per replay."""
    per_m, per_linear = {}, {}
    for m in BATCHES_7B:
        g = TimedGraph(lambda m=m: d.batch(m), LAYERS * len(LINEARS_7B))
        ms = g.time_ms(reps) / LAYERS
        del g
        nb = sum(bytes_linear_bf16(m, n, k) for _, n, k in LINEARS_7B)
        no = sum(ops_linear(m, n, k) for _, n, k in LINEARS_7B)
        per_m["m%d" % m] = {"us_per_layer": round(ms * 1e3, 2), "TOPS": round(no / ms / 1e9, 1),
                            "GB/s": round(nb / ms / 1e6, 1), "bound": bound_of(m),
                            "frac": round(frac_of(m, nb, no, ms), 4)}
        for name, n, k in LINEARS_7B:
            g = TimedGraph(lambda m=m, name=name: [d.linear_codes(name, m, l) for l in range(LAYERS)], LAYERS)
            ms = g.time_ms(reps) / LAYERS
            del g
            g = TimedGraph(lambda m=m, name=name: [d.acts(name, m, l) for l in range(LAYERS)], LAYERS)
            ms_a = g.time_ms(reps) / LAYERS
            del g
            g = TimedGraph(lambda m=m, name=name: [d.linear_bf16(name, m, l) for l in range(LAYERS)], LAYERS)
            ms_b = g.time_ms(reps) / LAYERS
            del g
            nb, no = bytes_linear(m, n, k), ops_linear(m, n, k)
            per_linear["m%d_%s" % (m, name)] = {
                "us": round(ms * 1e3, 2), "TOPS": round(no / ms / 1e9, 1), "GB/s": round(nb / ms / 1e6, 1),
                "bound": bound_of(m), "frac": round(frac_of(m, nb, no, ms), 4),
                "a2_us": round(ms_a * 1e3, 2), "a2_a3_us": round(ms_b * 1e3, 2)}
    return per_m, per_linear


def measure_dominant(d, reps):
    """The dominant kernel: the FP8 gate/up GEMM at M = 2048 on codes, LAYERS distinct weights per replay; its
    average launch duration from HIP events on the stream it runs on."""
    name, m = DOMINANT
    n, k = dict((a, (b, c)) for a, b, c in LINEARS_7B)[name]
    g = TimedGraph(lambda: [d.linear_codes(name, m, l) for l in range(LAYERS)], LAYERS)
    ms = g.time_ms(reps) / LAYERS
    del g
    return ms, ops_linear(m, n, k), bytes_linear(m, n, k)


def cpu_baseline(budget_s):
    """The oracle (plain C, test infrastructure) on a bounded sample of the step: for every batch M and linear of
    the workload, the activation quantization (a2) of M bf16 rows and the W8A8 linear (a3) of those rows with a
    subset of the output channels, sized so that each (M, linear) pair is about the same number of
    multiply-adds. Run once on one thread and once on every host core (threads over output channels); the value
    is operations per second (2 multiply-adds) in TOPS. Inputs: seeded numpy draws of the workload's
    distributions, quantized by the oracle itself."""
    import numpy as np

    from oracle import core as O

    rng = np.random.default_rng(0)
    pairs = [(m, name, n, k) for m in BATCHES_7B for name, n, k in LINEARS_7B]
    # multiply-adds per pair: half the budget for each run, from the oracle's ~0.18 G MAC/s per thread
    macs_per_pair = budget_s / 2 * 0.18e9 / len(pairs)

    acts = {}

    def inputs(m, n_cols, k):
        if (m, k) not in acts:  # the same activations for both runs
            x = rng.standard_normal((m, k)).astype(np.float32)
            x[:, rng.choice(k, 4, replace=False)] *= np.float32(20)
            u = x.view(np.uint32).astype(np.uint64)
            acts[(m, k)] = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
        w = (rng.standard_normal((n_cols, k)) * WEIGHT_STD).astype(np.float32)
        wc, ws = O.quantize_rows_threaded(w, O.FP8)
        return acts[(m, k)], wc, ws

    def run(threads, scale):
        t_total, ops, cols_used = 0.0, 0, 0
        for m, name, n, k in pairs:
            n_cols = int(max(1, min(n, scale * macs_per_pair / (m * k))))
            xb, wc, ws = inputs(m, n_cols, k)
            t0 = time.perf_counter()
            if threads == 1:
                xc, xs = O.quantize_rows(xb, O.FP8, s_mode=O.S_MUL_RECIP)
                O.linear(O.FP8, xc, xs, wc, ws, O.BF16)
            else:
                xc, xs = O.quantize_rows_threaded(xb, O.FP8, s_mode=O.S_MUL_RECIP, threads=threads)
                O.linear_threaded(O.FP8, xc, xs, wc, ws, O.BF16, threads=threads)
            t_total += time.perf_counter() - t0
            ops += ops_linear(m, n_cols, k)
            cols_used += n_cols
        return ops / t_total / 1e12, t_total, ops

    cores = O.host_threads()
    v1, t1, o1 = run(1, 1.0)
    vn, tn, on = run(cores, float(cores))
    cpu = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(vn, 6), "unit": "TOPS", "cores": cores, "kind": "oracle",
            "sample": "every (M, linear) pair of the step, M in %s: a2 on the M bf16 rows and a3 on a subset of "
                      "the output channels (about equal multiply-adds per pair), %.2e FP8 ops in %.1f s on %d "
                      "threads; CPU %s" % (list(BATCHES_7B), on, tn, cores, cpu),
            "seconds": round(tn, 2),
            "single_thread": {"value": round(v1, 6), "unit": "TOPS", "cores": 1, "seconds": round(t1, 2),
                              "ops": o1}}


# ----------------------------------------------------------------------------------------------------------
# other configurations of the path (side measurements, not part of `value`)
# ----------------------------------------------------------------------------------------------------------
def measure_publish_7b(dev, reps):
    """The publish between RL steps on the four 7B-shaped linears (233 M parameters): fp32 masters W ~ N(0, 0.02)
    and W2 = W + dW, dW ~ N(0, 1e-5), per-input-channel s ~ U(0.5, 2). For INT8 and FP8, with and without s:
    a1 quantizes W (the previous publish, untimed) and W2 (timed), a5 counts the codes, values and scales that
    changed (timed), and the fused requantize + diff publishes W2 against W's codes in one pass (timed); the
    fused codes and counts must equal the separate ones. Counts are reported with their fraction of P."""
    import torch

    import quantized_rollout_amd as qr

    gen = torch.Generator(device=dev)
    gen.manual_seed(4)
    P = sum(n * k for _, n, k in LINEARS_7B)
    rows = sum(n for _, n, _ in LINEARS_7B)
    w, w2, s = {}, {}, {}
    for name, n, k in LINEARS_7B:
        w[name] = torch.randn((n, k), generator=gen, device=dev) * WEIGHT_STD
        w2[name] = w[name] + torch.randn((n, k), generator=gen, device=dev) * 1e-5
        s[name] = torch.rand((k,), generator=gen, device=dev) * 1.5 + 0.5
    codes = {name: [torch.empty((n, k), dtype=torch.uint8, device=dev) for _ in range(3)]
             for name, n, k in LINEARS_7B}
    scales = {name: [torch.empty((n,), dtype=torch.float32, device=dev) for _ in range(3)]
              for name, n, k in LINEARS_7B}
    rc = {name: torch.empty((n, 3), dtype=torch.int32, device=dev) for name, n, _ in LINEARS_7B}
    cnt = torch.zeros((len(LINEARS_7B), 3), dtype=torch.int64, device=dev)
    o3 = torch.zeros((len(LINEARS_7B), 3), dtype=torch.int64, device=dev)
    out = {"params": P}
    for qname, q in (("int8", qr.QR_INT8), ("fp8", qr.QR_FP8_E4M3)):
        for with_s in (False, True):
            key = "%s%s" % (qname, "_s" if with_s else "")
            sv = lambda name: s[name] if with_s else None  # noqa: E731

            def prev():
                for name, _, _ in LINEARS_7B:
                    qr.qr_quantize_weights(w[name], q, s=sv(name), codes=codes[name][0], scales=scales[name][0])

            def quant():
                for name, _, _ in LINEARS_7B:
                    qr.qr_quantize_weights(w2[name], q, s=sv(name), codes=codes[name][1], scales=scales[name][1])

            def count():
                for i, (name, _, _) in enumerate(LINEARS_7B):
                    qr.qr_count_code_changes(codes[name][0], codes[name][1], q, scales[name][0], scales[name][1],
                                             out3=cnt[i])

            def fused():
                for i, (name, _, _) in enumerate(LINEARS_7B):
                    qr.qr_requantize_weights(w2[name], q, codes[name][0], scales[name][0], s=sv(name),
                                             codes=codes[name][2], scales=scales[name][2], row_counts=rc[name],
                                             out3=o3[i])
            prev()
            gq, gc, gf = (TimedGraph(quant, len(LINEARS_7B)), TimedGraph(count, len(LINEARS_7B)),
                          TimedGraph(fused, 2 * len(LINEARS_7B)))
            ms_q, ms_c, ms_f = gq.time_ms(reps), gc.time_ms(reps), gf.time_ms(reps)
            del gq, gc, gf
            torch.cuda.synchronize()
            same = all(torch.equal(codes[name][1], codes[name][2]) and torch.equal(scales[name][1], scales[name][2])
                       for name, _, _ in LINEARS_7B) and torch.equal(cnt, o3)
            tot = cnt.sum(dim=0).tolist()
            nb_q = sum(bytes_quantize(n, k, 4) for _, n, k in LINEARS_7B) + (4 * sum(k for _, _, k in LINEARS_7B)
                                                                             if with_s else 0)
            nb_c = bytes_count(P, rows)
            nb_f = 4 * P + 2 * P + 8 * rows + 12 * rows
            out[key] = {
                "changed_bytes": int(tot[0]), "changed_values": int(tot[1]), "changed_scales": int(tot[2]),
                "changed_frac": round(tot[0] / P, 6), "changed_value_frac": round(tot[1] / P, 6),
                "changed_scale_frac": round(tot[2] / rows, 6),
                "per_linear_changed_bytes": {name: int(cnt[i, 0]) for i, (name, _, _) in enumerate(LINEARS_7B)},
                "a1_us": round(ms_q * 1e3, 1), "a1_GB/s": round(nb_q / ms_q / 1e6, 1),
                "a1_hbm_frac": round(nb_q / ms_q / 1e6 / HBM_PEAK_GBS, 4),
                "a5_us": round(ms_c * 1e3, 1), "a5_GB/s": round(nb_c / ms_c / 1e6, 1),
                "a5_hbm_frac": round(nb_c / ms_c / 1e6 / HBM_PEAK_GBS, 4),
                "fused_us": round(ms_f * 1e3, 1), "fused_GB/s": round(nb_f / ms_f / 1e6, 1),
                "fused_hbm_frac": round(nb_f / ms_f / 1e6 / HBM_PEAK_GBS, 4),
                "fused_equals_separate": bool(same)}
    del w, w2, s, codes, scales, rc
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def measure_int8_1p5b(dev, reps):
    """The Qwen2.5-1.5B-shaped INT8 W8A8 linears (qkv 1536->2048, o 1536->1536, gate/up 1536->2x8960, down
    8960->1536) at M = 1, 16, 64 on bf16 activations (a2 + a3 through qr_w8a8_linear_bf16), codes of 28 distinct
    layers (1.31 GB) rotated."""
    import torch

    import quantized_rollout_amd as qr

    L = 28
    gen = torch.Generator(device=dev)
    gen.manual_seed(3)
    wc, ws, x, y = {}, {}, {}, {}
    for name, n, k in LINEARS_1P5B:
        wc[name] = torch.empty((L * n, k), dtype=torch.uint8, device=dev)
        ws[name] = torch.empty((L * n,), dtype=torch.float32, device=dev)
        for l in range(L):
            qr.qr_quantize_weights(normal_bf16(gen, (n, k), WEIGHT_STD, dev), qr.QR_INT8,
                                   codes=wc[name][l * n:(l + 1) * n], scales=ws[name][l * n:(l + 1) * n])
        x[name] = activations_bf16(gen, L, max(BATCHES_1P5B), k, dev)
        y[name] = torch.empty((max(BATCHES_1P5B), n), dtype=torch.bfloat16, device=dev)
    wsp = qr.Workspace()
    wsp.get(max(qr.qr_w8a8_linear_bf16_workspace_bytes(qr.QR_INT8, m, n, k) for m in BATCHES_1P5B
                for _, n, k in LINEARS_1P5B))
    out = {}
    for m in BATCHES_1P5B:
        def run(m=m):
            for l in range(L):
                for name, n, k in LINEARS_1P5B:
                    qr.qr_w8a8_linear_bf16(qr.QR_INT8, x[name][l, :m], wc[name][l * n:(l + 1) * n],
                                           ws[name][l * n:(l + 1) * n], y=y[name][:m], workspace=wsp)
        g = TimedGraph(run, L * len(LINEARS_1P5B))
        ms = g.time_ms(reps) / L
        del g
        nb = sum(bytes_linear_bf16(m, n, k) for _, n, k in LINEARS_1P5B)
        out["m%d" % m] = {"us_per_layer": round(ms * 1e3, 2), "GB/s": round(nb / ms / 1e6, 1),
                          "hbm_frac": round(nb / ms / 1e6 / HBM_PEAK_GBS, 4)}
    del wc, ws, x, y, wsp
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


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
# measured HBM traffic of a kernel (rocprofv3 FETCH_SIZE / WRITE_SIZE counters, scaled by a plain copy)
# ----------------------------------------------------------------------------------------------------------
TRAFFIC_COPY_BYTES = 256 << 20  # the scale reference: a device copy of 256 MiB (reads and writes that many)

# the library sources each kernel is built from (plus the shared device and host headers and the ABI, which
# holds the planners' inputs): a measured traffic figure stays valid while these files are unchanged
ROW_SOURCES = {"a1": ["qr_quantize.hip"], "a2": ["qr_quantize.hip"], "a5": ["qr_grouped.hip"],
               "a3": ["qr_linear.hip", "qr_gemm.hip"]}
SHARED_SOURCES = ["qr_device.hpp", "qr_internal.hpp", "qr_abi.hip"]


def measure_rmsnorm_producer(dev, reps):
    """The RMSNorm producer of a linear's FP8 input on the 7B hidden size (3584) at every batch of the step, eps
    1e-6, with the invariant scale: the fused call against the two launches it replaces (the library RMSNorm of
    PyTorch on bf16, then the activation quantizer), and the quantizer alone. A 7B decoder layer has two such
    producers (ahead of qkv and of gate/up)."""
    import torch

    import quantized_rollout_amd as qr
    from quantized_rollout_amd import synth

    K, INNER = 3584, 20
    out = {}
    for m in BATCHES_7B:
        inp = synth.make_norm_inputs(m, K, seed=5)
        x = torch.from_numpy(inp.x.view("int16")).view(torch.bfloat16).to(dev)
        g, s = torch.from_numpy(inp.gamma).to(dev), torch.from_numpy(inp.s).to(dev)
        gb = g.to(torch.bfloat16)
        c = torch.empty((m, K), dtype=torch.uint8, device=dev)
        sc = torch.empty((m,), dtype=torch.float32, device=dev)

        def fused():
            for _ in range(INNER):
                qr.qr_rmsnorm_quantize(x, g, 1e-6, qr.QR_FP8_E4M3, s=s, codes=c, scales=sc)

        def pair():
            for _ in range(INNER):
                hn = torch.nn.functional.rms_norm(x, (K,), gb, 1e-6)
                qr.qr_quantize_acts(hn, qr.QR_FP8_E4M3, s=s, codes=c, scales=sc)

        def quant():
            for _ in range(INNER):
                qr.qr_quantize_acts(x, qr.QR_FP8_E4M3, s=s, codes=c, scales=sc)

        t = {name: TimedGraph(fn, INNER).time_ms(reps) * 1e3 / INNER
             for name, fn in (("fused", fused), ("norm_then_quantize", pair), ("quantize_alone", quant))}
        out["m%d" % m] = {"us_fused": round(t["fused"], 2), "us_norm_then_quantize": round(t["norm_then_quantize"], 2),
                          "us_quantize_alone": round(t["quantize_alone"], 2),
                          "saved_us_per_layer": round(2 * (t["norm_then_quantize"] - t["fused"]), 2),
                          "GB/s": round(m * K * 3 / t["fused"] / 1e3, 1)}
        log("rmsnorm producer m=%d: fused %.2f us, norm + quantize %.2f us, quantize alone %.2f us"
            % (m, t["fused"], t["norm_then_quantize"], t["quantize_alone"]))
    return out


def sources_digest(name):
    """sha256 over the library sources of `name`'s kernels: a traffic figure is only reported for the sources it
    was measured on."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_rollout_amd", "csrc")
    for fname in sorted(ROW_SOURCES[name.split("_")[0]] + SHARED_SOURCES):
        h.update(fname.encode())
        with open(os.path.join(csrc, fname), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def kernel_work(name):
    """(algorithmic bytes, ops) of one call of a profiled kernel"""
    _, m, n, k = PROFILE_KERNELS[name]
    return bytes_linear(m, n, k), ops_linear(m, n, k)


def profile_kernel(dev, name, reps):
    """One W8A8 linear shape for counter runs: distinct weight-code copies (together past the caches) are used in
    turn for `reps` calls between two elementwise copies (the markers that give the counters' scale)."""
    import torch

    import quantized_rollout_amd as qr

    qname, m, n, k = PROFILE_KERNELS[name]
    q = {"int8": qr.QR_INT8, "fp8": qr.QR_FP8_E4M3}[qname]
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
    log("profiled %d calls of %s (%s m=%d n=%d k=%d)" % (reps, name, qname, m, n, k))


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
    """Markdown summary of the two counter runs of `profile_kernel`: per-call FETCH_SIZE / WRITE_SIZE of the
    kernel's launches between the two copies, each scaled by what the counter reads for the copy."""
    nbytes, _ = kernel_work(name)
    out = {}
    for counter, directory in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        ds = _counter_dispatches(directory, counter)
        copies = [i for i, (_, kname, _) in enumerate(ds) if "qr::" not in kname and "neg" in kname]
        if len(copies) < 2:
            raise SystemExit("copy markers not found in %s" % directory)
        a, b = copies[-2], copies[-1]
        row = [d for d in ds[a + 1:b] if "qr::" in d[1]]
        # a call may run more than one kernel (a split-K reduction after the linear): every library dispatch
        # between the copies counts, per call
        if len(row) < reps:
            raise SystemExit("%s: %d dispatches between the copies, expected at least %d" % (counter, len(row), reps))
        copy_kib = (ds[a][2] + ds[b][2]) / 2
        scale = TRAFFIC_COPY_BYTES / (copy_kib * 1024.0)
        out[counter] = (sum(v for _, _, v in row) / reps, copy_kib, scale, len(row))
    per_call = sum(v * 1024.0 * sc for v, _, sc, _ in out.values())
    lines = [
        "# HBM traffic of `%s` (rocprofv3 FETCH_SIZE / WRITE_SIZE), one MI355X" % name,
        "",
        "Commands (from the repository root):",
        "",
        "```",
        command,
        "```",
        "",
        "The call (%s m=%d n=%d k=%d) runs %d times between two elementwise passes over %d MiB of fp32 (a plain "
        "copy that reads and writes %d MiB): %d kernel dispatches. Each counter's readings (KiB) are summed per "
        "call and scaled by the copy's to bytes." % (PROFILE_KERNELS[name] + (reps, TRAFFIC_COPY_BYTES >> 20,
                                                                              TRAFFIC_COPY_BYTES >> 20,
                                                                              out["FETCH_SIZE"][3])),
        "",
        "| counter | mean per call (KiB) | copy reading (KiB) | scale to bytes per KiB |",
        "|---|---|---|---|",
    ]
    for counter, (v, ck, sc, _) in out.items():
        lines.append("| %s | %.1f | %.1f | %.4f x 1024 |" % (counter, v, ck, sc))
    lines += [
        "",
        "| | bytes per call |",
        "|---|---|",
        "| algorithmic (what the method must move) | %d |" % nbytes,
        "| measured HBM traffic (fetch + write, scaled) | %d |" % int(per_call),
        "",
        "traffic_row: %s" % name,
        "traffic_bytes_per_launch: %d" % int(per_call),
        "traffic_sources_sha256: %s" % sources_digest(name),
        "",
    ]
    return "\n".join(lines)


def read_traffic(name):
    """Measured traffic per call of `name` from profiles/, or None when absent or taken on other sources."""
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
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--reps", type=int, default=20, help="replays per per-row timing")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="skip the side workloads in `extra`")
    ap.add_argument("--profile-kernel", metavar="NAME", choices=sorted(PROFILE_KERNELS),
                    help="only run one W8A8 linear shape --profile-reps times between two device copies (for the "
                    "rocprofv3 counter runs) and exit")
    ap.add_argument("--profile-reps", type=int, default=3)
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the markdown summary of the two counter runs of --profile-kernel NAME and exit")
    ap.add_argument("--traffic-command", default="",
                    help="the command lines recorded in that summary (default: the two counter runs and this one, "
                    "with the given directories)")
    args = ap.parse_args()

    if args.traffic_summary:
        fdir, wdir = args.traffic_summary
        run = "python3 bench.py --profile-kernel %s --profile-reps %d" % (args.profile_kernel, args.profile_reps)
        command = args.traffic_command or "\n".join([
            "rocprofv3 --pmc FETCH_SIZE -d %s -o t --output-format csv -- %s" % (fdir, run),
            "rocprofv3 --pmc WRITE_SIZE -d %s -o t --output-format csv -- %s" % (wdir, run),
            "%s --traffic-summary %s %s" % (run, fdir, wdir)])
        print(traffic_summary(fdir, wdir, args.profile_kernel, args.profile_reps, command))
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

    if args.profile_kernel:
        profile_kernel(dev, args.profile_kernel, args.profile_reps)
        return 0

    d = Dense7B(dev)
    step_bytes, step_ops = d.step_work()
    log("inputs resident: %d layers of 7B-shaped FP8 codes (%.2f GB), bf16 activations up to M = %d"
        % (LAYERS, LAYERS * sum(n * k for _, n, k in LINEARS_7B) / 1e9, max(BATCHES_7B)))

    # eager reference of one step, then the graph of the whole step
    d.step()
    ref = d.snapshot()
    step_graph = TimedGraph(d.step, None)
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
    # the replays reproduce the eager step bit for bit (FP8 outputs are deterministic for a given shape)
    got = d.snapshot()
    replay_ok = all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(ref, got))
    if not replay_ok:
        log("ERROR: graph replay differs from the eager step")
    del step_graph

    per_m, per_linear = measure_rows(d, args.reps)
    ms_dom, ops_dom, bytes_dom = measure_dominant(d, args.reps)
    dom_name = "a3_fp8_%s_m%d" % DOMINANT
    achieved = ops_dom / ms_dom / 1e9  # TFLOP/s
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_PEAK_TOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_PEAK_TOPS, 4), "traffic": read_traffic(dom_name),
                "kernel": dom_name, "flops_per_launch": int(ops_dom), "bytes_per_launch": int(bytes_dom),
                "us_per_launch": round(ms_dom * 1e3, 2)}
    decode = {}
    for m in (1, 16):
        r = per_m["m%d" % m]
        decode["m%d" % m] = {"bound": "hbm", "achieved": r["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": r["frac"], "us_per_layer": r["us_per_layer"]}

    extra = {}
    if not args.quick:
        del d
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        r = max(5, args.reps // 2)
        log("publish of the 7B linears (fp32 masters, INT8 / FP8, with and without s)")
        extra["publish_7b"] = measure_publish_7b(dev, r)
        log("MoE grouped FFN (Qwen3-30B-A3B-shaped, FP8)")
        extra["moe_fp8"] = measure_moe(dev, r)
        log("1.5B-shaped INT8 linears")
        extra["int8_1p5b_linears"] = measure_int8_1p5b(dev, r)
        log("W4A16 7B-shaped linears")
        extra["w4a16_7b_linears"] = measure_w4a16_7b(dev, r)
        log("RMSNorm producer of the FP8 linears' input (7B hidden size)")
        extra["rmsnorm_producer_7b"] = measure_rmsnorm_producer(dev, r)

    cpu = None
    if not args.no_cpu_baseline:
        log("CPU oracle baseline (%.0f s budget)" % args.cpu_budget)
        cpu = cpu_baseline(args.cpu_budget)

    value = step_ops * args.steps / (ms_total / 1e3) / 1e12
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic",
        "config": {"workload": "7B-shaped FP8 E4M3 W8A8 decoder-layer linears at M=%s: per-token activation "
                               "quantization (a2) + W8A8 linear with dequant epilogue (a3), bf16 in and out, "
                               "%d distinct layers of codes per step" % (",".join(map(str, BATCHES_7B)), LAYERS),
                   "linears": {n: [nn, k] for n, nn, k in LINEARS_7B}, "batches": list(BATCHES_7B),
                   "layers": LAYERS, "weights": "bf16 N(0,0.02) published to FP8 codes (a1, before timing)",
                   "acts": "bf16 N(0,1), 4 outlier channels x20"},
        "hbm_GBps": round(step_bytes * args.steps / (ms_total / 1e3) / 1e9, 1),
        "step_bytes": int(step_bytes), "step_ops": int(step_ops), "replay_matches_eager": bool(replay_ok),
        "roofline": roofline, "roofline_decode": decode, "cpu_baseline": cpu,
        "per_m": per_m, "per_linear": per_linear, "extra": extra,
    }
    print(json.dumps(line), flush=True)
    return 0 if replay_ok else 1


if __name__ == "__main__":
    sys.exit(main())
