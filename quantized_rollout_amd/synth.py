"""Seeded synthetic inputs for the quantized-actor linear (no step of the method is computed here).

Both the HIP path (through the tests and the benchmark) and the CPU oracle consume the arrays made here;
this module is the only thing they share. Recipe, per workload:

  * ``rng = numpy.random.default_rng(seed)`` (PCG64), one fresh generator per workload, seed 0 by default;
  * draws are float64 ``standard_normal`` / ``uniform``, scaled in float64, rounded to fp32 (round to
    nearest even), then to bfloat16 (round to nearest even, kept as uint16 bit patterns) where the workload
    has bfloat16 tensors;
  * draw order: every weight matrix in the listed order, then the weight updates, then the invariant
    scales, then per linear the activations followed by their 4 outlier input channels
    (``rng.choice(K, 4, replace=False)``, those columns multiplied by 20 in fp32), then router logits;
  * activations are drawn once at the largest batch; smaller batches take row prefixes;
  * the RMSNorm producer's inputs (``make_norm_inputs``): hidden states N(0, 1) with the 4 outlier channels, each
    row multiplied by 10^u, u ~ U(-1, 2) (the residual stream's token-to-token magnitude spread), then the norm
    weight gamma = |N(1, 0.3)| rounded to bfloat16 (held as fp32), then the invariant scale s ~ U(0.5, 2).

Shapes follow the pages' models: a 1.5B-class dense decoder layer (QuRL section 5.1, the DeepScaleR
model), a 7B-class layer (QuRL sections 5.1 and 5.2) and the Qwen3-30B-A3B mixture-of-experts layer (QaRL
abstract). Weights ~ N(0, 0.02) (standard deviation), activations ~ N(0, 1) with outlier channels (the
channel-outlier premise of the invariant-scaling technique cited in QuRL section 4.3).
"""
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

WEIGHT_STD = 0.02
OUTLIER_CHANNELS = 4
OUTLIER_GAIN = 20.0


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal(rng, shape, std, chunk_rows=4096) -> np.ndarray:
    """float64 N(0, std) draws rounded to fp32, drawn row-block by row-block to bound host memory (the
    generator state advances exactly as for one large draw)."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, np.float32)
    flat = out.reshape(-1, shape[-1]) if len(shape) > 1 else out.reshape(1, -1)
    for r0 in range(0, flat.shape[0], chunk_rows):
        r1 = min(flat.shape[0], r0 + chunk_rows)
        flat[r0:r1] = (rng.standard_normal((r1 - r0, flat.shape[1])) * std).astype(np.float32)
    return out


def _activations(rng, m, k) -> np.ndarray:
    x = _normal(rng, (m, k), 1.0)
    cols = rng.choice(k, OUTLIER_CHANNELS, replace=False)
    x[:, cols] *= np.float32(OUTLIER_GAIN)
    return x


@dataclass
class Linear:
    name: str
    n: int  # output channels
    k: int  # input channels


@dataclass
class DenseWorkload:
    name: str
    qtype: str            # "int8" or "fp8"
    weight_dtype: str     # "f32" or "bf16"
    linears: List[Linear]
    batches: List[int]
    seed: int = 0


TOY = DenseWorkload("toy-int8-m4-k256-n512", "int8", "f32", [Linear("toy", 512, 256)], [4])
QWEN_1P5B = DenseWorkload(
    "qwen2.5-1.5b-layer-int8", "int8", "bf16",
    [Linear("qkv", 2048, 1536), Linear("o", 1536, 1536), Linear("gate_up", 17920, 1536),
     Linear("down", 1536, 8960)],
    [1, 16, 64])
DENSE_7B = DenseWorkload(
    "7b-layer-fp8", "fp8", "bf16",
    [Linear("qkv", 4608, 3584), Linear("o", 3584, 3584), Linear("gate_up", 37888, 3584),
     Linear("down", 3584, 18944)],
    [1, 16, 128, 512, 2048])


@dataclass
class DenseInputs:
    workload: DenseWorkload
    weights: Dict[str, np.ndarray] = field(default_factory=dict)  # fp32, or uint16 bf16 bits
    acts: Dict[str, np.ndarray] = field(default_factory=dict)     # [M_max, K], same dtype convention


def make_dense(wl: DenseWorkload, m_max: Optional[int] = None, linears: Optional[List[str]] = None,
               row_limit: Optional[int] = None) -> DenseInputs:
    """Weights of every linear (all are drawn, so the stream is the same whichever are kept) and
    activations [m_max, K] per linear. ``row_limit`` keeps only the first rows of each kept weight
    (still drawing all of them)."""
    rng = np.random.default_rng(wl.seed)
    m_max = max(wl.batches) if m_max is None else m_max
    out = DenseInputs(wl)
    keep = set(l.name for l in wl.linears) if linears is None else set(linears)
    for lin in wl.linears:
        if lin.name in keep:
            w = _normal(rng, (lin.n, lin.k), WEIGHT_STD)
            if row_limit is not None:
                w = np.ascontiguousarray(w[:row_limit])
            out.weights[lin.name] = f32_to_bf16_bits(w) if wl.weight_dtype == "bf16" else w
        else:
            _normal(rng, (lin.n, lin.k), WEIGHT_STD)  # advance the stream identically
    for lin in wl.linears:
        x = _activations(rng, m_max, lin.k)
        if lin.name in keep:
            out.acts[lin.name] = f32_to_bf16_bits(x) if wl.weight_dtype == "bf16" else x
    return out


@dataclass
class RequantInputs:
    """7B-class fp32 master weights W, W2 = fl32(W + dW) with dW ~ N(0, 1e-5), and s ~ U(0.5, 2)."""
    w: Dict[str, np.ndarray]
    w2: Dict[str, np.ndarray]
    s: Dict[str, np.ndarray]


def make_requant(linears: Optional[List[str]] = None, row_limit: Optional[int] = None,
                 seed: int = 0) -> RequantInputs:
    rng = np.random.default_rng(seed)
    lins = DENSE_7B.linears
    keep = set(l.name for l in lins) if linears is None else set(linears)

    def trim(a):
        return a if row_limit is None else np.ascontiguousarray(a[:row_limit])

    w = {}
    for lin in lins:
        a = _normal(rng, (lin.n, lin.k), WEIGHT_STD)
        if lin.name in keep:
            w[lin.name] = trim(a)
    w2 = {}
    for lin in lins:
        d = _normal(rng, (lin.n, lin.k), 1e-5)
        if lin.name in keep:
            w2[lin.name] = (w[lin.name] + trim(d)).astype(np.float32)  # one fp32 rounding of W + dW
    s = {}
    for lin in lins:
        a = rng.uniform(0.5, 2.0, lin.k).astype(np.float32)
        if lin.name in keep:
            s[lin.name] = a
    return RequantInputs(w, w2, s)


@dataclass
class MoEWorkload:
    name: str = "qwen3-30b-a3b-moe-fp8"
    hidden: int = 2048
    experts: int = 128
    inter: int = 768
    top_k: int = 8
    tokens: int = 256
    seed: int = 0


QWEN3_MOE = MoEWorkload()


@dataclass
class MoEInputs:
    wl: MoEWorkload
    w_gate_up: np.ndarray  # [E, 2*inter, hidden] bf16 bits (gate rows first, then up rows)
    w_down: np.ndarray     # [E, hidden, inter] bf16 bits
    x: np.ndarray          # [tokens, hidden] bf16 bits
    logits: np.ndarray     # [tokens, E] fp32
    h: np.ndarray          # [tokens*top_k, inter] bf16 bits: stand-in input of the down projection
    expert_offsets: np.ndarray  # [E+1] int32 CSR over (token, expert) rows
    row_ids: np.ndarray    # [tokens*top_k] int32 token id of each row


def route_top_k(logits: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Token lists from router logits: each token picks its k largest logits (ties to the lower expert
    index); rows are grouped by expert (ascending) with token ids ascending inside each expert."""
    t, e = logits.shape
    order = np.lexsort((np.tile(np.arange(e), (t, 1)), -logits.astype(np.float64)), axis=1)[:, :k]
    pairs = sorted((int(ex), tok) for tok in range(t) for ex in order[tok])
    counts = np.bincount([p[0] for p in pairs], minlength=e)
    offsets = np.zeros(e + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    row_ids = np.array([p[1] for p in pairs], np.int32)
    return offsets, row_ids


def make_moe(wl: MoEWorkload = QWEN3_MOE, experts: Optional[int] = None) -> MoEInputs:
    """``experts`` (optional) keeps only the first experts' weights; the stream is unchanged."""
    rng = np.random.default_rng(wl.seed)
    E = wl.experts
    keep = E if experts is None else experts
    wgu = np.empty((keep, 2 * wl.inter, wl.hidden), np.uint16)
    for e in range(E):
        a = _normal(rng, (2 * wl.inter, wl.hidden), WEIGHT_STD)
        if e < keep:
            wgu[e] = f32_to_bf16_bits(a)
    wd = np.empty((keep, wl.hidden, wl.inter), np.uint16)
    for e in range(E):
        a = _normal(rng, (wl.hidden, wl.inter), WEIGHT_STD)
        if e < keep:
            wd[e] = f32_to_bf16_bits(a)
    x = f32_to_bf16_bits(_activations(rng, wl.tokens, wl.hidden))
    logits = _normal(rng, (wl.tokens, E), 1.0)
    h = f32_to_bf16_bits(_activations(rng, wl.tokens * wl.top_k, wl.inter))
    offsets, row_ids = route_top_k(logits, wl.top_k)
    return MoEInputs(wl, wgu, wd, x, logits, h, offsets, row_ids)


@dataclass
class NormInputs:
    x: np.ndarray  # hidden states [rows, k], bfloat16 bits
    gamma: np.ndarray  # norm weight [k], fp32 holding bfloat16 values
    s: np.ndarray  # invariant scale [k], fp32


def make_norm_inputs(rows: int, k: int, seed: int = 0) -> NormInputs:
    """Inputs of the RMSNorm producer of a linear's quantized input, at the hidden size k of the pages' models."""
    rng = np.random.default_rng(seed)
    x = _activations(rng, rows, k)
    x *= (10.0 ** rng.uniform(-1.0, 2.0, (rows, 1))).astype(np.float32)
    gamma = bf16_bits_to_f32(f32_to_bf16_bits(np.abs(1.0 + 0.3 * rng.standard_normal(k)).astype(np.float32)))
    s = rng.uniform(0.5, 2.0, k).astype(np.float32)
    return NormInputs(f32_to_bf16_bits(x), gamma, s)
