"""GPU parity of the MoE glue (the next row around the grouped linear): routing, the SiLU-gated product fused
with the down projection's activation quantization, the routing-weighted combine, and the whole expert FFN.

Routing indices, CSR lists, h, its codes and scales, and the combined output are compared bit for bit with the
oracle: both sides evaluate every floating-point decision in fp64 and round once (the exponentials come from two
libm implementations, so a result could differ only if an fp64 value fell within an ulp or two of a rounding
boundary of its fp32/bf16 target). The routing weights are fp32 results and are allowed one ulp. The whole FFN is
checked against the oracle's own chain within the stated 1e-2 max|ref| tolerance (its FP8 accumulations may
round in a different order)."""
import numpy as np
import pytest
import torch

import quantized_rollout_amd as qr
from oracle import core as O
from quantized_rollout_amd import synth

from gpu_util import assert_codes_equal, assert_scales_equal, assert_y_close, dev, host, log

pytestmark = pytest.mark.gpu

QT = [(O.INT8, qr.QR_INT8), (O.FP8, qr.QR_FP8_E4M3)]


def _ulp_diff(a, b):
    ia = a.view(np.int32).astype(np.int64)
    ib = b.view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


def _check_route(logits, k, what):
    T, E = logits.shape
    ref = O.moe_route(logits, k)
    got = qr.qr_moe_route(dev(logits), k)
    torch.cuda.synchronize()
    got = {name: host(t) for name, t in got.items()}
    for name in ("topk_expert", "pair_rows", "row_ids"):
        assert np.array_equal(got[name], ref[name]), "%s: %s differs" % (what, name)
    assert np.array_equal(got["expert_offsets"], ref["offsets"]), "%s: offsets differ" % what
    for name in ("topk_weight", "row_weights"):
        d = _ulp_diff(got[name], ref[name])
        assert d.size == 0 or d.max() <= 1, "%s: %s differs by %d ulp" % (what, name, d.max())
    log("route %s T=%d E=%d k=%d: weights bitwise equal %d of %d" % (what, T, E, k,
                                                                   int((_ulp_diff(got["topk_weight"],
                                                                                  ref["topk_weight"]) == 0).sum()),
                                                                   T * k))
    return got, ref


@pytest.mark.parametrize("T,E,k", [(256, 128, 8), (37, 8, 3), (5, 64, 1), (70, 200, 32), (1300, 512, 6),
                                   (3, 65, 65 // 65 + 1), (1, 1, 1)])
def test_route_parity(T, E, k):
    """Routing of seeded logits N(0, 1), with ties planted: a token whose logits are all equal (the lowest
    experts win, equal weights), a tie at the top, -0 against +0, and a token with one large logit. Shapes: the
    Qwen3-30B-A3B router (256 tokens, 128 experts, top 8), experts not a multiple of 64, top_k 1 and 32, more
    tokens than one pass of the list builder (512), the maximum of 512 experts, one token and one expert."""
    rng = np.random.default_rng(700 + T + E + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    if T >= 4 and E >= 4:
        logits[0, :] = 0.5
        logits[1, 2] = logits[1, E - 1] = logits[1].max() + 1.0
        logits[2, :] = -1.0
        logits[2, 1] = -0.0
        logits[2, 3] = 0.0
        logits[3, E // 2] = 40.0
    _check_route(logits, k, "T=%d E=%d k=%d" % (T, E, k))


def test_route_empty_batch_writes_offsets():
    out = qr.qr_moe_route(torch.empty((0, 16), dtype=torch.float32, device="cuda"), 4)
    out["expert_offsets"].fill_(-7)
    qr.qr_moe_route(torch.empty((0, 16), dtype=torch.float32, device="cuda"), 4, out=out)
    torch.cuda.synchronize()
    assert host(out["expert_offsets"]).tolist() == [0] * 17


def _gate_up_rows(rng, rows, inter, spread=1.0):
    """Seeded bf16 gate/up outputs [rows, 2 inter]: N(0, spread) with a few large and zero values, one row of
    zeros and one of negative zeros (their codes are zero and the scale 1)."""
    y = (rng.standard_normal((rows, 2 * inter)) * spread).astype(np.float32)
    if rows >= 3:
        y[0, :inter // 2] = 0.0
        y[0, 3] = 35.0
        y[0, inter + 5] = -60.0
        y[1, :] = 0.0
        y[2, :inter] = -0.0
        y[2, inter:] = 1.0
    return synth.f32_to_bf16_bits(y)


@pytest.mark.parametrize("oq,gq", QT)
@pytest.mark.parametrize("rows,inter", [(2048, 768), (7, 16), (5, 4112), (1, 256)])
@pytest.mark.parametrize("with_s", [False, True])
def test_silu_mul_quantize_parity(oq, gq, rows, inter, with_s):
    """h = bf16(silu(g) u) bit for bit, and its per-row codes and scales bit for bit against the oracle's
    activation quantizer applied to the oracle's h. Shapes: the MoE FFN (2048 (token, expert) rows, intermediate
    768), a ragged tiny one, a long row past the registers a lane holds (recomputed for the codes), one row."""
    rng = np.random.default_rng(710 + rows + inter + int(with_s))
    y = _gate_up_rows(rng, rows, inter)
    s = rng.uniform(0.5, 2.0, inter).astype(np.float32) if with_s else None
    h_ref = O.silu_mul(y)
    c_ref, s_ref = O.quantize_rows(h_ref, oq, s=s, s_mode=O.S_MUL_RECIP)
    log("silu_mul_quantize %s rows=%d inter=%d s=%s" % (oq, rows, inter, with_s))
    codes, scales, h = qr.qr_silu_mul_quantize(dev(y), gq, s=None if s is None else dev(s), want_h=True)
    codes2, scales2 = qr.qr_silu_mul_quantize(dev(y), gq, s=None if s is None else dev(s))
    torch.cuda.synchronize()
    h = host(h)
    if not np.array_equal(h, h_ref):
        bad = np.argwhere(h != h_ref)
        raise AssertionError("%d h values differ, first at %s" % (len(bad), tuple(bad[0])))
    assert_codes_equal(host(codes), c_ref, "h codes")
    assert_scales_equal(host(scales), s_ref, "h scales")
    assert np.array_equal(host(codes2), c_ref) and np.array_equal(host(scales2).view(np.uint32), s_ref.view(np.uint32))
    if rows >= 3:
        assert not c_ref[1].any() and s_ref[1] == 1.0


@pytest.mark.parametrize("T,E,k,H", [(256, 128, 8, 2048), (33, 16, 4, 72), (2, 4, 4, 8)])
def test_combine_parity(T, E, k, H):
    """out[t] = bf16(sum_j w[t,j] y_down[pair_rows[t,j]]) bit for bit against the oracle (both in fp64, j in
    order), with the routing of seeded logits and seeded bf16 expert outputs."""
    rng = np.random.default_rng(720 + T + H)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    r = O.moe_route(logits, k)
    y_down = synth.f32_to_bf16_bits((rng.standard_normal((T * k, H)) * 0.5).astype(np.float32))
    ref = O.moe_combine(y_down, r["topk_weight"], r["pair_rows"])
    out = qr.qr_moe_combine(dev(y_down), dev(r["topk_weight"]), dev(r["pair_rows"]))
    torch.cuda.synchronize()
    assert np.array_equal(host(out), ref)


def test_combine_row_out_of_range_adds_nothing():
    """A pair row outside the expert outputs contributes nothing (the device never reads outside y_down): equal
    to the oracle's combine with that pair pointed at an appended row of zeros."""
    rng = np.random.default_rng(730)
    T, k, H, rows = 6, 3, 64, 18
    y_down = synth.f32_to_bf16_bits(rng.standard_normal((rows, H)).astype(np.float32))
    w = rng.uniform(0.1, 1.0, (T, k)).astype(np.float32)
    pr = rng.permutation(rows).astype(np.int32).reshape(T, k)
    pr_bad = pr.copy()
    pr_bad[2, 1] = -1
    pr_bad[4, 0] = rows + 5
    out = qr.qr_moe_combine(dev(y_down), dev(w), dev(pr_bad))
    torch.cuda.synchronize()
    y_pad = np.concatenate([y_down, np.zeros((1, H), np.uint16)])
    pr_ref = pr.copy()
    pr_ref[2, 1] = rows
    pr_ref[4, 0] = rows
    assert np.array_equal(host(out), O.moe_combine(y_pad, w, pr_ref))


def _ffn_gpu(gq, x, logits, wgu_c, wgu_s, wd_c, wd_s, k):
    """The MoE FFN on the GPU, every step through the library: routing, per-token activation codes, the
    grouped gate/up linear over the token lists, the SiLU product with its per-row codes, the grouped down
    linear over the (token, expert) rows, the weighted combine."""
    T = x.shape[0]
    r = qr.qr_moe_route(logits, k)
    xc, xs = qr.qr_quantize_acts(x, gq)
    rows = T * k
    y_gu = qr.qr_w8a8_grouped_linear(gq, r["expert_offsets"], r["row_ids"], rows, xc, xs, wgu_c, wgu_s)
    hc, hs = qr.qr_silu_mul_quantize(y_gu, gq)
    y_d = qr.qr_w8a8_grouped_linear(gq, r["expert_offsets"], None, rows, hc, hs, wd_c, wd_s)
    return r, qr.qr_moe_combine(y_d, r["topk_weight"], r["pair_rows"])


def _ffn_oracle_tokens(oq, x_bits, logits, wgu_c, wgu_s, wd_c, wd_s, k, tokens):
    """The oracle's chain for the given tokens: its routing, its activation codes, per chosen expert the plain
    linear, its SiLU product and quantizer, the down linear, its combine."""
    r = O.moe_route(logits, k)
    out = {}
    for t in tokens:
        xc, xs = O.quantize_rows(x_bits[t:t + 1], oq, s_mode=O.S_MUL_RECIP)
        y_down = []
        for e in r["topk_expert"][t]:
            y_gu, _, _ = O.linear(oq, xc, xs, wgu_c[e], wgu_s[e], O.BF16)
            h = O.silu_mul(y_gu)
            hc, hs = O.quantize_rows(h, oq, s_mode=O.S_MUL_RECIP)
            yd, _, _ = O.linear(oq, hc, hs, wd_c[e], wd_s[e], O.BF16)
            y_down.append(yd[0])
        out[t] = O.moe_combine(np.stack(y_down), r["topk_weight"][t:t + 1], np.arange(k, dtype=np.int32)[None, :])[0]
    return out


@pytest.mark.parametrize("oq,gq", QT)
def test_moe_ffn_small_every_token(oq, gq):
    """A small expert FFN (16 experts, hidden 256, intermediate 128, 48 tokens, top 4) checked on every token."""
    rng = np.random.default_rng(740)
    E, H, I, T, k = 16, 256, 128, 48, 4
    wgu = (rng.standard_normal((E, 2 * I, H)) * 0.02).astype(np.float32)
    wd = (rng.standard_normal((E, H, I)) * 0.02).astype(np.float32)
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    wgu_c, wgu_s = zip(*[O.quantize_rows(synth.f32_to_bf16_bits(wgu[e]), oq) for e in range(E)])
    wd_c, wd_s = zip(*[O.quantize_rows(synth.f32_to_bf16_bits(wd[e]), oq) for e in range(E)])
    wgu_c, wgu_s, wd_c, wd_s = map(np.stack, (wgu_c, wgu_s, wd_c, wd_s))
    r, out = _ffn_gpu(gq, dev(x), dev(logits), dev(wgu_c), dev(wgu_s), dev(wd_c), dev(wd_s), k)
    torch.cuda.synchronize()
    ref = _ffn_oracle_tokens(oq, x, logits, wgu_c, wgu_s, wd_c, wd_s, k, range(T))
    assert_y_close(host(out), np.stack([ref[t] for t in range(T)]), "moe ffn small %s" % oq)


def test_moe_ffn_full_size_qwen3_fp8_sampled():
    """The Qwen3-30B-A3B-shaped FFN (128 experts, hidden 2048, intermediate 768, top 8 of 256 tokens, FP8) with
    every step on the GPU, the weights quantized there too; the oracle's chain checks sampled tokens."""
    inp = synth.make_moe()
    wl = inp.wl
    log("moe ffn full size: E=%d hidden=%d inter=%d tokens=%d" % (wl.experts, wl.hidden, wl.inter, wl.tokens))
    wgu = dev(inp.w_gate_up.reshape(-1, wl.hidden))
    wd = dev(inp.w_down.reshape(-1, wl.inter))
    gq = qr.QR_FP8_E4M3
    wgu_c, wgu_s = qr.qr_quantize_weights(wgu, gq)
    wd_c, wd_s = qr.qr_quantize_weights(wd, gq)
    E = wl.experts
    r, out = _ffn_gpu(gq, dev(inp.x), dev(inp.logits), wgu_c.view(E, 2 * wl.inter, wl.hidden),
                      wgu_s.view(E, 2 * wl.inter), wd_c.view(E, wl.hidden, wl.inter), wd_s.view(E, wl.hidden),
                      wl.top_k)
    torch.cuda.synchronize()
    out = host(out)
    ref_route = O.moe_route(inp.logits, wl.top_k)
    assert np.array_equal(host(r["row_ids"]), ref_route["row_ids"])
    assert np.array_equal(host(r["expert_offsets"]), inp.expert_offsets)
    tokens = np.sort(np.random.default_rng(741).choice(wl.tokens, 5, replace=False))
    experts = sorted({int(e) for t in tokens for e in ref_route["topk_expert"][t]})
    wgu_c_ref = np.zeros((E, 2 * wl.inter, wl.hidden), np.uint8)
    wgu_s_ref = np.zeros((E, 2 * wl.inter), np.float32)
    wd_c_ref = np.zeros((E, wl.hidden, wl.inter), np.uint8)
    wd_s_ref = np.zeros((E, wl.hidden), np.float32)
    for e in experts:
        wgu_c_ref[e], wgu_s_ref[e] = O.quantize_rows(inp.w_gate_up[e], O.FP8)
        wd_c_ref[e], wd_s_ref[e] = O.quantize_rows(inp.w_down[e], O.FP8)
    ref = _ffn_oracle_tokens(O.FP8, inp.x, inp.logits, wgu_c_ref, wgu_s_ref, wd_c_ref, wd_s_ref, wl.top_k, tokens)
    for t in tokens:
        assert_y_close(out[t:t + 1], ref[t][None, :], "moe ffn token %d" % t)
