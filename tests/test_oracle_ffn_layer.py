"""Pins of the oracle expert FFN, combine and whole layer (brute force, closed forms)."""
import json
import math
import os

import numpy as np

import oracle
import synth
from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_codes(rng, shape):
    c = rng.integers(0, 0x7F, shape).astype(np.uint8)          # finite magnitudes
    return c | (rng.integers(0, 2, shape).astype(np.uint8) << 7)


def _rand_scales(rng, shape):
    return rng.uniform(0.001, 0.01, shape).astype(np.float32)


def _tiny_expert(rng, H=256, I=256):
    return (_rand_codes(rng, (I, H)), _rand_scales(rng, (I // 128, H // 128)),
            _rand_codes(rng, (I, H)), _rand_scales(rng, (I // 128, H // 128)),
            _rand_codes(rng, (H, I)), _rand_scales(rng, (H // 128, I // 128)))


def test_silu_closed_forms():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    z = math.log(3.0)                       # sigmoid(ln 3) = 3/4
    assert abs(oracle.silu(np.array([z]))[0] - 0.75 * z) < 1e-15
    v = np.linspace(-30, 30, 61)
    assert np.allclose(oracle.silu(v) - oracle.silu(-v), v, rtol=0, atol=1e-12)
    assert oracle.silu(np.array([-1000.0]))[0] == 0.0


def test_expert_ffn_matches_loop_bruteforce():
    """Scalar loops over K with per-element block-scale lookup (catches transposed or
    mis-indexed scales), against the oracle's dequantise-then-matmul."""
    rng = np.random.default_rng(30)
    H = I = 256
    M = 2
    aq = _rand_codes(rng, (M, H))
    a_s = _rand_scales(rng, (M, H // 128))
    w1q, w1s, w3q, w3s, w2q, w2s = _tiny_expert(rng, H, I)
    val = e4m3.decode
    av, w1v, w3v, w2v = val(aq), val(w1q), val(w3q), val(w2q)
    h = np.zeros((M, I), np.float32)
    for m in range(M):
        for n in range(I):
            g = u = 0.0
            for k in range(H):
                a = av[m, k] * float(a_s[m, k // 128])
                g += a * w1v[n, k] * float(w1s[n // 128, k // 128])
                u += a * w3v[n, k] * float(w3s[n // 128, k // 128])
            h[m, n] = np.float32(g / (1.0 + math.exp(-g)) * u)
    y, hq, hs, h_or = oracle.expert_ffn(aq, a_s, w1q, w1s, w3q, w3s, w2q, w2s)
    assert np.allclose(h_or, h, rtol=1e-6, atol=0)
    hv = val(hq)
    y_ref = np.zeros((M, H))
    for m in range(M):
        for n in range(H):
            acc = 0.0
            for k in range(I):
                acc += hv[m, k] * float(hs[m, k // 128]) * w2v[n, k] * float(w2s[n // 128, k // 128])
            y_ref[m, n] = acc
    assert np.allclose(y, y_ref, rtol=1e-12, atol=1e-15)


def test_chunk_promotion_equals_dequant_matmul_exactly():
    """Per-128-K integer partial sums promoted by sa*sb equal the FP64 dequantised GEMM."""
    rng = np.random.default_rng(31)
    M, N, K = 5, 128, 512
    aq = _rand_codes(rng, (M, K))
    a_s = _rand_scales(rng, (M, K // 128))
    wq = _rand_codes(rng, (N, K))
    ws = _rand_scales(rng, (1, K // 128))
    ai = np.rint(e4m3.decode(aq) * 512).astype(np.int64)     # E4M3 values * 2^9 are integers
    wi = np.rint(e4m3.decode(wq) * 512).astype(np.int64)
    acc = np.zeros((M, N))
    for c in range(K // 128):
        part = ai[:, c * 128:(c + 1) * 128] @ wi[:, c * 128:(c + 1) * 128].T   # exact int64
        acc += part * 2.0 ** -18 * a_s[:, c:c + 1].astype(np.float64) * float(ws[0, c])
    ref = oracle.dequant_1x128(aq, a_s) @ oracle.dequant_128x128(wq, ws).T
    assert np.allclose(acc, ref, rtol=1e-13, atol=0)


def test_zero_up_projection_gives_zero():
    rng = np.random.default_rng(32)
    w = list(_tiny_expert(rng))
    w[2] = np.zeros_like(w[2])
    aq = _rand_codes(rng, (3, 256))
    y, hq, hs, h = oracle.expert_ffn(aq, _rand_scales(rng, (3, 2)), *w)
    assert np.all(y == 0) and np.all(h == 0) and np.all(hs == 1.0)


def test_down_scale_linearity():
    rng = np.random.default_rng(33)
    w = list(_tiny_expert(rng))
    aq = _rand_codes(rng, (3, 256))
    a_s = _rand_scales(rng, (3, 2))
    y1 = oracle.expert_ffn(aq, a_s, *w)[0]
    w[5] = (w[5] * np.float32(2.0)).astype(np.float32)
    y2 = oracle.expert_ffn(aq, a_s, *w)[0]
    assert np.array_equal(y2, 2 * y1)


def test_combine_special_cases():
    rng = np.random.default_rng(34)
    T, k, H = 6, 3, 16
    y_rows = rng.standard_normal((T * k, H))
    row_of = rng.permutation(T * k).reshape(T, k)
    ysh = [rng.standard_normal((T, H))]
    assert np.array_equal(oracle.combine(y_rows, row_of, np.zeros((T, k)), ysh), ysh[0])
    onehot = np.zeros((T, k))
    onehot[:, 1] = 1.0
    assert np.array_equal(oracle.combine(y_rows, row_of, onehot), y_rows[row_of[:, 1]])
    g1, g2 = rng.random((T, k)), rng.random((T, k))
    lhs = oracle.combine(y_rows, row_of, g1 + g2)
    rhs = oracle.combine(y_rows, row_of, g1) + oracle.combine(y_rows, row_of, g2)
    assert np.allclose(lhs, rhs, rtol=1e-14)


def _tiny_layer_inputs(cfg):
    x = synth.hidden_states(cfg)
    wr = synth.router_weight(cfg)
    b = synth.expert_bias(cfg)

    def q(w):
        w1, w3, w2 = w
        return (*oracle.quantize_128x128(w1), *oracle.quantize_128x128(w3), *oracle.quantize_128x128(w2))
    routed = [q(synth.routed_expert_weights(cfg, e)) for e in range(cfg.num_experts)]
    shared = [q(synth.shared_expert_weights(cfg, s)) for s in range(cfg.num_shared_experts)]
    return x, wr, b, routed, shared


def test_identical_experts_reduce_to_rho_times_one_expert():
    cfg = synth.PRESETS["tiny"]
    x, wr, b, routed, shared = _tiny_layer_inputs(cfg)
    res = oracle.layer_forward(x, wr, b, cfg, lambda e: routed[0], lambda s: shared[s])
    xq, xs = oracle.quantize_1x128(x)
    y0 = oracle.expert_ffn(xq, xs, *routed[0])[0]
    ysh = oracle.expert_ffn(xq, xs, *shared[0])[0]
    assert np.allclose(res["out"], cfg.routed_scaling_factor * y0 + ysh, rtol=1e-12, atol=1e-12)


def test_zero_routed_experts_leave_shared_only():
    cfg = synth.PRESETS["tiny"]
    x, wr, b, routed, shared = _tiny_layer_inputs(cfg)
    zero = list(routed[0])
    zero[2] = np.zeros_like(zero[2])
    res = oracle.layer_forward(x, wr, b, cfg, lambda e: tuple(zero), lambda s: shared[s])
    xq, xs = oracle.quantize_1x128(x)
    assert np.array_equal(res["out"], oracle.expert_ffn(xq, xs, *shared[0])[0])


def test_tiny_layer_invariants_and_golden():
    cfg = synth.PRESETS["tiny"]
    x, wr, b, routed, shared = _tiny_layer_inputs(cfg)
    res = oracle.layer_forward(x, wr, b, cfg, lambda e: routed[e], lambda s: shared[s])
    r = res["route"]
    assert r["counts"].sum() == cfg.tokens * cfg.num_experts_per_tok
    assert np.allclose(r["gate"].sum(1), cfg.routed_scaling_factor)
    g = np.load(os.path.join(GOLDEN, "tiny_layer_oracle.npz"))
    assert np.array_equal(g["idx"], r["idx"]) and np.array_equal(g["counts"], r["counts"])
    assert np.array_equal(g["xq"], res["xq"]) and np.array_equal(g["xs"], res["xs"])
    assert np.allclose(g["out"], res["out"], rtol=1e-12, atol=1e-12)


def test_page_config_values():
    """The presets carry the values the pages print for the V3 MoE layer."""
    g = json.load(open(os.path.join(GOLDEN, "v3_moe_config.json")))
    c = synth.PRESETS["v3_prefill"]
    assert c.num_experts == g["num_experts"] and c.num_shared_experts == g["num_shared_experts"]
    assert c.num_experts_per_tok == g["num_experts_per_tok"]
    assert c.moe_intermediate_size == g["moe_intermediate_size"] and c.hidden_size == g["hidden_size"]
    assert c.routed_scaling_factor == g["routed_scaling_factor"]
    assert c.expert_bias_update_rate == g["expert_bias_update_rate"]
    assert c.topk_group == g["max_groups_per_token"]
    assert g["experts_per_layer"] == c.num_experts + c.num_shared_experts
    assert g["total_experts"] == (g["num_layers"] - g["first_moe_layer"] + 1) * g["experts_per_layer"]
