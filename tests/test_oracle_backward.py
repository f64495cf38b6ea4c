"""Pins of the oracle's backward (CPU): the chain rule against torch autograd in float64,
the quantisation granularity of each GEMM operand through inputs that one granularity
represents exactly and the other does not, closed forms, brute force and error bounds."""
import numpy as np
import pytest
import torch

import oracle
from oracle import e4m3

TILE = 128


def _codes_pow2_scales(rng, rows, cols, tile_rows, tile_cols, lo=-6, hi=2):
    """E4M3 codes with power-of-two scales per (tile_rows x tile_cols) block: the
    dequantised values are exact float32 numbers."""
    codes = rng.integers(0, 256, (rows, cols)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38          # no NaN codes
    sc = 2.0 ** rng.integers(lo, hi, ((rows + tile_rows - 1) // tile_rows,
                                      (cols + tile_cols - 1) // tile_cols))
    return codes, sc.astype(np.float32)


def _expert(rng, H, I):
    w1q, w1s = _codes_pow2_scales(rng, I, H, TILE, TILE, -9, -5)
    w3q, w3s = _codes_pow2_scales(rng, I, H, TILE, TILE, -9, -5)
    w2q, w2s = _codes_pow2_scales(rng, H, I, TILE, TILE, -9, -5)
    return w1q, w1s, w3q, w3s, w2q, w2s


def _acts(rng, M, H):
    aq, a_s = _codes_pow2_scales(rng, M, H, 1, TILE, -8, -5)
    return aq, a_s


# ---------------------------------------------------------------------------------------
# Chain rule: exact mode against torch autograd (float64)
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("M,H,I", [(5, 128, 128), (37, 256, 384)])
def test_expert_backward_exact_matches_autograd(M, H, I):
    rng = np.random.default_rng(M + H)
    aq, a_s = _acts(rng, M, H)
    ws = _expert(rng, H, I)
    A = oracle.dequant_1x128(aq, a_s)
    dy = rng.standard_normal((M, H)).astype(np.float32)
    b = oracle.expert_ffn_backward(aq, a_s, A.astype(np.float32), *ws, dy, exact=True)

    tA = torch.tensor(A, dtype=torch.float64, requires_grad=True)
    W1 = torch.tensor(oracle.dequant_128x128(ws[0], ws[1]), requires_grad=True)
    W3 = torch.tensor(oracle.dequant_128x128(ws[2], ws[3]), requires_grad=True)
    W2 = torch.tensor(oracle.dequant_128x128(ws[4], ws[5]), requires_grad=True)
    y = (torch.nn.functional.silu(tA @ W1.T) * (tA @ W3.T)) @ W2.T
    (y * torch.tensor(dy, dtype=torch.float64)).sum().backward()
    # the oracle rounds dg, du and h to float32 before the next GEMM: relative 2^-24 each
    for got, ref in ((b["dx"], tA.grad), (b["dw1"], W1.grad), (b["dw3"], W3.grad),
                     (b["dw2"], W2.grad)):
        ref = ref.numpy()
        assert np.linalg.norm(got - ref) <= 1e-6 * np.linalg.norm(ref)


def test_silu_grad_closed_forms_and_finite_differences():
    assert oracle.silu_grad(np.array([0.0]))[0] == 0.5
    assert abs(oracle.silu_grad(np.array([40.0]))[0] - 1.0) < 1e-12
    assert abs(oracle.silu_grad(np.array([-40.0]))[0]) < 1e-12
    z = np.linspace(-8, 8, 41)
    eps = 1e-6
    fd = (oracle.silu(z + eps) - oracle.silu(z - eps)) / (2 * eps)
    assert np.max(np.abs(oracle.silu_grad(z) - fd)) < 1e-8


def test_route_backward_matches_autograd():
    rng = np.random.default_rng(3)
    T, H, N, k, rho = 6, 64, 16, 4, 2.5
    x = rng.standard_normal((T, H))
    wr = rng.standard_normal((N, H)) * 0.1
    idx = np.stack([rng.choice(N, k, replace=False) for _ in range(T)])
    dgate = rng.standard_normal((T, k))
    tx = torch.tensor(x, requires_grad=True)
    tw = torch.tensor(wr, requires_grad=True)
    s = torch.sigmoid(tx @ tw.T)
    sel = torch.gather(s, 1, torch.tensor(idx))
    g = rho * sel / sel.sum(1, keepdim=True)
    (g * torch.tensor(dgate)).sum().backward()
    r = oracle.route_backward(x, wr, s.detach().numpy(), idx, dgate, rho)
    assert np.allclose(r["dx"], tx.grad.numpy(), rtol=1e-12, atol=1e-14)
    assert np.allclose(r["dw"], tw.grad.numpy(), rtol=1e-12, atol=1e-14)
    # experts outside the selection get no gradient; the gates' gradient sums to zero
    # along dgate = const (the gates always sum to rho)
    mask = np.ones((T, N), bool)
    np.put_along_axis(mask, idx, False, axis=1)
    assert np.all(r["ds"][mask] == 0)
    r1 = oracle.route_backward(x, wr, s.detach().numpy(), idx, np.ones((T, k)), rho)
    assert np.max(np.abs(r1["ds"])) < 1e-12


def test_combine_backward_matches_autograd_and_shared_rows():
    rng = np.random.default_rng(4)
    T, H, k, S = 5, 32, 3, 2
    N = 8
    idx = np.stack([rng.choice(N, k, replace=False) for _ in range(T)]).astype(np.int32)
    _, _, row_of = oracle.permute(idx, N)
    rows = T * k + S * T
    y = rng.standard_normal((rows, H))
    gate = rng.uniform(0.1, 1, (T, k)).astype(np.float32)
    dout = oracle.round_bf16(rng.standard_normal((T, H)).astype(np.float32))
    ty = torch.tensor(y, requires_grad=True)
    tg = torch.tensor(gate.astype(np.float64), requires_grad=True)
    out = sum(ty[T * k + s * T:T * k + (s + 1) * T] for s in range(S))
    for j in range(k):
        out = out + tg[:, j:j + 1] * ty[torch.tensor(row_of[:, j], dtype=torch.long)]
    (out * torch.tensor(dout.astype(np.float64))).sum().backward()
    dy, dgate = oracle.combine_backward(dout, y, row_of, gate, S)
    assert np.allclose(dy, ty.grad.numpy(), rtol=2 ** -23, atol=0)
    assert np.allclose(dgate, tg.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_round_bf16():
    v = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0, 65504.0], np.float32)
    assert np.array_equal(oracle.round_bf16(v), torch.tensor(v).to(torch.bfloat16).float().numpy())
    r = np.random.default_rng(1).standard_normal(10000).astype(np.float32)
    assert np.array_equal(oracle.round_bf16(r), torch.tensor(r).to(torch.bfloat16).float().numpy())


# ---------------------------------------------------------------------------------------
# Token-axis quantiser
# ---------------------------------------------------------------------------------------
def test_quantize_128x1_brute_force_and_closed_forms():
    rng = np.random.default_rng(5)
    M, C = 300, 5                  # ragged: tiles of 128, 128, 44 rows
    v = rng.standard_normal((M, C)).astype(np.float32)
    v[200, 3] = 1000.0
    v[:128, 4] = 0.0               # an all-zero tile gets scale 1
    q, s = oracle.quantize_128x1(v)
    assert s.shape == (3, C)
    for c in range(C):
        for t in range(3):
            blk = v[t * 128:(t + 1) * 128, c]
            amax = np.float32(np.max(np.abs(blk)))
            sc = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
            assert s[t, c] == sc
            for i, val in enumerate(blk):
                assert q[t * 128 + i, c] == e4m3.encode(np.array([np.float32(val / sc)]))[0]
    assert e4m3.decode(q[200:201, 3])[0] == 448.0
    assert np.all(q[:128, 4] == 0) and s[0, 4] == 1.0
    # the dequantisation error bound: half an E4M3 step (relative 2^-4) for normal codes
    d = oracle.dequant_128x1(q, s)
    big = np.abs(v) > np.repeat(s, 128, axis=0)[:M] * 2 ** -6
    assert np.all(np.abs(d - v)[big] <= np.abs(v)[big] * 2 ** -4 + 1e-30)


# ---------------------------------------------------------------------------------------
# Granularity of each GEMM operand
# ---------------------------------------------------------------------------------------
def _grid_values(rng, shape):
    """E4M3 grid values of magnitude 2^-3..448 (normal codes), random signs."""
    codes = rng.integers(0x20, 0x7F, shape).astype(np.uint8) | (rng.integers(0, 2, shape) << 7).astype(np.uint8)
    return e4m3.decode(codes).astype(np.float32)


def test_dgrad_quantises_dy_along_hidden():
    """dy exact in 1x128 tiles along H (each row tile holds +-448 * 2^k_row on the grid),
    lossy in tiles along tokens (rows of very different scale share a column tile): the
    dgrad GEMM must see dy unchanged."""
    rng = np.random.default_rng(6)
    M, H, I = 130, 256, 128
    aq, a_s = _acts(rng, M, H)
    ws = _expert(rng, H, I)
    dy = _grid_values(rng, (M, H))
    dy[:, ::TILE] = 448.0
    dy *= (2.0 ** rng.integers(-20, 0, (M, 1))).astype(np.float32)
    assert not np.array_equal(oracle.dequant_128x1(*oracle.quantize_128x1(dy)), dy)
    b = oracle.expert_ffn_backward(aq, a_s, np.zeros((M, H), np.float32), *ws, dy)
    W2 = oracle.dequant_128x128(ws[4], ws[5])
    assert np.array_equal(b["dh"], dy.astype(np.float64) @ W2)


def test_wgrad_quantises_dy_and_x_along_tokens():
    """dy and x exact in 128-row tiles of each column (column scales 2^k_col, a +-448 in
    every column tile), lossy in 1x128 row tiles: dw2's dy operand and dw1/dw3's x
    operand must be unchanged."""
    rng = np.random.default_rng(7)
    M, H, I = 200, 256, 128
    aq, a_s = _acts(rng, M, H)
    ws = _expert(rng, H, I)

    def tok_exact(shape):
        v = _grid_values(rng, shape)
        v[::TILE, :] = 448.0
        return (v * (2.0 ** rng.integers(-20, 0, (1, shape[1]))).astype(np.float32)).astype(np.float32)

    dy = tok_exact((M, H))
    x = tok_exact((M, H))
    assert not np.array_equal(oracle.dequant_1x128(*oracle.quantize_1x128(dy)), dy)
    b = oracle.expert_ffn_backward(aq, a_s, x, *ws, dy)
    qh = oracle.dequant_128x1(*oracle.quantize_128x1(b["h"]))
    qg = oracle.dequant_128x1(*oracle.quantize_128x1(b["dg"]))
    assert np.array_equal(b["dw2"], dy.astype(np.float64).T @ qh)
    assert np.array_equal(b["dw1"], qg.T @ x.astype(np.float64))


def test_dgrad_quantises_dg_du_along_intermediate():
    """With the forward activations and dy chosen so that dg, du happen to be exact per
    1x128 row tile is impractical; instead: the dx GEMM equals the product of the
    row-tile quantisations of dg and du with the weights, and not that of the token-tile
    ones (they differ on this input)."""
    rng = np.random.default_rng(8)
    M, H, I = 140, 128, 256
    aq, a_s = _acts(rng, M, H)
    ws = _expert(rng, H, I)
    dy = rng.standard_normal((M, H)).astype(np.float32) * (2.0 ** rng.integers(-12, 0, (M, 1))).astype(np.float32)
    b = oracle.expert_ffn_backward(aq, a_s, np.zeros((M, H), np.float32), *ws, dy)
    W1 = oracle.dequant_128x128(ws[0], ws[1])
    W3 = oracle.dequant_128x128(ws[2], ws[3])
    rows = (oracle.dequant_1x128(*oracle.quantize_1x128(b["dg"])) @ W1
            + oracle.dequant_1x128(*oracle.quantize_1x128(b["du"])) @ W3)
    toks = (oracle.dequant_128x1(*oracle.quantize_128x1(b["dg"])) @ W1
            + oracle.dequant_128x1(*oracle.quantize_128x1(b["du"])) @ W3)
    assert np.array_equal(b["dx"], rows)
    assert not np.allclose(b["dx"], toks, rtol=1e-3, atol=0)


def test_quantised_backward_within_fp8_bound_of_exact():
    """Each quantised operand is within 2^-4 relative per element (normal codes), so a
    GEMM of two such operands is within about 2^-3 of the exact product, summed in
    absolute value; a transposed operand or a wrong scale would break this."""
    rng = np.random.default_rng(9)
    M, H, I = 96, 256, 256
    aq, a_s = _acts(rng, M, H)
    ws = _expert(rng, H, I)
    x = oracle.dequant_1x128(aq, a_s).astype(np.float32)
    dy = rng.standard_normal((M, H)).astype(np.float32)
    q = oracle.expert_ffn_backward(aq, a_s, x, *ws, dy)
    e = oracle.expert_ffn_backward(aq, a_s, x, *ws, dy, exact=True)
    h32 = e["h"].astype(np.float64)
    bound = 0.14 * (np.abs(dy.astype(np.float64)).T @ np.abs(h32))
    assert np.all(np.abs(q["dw2"] - e["dw2"]) <= bound + 1e-30)
    assert np.linalg.norm(q["dw2"] - e["dw2"]) < 0.05 * np.linalg.norm(e["dw2"])
    assert np.linalg.norm(q["dw1"] - e["dw1"]) < 0.1 * np.linalg.norm(e["dw1"])
    assert np.linalg.norm(q["dx"] - e["dx"]) < 0.1 * np.linalg.norm(e["dx"])


def test_layer_backward_exact_matches_autograd_tiny():
    """The whole layer in exact mode (no FP8 in the backward GEMMs; the forward's FP8
    codes fixed) against autograd of the same forward function on a tiny config."""
    import dataclasses
    import synth
    cfg = dataclasses.replace(synth.PRESETS["tiny"], tokens=24)
    # x that the forward's 1x128 quantisation represents exactly (grid values, a 448 in
    # every row tile, power-of-two tile scales), so the FP8 forward operand equals x
    rng0 = np.random.default_rng(11)
    x = _grid_values(rng0, (cfg.tokens, cfg.hidden_size))
    x[:, ::TILE] = 448.0
    x = (x * np.repeat(2.0 ** rng0.integers(-12, -8, (cfg.tokens, cfg.hidden_size // TILE)),
                       TILE, axis=1)).astype(np.float32)
    xq0, xs0 = oracle.quantize_1x128(x)
    assert np.array_equal(oracle.dequant_1x128(xq0, xs0), x)
    wr = synth.router_weight(cfg)
    b = synth.expert_bias(cfg)
    experts = {}
    synth.map_experts(cfg, lambda e, w: experts.__setitem__(e, w), range(cfg.num_experts))
    shared = {}
    synth.map_experts(cfg, lambda e, w: shared.__setitem__(e, w), range(cfg.num_shared_experts), shared=True)

    def q(w):
        w1q, w1s = oracle.quantize_128x128(w[0])
        w3q, w3s = oracle.quantize_128x128(w[1])
        w2q, w2s = oracle.quantize_128x128(w[2])
        return w1q, w1s, w3q, w3s, w2q, w2s
    rq = {e: q(w) for e, w in experts.items()}
    sq = {e: q(w) for e, w in shared.items()}
    fwd = oracle.layer_forward(x, wr, b, cfg, lambda e: rq[e], lambda s: sq[s])
    rng = np.random.default_rng(10)
    dout = oracle.round_bf16(rng.standard_normal(x.shape).astype(np.float32))
    yfull = np.concatenate([fwd["y_rows"]] + list(fwd["y_shared"]), axis=0)
    bw = oracle.layer_backward(x, wr, cfg, fwd, lambda e: rq[e], lambda s: sq[s], dout,
                               y_rows=yfull, exact=True)

    # autograd: the gates through the router, the experts on the FP8 forward activations
    # (straight-through: their gradient reaches x as the gradient of the codes' values)
    T, H = x.shape
    k, N = cfg.num_experts_per_tok, cfg.num_experts
    tx = torch.tensor(x.astype(np.float64), requires_grad=True)
    A = torch.tensor(oracle.dequant_1x128(fwd["xq"], fwd["xs"]))
    Ast = A + (tx - tx.detach())                       # straight-through quantiser
    tw = torch.tensor(wr.astype(np.float64), requires_grad=True)
    s = torch.sigmoid(tx @ tw.T)
    idx = torch.tensor(fwd["route"]["idx"], dtype=torch.long)
    sel = torch.gather(s, 1, idx)
    gate = cfg.routed_scaling_factor * sel / sel.sum(1, keepdim=True)
    Ws = {}

    def ffn(Ain, key, w):
        W1 = torch.tensor(oracle.dequant_128x128(w[0], w[1]), requires_grad=True)
        W3 = torch.tensor(oracle.dequant_128x128(w[2], w[3]), requires_grad=True)
        W2 = torch.tensor(oracle.dequant_128x128(w[4], w[5]), requires_grad=True)
        Ws[key] = (W1, W3, W2)
        return (torch.nn.functional.silu(Ain @ W1.T) * (Ain @ W3.T)) @ W2.T
    out = sum(ffn(Ast, ("s", s_), sq[s_]) for s_ in range(cfg.num_shared_experts))
    ycache = torch.tensor(yfull[:T * k])
    row_of = fwd["row_of"]
    ys = torch.zeros((T * k, H), dtype=torch.float64)
    for e in range(N):
        lo, hi = int(fwd["offsets"][e]), int(fwd["offsets"][e + 1])
        if hi > lo:
            toks = torch.tensor(fwd["row_token"][lo:hi], dtype=torch.long)
            ys = ys.index_put((torch.arange(lo, hi),), ffn(Ast[toks], ("r", e), rq[e]))
    # The forward quantises h to FP8 before W2; the backward passes it straight through.
    # Autograd runs the unquantised expert function, with the forward's output values
    # put back on the value path only (what the gates' gradient sees).
    assert torch.linalg.norm(ys - ycache) < 0.1 * torch.linalg.norm(ycache)
    ys = ys + (ycache - ys).detach()
    for j in range(k):
        out = out + gate[:, j:j + 1] * ys[torch.tensor(row_of[:, j], dtype=torch.long)]
    (out * torch.tensor(dout.astype(np.float64))).sum().backward()
    rel = np.linalg.norm(bw["dx"] - tx.grad.numpy()) / np.linalg.norm(tx.grad.numpy())
    assert rel < 1e-6, rel
    rel_r = np.linalg.norm(bw["dw_router"] - tw.grad.numpy()) / np.linalg.norm(tw.grad.numpy())
    assert rel_r < 1e-9, rel_r
    for e in range(N):
        if ("r", e) in Ws:
            for got, ref in zip(bw["dw"][e], Ws[("r", e)]):
                assert np.linalg.norm(got - ref.grad.numpy()) <= 1e-6 * np.linalg.norm(ref.grad.numpy())
        else:
            assert bw["dw"][e] is None
    for s_ in range(cfg.num_shared_experts):
        for got, ref in zip(bw["dw"][N + s_], Ws[("s", s_)]):
            assert np.linalg.norm(got - ref.grad.numpy()) <= 1e-6 * np.linalg.norm(ref.grad.numpy())
