"""Oracle of the DeepSeekMoE layer backward with FP8 GEMMs (float64 unless a step fixes
float32). Test infrastructure only: see the package docstring for who may call this.

Passages followed, by page and section:
  * lpnh.cn guide "从技术报告到可跑配置", section 3: the [fp8] block runs fprop, dgrad
    and wgrad GEMMs in FP8 (format e4m3) with 1x128 tile-wise inputs and 128x128
    block-wise weights, and keeps moe_gating in BF16/FP32;
  * zhihu infra commentary, training part: E4M3 in both directions (no E5M2 for
    gradients), per-tile 1x128 and per-group 128x128 scaling, GEMMs by partial-sum
    promotion;
  * 2kiu.com digest, section 3.2: gates are the normalised unbiased sigmoid affinities of
    the selected experts times the scaling factor; the bias only ranks.

Readings (where the pages leave a step open):
  * Quantisers are straight-through: the backward differentiates the forward's real
    function, and every FP8 GEMM quantises its two operands at the pages' granularity
    along its own contraction axis. Weights are 128x128 blocks in every GEMM (a block is
    the same block of the transposed matrix). Activations and gradients are 1x128 tiles
    along K: along the hidden or intermediate axis for dgrad, along the token axis for
    wgrad (tiles of 128 consecutive rows of one expert's segment, from its first row; the
    last tile of a segment may be shorter).
  * The SwiGLU inputs a = x W1^T and b = x W3^T are recomputed from the forward's FP8
    activation codes; dg = dh * b * silu'(a), du = dh * silu(a) and h = silu(a) * b are
    float32 values when they are quantised.
  * The wgrad activation operand is the layer input x (its bf16 values) quantised along
    the token axis; the dgrad of the combine keeps the forward's bf16 expert outputs.
  * Weight gradients are the FP32-accumulated GEMM results (this oracle: float64).
  * Routing is not differentiated through the selection (the bias and the group limit
    only choose experts); the gates are, through the normalisation and the sigmoid, to
    the router logits, in float64 (gating stays out of FP8).
"""
from __future__ import annotations

from typing import Callable, Optional

import numpy as np

from .e4m3 import decode, encode
from .moe import _scale_from_amax, dequant_1x128, dequant_128x128, quantize_1x128, silu

TILE = 128


# ----------------------------------------------------------------------------------------
# 1x128 tiles along the token axis: per column, groups of 128 consecutive rows (the last
# group of a segment may be shorter). Same scale and rounding rule as the 1x128 tiles of
# the forward (s = fl32(amax / 448), codes = E4M3(fl32(v / s)), s = 1 for a zero group).
# ----------------------------------------------------------------------------------------
def quantize_128x1(v: np.ndarray):
    """v [M, C] float32 -> (codes [M, C] uint8, scales [ceil(M/128), C] float32)."""
    v = np.asarray(v, dtype=np.float32)
    M, C = v.shape
    nt = (M + TILE - 1) // TILE
    codes = np.zeros((M, C), dtype=np.uint8)
    scales = np.zeros((nt, C), dtype=np.float32)
    for t in range(nt):
        blk = v[t * TILE:(t + 1) * TILE]
        s = _scale_from_amax(np.max(np.abs(blk), axis=0))
        scales[t] = s
        codes[t * TILE:(t + 1) * TILE] = encode((blk / s[None, :]).astype(np.float32))
    return codes, scales


def dequant_128x1(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    M = codes.shape[0]
    s = np.repeat(np.asarray(scales, dtype=np.float64), TILE, axis=0)[:M]
    return decode(codes).astype(np.float64) * s


def round_bf16(v: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32. NaN stays NaN."""
    f = np.asarray(v, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    out = r.view(np.float32)
    return np.where(np.isnan(f), f, out).astype(np.float32)


def _q_rows(v):
    """Quantise-dequantise along the columns axis (1x128 tiles of each row)."""
    q, s = quantize_1x128(np.asarray(v, dtype=np.float32))
    return dequant_1x128(q, s)


def _q_tokens(v):
    """Quantise-dequantise along the token axis (128x1 tiles of each column)."""
    q, s = quantize_128x1(np.asarray(v, dtype=np.float32))
    return dequant_128x1(q, s)


def _identity(v):
    return np.asarray(v, dtype=np.float64)


# ----------------------------------------------------------------------------------------
# Combine backward (2kiu.com digest section 3.2: out_t = sum_j g_tj * y_{e_j}(t), plus the
# shared experts with weight 1). dy of a routed row is the float32 product g * dout; a
# shared row gets dout itself; dgate is the dot product of dout with the expert's output
# row.
# ----------------------------------------------------------------------------------------
def combine_backward(dout: np.ndarray, y_rows: np.ndarray, row_of: np.ndarray,
                     gate: np.ndarray, n_shared: int):
    """dout [T, H] (bf16 values), y_rows [T*k + n_shared*T, H] (the forward's rows),
    gate [T, k] float32 -> (dy [T*k + n_shared*T, H] float32, dgate [T, k] float64).
    Rows that no (token, slot) names stay zero."""
    dout = np.asarray(dout, dtype=np.float32)
    T, H = dout.shape
    k = row_of.shape[1]
    dy = np.zeros((T * k + n_shared * T, H), dtype=np.float32)
    dgate = np.zeros((T, k), dtype=np.float64)
    g32 = np.asarray(gate, dtype=np.float32)
    yr = np.asarray(y_rows, dtype=np.float64)
    for t in range(T):
        for j in range(k):
            r = int(row_of[t, j])
            if r < 0:
                continue
            dy[r] = (g32[t, j] * dout[t]).astype(np.float32)
            dgate[t, j] = float(np.dot(dout[t].astype(np.float64), yr[r]))
    for s in range(n_shared):
        dy[T * k + s * T:T * k + (s + 1) * T] = dout
    return dy, dgate


# ----------------------------------------------------------------------------------------
# Router backward (2kiu.com digest section 3.2; lpnh.cn guide section 3: gating in
# FP32). gate_j = rho * s_j / Z, Z = sum of the selected s; s = sigmoid(logit);
# logit = x W_r^T. Only the selected experts' affinities receive a gradient.
# ----------------------------------------------------------------------------------------
def route_backward(x: np.ndarray, w_router: np.ndarray, s: np.ndarray, idx: np.ndarray,
                   dgate: np.ndarray, rho: float):
    """-> dict(ds [T,N] (non-zero on the selected experts), dlogit [T,N], dx [T,H],
    dw [N,H]), float64."""
    x = np.asarray(x, dtype=np.float64)
    wr = np.asarray(w_router, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    T, N = s.shape
    ds = np.zeros((T, N), dtype=np.float64)
    for t in range(T):
        sel = np.asarray(idx[t], dtype=np.int64)
        z = s[t, sel].sum()
        g = rho * s[t, sel] / z
        inner = float(np.dot(dgate[t], g)) / rho
        # d gate_j / d s_m = rho (delta_jm / Z - s_j / Z^2)
        ds[t, sel] = rho / z * (np.asarray(dgate[t], dtype=np.float64) - inner)
    dlogit = ds * s * (1.0 - s)
    return {"ds": ds, "dlogit": dlogit, "dx": dlogit @ wr, "dw": dlogit.T @ x}


# ----------------------------------------------------------------------------------------
# One SwiGLU expert, backward, with FP8 GEMMs (zhihu commentary, training part; lpnh.cn
# guide section 3: gemm_dgrad and gemm_wgrad in e4m3).
# ----------------------------------------------------------------------------------------
def silu_grad(z: np.ndarray) -> np.ndarray:
    """d/dz [z * sigmoid(z)] = sigmoid(z) * (1 + z * (1 - sigmoid(z)))."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        sg = 1.0 / (1.0 + np.exp(-z))
    return sg * (1.0 + z * (1.0 - sg))


def expert_ffn_backward(aq, a_s, x_rows, w1q, w1s, w3q, w3s, w2q, w2s, dy,
                        exact: bool = False) -> dict:
    """Backward of y = (silu(A W1^T) * (A W3^T)) W2^T over M rows of one expert.

    aq, a_s: the forward's 1x128 activation codes and scales of the rows ([M, H]);
    x_rows: the rows' input values (float32, [M, H]) for the wgrad operand;
    w*q, w*s: E4M3 codes and 128x128 block scales (W1, W3 [I, H]; W2 [H, I]);
    dy: the gradient of the rows' outputs, float32 [M, H].
    ``exact`` skips every quantisation of the backward GEMMs' operands (the weights and
    the forward activation codes stay as given): the chain rule alone.
    Returns float64 dx [M, H], dw1, dw3 [I, H], dw2 [H, I] and the float32 values
    dg, du, h [M, I] that the GEMMs quantise.
    """
    q_rows = _identity if exact else _q_rows
    q_tok = _identity if exact else _q_tokens
    A = dequant_1x128(aq, a_s)
    W1 = dequant_128x128(w1q, w1s)
    W3 = dequant_128x128(w3q, w3s)
    W2 = dequant_128x128(w2q, w2s)
    dy = np.asarray(dy, dtype=np.float32)
    # recompute the SwiGLU inputs (fprop GEMMs, FP64 here)
    g = A @ W1.T
    u = A @ W3.T
    # dgrad of the down projection: K = H, dy in 1x128 tiles along H
    dh = q_rows(dy) @ W2
    dg = (dh * u * silu_grad(g)).astype(np.float32)
    du = (dh * silu(g)).astype(np.float32)
    h = (silu(g) * u).astype(np.float32)
    # dgrad of gate/up: K = I, dg and du in 1x128 tiles along I
    dx = q_rows(dg) @ W1 + q_rows(du) @ W3
    # wgrad: K = tokens, both operands in 128x1 tiles along the token axis
    xr = np.asarray(x_rows, dtype=np.float32)
    qx = q_tok(xr)
    dw2 = q_tok(dy).T @ q_tok(h)
    dw1 = q_tok(dg).T @ qx
    dw3 = q_tok(du).T @ qx
    return {"dx": dx, "dw1": dw1, "dw3": dw3, "dw2": dw2, "dg": dg, "du": du, "h": h,
            "g": g, "u": u, "dh": dh}


# ----------------------------------------------------------------------------------------
# Whole layer backward.
# ----------------------------------------------------------------------------------------
def layer_backward(x: np.ndarray, w_router: np.ndarray, cfg, fwd: dict,
                   routed: Callable[[int], tuple], shared: Callable[[int], tuple],
                   dout: np.ndarray, y_rows: Optional[np.ndarray] = None,
                   exact: bool = False) -> dict:
    """Gradients of the layer output for upstream gradient dout [T, H].

    ``fwd`` is the dict of moe.layer_forward for the same x; ``y_rows`` are the expert
    output rows the combine saw (permuted layout, shared segments appended), default the
    forward's rows rounded to bf16. Returns dx [T, H], per-expert dw (lists of (dw1, dw3,
    dw2), routed then shared), dw_router [N, H], dgate [T, k], the dy rows and the routing
    gradient parts.
    """
    x = np.asarray(x, dtype=np.float32)
    T, H = x.shape
    N, k, S = cfg.num_experts, cfg.num_experts_per_tok, cfg.num_shared_experts
    r = fwd["route"]
    offsets, row_token, row_of = fwd["offsets"], fwd["row_token"], fwd["row_of"]
    if y_rows is None:
        ys = [fwd["y_rows"]] + list(fwd["y_shared"])
        full = np.concatenate(ys, axis=0) if S > 0 else fwd["y_rows"]
        y_rows = round_bf16(full).astype(np.float64)
    gate32 = np.asarray(r["gate"], dtype=np.float32)
    dy, dgate = combine_backward(dout, y_rows, row_of, gate32, S)
    xq, xs = fwd["xq"], fwd["xs"]
    dx = np.zeros((T, H), dtype=np.float64)
    dw = []
    for e in range(N):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            dw.append(None)
            continue
        toks = row_token[lo:hi]
        b = expert_ffn_backward(xq[toks], xs[toks], x[toks], *routed(e), dy[lo:hi], exact=exact)
        np.add.at(dx, toks, b["dx"])
        dw.append((b["dw1"], b["dw3"], b["dw2"]))
    for s in range(S):
        lo = T * k + s * T
        b = expert_ffn_backward(xq, xs, x, *shared(s), dy[lo:lo + T], exact=exact)
        dx += b["dx"]
        dw.append((b["dw1"], b["dw3"], b["dw2"]))
    # routing: the gates' gradient, through the normalisation and the sigmoid
    rb = route_backward(x, w_router, r["s"], r["idx"], dgate, cfg.routed_scaling_factor)
    dx_total = dx + rb["dx"]
    return {"dx": dx_total, "dx_experts": dx, "dw": dw, "dw_router": rb["dw"], "dgate": dgate,
            "dy": dy, "route": rb}
