"""Oracle steps of the DeepSeekMoE layer forward (float64 unless a step fixes float32).

Test infrastructure only: see the package docstring for who may call this.
Each function states the passage it follows and the reading taken where the pages
are silent. No blocking, fusion or reordering beyond the plain definitions.
"""
from __future__ import annotations

from typing import Callable, Optional, Sequence

import numpy as np

from .e4m3 import E4M3_MAX, decode, encode

TILE = 128


# ----------------------------------------------------------------------------------------
# Fine-grained quantisation (lpnh.cn guide section 3 [fp8] block: inputs tile_wise_1x128,
# weights block_wise_128x128, format e4m3; 2kiu.com digest section 4.3: every group gets
# its own scale so an outlier only affects its own group; zhihu commentary: per-tile 1x128
# and per-group 128x128).
# Reading: online scale s = fl32(amax / 448) (not a power of two), codes =
# E4M3_RNE_SAT(fl32(x / s)) with a correctly rounded float32 division; a group whose
# fl32(amax/448) is 0 (all-zero group, or float32 underflow) gets s = 1.
# ----------------------------------------------------------------------------------------
def _scale_from_amax(amax: np.ndarray) -> np.ndarray:
    amax = np.asarray(amax, dtype=np.float32)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    return np.where(s == np.float32(0.0), np.float32(1.0), s).astype(np.float32)


def quantize_1x128(x: np.ndarray):
    """x [R, C] (float32 values, C % 128 == 0) -> (codes [R, C] u8, scales [R, C/128] f32)."""
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    assert C % TILE == 0
    xt = x.reshape(R, C // TILE, TILE)
    amax = np.max(np.abs(xt), axis=2)
    s = _scale_from_amax(amax)
    q = (xt / s[:, :, None]).astype(np.float32)
    return encode(q).reshape(R, C), s


def quantize_128x128(w: np.ndarray):
    """w [N, K] float32 -> (codes [N, K] u8, scales [N/128, K/128] f32)."""
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    assert N % TILE == 0 and K % TILE == 0
    wb = w.reshape(N // TILE, TILE, K // TILE, TILE)
    amax = np.max(np.abs(wb), axis=(1, 3))
    s = _scale_from_amax(amax)
    q = (wb / s[:, None, :, None]).astype(np.float32)
    return encode(q).reshape(N, K), s


# ----------------------------------------------------------------------------------------
# Power-of-two scale variant (opt-in; the pages call the fine-grained scheme close to
# micro-scaling, zhihu commentary training part and 2kiu.com digest section 4.3, without
# fixing this variant). Reading: the same 1x128 / 128x128 groups, each with the smallest
# power of two s such that amax / s <= 448 (s = 1 for an all-zero group; s >= 2^-126),
# codes = E4M3_RNE_SAT(x / s), where the division by a power of two is exact.
# ----------------------------------------------------------------------------------------
def _pow2_scale_from_amax(amax: np.ndarray) -> np.ndarray:
    amax = np.asarray(amax, dtype=np.float64)
    out = np.ones(amax.shape, dtype=np.float32)
    for i in np.ndindex(amax.shape):
        a = float(amax[i])
        if a == 0.0:
            continue
        k = int(np.ceil(np.log2(a / E4M3_MAX)))
        while E4M3_MAX * 2.0 ** (k - 1) >= a:   # smallest k with 448 * 2^k >= amax
            k -= 1
        while E4M3_MAX * 2.0 ** k < a:
            k += 1
        out[i] = np.float32(2.0 ** max(k, -126))
    return out


def quantize_1x128_pow2(x: np.ndarray):
    """x [R, C] float32 -> (codes [R, C] u8, power-of-two scales [R, C/128] f32)."""
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    assert C % TILE == 0
    xt = x.reshape(R, C // TILE, TILE)
    s = _pow2_scale_from_amax(np.max(np.abs(xt), axis=2))
    q = (xt.astype(np.float64) / s[:, :, None]).astype(np.float32)
    return encode(q).reshape(R, C), s


def quantize_128x128_pow2(w: np.ndarray):
    """w [N, K] float32 -> (codes [N, K] u8, power-of-two scales [N/128, K/128] f32)."""
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    assert N % TILE == 0 and K % TILE == 0
    wb = w.reshape(N // TILE, TILE, K // TILE, TILE)
    s = _pow2_scale_from_amax(np.max(np.abs(wb), axis=(1, 3)))
    q = (wb.astype(np.float64) / s[:, None, :, None]).astype(np.float32)
    return encode(q).reshape(N, K), s


def dequant_1x128(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """DQ of a 1x128-tiled operand: value(code) * scale, float64 (exact)."""
    v = decode(codes)
    return v * np.repeat(np.asarray(scales, dtype=np.float64), TILE, axis=1)


def dequant_128x128(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """DQ of a 128x128-blocked weight: value(code) * block scale, float64 (exact)."""
    v = decode(codes)
    s = np.asarray(scales, dtype=np.float64)
    return v * np.repeat(np.repeat(s, TILE, axis=0), TILE, axis=1)


# ----------------------------------------------------------------------------------------
# Routing (2kiu.com digest section 3.2 pseudocode and prose; section 3.4 group limit;
# lpnh.cn guide section 3 model JSON: norm_topk_prob, routed_scaling_factor 2.5; the
# [fp8] block keeps moe_gating out of FP8).
# ----------------------------------------------------------------------------------------
def route(x: np.ndarray, w_router: np.ndarray, bias: np.ndarray, top_k: int,
          n_group: int = 1, topk_group: int = 1, group_topn: int = 2,
          routed_scaling_factor: float = 2.5, force_idx: Optional[np.ndarray] = None):
    """Sigmoid affinities, bias-ranked (group-limited) top-k, normalised gates, load.

    * affinity s = sigmoid(x . W_r^T) on unquantised x, float64;
    * ranking score s + b: the bias only decides who is selected (section 3.2);
    * group limit (section 3.4), if n_group > 1: a group's score is the sum of its
      ``group_topn`` largest ranking scores; the ``topk_group`` best groups are kept
      (ties: lower group index) and experts of the other groups are excluded;
    * top-k by ranking score, descending, ties to the lower expert index;
    * gate = s[idx] / sum(s[idx]) * routed_scaling_factor, from the unbiased s;
    * load = bincount of the selected experts.
    ``force_idx`` evaluates gates and load for a given selection instead.
    Returns a dict with idx [T,k] int32, gate [T,k] f64, counts [N_r] int64, s, score,
    and the ranking gaps used to declare near-ties.
    """
    x = np.asarray(x, dtype=np.float64)
    wr = np.asarray(w_router, dtype=np.float64)
    T = x.shape[0]
    N = wr.shape[0]
    logits = x @ wr.T
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-logits))
    score = s + np.asarray(bias, dtype=np.float64)[None, :]

    allowed = np.ones((T, N), dtype=bool)
    group_gap = np.full(T, np.inf)
    if n_group > 1:
        assert N % n_group == 0
        gsz = N // n_group
        grouped = score.reshape(T, n_group, gsz)
        gscore = np.sort(grouped, axis=2)[:, :, gsz - group_topn:].sum(axis=2)
        gorder = np.argsort(-gscore, axis=1, kind="stable")
        keep = gorder[:, :topk_group]
        gmask = np.zeros((T, n_group), dtype=bool)
        np.put_along_axis(gmask, keep, True, axis=1)
        allowed = np.repeat(gmask, gsz, axis=1)
        gs_sorted = np.take_along_axis(gscore, gorder, axis=1)
        if topk_group < n_group:
            group_gap = gs_sorted[:, topk_group - 1] - gs_sorted[:, topk_group]

    masked = np.where(allowed, score, -np.inf)
    order = np.argsort(-masked, axis=1, kind="stable")
    idx = order[:, :top_k] if force_idx is None else np.asarray(force_idx, dtype=np.int64)
    ranked = np.take_along_axis(masked, order, axis=1)
    kth_gap = np.full(T, np.inf)
    if top_k < N:
        kth_gap = ranked[:, top_k - 1] - ranked[:, top_k]

    s_sel = np.take_along_axis(s, idx, axis=1)
    gate = s_sel / s_sel.sum(axis=1, keepdims=True) * routed_scaling_factor
    counts = np.bincount(idx.reshape(-1), minlength=N)
    return {
        "idx": idx.astype(np.int32), "gate": gate, "counts": counts, "s": s, "score": score,
        "logits": logits, "kth_gap": kth_gap, "group_gap": group_gap,
    }


# ----------------------------------------------------------------------------------------
# Permutation (2kiu.com digest section 3.2: y sums ffn_expert[idx[j]](h) over the slots;
# section 3.4: tokens go to the experts' owners, none is dropped).
# Reading: rows grouped by expert in expert order; within an expert, ascending token.
# ----------------------------------------------------------------------------------------
def permute(idx: np.ndarray, n_experts: int):
    """idx [T,k] -> offsets [N_r+1], row_token [T*k], row_of [T,k] (all int32)."""
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    counts = np.bincount(idx.reshape(-1), minlength=n_experts)
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    row_token = np.empty(T * k, dtype=np.int64)
    row_of = np.empty((T, k), dtype=np.int64)
    fill = offsets[:-1].copy()
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            r = fill[e]
            fill[e] += 1
            row_token[r] = t
            row_of[t, j] = r
    return offsets.astype(np.int32), row_token.astype(np.int32), row_of.astype(np.int32)


# ----------------------------------------------------------------------------------------
# Expert FFN (zhihu commentary: SwiGLU is one of the recomputed ops; lpnh.cn guide
# section 3: moe_intermediate_size, every GEMM input 1x128-quantised; 2kiu.com digest
# section 4.3 and zhihu commentary: FP8 GEMM with higher-precision accumulation).
# Reading: y = W2 (silu(W1 a) * (W3 a)), W1 the gate; the intermediate h is rounded to
# float32 and re-quantised 1x128 before the down GEMM. The GEMMs are evaluated as
# float64 products of the dequantised operands, which is what the per-128-K partial-sum
# promotion computes in exact arithmetic.
# ----------------------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(aq, a_s, w1q, w1s, w3q, w3s, w2q, w2s, pow2: bool = False):
    """One SwiGLU expert on M rows. Returns (y [M,H] f64, hq, hs, h f32).
    ``pow2``: h is re-quantised with power-of-two scales (the opt-in variant)."""
    a = dequant_1x128(aq, a_s)
    g = a @ dequant_128x128(w1q, w1s).T
    u = a @ dequant_128x128(w3q, w3s).T
    h = (silu(g) * u).astype(np.float32)
    hq, hs = quantize_1x128_pow2(h) if pow2 else quantize_1x128(h)
    y = dequant_1x128(hq, hs) @ dequant_128x128(w2q, w2s).T
    return y, hq, hs, h


# ----------------------------------------------------------------------------------------
# Combine (2kiu.com digest section 3.2: y = sum_j gate[j] * ffn_expert[idx[j]](h)) plus the
# shared expert with gate 1 (lpnh.cn guide section 3: num_shared_experts 1; 0539edu.com
# overview section 1.2: shared expert as a safety net). Residual excluded.
# ----------------------------------------------------------------------------------------
def combine(y_rows: np.ndarray, row_of: np.ndarray, gate: np.ndarray,
            y_shared: Optional[Sequence[np.ndarray]] = None) -> np.ndarray:
    y_rows = np.asarray(y_rows, dtype=np.float64)
    T, k = row_of.shape
    out = np.zeros((T, y_rows.shape[1]), dtype=np.float64)
    if y_shared is not None:
        for ys in y_shared:
            out += np.asarray(ys, dtype=np.float64)
    for j in range(k):
        out += np.asarray(gate, dtype=np.float64)[:, j:j + 1] * y_rows[row_of[:, j]]
    return out


# ----------------------------------------------------------------------------------------
# Bias update (2kiu.com digest section 3.2 pseudocode: after each step compare each
# expert's load with T*K/N_r, subtract gamma if over, add gamma if under; section 5.2:
# batch-level statistics, gamma around 1e-3; lpnh.cn guide: expert_bias_update_rate).
# Reading: eps = 0 (pure sign, equal load leaves b unchanged), compared in integers as
# T*k vs N_r*load; one float32 rounding of b + (+-gamma).
# ----------------------------------------------------------------------------------------
def bias_update(bias: np.ndarray, counts: np.ndarray, tokens: int, top_k: int,
                gamma: float) -> np.ndarray:
    bias = np.asarray(bias, dtype=np.float32)
    c = np.asarray(counts, dtype=np.int64)
    n = bias.shape[0]
    delta = np.sign(np.int64(tokens) * top_k - np.int64(n) * c).astype(np.float32)
    return (bias + np.float32(gamma) * delta).astype(np.float32)


# ----------------------------------------------------------------------------------------
# Sequence-wise balance statistic (2kiu.com digest section 3.3: a complementary
# sequence-level balance loss, the sum over experts of each expert's share of the
# sequence's assignments times its mean affinity, times a small coefficient alpha;
# lpnh.cn guide section 3: aux_loss_alpha 0.001 with seq_aux). Reading: for each sequence of
# L consecutive tokens, f_i = (assignments of expert i) / (k L), P_i = mean over the L
# tokens of the sigmoid affinity s_{t,i}, loss = alpha * sum_i f_i P_i.
# ----------------------------------------------------------------------------------------
def _seq_counts(idx_rows: np.ndarray, n: int) -> np.ndarray:
    """Assignments per expert; entries outside [0, n) name no expert and count for none
    (the same reading as the permutation's, where such entries route nowhere)."""
    v = np.asarray(idx_rows).ravel()
    return np.bincount(v[(v >= 0) & (v < n)], minlength=n)


def seq_balance_loss(scores: np.ndarray, idx: np.ndarray, seq_len: int, alpha: float) -> np.ndarray:
    scores = np.asarray(scores, dtype=np.float64)
    T, N = scores.shape
    k = idx.shape[1]
    assert T % seq_len == 0
    out = np.zeros(T // seq_len, dtype=np.float64)
    for q in range(T // seq_len):
        rows = slice(q * seq_len, (q + 1) * seq_len)
        f = _seq_counts(idx[rows], N) / (k * seq_len)
        p = scores[rows].mean(axis=0)
        out[q] = alpha * float(np.sum(f * p))
    return out


def seq_assignment_entropy(idx: np.ndarray, n_experts: int, seq_len: int) -> np.ndarray:
    """Entropy (natural log) of each sequence's expert allocation f_i = count_i / (k L)
    (2kiu.com digest section 5.5: the per-sequence allocation entropy is the quantity to
    watch before turning the sequence loss on). Terms with f_i = 0 contribute 0."""
    T, k = idx.shape
    assert T % seq_len == 0
    out = np.zeros(T // seq_len, dtype=np.float64)
    for q in range(T // seq_len):
        f = _seq_counts(idx[q * seq_len:(q + 1) * seq_len], n_experts) / (k * seq_len)
        nz = f[f > 0]
        out[q] = float(-np.sum(nz * np.log(nz)))
    return out


# ----------------------------------------------------------------------------------------
# Whole layer.
# ----------------------------------------------------------------------------------------
ExpertGetter = Callable[[int], tuple]  # e -> (w1q, w1s, w3q, w3s, w2q, w2s)


def layer_forward(x: np.ndarray, w_router: np.ndarray, bias: np.ndarray, cfg,
                  routed: ExpertGetter, shared: ExpertGetter,
                  force_idx: Optional[np.ndarray] = None, pow2: bool = False) -> dict:
    """Full MoE-layer forward for the tokens of x (float32 values).

    ``cfg`` supplies num_experts, num_shared_experts, num_experts_per_tok, n_group,
    topk_group, group_score_topn and routed_scaling_factor. ``routed``/``shared`` return
    the E4M3 codes and scales of one expert. Returns every intermediate and ``out``
    (float64) before the bf16 rounding of the output. ``pow2`` selects the power-of-two
    scale variant for x and h (the experts' codes come quantised already).
    """
    x = np.asarray(x, dtype=np.float32)
    T = x.shape[0]
    xq, xs = quantize_1x128_pow2(x) if pow2 else quantize_1x128(x)
    r = route(x, w_router, bias, cfg.num_experts_per_tok, cfg.n_group, cfg.topk_group,
              cfg.group_score_topn, cfg.routed_scaling_factor, force_idx=force_idx)
    offsets, row_token, row_of = permute(r["idx"], cfg.num_experts)
    H = x.shape[1]
    y_rows = np.zeros((row_token.shape[0], H), dtype=np.float64)
    for e in range(cfg.num_experts):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        toks = row_token[lo:hi]
        y, _, _, _ = expert_ffn(xq[toks], xs[toks], *routed(e), pow2=pow2)
        y_rows[lo:hi] = y
    y_shared = []
    for s in range(cfg.num_shared_experts):
        y, _, _, _ = expert_ffn(xq, xs, *shared(s), pow2=pow2)
        y_shared.append(y)
    out = combine(y_rows, row_of, r["gate"], y_shared)
    return {"xq": xq, "xs": xs, "route": r, "offsets": offsets, "row_token": row_token,
            "row_of": row_of, "y_rows": y_rows, "y_shared": y_shared, "out": out}
