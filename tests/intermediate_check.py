"""Check of the grouped FFN's quantised intermediate (hq, hs) against the oracle (helper).

The gate/up GEMMs give G and U with FP32 accumulation differences against the oracle's
exact FP64 sums (zhihu commentary, training part: per-chunk partial sums promoted to
FP32; the FP8 MFMA is not an exact 128-deep dot product), and h = silu(G) U is then
1x128-quantised (lpnh.cn guide section 3: every GEMM input 1x128 tile-wise). So hq and hs
are not bit-exact quantities. This module bounds, element by element, how far the GPU's
h can be from the oracle's:

  |dG| <= (EPS_CHUNK + (nkc + 1) * 2^-24) * sum_k |a_k w1_k|      (same for U with W3)
  |dh| <= 1.1 |dG| (|U| + |dU|) + (|silu(G)| + 1.1 |dG|) |dU| + 4e-6 |h|-bound

(1.1 bounds |silu'|; 4e-6 covers the hardware exp2/reciprocal and the FP32 roundings),
then the group scale s = amax / 448 moves by at most max|dh| / 448 plus two ulps, and a
GPU code must be the E4M3 code of some quotient in [q - dq, q + dq] around the oracle's
quotient q = h / s. EPS_CHUNK is the per-128-chunk error of the FP8 MFMA relative to
sum |a_k b_k|: a probe measured up to 2.9e-4; 2^-11 (4.9e-4) is used.
"""
from __future__ import annotations

import numpy as np

import oracle

EPS_CHUNK = 2.0 ** -11
U32 = 2.0 ** -24


def ordinal(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes -> integers that grow with the encoded value (+0 and -0 both 0)."""
    c = np.asarray(codes, dtype=np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def h_band(aq, a_s, w1q, w1s, w3q, w3s):
    """Oracle h (float32, as expert_ffn rounds it) and the bound on |h_gpu - h| per element."""
    a = oracle.dequant_1x128(aq, a_s)
    w1 = oracle.dequant_128x128(w1q, w1s)
    w3 = oracle.dequant_128x128(w3q, w3s)
    g, u = a @ w1.T, a @ w3.T
    aa = np.abs(a)
    nkc = aq.shape[1] // 128
    k = EPS_CHUNK + (nkc + 1) * U32
    dg = k * (aa @ np.abs(w1).T)
    du = k * (aa @ np.abs(w3).T)
    sg = np.abs(oracle.silu(g))
    dh = 1.1 * dg * (np.abs(u) + du) + (sg + 1.1 * dg) * du
    dh += 4e-6 * (sg + 1.1 * dg) * (np.abs(u) + du)
    h = (oracle.silu(g) * u).astype(np.float32)
    return h, dh


def check_intermediate(hq_gpu, hs_gpu, h, dh):
    """hq_gpu [M, I] codes, hs_gpu [M, I/128] scales; h, dh from h_band. Returns a dict of
    statistics; raises AssertionError where a scale or a code leaves its band."""
    M, I = h.shape
    rq, rs = oracle.quantize_1x128(h)
    dmax = dh.reshape(M, I // 128, 128).max(axis=2)
    ds = dmax / 448.0 + 2 * np.spacing(rs.astype(np.float32)).astype(np.float64)
    hs_gpu = np.asarray(hs_gpu, np.float64)
    rs64 = rs.astype(np.float64)
    bad_s = np.abs(hs_gpu - rs64) > ds
    assert not bad_s.any(), f"scales outside their band at (row, group) {np.argwhere(bad_s)[:5].tolist()}"
    s = np.repeat(rs64, 128, axis=1).reshape(M, I)
    dsr = np.repeat(ds, 128, axis=1).reshape(M, I)
    q = h.astype(np.float64) / s
    dq = (dh + np.abs(h) * dsr / s) / (s - dsr) + 4 * U32 * np.abs(q)
    lo = oracle.encode(np.nextafter((q - dq).astype(np.float32), np.float32(-np.inf)))
    hi = oracle.encode(np.nextafter((q + dq).astype(np.float32), np.float32(np.inf)))
    og = ordinal(hq_gpu)
    bad = (og < ordinal(lo)) | (og > ordinal(hi))
    assert not bad.any(), f"codes outside their band at {np.argwhere(bad)[:5].tolist()}"
    diff = og != ordinal(rq)
    return {"codes": int(h.size), "code_flips": int(diff.sum()),
            "flip_rate": float(diff.mean()),
            "max_step": int(np.abs(og - ordinal(rq)).max()),
            "hs_max_rel": float(np.max(np.abs(hs_gpu - rs64) / rs64)),
            "hs_exact": float(np.mean(hs_gpu == rs64))}
