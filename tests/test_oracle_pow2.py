"""Pins of the oracle's power-of-two scale variant (opt-in; CPU).

The variant keeps the 1x128 / 128x128 groups and gives each group the smallest power
of two s with amax / s <= 448. The pins below fix it by closed forms, by the special
case in which it coincides with the float32-scale quantiser, and by invariants.
"""
import numpy as np
import pytest

import oracle


def _tile(amax, n=128, seed=0):
    rng = np.random.default_rng(seed)
    t = rng.uniform(-1, 1, n).astype(np.float32) * np.float32(amax)
    t[7] = np.float32(amax)
    t = np.clip(t, -amax, amax).astype(np.float32)
    return t[None, :]


@pytest.mark.parametrize("k", [-20, -3, 0, 5, 30])
def test_scale_closed_forms(k):
    exact = np.float32(448.0 * 2.0 ** k)
    _, s = oracle.quantize_1x128_pow2(_tile(exact))
    assert s[0, 0] == np.float32(2.0 ** k)              # amax = 448 * 2^k -> 2^k
    above = np.nextafter(exact, np.float32(np.inf))
    _, s = oracle.quantize_1x128_pow2(_tile(above))
    assert s[0, 0] == np.float32(2.0 ** (k + 1))        # just above -> next power
    half = np.nextafter(np.float32(224.0 * 2.0 ** k), np.float32(np.inf))
    _, s = oracle.quantize_1x128_pow2(_tile(half))
    assert s[0, 0] == np.float32(2.0 ** k)              # (224, 448] * 2^k -> 2^k
    _, s = oracle.quantize_1x128_pow2(_tile(np.float32(224.0 * 2.0 ** k)))
    assert s[0, 0] == np.float32(2.0 ** (k - 1))        # 224 * 2^k = 448 * 2^(k-1)


def test_zero_group_and_floor():
    q, s = oracle.quantize_1x128_pow2(np.zeros((2, 256), np.float32))
    assert np.all(s == 1.0) and np.all(q == 0)
    tiny = np.full((1, 128), np.float32(1e-44), np.float32)   # subnormal input
    _, s = oracle.quantize_1x128_pow2(tiny)
    assert s[0, 0] == np.float32(2.0 ** -126)


def test_invariants_random():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 512)) * np.exp(rng.uniform(-8, 8, (64, 1)))).astype(np.float32)
    q, s = oracle.quantize_1x128_pow2(x)
    m, e = np.frexp(s.astype(np.float64))
    assert np.all(m == 0.5)                                # powers of two
    amax = np.abs(x.reshape(64, 4, 128)).max(axis=2)
    r = amax / s
    assert np.all(r <= 448.0) and np.all(r > 224.0)        # the smallest such power
    v = oracle.decode(q).reshape(64, 4, 128)
    xs = x.reshape(64, 4, 128).astype(np.float64) / s[:, :, None]
    # each code is the E4M3 rounding of the exact quotient: within half a step
    step = np.where(np.abs(xs) < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(xs), 1e-300))) - 3))
    assert np.all(np.abs(v - xs) <= step / 2 + 1e-12)


def test_coincides_with_fp32_scales_when_amax_is_448_times_power_of_two():
    rng = np.random.default_rng(9)
    rows = []
    for k in range(-6, 6):
        t = rng.uniform(-1, 1, 128).astype(np.float32) * np.float32(448.0 * 2.0 ** k)
        t[0] = np.float32(448.0 * 2.0 ** k)
        rows.append(t)
    x = np.stack(rows)
    assert np.array_equal(oracle.quantize_1x128_pow2(x)[0], oracle.quantize_1x128(x)[0])
    assert np.array_equal(oracle.quantize_1x128_pow2(x)[1], oracle.quantize_1x128(x)[1])
    w = np.zeros((128, 256), np.float32)
    w[:, :128] = rng.uniform(-1, 1, (128, 128)) * 448.0 * 0.25
    w[3, 5] = 112.0
    w[:, 128:] = rng.uniform(-1, 1, (128, 128)) * 448.0 * 8
    w[9, 200] = 448.0 * 8
    a, b = oracle.quantize_128x128_pow2(w), oracle.quantize_128x128(w)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_pow2_ffn_matches_dequantised_reference():
    """The variant's FFN: exact FP64 products of the dequantised operands, h re-quantised
    with power-of-two scales (checked here against a direct scalar evaluation)."""
    rng = np.random.default_rng(4)
    H, I, M = 256, 128, 5
    a = rng.standard_normal((M, H)).astype(np.float32)
    aq, a_s = oracle.quantize_1x128_pow2(a)
    ws = [oracle.quantize_128x128_pow2((rng.standard_normal(sh) / np.sqrt(sh[1])).astype(np.float32))
          for sh in ((I, H), (I, H), (H, I))]
    y, hq, hs, h = oracle.expert_ffn(aq, a_s, *ws[0], *ws[1], *ws[2], pow2=True)
    av = oracle.decode(aq) * np.repeat(a_s.astype(np.float64), 128, axis=1)
    wv = [oracle.decode(q) * np.kron(s.astype(np.float64), np.ones((128, 128))) for q, s in ws]
    g, u = av @ wv[0].T, av @ wv[1].T
    h_ref = (g / (1 + np.exp(-g)) * u).astype(np.float32)
    assert np.array_equal(h, h_ref)
    hq2, hs2 = oracle.quantize_1x128_pow2(h_ref)
    assert np.array_equal(hq, hq2) and np.array_equal(hs, hs2)
    y_ref = (oracle.decode(hq2) * np.repeat(hs2.astype(np.float64), 128, axis=1)) @ wv[2].T
    assert np.allclose(y, y_ref, rtol=1e-12, atol=1e-12)
