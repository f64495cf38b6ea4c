"""Pins of the oracle's 1x128 / 128x128 quantisers (closed forms and invariants)."""
import numpy as np

import oracle
from oracle import e4m3


def test_power_of_two_tile_closed_form():
    # amax = 56 -> s = 56/448 = 0.125 exactly, so x/s = 8x exactly
    x = np.zeros((1, 128), dtype=np.float32)
    x[0, 0] = 56.0     # -> 448 -> 0x7E
    x[0, 1] = -1.0     # -> -8 = 2^3 -> exp field 10 -> 0xD0
    x[0, 2] = 0.001    # -> 0.008 -> subnormal 4.096 * 2^-9 -> 4 -> 0x04
    x[0, 3] = 1.5      # -> 12 = 1.5*2^3 -> 0x54
    x[0, 4] = 0.0
    q, s = oracle.quantize_1x128(x)
    assert s.dtype == np.float32 and s.shape == (1, 1) and s[0, 0] == np.float32(0.125)
    assert list(q[0, :5]) == [0x7E, 0xD0, 0x04, 0x54, 0x00]


def test_amax_element_encodes_to_448():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((37, 512)).astype(np.float32) * np.float32(3.0)
    q, s = oracle.quantize_1x128(x)
    xt = x.reshape(37, 4, 128)
    am = np.argmax(np.abs(xt), axis=2)
    codes = np.take_along_axis(q.reshape(37, 4, 128), am[:, :, None], axis=2)[:, :, 0]
    signs = np.take_along_axis(xt, am[:, :, None], axis=2)[:, :, 0] < 0
    assert np.all(codes == np.where(signs, 0xFE, 0x7E))


def test_zero_tile_scale_one():
    x = np.zeros((2, 256), dtype=np.float32)
    x[1, 130] = 3.0
    q, s = oracle.quantize_1x128(x)
    assert s[0, 0] == 1.0 and s[0, 1] == 1.0 and s[1, 0] == 1.0
    assert s[1, 1] == np.float32(3.0) / np.float32(448.0)
    assert np.all(q[0] == 0) and np.all(q[1, :128] == 0)


def test_scale_is_rounded_quotient():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((64, 1024)) * np.exp2(rng.integers(-20, 20, (64, 1)))).astype(np.float32)
    _, s = oracle.quantize_1x128(x)
    amax = np.abs(x.reshape(64, 8, 128)).max(axis=2).astype(np.float64)
    exact = amax / 448.0
    # s is a float32 within half an ulp of amax/448
    ulp = np.spacing(s.astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(s.astype(np.float64) - exact) <= ulp / 2)


def test_outlier_isolation():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 512)).astype(np.float32)
    q0, s0 = oracle.quantize_1x128(x)
    x2 = x.copy()
    x2[2, 300] = 1e4
    q1, s1 = oracle.quantize_1x128(x2)
    diff_s = s0 != s1
    assert diff_s.sum() == 1 and diff_s[2, 2]
    diff_q = (q0 != q1).reshape(4, 4, 128).any(axis=2)
    assert np.array_equal(diff_q, diff_s)


def test_dequant_error_bound():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((16, 768)) * np.float32(0.7)).astype(np.float32)
    q, s = oracle.quantize_1x128(x)
    dq = oracle.dequant_1x128(q, s)
    sr = np.repeat(s.astype(np.float64), 128, axis=1)
    qv = np.abs(x / sr)
    e = np.floor(np.log2(np.maximum(qv, 2.0 ** -6)))
    bound = (np.exp2(e - 3) / 2) * sr * (1 + 2.0 ** -22) + np.abs(x) * 2.0 ** -23
    assert np.all(np.abs(dq - x) <= bound)


def test_128x128_blocks_independent_and_closed_form():
    rng = np.random.default_rng(5)
    w = rng.standard_normal((256, 384)).astype(np.float32)
    q, s = oracle.quantize_128x128(w)
    assert s.shape == (2, 3)
    blocks = np.abs(w.reshape(2, 128, 3, 128)).max(axis=(1, 3))
    assert np.array_equal(s, (blocks / np.float32(448)).astype(np.float32))
    # each block's max element hits +-448
    for i in range(2):
        for j in range(3):
            b = w[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            r, c = np.unravel_index(np.argmax(np.abs(b)), b.shape)
            assert q[i * 128 + r, j * 128 + c] in (0x7E, 0xFE)
    w2 = w.copy()
    w2[200, 10] = 100.0
    q2, s2 = oracle.quantize_128x128(w2)
    changed = s2 != s
    assert changed.sum() == 1 and changed[1, 0]
    # a block that is a power-of-two multiple of E4M3 values is reproduced exactly
    vals = e4m3.decode(rng.integers(0, 126, (128, 128)).astype(np.uint8)) * 0.25
    vals[0, 0] = 448 * 0.25
    qb, sb = oracle.quantize_128x128(vals.astype(np.float32))
    assert sb[0, 0] == 0.25 and np.array_equal(oracle.dequant_128x128(qb, sb), vals)
