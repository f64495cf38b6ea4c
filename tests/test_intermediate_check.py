"""The intermediate-check helper used by the GPU parity tests: the oracle's own (hq, hs)
pass; an h perturbed inside the stated accumulation bound and quantised with the
reference rule passes; planted mistakes fail (a code two steps off, a scale 1% off, the
gate and up projections swapped)."""
import numpy as np
import pytest

import oracle
from intermediate_check import EPS_CHUNK, check_intermediate, h_band


def _expert(seed=0, M=40, H=384, I=256):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, H)).astype(np.float32)
    aq, a_s = oracle.quantize_1x128(x)
    w = [oracle.quantize_128x128((rng.standard_normal((I, H)) / np.sqrt(H)).astype(np.float32))
         for _ in range(2)]
    return aq, a_s, w[0][0], w[0][1], w[1][0], w[1][1]


def test_oracle_intermediate_passes():
    e = _expert()
    h, dh = h_band(*e)
    hq, hs = oracle.quantize_1x128(h)
    st = check_intermediate(hq, hs, h, dh)
    assert st["code_flips"] == 0 and st["hs_exact"] == 1.0


def test_perturbed_inside_the_bound_passes():
    aq, a_s, w1q, w1s, w3q, w3s = _expert(1)
    a = oracle.dequant_1x128(aq, a_s)
    w1, w3 = oracle.dequant_128x128(w1q, w1s), oracle.dequant_128x128(w3q, w3s)
    rng = np.random.default_rng(2)
    g = a @ w1.T
    u = a @ w3.T
    dg = EPS_CHUNK * (np.abs(a) @ np.abs(w1).T)
    du = EPS_CHUNK * (np.abs(a) @ np.abs(w3).T)
    gp = g + rng.uniform(-0.9, 0.9, g.shape) * dg
    up = u + rng.uniform(-0.9, 0.9, u.shape) * du
    hp = (oracle.silu(gp) * up).astype(np.float32)
    hq, hs = oracle.quantize_1x128(hp)
    h, dh = h_band(aq, a_s, w1q, w1s, w3q, w3s)
    st = check_intermediate(hq, hs, h, dh)
    assert st["code_flips"] > 0   # the perturbation does flip codes, all inside the band


def test_planted_mistakes_fail():
    e = _expert(3)
    h, dh = h_band(*e)
    hq, hs = oracle.quantize_1x128(h)
    bad = hq.copy()
    i = np.unravel_index(np.argmax(np.abs(h)), h.shape)
    bad[i] = bad[i] - 2 if bad[i] & 0x7F >= 2 else bad[i] + 2
    with pytest.raises(AssertionError):
        check_intermediate(bad, hs, h, dh)
    bs = hs.copy()
    bs[3, 1] *= np.float32(1.01)
    with pytest.raises(AssertionError):
        check_intermediate(hq, bs, h, dh)
    aq, a_s, w1q, w1s, w3q, w3s = e
    hw, _ = h_band(aq, a_s, w3q, w3s, w1q, w1s)   # silu applied to the up projection
    sq, ss = oracle.quantize_1x128(hw)
    with pytest.raises(AssertionError):
        check_intermediate(sq, ss, h, dh)
