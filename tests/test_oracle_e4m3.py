"""Pins of the oracle's E4M3 codec against the format definition and torch's cast."""
import os

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_ocp_points.txt")


def _torch_encode(v: np.ndarray) -> np.ndarray:
    """Library routine: torch's float32 -> float8_e4m3fn cast, after clamping to +-448."""
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    t = torch.clamp(t, -448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_matches_ocp_points():
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        code, val = line.split()
        got = e4m3.decode(np.array([int(code, 16)], dtype=np.uint8))[0]
        if val == "nan":
            assert np.isnan(got), code
        else:
            assert got == float(val) and np.signbit(got) == val.startswith("-"), (code, got, val)


def test_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = e4m3.decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))
    assert e4m3.finite_values().max() == 448.0 and len(e4m3.finite_values()) == 127


def _boundary_sweep() -> np.ndarray:
    """Every E4M3 value and midpoint, +-16 float32 ulps around each, both signs."""
    pos = e4m3.finite_values()
    mids = (pos[:-1] + pos[1:]) / 2
    pts = np.concatenate([pos, mids, [448.0, 464.0, 480.0, 500.0, 1e4, 3e38]]).astype(np.float32)
    bits = pts.view(np.uint32)
    offs = np.arange(-16, 17, dtype=np.int64)
    allb = (bits[:, None].astype(np.int64) + offs[None, :]).reshape(-1)
    allb = allb[(allb >= 0) & (allb < 0x7F800000)].astype(np.uint32)
    v = allb.view(np.float32)
    return np.concatenate([v, -v])


def test_encode_matches_torch_on_boundaries():
    v = _boundary_sweep()
    assert np.array_equal(e4m3.encode(v), _torch_encode(v))


def test_encode_matches_torch_on_strided_bit_patterns():
    # every 65537th float32 bit pattern (all exponents, both signs), NaNs excluded
    b = np.arange(0, 1 << 32, 65537, dtype=np.uint64).astype(np.uint32)
    v = b.view(np.float32)
    v = v[~np.isnan(v)]
    assert np.array_equal(e4m3.encode(v), _torch_encode(v))


def test_encode_random_within_half_ulp():
    rng = np.random.default_rng(5)
    v = (rng.standard_normal(200000) * np.exp2(rng.integers(-14, 9, 200000))).astype(np.float32)
    v = np.clip(v, -448, 448)
    back = e4m3.decode(e4m3.encode(v))
    a = np.abs(v.astype(np.float64))
    # spacing of E4M3 at |v|: 2^(e-3) for normals (e = floor(log2|v|) >= -6), 2^-9 below
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    half_ulp = np.exp2(e - 3) / 2
    assert np.all(np.abs(back - v) <= half_ulp)


def test_encode_special_cases():
    enc = lambda x: int(e4m3.encode(np.array([x], dtype=np.float32))[0])
    assert enc(448.0) == 0x7E and enc(-448.0) == 0xFE
    assert enc(449.0) == 0x7E and enc(463.9) == 0x7E and enc(464.0) == 0x7E and enc(1e30) == 0x7E
    assert enc(float("inf")) == 0x7E and enc(float("-inf")) == 0xFE
    assert enc(0.0) == 0x00 and enc(-0.0) == 0x80 and enc(-1e-10) == 0x80
    assert enc(float("nan")) & 0x7F == 0x7F
    # ties to even: 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39)
    assert enc(1.0625) == 0x38 and enc(1.1875) == 0x3A
    # subnormal ties: 2^-10 halfway between 0 and 2^-9 -> 0 (even); 3*2^-10 -> 2*2^-9 (0x02)
    assert enc(2.0 ** -10) == 0x00 and enc(3 * 2.0 ** -10) == 0x02


@pytest.mark.slow
def test_encode_matches_torch_dense_normal_range():
    # all float32 bit patterns with exponent field in [110, 136) (|x| ~ 2^-17 .. 2^9),
    # sampled every 61st pattern: ~3.4M values covering every rounding position
    lo, hi = 110 << 23, 136 << 23
    b = np.arange(lo, hi, 61, dtype=np.uint32)
    v = b.view(np.float32)
    v = np.concatenate([v, -v])
    assert np.array_equal(e4m3.encode(v), _torch_encode(v))
