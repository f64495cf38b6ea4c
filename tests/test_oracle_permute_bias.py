"""Pins of the oracle's permutation and bias update (invariants and closed forms)."""
import numpy as np

import oracle


def _random_idx(rng, T, N, k):
    return np.stack([rng.permutation(N)[:k] for _ in range(T)]).astype(np.int32)


def test_permutation_is_bijection_and_stable():
    rng = np.random.default_rng(20)
    T, N, k = 300, 16, 4
    idx = _random_idx(rng, T, N, k)
    offsets, row_token, row_of = oracle.permute(idx, N)
    assert offsets[0] == 0 and offsets[-1] == T * k and np.all(np.diff(offsets) >= 0)
    assert np.array_equal(np.diff(offsets), np.bincount(idx.ravel(), minlength=N))
    assert np.array_equal(np.sort(row_of.ravel()), np.arange(T * k))
    assert np.all(row_token[row_of] == np.arange(T)[:, None])
    for e in range(N):
        seg = row_token[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)
        # row r of expert e holds a token that selected e
        assert all(e in idx[t] for t in seg)


def test_forced_collapse_closed_form():
    T, N, k = 50, 8, 3
    idx = np.tile(np.array([6, 1, 3], np.int32), (T, 1))
    offsets, row_token, row_of = oracle.permute(idx, N)
    counts = np.diff(offsets)
    assert list(counts) == [0, T, 0, T, 0, 0, T, 0]
    assert np.array_equal(row_of[:, 1], np.arange(T))           # expert 1 first
    assert np.array_equal(row_of[:, 2], T + np.arange(T))       # then expert 3
    assert np.array_equal(row_of[:, 0], 2 * T + np.arange(T))   # then expert 6


def test_bias_update_closed_form():
    T, k, N = 100, 4, 8           # target load T*k/N = 50
    counts = np.array([50, 51, 49, 0, 400, 50, 0, 0])
    b = np.array([0, 0.5, -0.5, 1e-3, 0, 7, -7, 1e-9], np.float32)
    nb = oracle.bias_update(b, counts, T, k, 0.001)
    g = np.float32(0.001)
    want = np.array([b[0], b[1] - g, b[2] + g, b[3] + g, b[4] - g, b[5], b[6] + g, b[7] + g],
                    np.float32)
    assert nb.dtype == np.float32 and np.array_equal(nb, want)
    # each step moves a bias by exactly +-fl32(gamma) or 0 when that is exact
    b0 = np.zeros(8, np.float32)
    d = oracle.bias_update(b0, counts, T, k, 0.001) - b0
    assert set(np.abs(d).tolist()) <= {0.0, float(g)}


def test_bias_update_integer_compare_at_fractional_target():
    # T*k/N = 10*3/4 = 7.5: load 7 is under, load 8 is over, never "equal"
    nb = oracle.bias_update(np.zeros(4, np.float32), np.array([7, 8, 7, 8]), 10, 3, 0.25)
    assert list(nb) == [0.25, -0.25, 0.25, -0.25]


def test_bias_trajectory_resume_is_bitwise_equal():
    rng = np.random.default_rng(21)
    N, T, k = 16, 64, 4
    loads = [np.bincount(_random_idx(rng, T, N, k).ravel(), minlength=N) for _ in range(10)]
    b = np.zeros(N, np.float32)
    traj = []
    for c in loads:
        b = oracle.bias_update(b, c, T, k, 0.001)
        traj.append(b.copy())
    saved = traj[4].copy()
    b2 = saved
    for c in loads[5:]:
        b2 = oracle.bias_update(b2, c, T, k, 0.001)
    assert np.array_equal(b2.view(np.uint32), traj[-1].view(np.uint32))
