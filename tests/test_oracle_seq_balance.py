"""Pins of the oracle's sequence-wise balance statistic (CPU): closed forms and a
scalar-loop evaluation of the definition."""
import numpy as np

import oracle


def test_uniform_assignment_closed_form():
    N, k, L, c = 16, 4, 32, 0.3
    idx = np.array([[(t * k + j) % N for j in range(k)] for t in range(L)], np.int32)
    s = np.full((L, N), c)
    assert np.allclose(oracle.seq_balance_loss(s, idx, L, 0.001), [0.001 * c], rtol=1e-14)


def test_collapsed_assignment_closed_form():
    N, k, L, a, b = 32, 8, 10, 0.9, 0.1
    idx = np.tile(np.arange(k, dtype=np.int32), (L, 1))
    s = np.full((L, N), b)
    s[:, :k] = a
    # f = 1/k on the k chosen experts, P = a there: loss = alpha * a (N times the uniform
    # value a/N would give)
    assert np.allclose(oracle.seq_balance_loss(s, idx, L, 0.001), [0.001 * a], rtol=1e-14)


def test_matches_scalar_loops_and_splits_sequences():
    rng = np.random.default_rng(2)
    N, k, L, n = 12, 3, 7, 4
    s = rng.uniform(0, 1, (L * n, N))
    idx = np.stack([rng.choice(N, k, replace=False) for _ in range(L * n)]).astype(np.int32)
    got = oracle.seq_balance_loss(s, idx, L, 0.25)
    for q in range(n):
        tot = 0.0
        for i in range(N):
            cnt = sum(1 for t in range(q * L, (q + 1) * L) for j in range(k) if idx[t, j] == i)
            mean = sum(s[t, i] for t in range(q * L, (q + 1) * L)) / L
            tot += cnt / (k * L) * mean
        assert abs(got[q] - 0.25 * tot) <= 1e-15
    # one sequence over everything is the assignment-weighted mean of the per-sequence sums
    whole = oracle.seq_balance_loss(s, idx, L * n, 0.25)
    assert whole.shape == (1,)


def test_entropy_closed_forms():
    N, k, L = 16, 4, 32
    spread = np.array([[(t * k + j) % N for j in range(k)] for t in range(L)], np.int32)
    assert np.allclose(oracle.seq_assignment_entropy(spread, N, L), [np.log(N)], rtol=1e-14)
    collapsed = np.tile(np.arange(k, dtype=np.int32), (L, 1))
    assert np.allclose(oracle.seq_assignment_entropy(collapsed, N, L), [np.log(k)], rtol=1e-14)
    # two experts with shares 3/4 and 1/4 (k = 1)
    two = np.array([[0], [0], [0], [5]], np.int32)
    h = -(0.75 * np.log(0.75) + 0.25 * np.log(0.25))
    assert abs(oracle.seq_assignment_entropy(two, 8, 4)[0] - h) < 1e-15


def test_entropy_matches_scipy_and_loss_bounds():
    from scipy.stats import entropy
    rng = np.random.default_rng(9)
    N, k, L, n = 20, 4, 50, 3
    idx = np.stack([rng.choice(N, k, replace=False) for _ in range(L * n)]).astype(np.int32)
    s = rng.uniform(0, 1, (L * n, N))
    got = oracle.seq_assignment_entropy(idx, N, L)
    loss = oracle.seq_balance_loss(s, idx, L, 1.0)
    for q in range(n):
        cnt = np.bincount(idx[q * L:(q + 1) * L].ravel(), minlength=N)
        assert abs(got[q] - entropy(cnt)) < 1e-12
        # f sums to 1, so the loss is a convex combination of mean affinities
        p = s[q * L:(q + 1) * L].mean(axis=0)
        assert p.min() - 1e-15 <= loss[q] <= p.max() + 1e-15


def test_entries_naming_no_expert_count_for_none():
    # k = 2, L = 2: three valid entries on expert 1, one entry -1; f_1 = 3/4
    idx = np.array([[1, -1], [1, 1]], np.int32)
    s = np.zeros((2, 4))
    s[:, 1] = [0.2, 0.6]
    assert abs(oracle.seq_balance_loss(s, idx, 2, 1.0)[0] - 0.75 * 0.4) < 1e-15
    assert abs(oracle.seq_assignment_entropy(idx, 4, 2)[0] - (-0.75 * np.log(0.75))) < 1e-15
