"""Pins of the oracle router: brute force, library top-k, closed forms, invariants."""
import itertools

import numpy as np
import torch

import oracle


def _brute_route(score, k, n_group=1, topk_group=1, topn=2):
    """Exhaustive search: the kept groups maximise the summed group score, the chosen
    experts maximise the summed ranking score (inputs drawn without ties)."""
    N = score.shape[0]
    allowed = list(range(N))
    if n_group > 1:
        gsz = N // n_group
        gscore = []
        for g in range(n_group):
            members = score[g * gsz:(g + 1) * gsz]
            gscore.append(max(sum(c) for c in itertools.combinations(members, topn)))
        best = max(itertools.combinations(range(n_group), topk_group),
                   key=lambda gs: sum(gscore[g] for g in gs))
        allowed = [e for e in range(N) if e // gsz in best]
    chosen = max(itertools.combinations(allowed, k), key=lambda es: sum(score[e] for e in es))
    return sorted(chosen, key=lambda e: -score[e])


def test_bruteforce_plain_topk():
    rng = np.random.default_rng(10)
    T, H, N, k = 20, 128, 9, 3
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (rng.standard_normal((N, H)) / np.sqrt(H)).astype(np.float32)
    b = rng.uniform(-0.05, 0.05, N).astype(np.float32)
    r = oracle.route(x, wr, b, k)
    for t in range(T):
        assert list(r["idx"][t]) == _brute_route(r["score"][t], k)


def test_bruteforce_group_limited():
    rng = np.random.default_rng(11)
    T, H, N, k, G, Gk = 24, 128, 12, 3, 4, 2
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (rng.standard_normal((N, H)) / np.sqrt(H)).astype(np.float32)
    b = rng.uniform(-0.1, 0.1, N).astype(np.float32)
    r = oracle.route(x, wr, b, k, n_group=G, topk_group=Gk, group_topn=2)
    for t in range(T):
        assert list(r["idx"][t]) == _brute_route(r["score"][t], k, G, Gk, 2)
    # the limit actually binds for some token (otherwise this test pins nothing)
    free = oracle.route(x, wr, b, k)
    assert np.any(free["idx"] != r["idx"])


def test_unbiased_ungrouped_equals_torch_topk_of_logits():
    rng = np.random.default_rng(12)
    T, H, N, k = 50, 256, 32, 6
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (rng.standard_normal((N, H)) / np.sqrt(H)).astype(np.float32)
    r = oracle.route(x, wr, np.zeros(N, np.float32), k)
    logits = torch.from_numpy(x.astype(np.float64)) @ torch.from_numpy(wr.astype(np.float64)).T
    ref = torch.topk(logits, k, dim=1).indices.numpy()
    assert np.array_equal(r["idx"], ref)


def test_all_groups_kept_reduces_to_plain():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((40, 128)).astype(np.float32)
    wr = (rng.standard_normal((16, 128)) / np.sqrt(128)).astype(np.float32)
    b = rng.uniform(-0.01, 0.01, 16).astype(np.float32)
    a = oracle.route(x, wr, b, 4, n_group=4, topk_group=4)
    p = oracle.route(x, wr, b, 4)
    assert np.array_equal(a["idx"], p["idx"])


def test_k_equals_n_selects_all():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((10, 128)).astype(np.float32)
    wr = rng.standard_normal((8, 128)).astype(np.float32)
    r = oracle.route(x, wr, np.zeros(8, np.float32), 8)
    assert np.all(r["counts"] == 10)
    assert np.allclose(r["gate"].sum(1), 2.5)


def test_gate_invariants():
    rng = np.random.default_rng(15)
    T, H, N, k = 64, 256, 16, 4
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (rng.standard_normal((N, H)) / np.sqrt(H)).astype(np.float32)
    b = rng.uniform(-0.2, 0.2, N).astype(np.float32)
    r = oracle.route(x, wr, b, k, routed_scaling_factor=2.5)
    assert np.allclose(r["gate"].sum(1), 2.5, rtol=0, atol=1e-12)
    assert np.all(r["gate"] > 0)
    assert r["counts"].sum() == T * k
    # gates come from the unbiased affinities: closed form s_sel / sum * rho
    s = 1 / (1 + np.exp(-(x.astype(np.float64) @ wr.astype(np.float64).T)))
    sel = np.take_along_axis(s, r["idx"].astype(np.int64), 1)
    assert np.allclose(r["gate"], sel / sel.sum(1, keepdims=True) * 2.5, rtol=1e-14)
    r1 = oracle.route(x, wr, b, 1)
    assert np.all(r1["gate"] == 2.5)


def test_bias_changes_selection_not_gate_formula():
    rng = np.random.default_rng(16)
    T, H, N, k = 32, 128, 8, 2
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (rng.standard_normal((N, H)) / np.sqrt(H)).astype(np.float32)
    b = np.zeros(N, np.float32)
    b[5] = 10.0   # expert 5 always ranks first
    r = oracle.route(x, wr, b, k)
    assert np.all(r["idx"][:, 0] == 5)
    s = r["s"]
    other = r["idx"][:, 1]
    g5 = s[:, 5] / (s[:, 5] + s[np.arange(T), other]) * 2.5
    assert np.allclose(r["gate"][:, 0], g5, rtol=1e-14)


def test_ties_go_to_lower_index():
    x = np.ones((3, 128), np.float32)
    wr = np.tile(np.linspace(-1, 1, 128, dtype=np.float32), (8, 1)) * np.float32(0.01)
    r = oracle.route(x, wr, np.zeros(8, np.float32), 3)
    assert np.all(r["idx"] == [0, 1, 2])
    r = oracle.route(x, wr, np.zeros(8, np.float32), 2, n_group=4, topk_group=2)
    assert np.all(r["idx"] == [0, 1])
