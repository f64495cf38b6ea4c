"""The routing-validity helper used by the GPU parity tests: the oracle's own choice
passes; near-tie swaps inside the band pass; planted mistakes (a worse expert, an expert
from a dropped group, a duplicate, a wrong slot order, a changed set on a clear token)
each break the rule that names them."""
import dataclasses

import numpy as np

import oracle
import synth
from routing_check import NEAR_TIE, routing_violations


def _case(n_group=8, topk_group=4, seed=0, T=200):
    cfg = dataclasses.replace(synth.PRESETS["tiny"], num_experts=64, num_experts_per_tok=6,
                              n_group=n_group, topk_group=topk_group, group_score_topn=2, tokens=T)
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, cfg.hidden_size)).astype(np.float32)
    wr = (rng.standard_normal((64, cfg.hidden_size)) / 16).astype(np.float32)
    b = rng.uniform(-0.05, 0.05, 64).astype(np.float32)
    r = oracle.route(x, wr, b, 6, n_group, topk_group, 2, 2.5)
    return cfg, r


def _broken(bad):
    return {k for k, v in bad.items() if len(v)}


def test_oracle_choice_is_valid():
    for g, gk in ((1, 1), (8, 4), (8, 8)):
        cfg, r = _case(g, gk)
        assert not _broken(routing_violations(r, r["idx"], cfg))


def test_planted_mistakes_are_caught():
    cfg, r = _case()
    score, idx = r["score"], r["idx"].astype(np.int64)
    t = int(np.argmax((r["kth_gap"] > 1e-3) & (r["group_gap"] > 1e-3)))   # a clear token
    gsz = 64 // 8
    # a worse expert inside a kept group replaces the last choice
    g = idx.copy()
    kept = {int(e) // gsz for e in idx[t]}
    worse = [e for e in range(64) if e // gsz in kept and e not in idx[t]
             and score[t, e] < score[t, idx[t, -1]] - 1e-3]
    g[t, -1] = worse[0]
    assert {"skipped_better_expert", "set_differs_without_tie"} <= _broken(routing_violations(r, g, cfg))
    # an expert of a dropped group
    gs = np.sort(score[t].reshape(8, gsz), axis=1)[:, -2:].sum(1)
    dropped = int(np.argsort(gs)[0])
    g = idx.copy()
    g[t, -1] = dropped * gsz
    assert "group_outside_band" in _broken(routing_violations(r, g, cfg))
    # a duplicate
    g = idx.copy()
    g[t, 1] = g[t, 0]
    assert "range_or_duplicate" in _broken(routing_violations(r, g, cfg))
    # reversed slots (scores differ by more than the band)
    g = idx.copy()
    g[t] = g[t, ::-1]
    assert _broken(routing_violations(r, g, cfg)) == {"slot_order"}


def test_swaps_inside_the_band_are_accepted():
    cfg, r = _case(n_group=1, topk_group=1, seed=3)
    score = r["score"].copy()
    idx = r["idx"].astype(np.int64)
    t = 5
    # make the k-th and (k+1)-th scores a near-tie and pick the other one
    order = np.argsort(-score[t], kind="stable")
    a, b = order[5], order[6]
    score[t, b] = score[t, a] - NEAR_TIE / 4
    r2 = dict(r, score=score)
    r2["kth_gap"] = r["kth_gap"].copy()
    r2["kth_gap"][t] = NEAR_TIE / 4
    g = idx.copy()
    g[t, 5] = b
    assert not _broken(routing_violations(r2, g, cfg))
    # the same swap on a token without a declared tie is a mistake
    r2["kth_gap"][t] = 1.0
    assert "set_differs_without_tie" in _broken(routing_violations(r2, g, cfg))
