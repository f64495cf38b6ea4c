"""Validity of a GPU routing choice against the oracle's FP64 scores (test helper).

The method selects top-k experts by biased affinity, inside the G_k best groups (2kiu.com
digest section 3.2 pseudocode, section 3.4 group limit). The GPU ranks in FP32 and the
oracle in FP64, so where two oracle scores lie within NEAR_TIE of each other either order
is correct (a declared near-tie). This module checks a GPU selection against that rule
and nothing looser:

* every token: k distinct experts in [0, N_r); every selected expert's group is one the
  oracle could keep (its group score is at least the G_k-th best minus the band); no
  expert of a group the oracle surely keeps, left out, beats a selected one by more than
  the band; and the slots are in descending oracle score wherever two scores differ by
  more than the band;
* tokens without a declared near-tie: the selected set equals the oracle's exactly.
"""
from __future__ import annotations

import numpy as np

NEAR_TIE = 1e-6


def group_scores(score: np.ndarray, n_group: int, topn: int) -> np.ndarray:
    """Oracle group scores: the sum of each group's ``topn`` best biased affinities."""
    T, N = score.shape
    g = np.sort(score.reshape(T, n_group, N // n_group), axis=2)
    return g[:, :, -topn:].sum(axis=2)


def routing_violations(r: dict, g_idx: np.ndarray, cfg, band: float = NEAR_TIE) -> dict:
    """``r`` is ``oracle.route(...)`` on the same inputs, ``g_idx`` the GPU's [T, k] choice.
    Returns {rule name: token indices that break it}; every list is empty for a valid
    choice."""
    score = np.asarray(r["score"], dtype=np.float64)
    T, N = score.shape
    k = g_idx.shape[1]
    g_idx = np.asarray(g_idx, dtype=np.int64)
    bad = {}
    in_range = np.all((g_idx >= 0) & (g_idx < N), axis=1)
    srt = np.sort(g_idx, axis=1)
    distinct = np.all(srt[:, 1:] != srt[:, :-1], axis=1) if k > 1 else np.ones(T, bool)
    bad["range_or_duplicate"] = np.nonzero(~(in_range & distinct))[0]
    gi = np.clip(g_idx, 0, N - 1)
    sel = np.take_along_axis(score, gi, axis=1)

    # groups: which ones the oracle may keep, which it surely keeps
    G = cfg.n_group
    if G > 1:
        gsz = N // G
        gs = group_scores(score, G, cfg.group_score_topn)
        gsort = -np.sort(-gs, axis=1)
        gk = gsort[:, cfg.topk_group - 1]                        # G_k-th best
        gnext = gsort[:, cfg.topk_group] if cfg.topk_group < G else np.full(T, -np.inf)
        may_keep = gs >= (gk - band)[:, None]
        sure_keep = gs > (gnext + band)[:, None]
        sel_group_ok = np.take_along_axis(may_keep, gi // gsz, axis=1).all(axis=1)
        bad["group_outside_band"] = np.nonzero(~sel_group_ok)[0]
        sure_expert = np.repeat(sure_keep, gsz, axis=1)
    else:
        sure_expert = np.ones((T, N), bool)

    # no surely-allowed expert left out beats a selected one by more than the band
    chosen = np.zeros((T, N), bool)
    np.put_along_axis(chosen, gi, True, axis=1)
    left = np.where(sure_expert & ~chosen, score, -np.inf).max(axis=1)
    bad["skipped_better_expert"] = np.nonzero(left > sel.min(axis=1) + band)[0]

    # slot order: descending oracle score except within the band
    if k > 1:
        later_higher = np.zeros(T, bool)
        for j in range(k - 1):
            later_higher |= (sel[:, j + 1:] > sel[:, j:j + 1] + band).any(axis=1)
        bad["slot_order"] = np.nonzero(later_higher)[0]

    # tokens without a declared near-tie: the same set as the oracle
    tie = (r["kth_gap"] < band) | (r["group_gap"] < band)
    same = np.all(np.sort(g_idx, 1) == np.sort(np.asarray(r["idx"], np.int64), 1), axis=1)
    bad["set_differs_without_tie"] = np.nonzero(~same & ~tie)[0]
    return bad


def assert_routing_valid(r: dict, g_idx: np.ndarray, cfg, band: float = NEAR_TIE) -> int:
    """Raises AssertionError naming the rule and the first tokens that break it; returns
    the number of declared near-tie tokens."""
    bad = routing_violations(r, g_idx, cfg, band)
    for rule, toks in bad.items():
        assert len(toks) == 0, f"routing rule '{rule}' broken at tokens {toks[:10].tolist()}"
    tie = (r["kth_gap"] < band) | (r["group_gap"] < band)
    return int(tie.sum())
