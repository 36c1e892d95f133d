"""Pins for the oracle's selection: a fixed budget of important tokens filled
greedily from the predicted scores with neighbour fetching, on top of the
always-kept sink and circular local window (TokenButler summary, "Inference
strategy" and its "Optimizations"; "Core architecture": selection under a
fixed budget).

The oracle implements the greedy fill loop. These tests pin it with: a
hand-worked golden case; an independent ranking formulation (each eligible
token ranked by its best candidate within distance r) on exhaustive tiny
tie-heavy inputs; a textbook full sort at r = 0; closed forms (isolated
centres, all-equal scores, +0 above -0); and the invariants the pages fix
(sink and window always kept, budget respected, full budget gives dense,
zero budget gives sink + window)."""
import json
import os
import struct

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def total_order_key(x):
    b = struct.unpack("<I", struct.pack("<f", float(x)))[0]
    return b ^ (0xFFFFFFFF if b >> 31 else 0x80000000)


def ranking_select(s, L, P, S, W, K, r):
    """Independent formulation: rank each eligible t by (best candidate c(t)
    within distance r, then c, then |t - c|, then t)."""
    e0, e1 = S, max(S, min(L - W, P))
    E = list(range(e0, e1))
    if not E:
        return set()
    key = {t: total_order_key(s[t]) for t in E}

    def best(t):
        nb = range(max(e0, t - r), min(e1 - 1, t + r) + 1)
        return min(nb, key=lambda u: (-key[u], u))

    ranked = sorted(E, key=lambda t: (-key[best(t)], best(t), abs(t - best(t)), t))
    return set(ranked[:min(K, len(E))])


def attended(idx, cnt, b=0, h=0):
    return [int(t) for t in idx[b, h, :cnt[b, h]]]


def run1(orc, s, L, P, S, W, K, r, Lmax=None):
    Lmax = Lmax or len(s)
    sc = np.full((1, 1, Lmax), np.nan, np.float32)
    sc[0, 0, :len(s)] = s
    idx, cnt = orc.select(sc, np.array([L], np.int32), np.array([P], np.int32),
                          S, W, K, r, cap=Lmax)
    return attended(idx, cnt)


def test_golden_hand_cases(orc):
    g = json.load(open(os.path.join(HERE, "golden", "select_hand.json")))
    for c in g["cases"]:
        got = run1(orc, np.array(g["scores"], np.float32), g["L"], g["P"], g["S"],
                   g["W"], c["K"], c["r"])
        assert got == c["attended"], c


def test_brute_force_vs_ranking_tie_heavy(orc):
    rng = np.random.default_rng(11)
    n = 0
    for L in range(1, 22):
        for trial in range(12):
            S = int(rng.integers(0, 4))
            W = int(rng.integers(0, 5))
            P = int(rng.integers(max(0, L - 6), L + 1))
            K = int(rng.integers(0, L + 2))
            r = int(rng.integers(0, 4))
            s = rng.integers(-2, 3, size=L).astype(np.float32)
            s[rng.random(L) < 0.2] = -0.0
            got = set(run1(orc, s, L, P, S, W, K, r))
            sink = set(range(min(S, L)))
            win = set(range(max(0, L - W), L))
            expect = ranking_select(s, L, P, S, W, K, r) | sink | win
            assert got == expect, (L, S, W, P, K, r, s.tolist())
            n += 1
    assert n > 200


def test_radius0_equals_full_sort(orc):
    rng = np.random.default_rng(12)
    for trial in range(50):
        L = int(rng.integers(30, 200))
        S, W = int(rng.integers(0, 8)), int(rng.integers(0, 20))
        K = int(rng.integers(0, L))
        s = rng.standard_normal(L).astype(np.float32)
        s[rng.random(L) < 0.3] = 1.0                      # many exact ties
        e0, e1 = S, max(S, L - W)
        E = np.arange(e0, e1)
        order = E[np.lexsort((E, -s[e0:e1]))]             # score desc, position asc
        expect = set(order[:K].tolist()) | set(range(min(S, L))) | set(range(max(0, L - W), L))
        got = run1(orc, s, L, L, S, W, K, 0)
        assert set(got) == expect
        assert got == sorted(got)


def test_plus_zero_ranks_above_minus_zero(orc):
    # E = {2, 3}; IEEE totalOrder puts -0 below +0, so K = 1 keeps position 3
    s = np.array([5, 5, -0.0, 0.0, 5], np.float32)
    assert run1(orc, s, 5, 5, 2, 1, 1, 0) == [0, 1, 3, 4]
    s = np.array([5, 5, 0.0, -0.0, 5], np.float32)
    assert run1(orc, s, 5, 5, 2, 1, 1, 0) == [0, 1, 2, 4]


def test_isolated_centres_closed_form(orc):
    # centres >= 2r+1 apart and away from E's edges, K a multiple of 2r+1:
    # the important set is exactly the full neighbourhoods of the top K/(2r+1)
    rng = np.random.default_rng(13)
    for r in (1, 2, 3):
        L, S, W = 400, 8, 16
        s = rng.uniform(-1, 0, L).astype(np.float32)
        centres = np.arange(S + 10, L - W - 10, 2 * r + 1 + 5)[:20]
        s[centres] = 1.0 + np.arange(len(centres), dtype=np.float32)
        m = 7
        top = centres[-m:]
        expect = set()
        for c in top:
            expect.update(range(c - r, c + r + 1))
        got = set(run1(orc, s, L, L, S, W, m * (2 * r + 1), r))
        assert got - set(range(S)) - set(range(L - W, L)) == expect


def test_all_equal_scores_take_lowest_positions(orc):
    for r in (0, 1, 2):
        L, S, W, K = 100, 4, 10, 17
        got = run1(orc, np.zeros(L, np.float32), L, L, S, W, K, r)
        assert got == list(range(0, S + K)) + list(range(L - W, L))


def test_invariants_random(orc):
    rng = np.random.default_rng(14)
    B, Hq, Lmax = 3, 4, 700
    for trial in range(6):
        S, W = int(rng.integers(0, 20)), int(rng.integers(0, 60))
        K, r = int(rng.integers(0, 300)), int(rng.integers(0, 4))
        L = rng.integers(1, Lmax + 1, size=B).astype(np.int32)
        P = np.array([rng.integers(max(0, l - W), l + 1) for l in L], np.int32)
        s = rng.standard_normal((B, Hq, Lmax)).astype(np.float32)
        idx, cnt = orc.select(s, L, P, S, W, K, r, cap=Lmax)
        for b in range(B):
            e0, e1 = S, max(S, min(L[b] - W, P[b]))
            for h in range(Hq):
                F = attended(idx, cnt, b, h)
                assert F == sorted(set(F)) and all(0 <= t < L[b] for t in F)
                Fs = set(F)
                assert set(range(min(S, L[b]))) <= Fs                 # sink kept
                assert set(range(max(0, L[b] - W), L[b])) <= Fs       # window kept
                imp = [t for t in F if e0 <= t < e1]
                assert len(imp) == min(K, e1 - e0)                    # fixed budget
                assert len(F) <= S + W + K
                # nothing outside sink, window and E
                assert all(t < S or t >= L[b] - W or e0 <= t < e1 for t in F)


def test_full_budget_is_dense_and_zero_budget_is_sink_window(orc):
    rng = np.random.default_rng(15)
    L, S, W = 257, 4, 16
    s = rng.standard_normal(L).astype(np.float32)
    assert run1(orc, s, L, L, S, W, L, 1) == list(range(L))
    assert run1(orc, s, L, L, S, W, 0, 2) == list(range(S)) + list(range(L - W, L))
    # short context: L <= S + W gives everything
    assert run1(orc, s[:15], 15, 15, 4, 16, 3, 1) == list(range(15))


def test_neighbour_fill_stays_in_region_and_covers_spans(orc):
    # each centre whose neighbourhood is not truncated brings all of [c-r, c+r]
    rng = np.random.default_rng(16)
    L, S, W, r = 300, 4, 16, 2
    s = rng.standard_normal(L).astype(np.float32)
    F = set(run1(orc, s, L, L, S, W, 40, r))
    e0, e1 = S, L - W
    E = np.arange(e0, e1)
    order = E[np.lexsort((E, -s[e0:e1]))]
    # first 8 centres: 8 * 5 = 40 tokens at most, so at least the first centre's
    # neighbourhood is complete and all picks stay in E
    c = order[0]
    assert set(range(max(e0, c - r), min(e1, c + r + 1))) <= F
    assert all(t < S or t >= L - W or e0 <= t < e1 for t in F)


def test_projection_lag_clips_region(orc):
    # positions [P, L-W) have no projected key yet: neither eligible nor kept
    L, S, W, P = 100, 2, 10, 60
    s = np.ones(L, np.float32)
    F = run1(orc, s, L, P, S, W, 1000, 0)
    assert F == list(range(0, 60)) + list(range(90, 100))


def test_ragged_batch_matches_single(orc):
    rng = np.random.default_rng(17)
    B, Hq, Lmax = 3, 2, 120
    L = np.array([120, 77, 33], np.int32)
    s = rng.standard_normal((B, Hq, Lmax)).astype(np.float32)
    idx, cnt = orc.select(s, L, L, 3, 9, 20, 1, cap=Lmax)
    for b in range(B):
        for h in range(Hq):
            single = run1(orc, s[b, h, :L[b]], int(L[b]), int(L[b]), 3, 9, 20, 1)
            assert attended(idx, cnt, b, h) == single
