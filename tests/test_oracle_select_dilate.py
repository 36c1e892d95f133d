"""Pins for the oracle's other reading of neighbour fetching (TokenButler
summary, "Optimizations": the chosen tokens are widened to their spatial
neighbours): the budget picks the top-K eligible tokens as centres and every
eligible token within distance r of a centre is attended on top of the
budget, together with the sink and the circular local window ("Inference
strategy").

The oracle marks each centre's neighbourhood. These tests pin it with a
hand-worked golden case; an independent formulation (a token is attended iff
some centre lies within distance r, centres found by counting the tokens that
outrank each one) on exhaustive tiny tie-heavy inputs; r = 0 equal to the
fill mode's r = 0 (a plain top-K, itself pinned to a full sort); a closed
form for isolated centres; and the invariants (sink and window kept, at most
(2r+1)K widened tokens, all of them inside the eligible region)."""
import json
import os
import struct

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def total_order_key(x):
    b = struct.unpack("<I", struct.pack("<f", float(x)))[0]
    return b ^ (0xFFFFFFFF if b >> 31 else 0x80000000)


def by_distance(s, L, P, S, W, K, r):
    """Independent formulation: rank(t) = number of eligible tokens that come
    before t (higher score, or equal score and lower position); the centres
    are the tokens of rank < min(K, |E|); t in E is attended iff a centre lies
    within distance r."""
    e0, e1 = S, max(S, min(L - W, P))
    E = list(range(e0, e1))
    key = {t: total_order_key(s[t]) for t in E}
    rank = {t: sum(1 for u in E if key[u] > key[t] or (key[u] == key[t] and u < t)) for t in E}
    need = min(K, len(E))
    centres = [t for t in E if rank[t] < need]
    return {t for t in E if any(abs(t - c) <= r for c in centres)}


def run1(orc, s, L, P, S, W, K, r, dilate=True):
    Lmax = len(s)
    sc = np.asarray(s, np.float32).reshape(1, 1, Lmax)
    idx, cnt = orc.select(sc, np.array([L], np.int32), np.array([P], np.int32), S, W, K, r,
                          cap=Lmax, dilate=dilate)
    return [int(t) for t in idx[0, 0, :cnt[0, 0]]]


def test_golden_hand_cases(orc):
    g = json.load(open(os.path.join(HERE, "golden", "select_dilate_hand.json")))
    for c in g["cases"]:
        got = run1(orc, np.array(g["scores"], np.float32), g["L"], g["P"], g["S"], g["W"],
                   c["K"], c["r"])
        assert got == c["attended"], c


def test_brute_force_by_distance_tie_heavy(orc):
    rng = np.random.default_rng(21)
    n = 0
    for L in range(1, 24):
        for trial in range(10):
            S = int(rng.integers(0, 4))
            W = int(rng.integers(0, 5))
            P = int(rng.integers(max(0, L - 6), L + 1))
            K = int(rng.integers(0, L + 2))
            r = int(rng.integers(0, 4))
            s = rng.integers(-2, 3, size=L).astype(np.float32)
            s[rng.random(L) < 0.2] = -0.0
            got = set(run1(orc, s, L, P, S, W, K, r))
            expect = (by_distance(s, L, P, S, W, K, r) | set(range(min(S, L)))
                      | set(range(max(0, L - W), L)))
            assert got == expect, (L, S, W, P, K, r, s.tolist())
            n += 1
    assert n > 200


def test_radius0_equals_fill_radius0(orc):
    rng = np.random.default_rng(22)
    for trial in range(40):
        L = int(rng.integers(20, 300))
        S, W = int(rng.integers(0, 8)), int(rng.integers(0, 20))
        K = int(rng.integers(0, L))
        s = rng.standard_normal(L).astype(np.float32)
        s[rng.random(L) < 0.3] = 0.5
        assert run1(orc, s, L, L, S, W, K, 0) == run1(orc, s, L, L, S, W, K, 0, dilate=False)


def test_isolated_centres_closed_form(orc):
    # the K highest tokens sit at least 2r+1 apart inside E: exactly (2r+1)K
    # widened tokens, the full neighbourhoods of the planted centres
    rng = np.random.default_rng(23)
    for r in (1, 2, 5):
        L, S, W, K = 600, 8, 16, 9
        s = rng.uniform(-1, 0, L).astype(np.float32)
        centres = S + r + 3 + np.arange(K) * (2 * r + 1 + int(rng.integers(0, 4)))
        s[centres] = 1.0 + rng.random(K).astype(np.float32)
        got = run1(orc, s, L, L, S, W, K, r)
        assert len(got) == S + W + (2 * r + 1) * K
        expect = set()
        for c in centres:
            expect.update(range(c - r, c + r + 1))
        assert set(got) - set(range(S)) - set(range(L - W, L)) == expect


def test_invariants_random(orc):
    rng = np.random.default_rng(24)
    for trial in range(30):
        L = int(rng.integers(50, 400))
        S, W = int(rng.integers(0, 10)), int(rng.integers(0, 30))
        P = int(rng.integers(L // 2, L + 1))
        K, r = int(rng.integers(0, 60)), int(rng.integers(0, 6))
        s = rng.standard_normal(L).astype(np.float32)
        got = run1(orc, s, L, P, S, W, K, r)
        assert got == sorted(set(got))
        e0, e1 = S, max(S, min(L - W, P))
        imp = [t for t in got if e0 <= t < e1]
        assert set(range(min(S, L))) | set(range(max(0, L - W), L)) <= set(got)
        assert all(t < S or t >= L - W or e0 <= t < e1 for t in got)
        assert len(imp) <= (2 * r + 1) * min(K, e1 - e0)
        assert len(imp) >= min(K, e1 - e0)


def test_full_budget_dense_zero_budget_sink_window(orc):
    rng = np.random.default_rng(25)
    L, S, W = 120, 5, 9
    s = rng.standard_normal(L).astype(np.float32)
    assert run1(orc, s, L, L, S, W, L, 2) == list(range(L))
    assert run1(orc, s, L, L, S, W, 0, 2) == list(range(S)) + list(range(L - W, L))
