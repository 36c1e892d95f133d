"""Pins for the oracle's compositions: the important buffer alone, the
attended sets of a prediction interval, and the one-layer decode step
(TokenButler summary, "Inference strategy": the sink, the circular local
window and the important buffer filled from the predicted scores; the
predictor runs once per interval while the window keeps sliding).

Checked against what the method and the mathematics fix, not against the
functions' own formulas: hand-worked interval sets, the top-K of a full sort
at radius 0, the whole eligible region when the budget covers it, dense
causal attention (torch SDPA, float64) for a decode step whose budget covers
the context, and masked SDPA for an interval whose budget covered the
context at its start (only the tokens that slid out of the window since are
dropped)."""
import numpy as np
import torch

from synthetic import bits_to_f32_bf16, normal_bf16, xavier_bf16


def _dense_last_row(q, k, v, L):
    """Dense causal attention of the newest position over [0, L), float64."""
    B, Hq, D = q.shape
    g = Hq // k.shape[1]
    kk = torch.from_numpy(np.repeat(bits_to_f32_bf16(k[:, :, :L]), g, axis=1)).double()
    vv = torch.from_numpy(np.repeat(bits_to_f32_bf16(v[:, :, :L]), g, axis=1)).double()
    qq = torch.from_numpy(bits_to_f32_bf16(q)).double()[:, :, None, :]
    return torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)[:, :, 0].numpy()


def test_interval_sets_hand_worked(orc):
    # sink 2, window 3, context 10 at the first step, important {4, 6}:
    # step 0 (length 10): {0, 1} + {7, 8, 9} + {4, 6}
    # step 2 (length 12): {0, 1} + {9, 10, 11} + {4, 6}
    imp = [[np.array([4, 6])]]
    s0 = orc.interval_attended(imp, [10], 0, 2, 3)[0][0].tolist()
    s2 = orc.interval_attended(imp, [10], 2, 2, 3)[0][0].tolist()
    assert s0 == [0, 1, 4, 6, 7, 8, 9]
    assert s2 == [0, 1, 4, 6, 9, 10, 11]
    # an important token that the window reaches is counted once
    s = orc.interval_attended([[np.array([4, 8])]], [10], 0, 2, 3)[0][0].tolist()
    assert s == [0, 1, 4, 7, 8, 9]
    # context shorter than the sink: the sink is cut at the length
    s = orc.interval_attended([[np.array([], np.int64)]], [1], 0, 4, 2)[0][0].tolist()
    assert s == [0]


def test_interval_window_slides_one_token_per_step(orc):
    rng = np.random.default_rng(5)
    S, W, L0, I = 8, 32, 500, 20
    imp = np.sort(rng.choice(np.arange(S, L0 - W), 40, replace=False))
    for j in range(I):
        L = L0 + j
        got = orc.interval_attended([[imp]], [L0], j, S, W)[0][0]
        assert got.max() == L - 1                      # the newest token
        assert set(range(L - W, L)) <= set(got.tolist())
        assert (L - W - 1) not in set(got.tolist()) or (L - W - 1) in set(imp.tolist())
        assert set(got.tolist()) == set(range(S)) | set(range(L - W, L)) | set(imp.tolist())
        assert np.all(np.diff(got) > 0)


def test_important_only_radius0_is_topk_of_a_full_sort(orc):
    rng = np.random.default_rng(6)
    B, Hq, L, S, W, K = 2, 3, 400, 5, 20, 37
    s = rng.standard_normal((B, Hq, L)).astype(np.float32)
    s[:, :, 100:110] = s[:, :, 200:210]                # repeated values: ties by position
    Lb = np.array([400, 333], np.int32)
    imp = orc.important_only(s, Lb, Lb, S, W, K, 0)
    for b in range(B):
        e0, e1 = S, int(Lb[b]) - W
        for h in range(Hq):
            pos = np.arange(e0, e1)
            order = np.lexsort((pos, -s[b, h, e0:e1].astype(np.float64)))
            ref = np.sort(pos[order[:K]])
            assert np.array_equal(imp[b][h], ref), (b, h)


def test_important_only_budget_and_region(orc):
    rng = np.random.default_rng(7)
    B, Hq, L, S, W = 1, 4, 300, 4, 16
    s = rng.standard_normal((B, Hq, L)).astype(np.float32)
    Lb = np.array([L], np.int32)
    nE = L - W - S
    for K, r in ((10, 1), (50, 2), (nE, 1), (nE + 30, 2)):
        imp = orc.important_only(s, Lb, Lb, S, W, K, r)
        for h in range(Hq):
            t = imp[0][h]
            assert len(t) == min(K, nE)
            assert t.min() >= S and t.max() < L - W
            if K >= nE:
                assert np.array_equal(t, np.arange(S, L - W))


def test_decode_step_dense_budget_equals_causal_attention(orc):
    rng = np.random.default_rng(8)
    B, Hq, Hkv, L, D, E, Eh, dp = 1, 4, 2, 120, 64, 64, 32, 16
    x = normal_bf16(rng, (B, E))
    w1 = xavier_bf16(rng, Eh, E)
    w2 = xavier_bf16(rng, Hq * dp, Eh)
    wk = xavier_bf16(rng, dp, D, lead=(Hkv,))
    kc = normal_bf16(rng, (B, Hkv, L, D))
    vc = normal_bf16(rng, (B, Hkv, L, D))
    q = normal_bf16(rng, (B, Hq, D))
    kp = np.zeros((B, Hkv, L, dp), np.uint16)
    Lb = np.array([L], np.int32)
    orc.project_keys(kc, wk, kp, np.zeros(B, np.int32), L - 1)
    res = orc.decode_step(x, w1, w2, kc, vc, wk, kp, q, Lb, Lb, np.array([L - 1], np.int32), 1,
                          4, 8, L, 1)
    assert np.all(res["count"] == L)
    np.testing.assert_allclose(res["out"], _dense_last_row(q, kc, vc, L), rtol=1e-6, atol=1e-6)


def test_interval_dense_budget_drops_only_what_left_the_window(orc):
    # budget over the whole eligible region at the interval start: step j
    # attends to every token so far except the j + 1 that have slid out of
    # the window since (they were window tokens, not candidates, when the
    # important buffer was filled); attention equals masked SDPA
    rng = np.random.default_rng(9)
    B, Hq, Hkv, L0, D, S, W, I = 1, 4, 2, 90, 64, 4, 12, 6
    kc = normal_bf16(rng, (B, Hkv, L0 + I, D))
    vc = normal_bf16(rng, (B, Hkv, L0 + I, D))
    q = normal_bf16(rng, (B, Hq, D))
    s = rng.standard_normal((B, Hq, L0 + I)).astype(np.float32)
    Lb = np.array([L0], np.int32)
    imp = orc.important_only(s, Lb, Lb, S, W, L0, 1)
    g = Hq // Hkv
    for j in range(I):
        L = L0 + 1 + j
        gone = np.arange(L0 - W, L0 - W + j + 1)
        expect = np.setdiff1d(np.arange(L), gone)
        sets = orc.interval_attended(imp, [L0 + 1], j, S, W)
        idx = np.zeros((B, Hq, L), np.int32)
        cnt = np.zeros((B, Hq), np.int32)
        for h in range(Hq):
            assert np.array_equal(sets[0][h], expect), (j, h)
            idx[0, h, :len(expect)] = expect
            cnt[0, h] = len(expect)
        out = orc.sparse_attention(q, kc, vc, idx, cnt)
        mask = np.ones((B, Hq, L), bool)
        mask[:, :, gone] = False
        kk = torch.from_numpy(np.repeat(bits_to_f32_bf16(kc[:, :, :L]), g, axis=1)).double()
        vv = torch.from_numpy(np.repeat(bits_to_f32_bf16(vc[:, :, :L]), g, axis=1)).double()
        qq = torch.from_numpy(bits_to_f32_bf16(q)).double()[:, :, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq, kk, vv, attn_mask=torch.from_numpy(mask)[:, :, None, :])[:, :, 0].numpy()
        np.testing.assert_allclose(out, ref, rtol=1e-6, atol=1e-6)


def test_interval_of_one_step_equals_per_step_selection(orc):
    # I = 1: the interval's only step attends exactly to the per-step
    # selection (sink U window U important at the same length)
    rng = np.random.default_rng(10)
    B, Hq, L, S, W, K = 2, 3, 700, 6, 40, 55
    s = rng.standard_normal((B, Hq, L)).astype(np.float32)
    Lb = np.array([700, 512], np.int32)
    for r in (0, 1, 3):
        imp = orc.important_only(s, Lb, Lb, S, W, K, r)
        idx, cnt = orc.select(s, Lb, Lb, S, W, K, r)
        sets = orc.interval_attended(imp, Lb, 0, S, W)
        for b in range(B):
            for h in range(Hq):
                assert np.array_equal(sets[b][h], idx[b, h, :cnt[b, h]]), (r, b, h)
