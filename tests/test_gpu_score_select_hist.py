"""tb_score_select above 8192 tokens with radius <= 2 (0 in the dilation mode)
takes the histogram route: scoring that counts every eligible token's pooled
key32 in 4096 bins, then one workgroup per segment that finds the bin holding
the budget's key, streams the segment's scores once and selects exactly
inside that bin (through a second histogram of the next 12 key bits). It must
equal tb_score followed by tb_select (the sampled-band route) bit for bit --
scores, list, count -- and the oracle's selection on the same scores,
including where the bin holds every eligible token (all scores equal,
integer-valued scores), more candidates than the workgroup stages in LDS, a
budget that takes a whole bin, budgets that cover the region or are empty,
contexts shorter than the sink, nothing projected, ragged and lagging
lengths, invalid lengths, a workspace shared with the band route, and a
histogram region that was not zero at first use."""
import numpy as np
import pytest
import torch

from synthetic import normal_f16, rng_for
from gpu_util import dev, dev32, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import learned_kv_cache_amd as tb
    tb.lib()
    return tb


def _run(tb, fused, qh, kp, L, P, S, W, K, r, mode, cap, ws):
    B, Hkv, Lmax, dp = kp.shape
    Hq = qh.shape[1] // dp
    scores = torch.full((B, Hq, Lmax), -3.5, device="cuda")
    idx = torch.full((B, Hq, cap), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, Hq), -7, dtype=torch.int32, device="cuda")
    ctx, pl = dev32(np.asarray(L, np.int32)), dev32(np.asarray(P, np.int32))
    if fused:
        tb.tb_score_select(qh, kp, ctx, pl, scores, S, W, K, r, idx, cnt, ws, mode=mode)
    else:
        tb.tb_score(qh, kp, pl, scores)
        tb.tb_select(scores, ctx, pl, S, W, K, r, idx, cnt, ws, mode=mode)
    torch.cuda.synchronize()
    return host(scores), host(idx), host(cnt)


def _check(tb, orc, kp_np, qh_np, L, P, S, W, K, r, dilate=False, omit=False, reps=2):
    B, Hkv, Lmax, dp = kp_np.shape
    Hq = qh_np.shape[1] // dp
    say("hist route", B, Hq, Hkv, Lmax, dp, L, P, S, W, K, r, dilate, omit)
    kp = dev(kp_np, torch.float16)
    qh = dev32(qh_np)
    mode = (tb.TB_NF_DILATE if dilate else tb.TB_NF_FILL) | (tb.TB_SEL_OMIT_WINDOW if omit else 0)
    imp = (2 * r + 1) * K if dilate else K
    cap = max(1, min(Lmax, S + (0 if omit else W) + imp))
    ws = tb.new_workspace(tb.tb_select_workspace_bytes(B, Hq, Lmax))
    s0, i0, c0 = _run(tb, False, qh, kp, L, P, S, W, K, r, mode, cap, ws)
    for rep in range(reps):   # the histogram and counters are left at zero for the next call
        s1, i1, c1 = _run(tb, True, qh, kp, L, P, S, W, K, r, mode, cap, ws)
        assert np.array_equal(s0.view(np.uint32), s1.view(np.uint32)), "scores differ"
        assert np.array_equal(c0, c1), ("counts differ", rep, c0, c1)
        for b in range(B):
            for h in range(Hq):
                n = c0[b, h]
                if n > 0:
                    assert np.array_equal(i0[b, h, :n], i1[b, h, :n]), (rep, b, h)
    # the band route after the histogram route on the same workspace
    s2, i2, c2 = _run(tb, False, qh, kp, L, P, S, W, K, r, mode, cap, ws)
    assert np.array_equal(c0, c2)
    ri, rc = orc.select(s1, np.asarray(L, np.int32), np.asarray(P, np.int32), S, W, K, r,
                        None, dilate=dilate)
    for b in range(B):
        for h in range(Hq):
            want = ri[b, h, :rc[b, h]]
            if omit and rc[b, h] >= 0:
                # the window left out of the list (the eligible region is the same)
                want = want[(want < S) | (want < L[b] - W)]
            assert c1[b, h] == (len(want) if rc[b, h] >= 0 else -1), (b, h)
            if rc[b, h] >= 0:
                assert np.array_equal(i1[b, h, :c1[b, h]], want), (b, h)
    # the two histograms (the workspace's last region) and the arrival
    # counters (its first) are back at zero
    ws_np = host(ws)
    hist_bytes = 2 * B * Hq * 4096 * 4
    assert not ws_np[-hist_bytes:].any()
    assert not ws_np[:B * Hq * 4].any()
    return c1


def _normal(seed, B, Hq, Hkv, Lmax, dp):
    rng = rng_for(72, seed, B, Hq, Lmax, dp)
    kp = normal_f16(rng, (B, Hkv, Lmax, dp), std=0.5)
    qh = rng.standard_normal((B, Hq * dp)).astype(np.float32)
    return kp, qh


@pytest.mark.parametrize("r", [0, 1, 2])
def test_hist_route_random(tb, orc, r):
    kp, qh = _normal(r, 2, 8, 2, 20000, 32)
    _check(tb, orc, kp, qh, [20000, 15000], [20000, 14990], 16, 64, 2000, r)


def test_hist_route_dilate_and_omit(tb, orc):
    kp, qh = _normal(5, 1, 8, 2, 30000, 16)
    _check(tb, orc, kp, qh, [30000], [30000], 32, 128, 1500, 2, dilate=True)
    _check(tb, orc, kp, qh, [30000], [30000], 32, 128, 1500, 1, omit=True)


def test_hist_route_all_scores_equal(tb, orc):
    # q = 0: every score is +0, every eligible token lands in one bin, far
    # more candidates than the threshold stages in LDS (its global path)
    kp, qh = _normal(6, 1, 8, 2, 16384, 16)
    qh[:] = 0.0
    for r in (0, 1, 2):
        _check(tb, orc, kp, qh, [16384], [16384], 8, 32, 3000, r)


def test_hist_route_integer_scores(tb, orc):
    # integer-valued projected keys and one-hot queries: integer scores with
    # heavy ties across and inside bins
    rng = rng_for(73)
    B, Hq, Hkv, Lmax, dp = 1, 8, 2, 24000, 16
    ints = rng.integers(-6, 7, size=(B, Hkv, Lmax, dp)).astype(np.float16)
    kp = ints.view(np.uint16)
    qh = np.zeros((B, Hq * dp), np.float32)
    for h in range(Hq):
        qh[0, h * dp + (h % dp)] = 1.0
    for r in (0, 1, 2):
        _check(tb, orc, kp, qh, [Lmax], [Lmax], 16, 64, 4000, r)


@pytest.mark.parametrize("n_mid,r,K", [(4000, 0, 2000), (5000, 0, 2500), (1500, 1, 750),
                                       (3000, 0, 3000), (9000, 0, 9000), (9000, 0, 4500)])
def test_hist_route_candidates_around_lds_capacity(tb, orc, n_mid, r, K):
    # n_mid tokens score in [1.5, 1.7) (one bin: [1.5, 1.75)), the rest in
    # [0.5, 0.9): the budget's key lies in that bin, whose candidates number
    # up to beyond the 8192 the selection workgroup stages in LDS (with
    # radius 1 each mid token's neighbours join the bin); a budget of n_mid
    # takes the whole bin
    rng = rng_for(74, n_mid, r)
    B, Hq, Hkv, Lmax, dp = 1, 4, 1, 12000, 16
    x = 0.5 + 0.4 * rng.random(Lmax)
    mid = rng.choice(np.arange(8, Lmax - 16), n_mid, replace=False)
    x[mid] = 1.5 + 0.2 * rng.random(n_mid)
    kpf = np.zeros((B, Hkv, Lmax, dp), np.float16)
    kpf[0, 0, :, 0] = x.astype(np.float16)
    qh = np.zeros((B, Hq * dp), np.float32)
    qh[0, ::dp] = 1.0
    _check(tb, orc, kpf.view(np.uint16), qh, [Lmax], [Lmax], 8, 16, K, r)


def test_hist_route_edges(tb, orc):
    kp, qh = _normal(8, 2, 8, 2, 12000, 16)
    # budget covering the eligible region; empty budget
    _check(tb, orc, kp, qh, [12000, 11000], [12000, 11000], 4, 16, 20000, 1)
    _check(tb, orc, kp, qh, [12000, 11000], [12000, 11000], 4, 16, 0, 1)
    # context shorter than the sink; nothing projected; lagging projection
    _check(tb, orc, kp, qh, [3, 12000], [3, 12000], 4, 16, 500, 1)
    _check(tb, orc, kp, qh, [12000, 9000], [0, 8000], 4, 16, 500, 2)
    # eligible region of a single token and of budget + 1 tokens
    _check(tb, orc, kp, qh, [12000, 12000], [4 + 1, 4 + 501], 4, 16, 500, 1)


def test_hist_route_bad_lengths_flagged(tb, orc):
    kp, qh = _normal(9, 3, 8, 2, 12000, 16)
    ctx = dev32(np.asarray([12000, 12001, -1], np.int32))
    pl = dev32(np.asarray([12000, 10, 5], np.int32))
    ws = tb.new_workspace(tb.tb_select_workspace_bytes(3, 8, 12000))
    scores = torch.empty((3, 8, 12000), device="cuda")
    idx = torch.zeros((3, 8, 600), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((3, 8), dtype=torch.int32, device="cuda")
    for _ in range(2):
        tb.tb_score_select(dev32(qh), dev(kp, torch.float16), ctx, pl, scores, 4, 16, 500, 1, idx,
                           cnt, ws)
        torch.cuda.synchronize()
        c = host(cnt)
        assert (c[0] == 4 + 16 + 500).all() and (c[1] == -1).all() and (c[2] == -1).all()


@pytest.mark.parametrize("fill", ["large", "small", "second"])
def test_hist_route_workspace_histogram_not_zero(tb, orc, fill):
    # histogram regions that were not zero at first use: counts far above the
    # segment's (the bin found disagrees with the pass), below its budget (no
    # bin holds the budget's rank), or junk in the second histogram only; the
    # selection stays exact and both regions are zero afterwards
    kp, qh = _normal(11, 2, 8, 2, 20000, 16)
    B, Hq, Lmax = 2, 8, 20000
    L, P, S, W, K, r = [20000, 17000], [20000, 17000], 16, 64, 2000, 1
    mode = tb.TB_NF_FILL
    cap = S + W + K
    ws = tb.new_workspace(tb.tb_select_workspace_bytes(B, Hq, Lmax))
    s0, i0, c0 = _run(tb, False, dev32(qh), dev(kp, torch.float16), L, P, S, W, K, r, mode, cap, ws)
    hw = B * Hq * 4096   # words of one histogram; the main one, then the second
    rng = rng_for(75, ["large", "small", "second"].index(fill))
    region = ws[-2 * hw * 4:].view(torch.int32)
    if fill == "large":
        region[:hw].copy_(torch.from_numpy(rng.integers(0, 5000, size=hw).astype(np.int32)))
    elif fill == "small":
        region[:hw].copy_(torch.from_numpy((rng.random(hw) < 0.02).astype(np.int32)))
    else:
        region[hw:].copy_(torch.from_numpy(rng.integers(0, 3, size=hw).astype(np.int32)))
    s1, i1, c1 = _run(tb, True, dev32(qh), dev(kp, torch.float16), L, P, S, W, K, r, mode, cap, ws)
    assert np.array_equal(c0, c1)
    for b in range(B):
        for h in range(Hq):
            assert np.array_equal(i0[b, h, :c0[b, h]], i1[b, h, :c1[b, h]]), (b, h)
    assert not host(ws)[-2 * hw * 4:].any()
    assert not host(ws)[:B * Hq * 4].any()
    # and the next call, on clean histograms, is exact too
    s2, i2, c2 = _run(tb, True, dev32(qh), dev(kp, torch.float16), L, P, S, W, K, r, mode, cap, ws)
    assert np.array_equal(c0, c2) and np.array_equal(i0, i2)
