"""tb_score_select (for small problems the selection's band is sampled by
extra workgroups of the scoring launch, from the projected keys; otherwise the
two calls' launches) equals tb_score followed by tb_select bit for bit --
scores, list and count -- over shapes covering every compiled (group size,
d', radius) variant of the fused launch and the separate launches (radius 2
and above, many heads), both neighbour modes, the window left out,
ragged and lagging projections, short contexts, a budget covering the
eligible region, an empty budget, invalid lengths and radii above the fused
variants; and its list equals the oracle's selection on the same scores."""
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


def _run(tb, fused, qh, kp, L, P, S, W, K, r, mode, cap, ws, ns=1, slot=0):
    B, Hkv, Lmax, dp = kp.shape
    Hq = qh.shape[1] // (ns * dp)
    scores = torch.full((B, Hq, Lmax), -3.5, device="cuda")
    idx = torch.full((B, Hq, cap), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, Hq), -7, dtype=torch.int32, device="cuda")
    ctx, pl = dev32(np.asarray(L, np.int32)), dev32(np.asarray(P, np.int32))
    if fused:
        tb.tb_score_select(qh, kp, ctx, pl, scores, S, W, K, r, idx, cnt, ws, mode=mode,
                           n_slots=ns, slot=slot)
    else:
        tb.tb_score(qh, kp, pl, scores, n_slots=ns, slot=slot)
        tb.tb_select(scores, ctx, pl, S, W, K, r, idx, cnt, ws, mode=mode)
    torch.cuda.synchronize()
    return host(scores), host(idx), host(cnt)


def _case(tb, seed, B, Hq, Hkv, Lmax, dp, L, P, S, W, K, r, dilate=False, omit=False, ns=1,
          slot=0, orc=None):
    say("score_select", seed, B, Hq, Hkv, Lmax, dp, L, P, S, W, K, r, dilate, omit)
    rng = rng_for(71, seed, B, Hq, Lmax, dp)
    kp = dev(normal_f16(rng, (B, Hkv, Lmax, dp), std=0.5), torch.float16)
    qh_np = rng.standard_normal((B, ns * Hq * dp)).astype(np.float32)
    qh = dev32(qh_np)
    mode = (tb.TB_NF_DILATE if dilate else tb.TB_NF_FILL) | (tb.TB_SEL_OMIT_WINDOW if omit else 0)
    imp = (2 * r + 1) * K if dilate else K
    cap = max(1, min(Lmax, S + (0 if omit else W) + imp))
    # one workspace shared by both runs: the fused call must leave its arrival
    # counters at zero like the separate calls do
    ws = tb.new_workspace(tb.tb_select_workspace_bytes(B, Hq, Lmax))
    s0, i0, c0 = _run(tb, False, qh, kp, L, P, S, W, K, r, mode, cap, ws, ns, slot)
    s1, i1, c1 = _run(tb, True, qh, kp, L, P, S, W, K, r, mode, cap, ws, ns, slot)
    s2, i2, c2 = _run(tb, True, qh, kp, L, P, S, W, K, r, mode, cap, ws, ns, slot)
    assert np.array_equal(s0.view(np.uint32), s1.view(np.uint32)), "scores differ"
    assert np.array_equal(c0, c1) and np.array_equal(c1, c2), "counts differ"
    for b in range(B):
        for h in range(Hq):
            n = c0[b, h]
            if n > 0:
                assert np.array_equal(i0[b, h, :n], i1[b, h, :n]), (b, h)
                assert np.array_equal(i1[b, h, :n], i2[b, h, :n]), (b, h)
    if orc is not None:
        ri, rc = orc.select(s1, np.asarray(L, np.int32), np.asarray(P, np.int32), S,
                            0 if omit else W, K, r, cap, dilate=dilate)
        if not omit:
            assert np.array_equal(c1, rc)
            for b in range(B):
                for h in range(Hq):
                    assert np.array_equal(i1[b, h, :rc[b, h]], ri[b, h, :rc[b, h]]), (b, h)
    return c1


def test_score_select_c2_shape_matches_separate_calls_and_oracle(tb, orc):
    L = 65536
    _case(tb, 0, 1, 32, 8, L, 32, [L], [L], 64, 256, 7872, 1, orc=orc)


def test_score_select_c1_shape_all_radii(tb, orc):
    for r in (0, 1, 2, 3):
        _case(tb, 1, 1, 8, 2, 300, 16, [300], [300], 4, 16, 32, r, orc=orc)


def test_score_select_ragged_qwen_shape(tb, orc):
    # group of 7, radius 2, ragged lengths, one sequence lagging in projection
    L = [20000, 13001, 17777, 9000]
    P = [20000, 13001, 17700, 9000]
    _case(tb, 2, 4, 28, 4, 20000, 32, L, P, 32, 128, 3936, 2, orc=orc)


@pytest.mark.parametrize("g,dp,r", [(1, 32, 0), (2, 16, 1), (3, 32, 1), (5, 16, 0), (6, 32, 1),
                                    (7, 16, 0), (8, 32, 1), (3, 32, 2), (8, 16, 2), (4, 16, 5)])
def test_score_select_group_sizes(tb, orc, g, dp, r):
    Hkv = 2
    Lmax = 12000
    _case(tb, 3 + g, 2, g * Hkv, Hkv, Lmax, dp, [Lmax, 7001], [Lmax, 6990], 16, 64, 900, r,
          orc=orc)


def test_score_select_dilate_and_omit_window(tb, orc):
    L = 65536
    _case(tb, 10, 1, 32, 8, L, 32, [L], [L], 64, 256, 7872, 1, dilate=True, orc=orc)
    _case(tb, 11, 1, 32, 8, L, 32, [L], [L], 64, 256, 7872, 1, omit=True)
    _case(tb, 12, 2, 8, 2, 5000, 16, [5000, 4000], [5000, 4000], 4, 16, 300, 2, dilate=True,
          omit=True)


def test_score_select_edges(tb, orc):
    # budget covering the eligible region, empty budget, context shorter than
    # the sink, nothing projected, a second slot of the predictor output
    _case(tb, 20, 1, 8, 2, 3000, 16, [3000], [3000], 4, 16, 5000, 1, orc=orc)
    _case(tb, 21, 1, 8, 2, 3000, 16, [3000], [3000], 4, 16, 0, 1, orc=orc)
    _case(tb, 22, 2, 8, 2, 3000, 16, [3, 2999], [3, 2999], 4, 16, 100, 1, orc=orc)
    _case(tb, 23, 1, 8, 2, 3000, 16, [3000], [0], 4, 16, 100, 1, orc=orc)
    _case(tb, 24, 1, 8, 2, 3000, 32, [3000], [2500], 4, 16, 100, 2, ns=2, slot=1, orc=orc)


def test_score_select_bad_lengths_flagged(tb):
    c = _case(tb, 30, 3, 8, 2, 3000, 16, [3000, 3001, -1], [3000, 10, 5], 4, 16, 100, 1)
    assert (c[0] >= 0).all() and (c[1] == -1).all() and (c[2] == -1).all()
