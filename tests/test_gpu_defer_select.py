"""The split selection: tb_score_select with TB_SEL_DEFER_SELECT (scores,
histogram and classification only) followed by tb_select_attn with the same
flag (every attention workgroup resolves the threshold for its chunk, writes
the chunk's list rows and attends). Scores, count and list equal those of
tb_score_select without the flag bit for bit; the output equals
tb_sparse_decode_attn over that list to fp32 rounding (other splits), and the
oracle's attention at the 64K shape. Covered: the 8B-layer decode shape,
ragged batches, radius 0-2, query groups of 1, 2 and 4, the window left out of
the list, budgets covering the region or empty, flagged lengths, shapes the
split does not apply to (the flag then acts as TB_SEL_DEFER_LIST, bit for
bit), calls twice in a row on the same workspaces, graph replays, a
workspace whose histograms hold junk (reported as count -1, then exact on
the next call), and random configurations on the route."""
import numpy as np
import pytest
import torch

from synthetic import normal_bf16, normal_f16, rng_for
from gpu_util import assert_attn_close, assert_rel, dev, dev32, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import learned_kv_cache_amd as tb
    tb.lib()
    return tb


def _inputs(seed, B, Hq, Hkv, Lmax, D, dp):
    rng = rng_for(98, seed, B, Hq, Lmax, D)
    kp = dev(normal_f16(rng, (B, Hkv, Lmax, dp), std=0.5), torch.float16)
    qh = dev32(rng.standard_normal((B, Hq * dp)).astype(np.float32))
    kc_h, vc_h, q_h = (normal_bf16(rng, (B, Hkv, Lmax, D)), normal_bf16(rng, (B, Hkv, Lmax, D)),
                       normal_bf16(rng, (B, Hq, D)))
    return kp, qh, kc_h, vc_h, q_h


def _case(tb, seed, B, Hq, Hkv, Lmax, D, dp, L, P, S, W, K, r, omit=False, orc=None,
          junk=False, expect_split=True, flat=False):
    say("defer_select", seed, B, Hq, Hkv, Lmax, D, dp, L, P, S, W, K, r, omit, junk, flat)
    kp, qh, kc_h, vc_h, q_h = _inputs(seed, B, Hq, Hkv, Lmax, D, dp)
    if flat:
        kp.zero_()   # every score 0: ties broken by position
    kc, vc, q = (dev(x, torch.bfloat16) for x in (kc_h, vc_h, q_h))
    ctx, pl = dev32(np.asarray(L, np.int32)), dev32(np.asarray(P, np.int32))
    mode = tb.TB_NF_FILL | (tb.TB_SEL_OMIT_WINDOW if omit else 0)
    cap = max(1, min(Lmax, S + (0 if omit else W) + K))
    # the reference: the selection without the flag, then the attention over its list
    ws_r = tb.new_workspace(tb.tb_select_workspace_bytes(B, Hq, Lmax))
    ws_ra = tb.new_workspace(tb.tb_attn_workspace_bytes(B, Hq, cap, 0, D))
    s_ref = torch.full((B, Hq, Lmax), -3.5, device="cuda")   # positions past P stay unwritten
    i_ref = torch.full((B, Hq, cap), -7, dtype=torch.int32, device="cuda")
    c_ref = torch.full((B, Hq), -7, dtype=torch.int32, device="cuda")
    o_ref = torch.full((B, Hq, D), float("nan"), device="cuda")
    tb.tb_score_select(qh, kp, ctx, pl, s_ref, S, W, K, r, i_ref, c_ref, ws_r, mode=mode)
    tb.tb_sparse_decode_attn(q, kc, vc, i_ref, c_ref, o_ref, ws_ra)
    torch.cuda.synchronize()
    s0, i0, c0, o0 = host(s_ref), host(i_ref), host(c_ref), host(o_ref)

    ws_s = tb.new_workspace(tb.tb_select_workspace_bytes(B, Hq, Lmax))
    ws_a = tb.new_workspace(tb.tb_attn_workspace_bytes(B, Hq, cap, 0, D))
    m = mode | tb.TB_SEL_DEFER_SELECT
    if junk:
        # histograms that were never zeroed: both hold junk before the first call
        nseg = B * Hq
        hb = 2 * nseg * 4096 * 4   # the last bytes of the selection workspace
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        ws_s.view(torch.uint8)[-hb:] = torch.randint(0, 3, (hb,), generator=g, device="cuda",
                                                     dtype=torch.uint8)
    res = []
    for rep in range(2):
        scores = torch.full((B, Hq, Lmax), -3.5, device="cuda")
        idx = torch.full((B, Hq, cap), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((B, Hq), -7, dtype=torch.int32, device="cuda")
        out = torch.full((B, Hq, D), float("nan"), device="cuda")
        tb.tb_score_select(qh, kp, ctx, pl, scores, S, W, K, r, idx, cnt, ws_s, mode=m)
        tb.tb_select_attn(ctx, pl, S, W, K, r, idx, cnt, ws_s, q, kc, vc, out, ws_a, mode=m)
        torch.cuda.synchronize()
        res.append((host(scores), host(idx), host(cnt), host(out)))
    for rep, (s1, i1, c1, o1) in enumerate(res):
        assert np.array_equal(s0.view(np.uint32), s1.view(np.uint32)), ("scores", rep)
        if junk and rep == 0:
            # segments whose state disagreed are flagged; the others are exact
            bad = c1 == -1
            assert np.array_equal(c1[~bad], c0[~bad]), "count"
            assert (np.abs(o1[bad]) == 0).all(), "flagged output"
            continue
        assert np.array_equal(c0, c1), ("count", rep, c0, c1)
        for b in range(B):
            for h in range(Hq):
                n = max(0, int(c0[b, h]))
                assert np.array_equal(i0[b, h, :n], i1[b, h, :n]), ("idx", rep, b, h)
        if expect_split:
            assert_rel(o1, o0, 1e-4, "out vs the attention over the list")
        else:
            assert np.array_equal(o0.view(np.uint32), o1.view(np.uint32)), "out"
    # the attention's arrival counters are back to zero
    assert int(ws_a[-B * Hq * 4:].count_nonzero()) == 0
    if orc is not None:
        ref = orc.sparse_attention(q_h, kc_h, vc_h, i0, np.maximum(c0, 0))
        assert_attn_close(res[-1][3], ref, "vs oracle")
    return res[-1][2]


def test_defer_select_c2_shape(tb, orc):
    L = 65536
    _case(tb, 0, 1, 32, 8, L, 128, 32, [L], [L], 64, 256, 7872, 1, orc=orc)


def test_defer_select_shapes(tb):
    # radius 0 and 2, ragged, groups of 1, 2, 4, D 64
    _case(tb, 1, 2, 8, 2, 20000, 128, 32, [20000, 12345], [20000, 12340], 16, 64, 2400, 2)
    _case(tb, 2, 2, 8, 8, 20000, 64, 16, [20000, 15000], [19990, 15000], 16, 64, 2400, 0)
    _case(tb, 3, 1, 16, 8, 131072, 64, 32, [131072], [131072], 32, 128, 16224, 1)
    _case(tb, 4, 3, 4, 1, 9000, 128, 16, [9000, 8999, 8193], [9000, 8000, 8193], 8, 32, 2200, 1)
    # the window left out of the list (cap = sink + budget)
    _case(tb, 5, 1, 32, 8, 65536, 128, 32, [65536], [65536], 64, 256, 8128, 1, omit=True)


def test_defer_select_edges(tb):
    _case(tb, 6, 1, 8, 2, 9000, 128, 16, [9000], [9000], 4, 16, 9000, 1)   # budget covers E
    _case(tb, 7, 1, 8, 2, 9000, 128, 16, [9000], [9000], 4, 16, 2300, 1)
    _case(tb, 8, 2, 8, 2, 9000, 64, 16, [3, 8999], [3, 8999], 4, 16, 2300, 1)   # short context
    c = _case(tb, 9, 3, 8, 2, 9000, 64, 16, [9000, 9001, -1], [9000, 10, 5], 4, 16, 2300, 1)
    assert (c[0] >= 0).all() and (c[1] == -1).all() and (c[2] == -1).all()
    # every score equal: the budget's tokens are the first positions, so the
    # chosen candidates of the first chunks outnumber what one workgroup's
    # row table holds at once
    _case(tb, 11, 1, 8, 2, 65536, 128, 32, [65536], [65536], 64, 256, 7872, 1, flat=True)
    _case(tb, 12, 1, 4, 1, 40000, 64, 16, [40000], [40000], 8, 64, 12000, 2, flat=True)


def test_defer_select_off_route_acts_as_defer_list(tb):
    # too many segments, too short, radius 3, group of 8, or a list too short
    # for one split per chunk: the flag acts as TB_SEL_DEFER_LIST (bit for bit)
    _case(tb, 10, 3, 32, 8, 20000, 64, 16, [20000] * 3, [20000] * 3, 16, 64, 2400, 1,
          expect_split=False)
    _case(tb, 11, 1, 8, 2, 5000, 64, 16, [5000], [5000], 4, 16, 1200, 1, expect_split=False)
    _case(tb, 12, 1, 8, 2, 20000, 64, 16, [20000], [20000], 16, 64, 2400, 3, expect_split=False)
    _case(tb, 13, 1, 16, 2, 20000, 64, 16, [20000], [20000], 16, 64, 2400, 1, expect_split=False)
    _case(tb, 14, 1, 8, 2, 20000, 64, 16, [20000], [20000], 16, 64, 1000, 1, expect_split=False)


def test_defer_select_junk_histograms(tb):
    _case(tb, 15, 1, 8, 2, 20000, 64, 16, [20000], [20000], 16, 64, 2400, 1, junk=True)


def test_defer_select_random_configs(tb):
    rng = rng_for(99)
    for trial in range(16):
        B = int(rng.integers(1, 3))
        Hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 2, 3, 4]))
        Lmax = int(rng.choice([8193, 9000, 20000, 40000, 65536, 100000]))
        D = int(rng.choice([64, 128]))
        dp = int(rng.choice([16, 32]))
        S, W = int(rng.integers(0, 80)), int(rng.integers(0, 400))
        nch = (Lmax + 2047) // 2048
        K = int(rng.integers(nch * 256, min(Lmax + 50, nch * 256 + 6000)))
        r = int(rng.choice([0, 1, 2]))
        L = rng.integers(0, Lmax + 1, size=B).astype(np.int32)
        L[0] = Lmax
        P = np.minimum(L, rng.integers(0, Lmax + 1, size=B)).astype(np.int32)
        P[0] = L[0]
        _case(tb, 200 + trial, B, Hkv * g, Hkv, Lmax, D, dp, L.tolist(), P.tolist(), S, W, K, r,
              omit=bool(rng.integers(0, 2)))


def test_defer_select_graph_replays(tb):
    """The pair captured in a graph and replayed with eager work in between:
    every replay gives the eager results."""
    B, Hq, Hkv, Lmax, D, dp, S, W, K, r = 1, 32, 8, 65536, 128, 32, 64, 256, 7872, 1
    say("defer_select graph", B, Hq, Lmax)
    kp, qh, kc_h, vc_h, q_h = _inputs(30, B, Hq, Hkv, Lmax, D, dp)
    kc, vc, q = (dev(x, torch.bfloat16) for x in (kc_h, vc_h, q_h))
    ctx = dev32(np.asarray([Lmax], np.int32))
    cap = S + W + K
    m = tb.TB_NF_FILL | tb.TB_SEL_DEFER_SELECT
    ws_s = tb.new_workspace(tb.tb_select_workspace_bytes(B, Hq, Lmax))
    ws_a = tb.new_workspace(tb.tb_attn_workspace_bytes(B, Hq, cap, 0, D))
    scores = torch.empty((B, Hq, Lmax), device="cuda")
    idx = torch.zeros((B, Hq, cap), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((B, Hq), dtype=torch.int32, device="cuda")
    out = torch.zeros((B, Hq, D), device="cuda")

    def step():
        tb.tb_score_select(qh, kp, ctx, ctx, scores, S, W, K, r, idx, cnt, ws_s, mode=m)
        tb.tb_select_attn(ctx, ctx, S, W, K, r, idx, cnt, ws_s, q, kc, vc, out, ws_a, mode=m)

    step()
    torch.cuda.synchronize()
    ref = (host(idx).copy(), host(cnt).copy(), host(out).copy())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    for rep in range(3):
        idx.zero_()
        cnt.zero_()
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(cnt), ref[1]), rep
        assert np.array_equal(host(idx), ref[0]), rep
        assert np.array_equal(host(out).view(np.uint32), ref[2].view(np.uint32)), rep
        step()   # eager work between replays
        torch.cuda.synchronize()
