"""The deferred list: a selection with TB_SEL_DEFER_LIST followed by
tb_select_attn (each attention workgroup rebuilds its list rows from the
selection's bitmap and candidates and writes them) equals the selection
without the flag followed by tb_sparse_decode_attn over its list -- scores,
count, list and output bit for bit -- after tb_score_select and after
tb_select, on the fused launch (up to 64 chunks) and on the compaction +
attention fallback (more chunks), with the window in the list or left out,
budgets covering the region or empty, short contexts and flagged lengths,
a query group of 7, twice in a row on the same workspaces, and 30 random
configurations; and the output against the oracle's attention at the 64K
shape.""" 
import numpy as np
import pytest
import torch

from synthetic import normal_bf16, normal_f16, rng_for
from gpu_util import assert_attn_close, dev, dev32, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import learned_kv_cache_amd as tb
    tb.lib()
    return tb


def _case(tb, seed, B, Hq, Hkv, Lmax, D, dp, L, P, S, W, K, r, omit=False, via_scores=False,
          orc=None):
    say("select_attn", seed, B, Hq, Hkv, Lmax, D, dp, L, P, S, W, K, r, omit, via_scores)
    rng = rng_for(96, seed, B, Hq, Lmax, D)
    kp = dev(normal_f16(rng, (B, Hkv, Lmax, dp), std=0.5), torch.float16)
    qh = dev32(rng.standard_normal((B, Hq * dp)).astype(np.float32))
    kc_h, vc_h, q_h = (normal_bf16(rng, (B, Hkv, Lmax, D)), normal_bf16(rng, (B, Hkv, Lmax, D)),
                       normal_bf16(rng, (B, Hq, D)))
    kc, vc, q = (dev(x, torch.bfloat16) for x in (kc_h, vc_h, q_h))
    ctx, pl = dev32(np.asarray(L, np.int32)), dev32(np.asarray(P, np.int32))
    mode = tb.TB_NF_FILL | (tb.TB_SEL_OMIT_WINDOW if omit else 0)
    cap = max(1, min(Lmax, S + (0 if omit else W) + K))
    ws_s = tb.new_workspace(tb.tb_select_workspace_bytes(B, Hq, Lmax))
    ws_a = tb.new_workspace(tb.tb_attn_workspace_bytes(B, Hq, cap, 0, D))
    pre = None
    if via_scores:
        pre = torch.empty((B, Hq, Lmax), device="cuda")
        tb.tb_score(qh, kp, pl, pre)
    res = []
    for deferred in (False, True, True):
        scores = torch.full((B, Hq, Lmax), -3.5, device="cuda") if pre is None else pre
        idx = torch.full((B, Hq, cap), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((B, Hq), -7, dtype=torch.int32, device="cuda")
        out = torch.full((B, Hq, D), float("nan"), device="cuda")
        m = mode | (tb.TB_SEL_DEFER_LIST if deferred else 0)
        if via_scores:
            tb.tb_select(scores, ctx, pl, S, W, K, r, idx, cnt, ws_s, mode=m)
        else:
            tb.tb_score_select(qh, kp, ctx, pl, scores, S, W, K, r, idx, cnt, ws_s, mode=m)
        if deferred:
            tb.tb_select_attn(ctx, pl, S, W, K, r, idx, cnt, ws_s, q, kc, vc, out, ws_a, mode=m)
        else:
            tb.tb_sparse_decode_attn(q, kc, vc, idx, cnt, out, ws_a)
        torch.cuda.synchronize()
        res.append((host(scores), host(idx), host(cnt), host(out)))
    s0, i0, c0, o0 = res[0]
    for s1, i1, c1, o1 in res[1:]:
        assert np.array_equal(s0.view(np.uint32), s1.view(np.uint32)), "scores"
        assert np.array_equal(c0, c1), "count"
        for b in range(B):
            for h in range(Hq):
                n = max(0, int(c0[b, h]))
                assert np.array_equal(i0[b, h, :n], i1[b, h, :n]), ("idx", b, h)
        assert np.array_equal(o0.view(np.uint32), o1.view(np.uint32)), "out"
    if orc is not None:
        ref = orc.sparse_attention(q_h, kc_h, vc_h, res[1][1], np.maximum(res[1][2], 0))
        assert_attn_close(res[1][3], ref, "vs oracle")
    return res[1][2]


def test_deferred_list_c2_shape(tb, orc):
    L = 65536
    _case(tb, 0, 1, 32, 8, L, 128, 32, [L], [L], 64, 256, 7872, 1, orc=orc)


def test_deferred_list_after_tb_select(tb):
    L = 65536
    _case(tb, 1, 1, 32, 8, L, 128, 32, [L], [L], 64, 256, 7872, 2, via_scores=True)
    _case(tb, 2, 2, 8, 2, 5000, 64, 16, [5000, 4000], [5000, 3990], 4, 16, 300, 0, via_scores=True)


def test_deferred_list_shapes(tb):
    _case(tb, 3, 1, 8, 2, 300, 64, 16, [300], [300], 4, 16, 32, 1)
    _case(tb, 4, 3, 16, 2, 20000, 128, 32, [20000, 12345, 777], [20000, 12340, 700], 16, 64, 2000, 2)
    _case(tb, 5, 2, 8, 1, 131072, 64, 16, [131072, 99999], [131072, 99999], 32, 128, 3000, 0)
    _case(tb, 6, 1, 8, 2, 140000, 64, 16, [140000], [140000], 64, 256, 4000, 1)   # fallback
    _case(tb, 7, 1, 32, 8, 65536, 128, 32, [65536], [65536], 64, 256, 7872, 1, omit=True)
    # Qwen-like group of 7, ragged, radius 2
    _case(tb, 12, 2, 14, 2, 70000, 128, 32, [70000, 51234], [70000, 51230], 32, 128, 3936, 2)


def test_deferred_list_random_configs(tb):
    rng = rng_for(97)
    for trial in range(30):
        B = int(rng.integers(1, 4))
        Hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.integers(1, 9))
        Lmax = int(rng.choice([1, 64, 300, 2047, 2049, 5000, 40000, 131072, 131073]))
        D = int(rng.choice([64, 128]))
        dp = int(rng.choice([16, 32]))
        S, W = int(rng.integers(0, 80)), int(rng.integers(0, 400))
        K = int(rng.integers(0, min(Lmax + 50, 9000)))
        r = int(rng.choice([0, 1, 2, 3]))
        L = rng.integers(0, Lmax + 1, size=B).astype(np.int32)
        P = np.minimum(L, rng.integers(0, Lmax + 1, size=B)).astype(np.int32)
        _case(tb, 100 + trial, B, Hkv * g, Hkv, Lmax, D, dp, L.tolist(), P.tolist(), S, W, K, r,
              omit=bool(rng.integers(0, 2)), via_scores=bool(rng.integers(0, 2)))


def test_deferred_list_edges(tb):
    _case(tb, 8, 1, 8, 2, 3000, 128, 16, [3000], [3000], 4, 16, 5000, 1)   # budget covers E
    _case(tb, 9, 1, 8, 2, 3000, 128, 16, [3000], [3000], 4, 16, 0, 1)      # empty budget
    _case(tb, 10, 2, 8, 2, 3000, 64, 16, [3, 2999], [3, 2999], 4, 16, 100, 1)
    c = _case(tb, 11, 3, 8, 2, 3000, 64, 16, [3000, 3001, -1], [3000, 10, 5], 4, 16, 100, 1)
    assert (c[0] >= 0).all() and (c[1] == -1).all() and (c[2] == -1).all()
