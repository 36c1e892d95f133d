"""Randomized GPU parity sweeps on small shapes (seeded): many (batch, heads,
context, sink, window, budget, radius, mode) combinations for the selection
in both neighbour modes, with and without the window, ragged lengths and
projection lag, bit-exact against the oracle; the same for scoring and
selection in one call (tb_score_select, either of its routes), its lists
bit-exact against the oracle's selection on its scores and its scores within
2e-3 of the oracle's; and projection + scoring +
attention (over a list, and over a list plus the implicit local window at a
random length) on random small shapes within their tolerances."""
import numpy as np
import pytest
import torch

from synthetic import bits_to_f32_f16, integer_scores, normal_bf16, rng_for, xavier_bf16
from gpu_util import assert_attn_close, assert_rel, bits, dev, dev32, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import learned_kv_cache_amd as tb
    tb.lib()
    return tb


def test_select_random_configs(tb, orc):
    rng = rng_for(120)
    for trial in range(60):
        B = int(rng.integers(1, 4))
        Hq = int(rng.choice([1, 2, 4, 8]))
        Lmax = int(rng.choice([1, 7, 64, 300, 2047, 2048, 2049, 5000, 12000]))
        S, W = int(rng.integers(0, 40)), int(rng.integers(0, 300))
        K = int(rng.integers(0, Lmax + 50))
        r = int(rng.choice([0, 1, 2, 3, 7, 64]))
        dilate = bool(rng.integers(0, 2))
        omit = bool(rng.integers(0, 2))
        L = rng.integers(0, Lmax + 1, size=B).astype(np.int32)
        P = np.minimum(L, rng.integers(0, Lmax + 1, size=B)).astype(np.int32)
        if rng.random() < 0.3:
            s = integer_scores(rng, (B, Hq, Lmax), -2, 3)
        else:
            s = rng.standard_normal((B, Hq, Lmax)).astype(np.float32)
        imp = (2 * r + 1) * K if dilate else K
        cap = max(1, min(Lmax, S + (0 if omit else W) + imp))
        what = (trial, B, Hq, Lmax, S, W, K, r, dilate, omit, L.tolist(), P.tolist())
        say("select fuzz", *what)
        ri, rc = orc.select(s, L, P, S, W, K, r, cap=min(Lmax, S + W + imp) or 1, dilate=dilate)
        idx = torch.full((B, Hq, cap), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((B, Hq), -7, dtype=torch.int32, device="cuda")
        ws = tb.new_workspace(tb.tb_select_workspace_bytes(B, Hq, Lmax))
        mode = (tb.TB_NF_DILATE if dilate else tb.TB_NF_FILL) | (tb.TB_SEL_OMIT_WINDOW if omit else 0)
        tb.tb_select(dev32(s), dev32(L), dev32(P), S, W, K, r, idx, cnt, ws, mode=mode)
        torch.cuda.synchronize()
        gi, gc = host(idx), host(cnt)
        for b in range(B):
            for h in range(Hq):
                ref = ri[b, h, :rc[b, h]]
                if omit:
                    ref = ref[(ref < S) | (ref < L[b] - W)]
                assert gc[b, h] == len(ref), what
                assert np.array_equal(gi[b, h, :gc[b, h]], ref), what


def test_score_select_random_configs(tb, orc):
    rng = rng_for(122)
    for trial in range(40):
        B = int(rng.integers(1, 4))
        Hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.integers(1, 9))
        Hq = Hkv * g
        dp = int(rng.choice([16, 32]))
        Lmax = int(rng.choice([1, 64, 300, 2047, 2049, 5000, 12000]))
        S, W = int(rng.integers(0, 40)), int(rng.integers(0, 300))
        K = int(rng.integers(0, Lmax + 50))
        r = int(rng.choice([0, 1, 1, 2, 3]))
        dilate = bool(rng.integers(0, 2))
        omit = bool(rng.integers(0, 2))
        L = rng.integers(0, Lmax + 1, size=B).astype(np.int32)
        P = np.minimum(L, rng.integers(0, Lmax + 1, size=B)).astype(np.int32)
        kp = (rng.standard_normal((B, Hkv, Lmax, dp)) * 0.5).astype(np.float16).view(np.uint16)
        qhat = rng.standard_normal((B, Hq * dp)).astype(np.float32)
        imp = (2 * r + 1) * K if dilate else K
        cap = max(1, min(Lmax, S + (0 if omit else W) + imp))
        what = (trial, B, Hq, Hkv, dp, Lmax, S, W, K, r, dilate, omit, L.tolist(), P.tolist())
        say("score_select fuzz", *what)
        scores = torch.full((B, Hq, Lmax), float("nan"), device="cuda")
        idx = torch.full((B, Hq, cap), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((B, Hq), -7, dtype=torch.int32, device="cuda")
        ws = tb.new_workspace(tb.tb_select_workspace_bytes(B, Hq, Lmax))
        mode = (tb.TB_NF_DILATE if dilate else tb.TB_NF_FILL) | (tb.TB_SEL_OMIT_WINDOW if omit else 0)
        tb.tb_score_select(dev32(qhat), dev(kp, torch.float16), dev32(L), dev32(P), scores, S, W,
                           K, r, idx, cnt, ws, mode=mode)
        torch.cuda.synchronize()
        gs, gi, gc = host(scores), host(idx), host(cnt)
        ref_s = orc.score(qhat, kp, P, Hq)
        for b in range(B):
            if P[b]:
                assert_rel(gs[b, :, :P[b]], ref_s[b, :, :P[b]], 2e-3, "scores %s" % (what,))
        # the oracle's selection on the GPU's scores (positions at or past the
        # projected length are never read; give them a finite value)
        s_in = np.where(np.isnan(gs), np.float32(0), gs).astype(np.float32)
        ri, rc = orc.select(s_in, L, P, S, W, K, r, cap=min(Lmax, S + W + imp) or 1, dilate=dilate)
        for b in range(B):
            for h in range(Hq):
                ref = ri[b, h, :rc[b, h]]
                if omit:
                    ref = ref[(ref < S) | (ref < L[b] - W)]
                assert gc[b, h] == len(ref), what
                assert np.array_equal(gi[b, h, :gc[b, h]], ref), what


def test_project_score_attention_random_shapes(tb, orc):
    rng = rng_for(121)
    for trial in range(12):
        B = int(rng.integers(1, 3))
        Hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 2, 4, 8]))
        Hq = Hkv * g
        D = int(rng.choice([64, 128]))
        dp = int(rng.choice([16, 32]))
        L = int(rng.integers(1, 3000))
        say("stage fuzz", trial, B, Hkv, Hq, D, dp, L)
        kc = normal_bf16(rng, (B, Hkv, L, D))
        vc = normal_bf16(rng, (B, Hkv, L, D))
        wk = xavier_bf16(rng, dp, D, lead=(Hkv,))
        kp = np.zeros((B, Hkv, L, dp), np.uint16)
        orc.project_keys(kc, wk, kp, np.zeros(B, np.int32), L)
        g_kp = torch.zeros((B, Hkv, L, dp), dtype=torch.float16, device="cuda")
        tb.tb_project_keys(dev(kc, torch.bfloat16), dev(wk, torch.bfloat16), g_kp,
                           dev32(np.zeros(B, np.int32)), L)
        qhat = rng.standard_normal((B, Hq * dp)).astype(np.float32)
        P = rng.integers(0, L + 1, size=B).astype(np.int32)
        ref_s = orc.score(qhat, kp, P, Hq)
        g_s = torch.full((B, Hq, L), float("nan"), device="cuda")
        tb.tb_score(dev32(qhat), dev(kp, torch.float16), dev32(P), g_s)
        q = normal_bf16(rng, (B, Hq, D))
        cap = int(rng.integers(1, L + 1))
        lists = np.zeros((B, Hq, cap), np.int32)
        cnt = rng.integers(0, cap + 1, size=(B, Hq)).astype(np.int32)
        for b in range(B):
            for h in range(Hq):
                lists[b, h, :cnt[b, h]] = np.sort(rng.choice(L, size=cnt[b, h], replace=False))
        ref_o = orc.sparse_attention(q, kc, vc, lists, cnt)
        g_o = torch.zeros((B, Hq, D), device="cuda")
        tb.tb_sparse_decode_attn(dev(q, torch.bfloat16), dev(kc, torch.bfloat16), dev(vc, torch.bfloat16),
                                 dev32(lists), dev32(cnt), g_o,
                                 tb.new_workspace(tb.tb_attn_workspace_bytes(B, Hq, cap, 0, D)))
        # the same lists plus the implicit local window: for each sequence a
        # length Lb and the window [max(Lb - W, last entry + 1, 0), Lb)
        W = int(rng.integers(1, 300))
        Lw = rng.integers(1, L + 1, size=B).astype(np.int32)
        wl = np.zeros((B, Hq, cap), np.int32)
        wc = np.zeros((B, Hq), np.int32)
        sets = []
        for b in range(B):
            for h in range(Hq):
                n = min(int(cnt[b, h]), int(Lw[b]))
                lst = np.sort(rng.choice(int(Lw[b]), size=n, replace=False)).astype(np.int32)
                wl[b, h, :n] = lst
                wc[b, h] = n
                w0 = max(int(Lw[b]) - W, (int(lst[-1]) + 1) if n else 0, 0)
                sets.append((b, h, np.concatenate([lst, np.arange(w0, int(Lw[b]), dtype=np.int32)])))
        n_max = max(len(x) for _, _, x in sets)
        ref_idx = np.zeros((B, Hq, max(1, n_max)), np.int32)
        ref_cnt = np.zeros((B, Hq), np.int32)
        for b, h, x in sets:
            ref_idx[b, h, :len(x)] = x
            ref_cnt[b, h] = len(x)
        ref_w = orc.sparse_attention(q, kc, vc, ref_idx, ref_cnt)
        g_w = torch.zeros((B, Hq, D), device="cuda")
        tb.tb_sparse_decode_attn(dev(q, torch.bfloat16), dev(kc, torch.bfloat16), dev(vc, torch.bfloat16),
                                 dev32(wl), dev32(wc), g_w,
                                 tb.new_workspace(tb.tb_attn_workspace_bytes(B, Hq, cap, W, D)),
                                 ctx_len=dev32(Lw), window=W)
        torch.cuda.synchronize()
        assert_attn_close(host(g_w), ref_w, "attention with window %d" % trial)
        assert_rel(bits_to_f32_f16(bits(g_kp)), bits_to_f32_f16(kp), 2e-3, "kp %d" % trial)
        gs = host(g_s)
        for b in range(B):
            assert_rel(gs[b, :, :P[b]], ref_s[b, :, :P[b]], 2e-3, "scores %d" % trial)
        assert_attn_close(host(g_o), ref_o, "attention %d" % trial)
