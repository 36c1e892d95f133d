"""End-to-end GPU parity of one decode step and of a prediction interval:
predict -> project -> score -> select -> sparse attention, all through the
C ABI, against the oracle chain on the same seeded inputs. Where the two
sides' fp32 scores differ in their last bits, selections may differ only by
tokens whose oracle rank score is within 1e-3 (relative) of the K-th."""
import numpy as np
import pytest
import torch

from synthetic import CONFIGS, bits_to_f32_f16, rng_for
from synthetic.workload import make_layer
from gpu_util import (assert_attn_close, assert_rel, bits, check_selection_band, dev, dev32, host,
                      say)
from workloads import oracle_direction, oracle_step, recovered

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import learned_kv_cache_amd as tb
    tb.lib()
    return tb


def gpu_step(tb, cfg, inp, K=None, r=None):
    K = cfg.K if K is None else K
    r = cfg.r if r is None else r
    B = inp["x"].shape[0]
    Lmax = inp["kc"].shape[2]
    L = inp["ctx_len"]
    x, w1, w2 = (dev(inp[k], torch.bfloat16) for k in ("x", "w1", "w2"))
    kc, vc, wk, q = (dev(inp[k], torch.bfloat16) for k in ("kc", "vc", "wk", "q"))
    kp = torch.zeros((B, cfg.Hkv, Lmax, cfg.dp), dtype=torch.float16, device="cuda")
    # the cache up to the newest token is already projected
    tb.tb_project_keys(kc, wk, kp, dev32(np.zeros(B, np.int32)), int(L.max()) - 1)
    ctx = dev32(L.astype(np.int32))
    qhat = torch.empty((B, cfg.n_out), device="cuda")
    tb.tb_predict_queries(x, w1, w2, qhat, tb.new_workspace(tb.tb_predict_workspace_bytes(B, cfg.E, cfg.Eh, cfg.n_out)))
    tb.tb_project_keys(kc, wk, kp, dev32((L - 1).astype(np.int32)), 1)
    scores = torch.full((B, cfg.Hq, Lmax), float("nan"), device="cuda")
    tb.tb_score(qhat, kp, ctx, scores)
    cap = min(Lmax, cfg.S + cfg.W + K)
    idx = torch.zeros((B, cfg.Hq, cap), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((B, cfg.Hq), dtype=torch.int32, device="cuda")
    tb.tb_select(scores, ctx, ctx, cfg.S, cfg.W, K, r, idx, cnt,
                 tb.new_workspace(tb.tb_select_workspace_bytes(B, cfg.Hq, Lmax)))
    out = torch.zeros((B, cfg.Hq, cfg.D), device="cuda")
    tb.tb_sparse_decode_attn(q, kc, vc, idx, cnt, out,
                             tb.new_workspace(tb.tb_attn_workspace_bytes(B, cfg.Hq, cap, 0, cfg.D)))
    torch.cuda.synchronize()
    return dict(qhat=host(qhat), kp=bits(kp), scores=host(scores), idx=host(idx), count=host(cnt),
                out=host(out), dev=dict(q=q, kc=kc, vc=vc))


def compare_step(tb, orc, cfg, inp, g, o, K=None, r=None, kp_rows=None):
    K = cfg.K if K is None else K
    r = cfg.r if r is None else r
    L = inp["ctx_len"]
    B = len(L)
    assert_rel(g["qhat"], o["qhat"], 2e-3, "qhat")
    for b in range(B):
        if kp_rows is None:
            assert_rel(bits_to_f32_f16(g["kp"][b, :, :L[b]]), bits_to_f32_f16(o["kp"][b, :, :L[b]]),
                       2e-3, "kp")
        else:
            for t in kp_rows:
                assert_rel(bits_to_f32_f16(g["kp"][b, :, t]), bits_to_f32_f16(o["kp"][b, :, t]), 2e-3,
                           "kp t=%d" % t)
        assert_rel(g["scores"][b, :, :L[b]], o["scores"][b, :, :L[b]], 2e-3, "scores")
    check_selection_band(g["idx"], g["count"], o["idx"], o["count"], o["scores"], L, L, cfg.S,
                         cfg.W, K, r, what="select")
    same = all(np.array_equal(g["idx"][b, h, :g["count"][b, h]], o["idx"][b, h, :o["count"][b, h]])
               for b in range(B) for h in range(cfg.Hq))
    if same:
        assert_attn_close(g["out"], o["out"], "attention end-to-end")
    else:
        # stage-isolated: both sides attend over the oracle's sets
        d = g["dev"]
        out = torch.zeros_like(torch.from_numpy(g["out"])).cuda()
        cap = o["idx"].shape[-1]
        tb.tb_sparse_decode_attn(d["q"], d["kc"], d["vc"], dev32(o["idx"]), dev32(o["count"]), out,
                                 tb.new_workspace(tb.tb_attn_workspace_bytes(B, cfg.Hq, cap, 0, cfg.D)))
        torch.cuda.synchronize()
        assert_attn_close(host(out), o["out"], "attention on oracle sets")
    return same


def test_c1_planted_step(tb, orc):
    cfg = CONFIGS[1]
    say("e2e c1 planted")
    inp = make_layer(cfg, seed=0, direction_fn=oracle_direction(orc, cfg))
    o = oracle_step(orc, cfg, inp)
    g = gpu_step(tb, cfg, inp)
    compare_step(tb, orc, cfg, inp, g, o)
    assert all(recovered(g, inp["spans"]))


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_c1_more_seeds_and_radii(tb, orc, seed):
    cfg = CONFIGS[1]
    say("e2e c1 seed", seed)
    inp = make_layer(cfg, seed=seed, direction_fn=oracle_direction(orc, cfg))
    for r in (0, 2):
        o = oracle_step(orc, cfg, inp, r=r)
        g = gpu_step(tb, cfg, inp, r=r)
        compare_step(tb, orc, cfg, inp, g, o, r=r)


def test_c2_full_step(tb, orc):
    cfg = CONFIGS[2]
    say("e2e c2 full size: generating")
    inp = make_layer(cfg, seed=0, direction_fn=oracle_direction(orc, cfg))
    say("e2e c2: oracle")
    o = oracle_step(orc, cfg, inp)
    say("e2e c2: gpu")
    g = gpu_step(tb, cfg, inp)
    rows = list(range(0, cfg.L, 997)) + [cfg.L - 1]
    compare_step(tb, orc, cfg, inp, g, o, kp_rows=rows)
    rec = recovered(g, inp["spans"])
    say("c2 planted spans recovered: %d / %d" % (sum(rec), len(rec)))


def test_c5_ragged_step(tb, orc):
    cfg = CONFIGS[5]
    say("e2e c5 ragged: generating")
    inp = make_layer(cfg, seed=0, B=2)
    say("e2e c5 lengths", inp["ctx_len"].tolist())
    o = oracle_step(orc, cfg, inp)
    g = gpu_step(tb, cfg, inp)
    compare_step(tb, orc, cfg, inp, g, o, kp_rows=list(range(0, 65536, 4093)))


def test_interval_reuses_selection_and_slides_window(tb, orc):
    """Prediction interval: select once with the window left out of the list,
    then attend for I steps while the context grows by one token per step; the
    attended set at step j is sink U window(L0 + 1 + j) U the important tokens
    chosen at L0 (the circular window keeps only the most recent W tokens)."""
    cfg = CONFIGS[1]
    I, L0, B = 6, 280, 1
    say("interval", I, L0)
    inp = make_layer(cfg, seed=4, L=L0 + I, Lmax=L0 + I)
    Ln = np.array([L0], np.int32)
    # oracle: projection of the first L0 tokens, predictor, scores, selection
    o_kp = np.zeros((B, cfg.Hkv, L0 + I, cfg.dp), np.uint16)
    orc.project_keys(inp["kc"], inp["wk"], o_kp, np.zeros(B, np.int32), L0)
    _, o_qhat = orc.predict_queries(inp["x"], inp["w1"], inp["w2"])
    o_scores = orc.score(o_qhat, o_kp, Ln, cfg.Hq)
    o_idx, o_cnt = orc.select(o_scores, Ln, Ln, cfg.S, cfg.W, cfg.K, cfg.r)
    important = orc.important_only(o_scores, Ln, Ln, cfg.S, cfg.W, cfg.K, cfg.r)
    # the oracle's sink U important list (window left out)
    cap = cfg.S + cfg.K
    o_list = np.zeros((B, cfg.Hq, cap), np.int32)
    o_lcnt = np.zeros((B, cfg.Hq), np.int32)
    for h in range(cfg.Hq):
        lst = sorted(set(range(min(cfg.S, L0))) | set(important[0][h].tolist()))
        o_list[0, h, :len(lst)] = lst
        o_lcnt[0, h] = len(lst)

    # GPU: the same interval-start work, selection with TB_SEL_OMIT_WINDOW
    kc, vc, wk, q = (dev(inp[k], torch.bfloat16) for k in ("kc", "vc", "wk", "q"))
    kp = torch.zeros((B, cfg.Hkv, L0 + I, cfg.dp), dtype=torch.float16, device="cuda")
    tb.tb_project_keys(kc, wk, kp, dev32(np.zeros(B, np.int32)), L0)
    qh = torch.empty((B, cfg.n_out), device="cuda")
    tb.tb_predict_queries(dev(inp["x"], torch.bfloat16), dev(inp["w1"], torch.bfloat16),
                          dev(inp["w2"], torch.bfloat16), qh,
                          tb.new_workspace(tb.tb_predict_workspace_bytes(B, cfg.E, cfg.Eh, cfg.n_out)))
    ctx = dev32(Ln.copy())
    scores = torch.zeros((B, cfg.Hq, L0 + I), device="cuda")
    tb.tb_score(qh, kp, ctx, scores)
    idx = torch.zeros((B, cfg.Hq, cap), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((B, cfg.Hq), dtype=torch.int32, device="cuda")
    tb.tb_select(scores, ctx, ctx, cfg.S, cfg.W, cfg.K, cfg.r, idx, cnt,
                 tb.new_workspace(tb.tb_select_workspace_bytes(B, cfg.Hq, L0 + I)),
                 mode=tb.TB_NF_FILL | tb.TB_SEL_OMIT_WINDOW)
    torch.cuda.synchronize()
    check_selection_band(host(idx), host(cnt), o_list, o_lcnt, o_scores, Ln, Ln, cfg.S, cfg.W,
                         cfg.K, cfg.r, what="omit-window select", window_in_list=False)

    # I steps over the oracle's list; the kernel adds the sliding window
    ws = tb.new_workspace(tb.tb_attn_workspace_bytes(B, cfg.Hq, cap, cfg.W, cfg.D))
    out = torch.zeros((B, cfg.Hq, cfg.D), device="cuda")
    d_list, d_cnt = dev32(o_list), dev32(o_lcnt)
    for j in range(I):
        step_ctx = dev32(np.array([L0 + 1 + j], np.int32))   # the step's token appended
        tb.tb_sparse_decode_attn(q, kc, vc, d_list, d_cnt, out, ws, ctx_len=step_ctx, window=cfg.W)
        torch.cuda.synchronize()
        sets = orc.interval_attended(important, [L0 + 1], j, cfg.S, cfg.W)
        ref_idx = np.zeros((1, cfg.Hq, cap + cfg.W), np.int32)
        ref_cnt = np.zeros((1, cfg.Hq), np.int32)
        for h in range(cfg.Hq):
            ref_idx[0, h, :len(sets[0][h])] = sets[0][h]
            ref_cnt[0, h] = len(sets[0][h])
        ref = orc.sparse_attention(inp["q"], inp["kc"], inp["vc"], ref_idx, ref_cnt)
        assert_attn_close(host(out), ref, "interval step %d" % j)
