"""GPU parity of CPU-offload decoding: the full K/V cache in pinned host
memory, the sink + important rows gathered once per interval into
per-query-head device buffers, the circular window filled and slid by the
append, attention on the buffers. Against the oracle: the appended host rows
and the gathered buffer rows bit for bit, the new keys' projections within
2e-3, and every step's attention output against the oracle's attention over
the same list plus that step's window (selection lists shared, so the test
isolates the offload path). Once at a small shape with both head sizes, once
at the 256K-context per-layer shape the offload benchmark times."""
import numpy as np
import pytest
import torch

from synthetic import CONFIGS, bits_to_f32_f16, normal_bf16, rng_for, xavier_bf16
from synthetic.workload import make_layer
from gpu_util import assert_attn_close, assert_rel, bits, dev, dev32, host, say
from workloads import oracle_direction

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import learned_kv_cache_amd as tb
    tb.lib()
    return tb


def pinned(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).pin_memory()


@pytest.mark.parametrize("D,dp", [(128, 32), (64, 16)])
def test_offload_interval_matches_oracle(tb, orc, D, dp):
    say("offload", D, dp)
    rng = rng_for(80, D)
    B, Hq, Hkv, Lmax = 2, 8, 2, 3000
    S, W, K, r, I = 16, 64, 300, 1, 5
    L0 = np.array([2500, 1800], np.int32)
    kc = normal_bf16(rng, (B, Hkv, Lmax, D))
    vc = normal_bf16(rng, (B, Hkv, Lmax, D))
    wk = xavier_bf16(rng, dp, D, lead=(Hkv,))
    q = normal_bf16(rng, (B, Hq, D))
    qhat = rng.standard_normal((B, Hq * dp)).astype(np.float32)
    k_host, v_host = pinned(kc), pinned(vc)
    g_wk = dev(wk, torch.bfloat16)
    # setup (not the offload path): project the context from a device copy
    kp = torch.zeros((B, Hkv, Lmax, dp), dtype=torch.float16, device="cuda")
    tb.tb_project_keys(dev(kc, torch.bfloat16), g_wk, kp, dev32(np.zeros(B, np.int32)), int(L0.max()))
    ctx, plen = dev32(L0), dev32(L0)
    scores = torch.empty((B, Hq, Lmax), device="cuda")
    tb.tb_score(dev32(qhat), kp, ctx, scores)
    cap = S + K
    idx = torch.zeros((B, Hq, cap), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((B, Hq), dtype=torch.int32, device="cuda")
    tb.tb_select(scores, ctx, plen, S, W, K, r, idx, cnt,
                 tb.new_workspace(tb.tb_select_workspace_bytes(B, Hq, Lmax)),
                 mode=tb.TB_NF_FILL | tb.TB_SEL_OMIT_WINDOW)
    buf_rows = cap + W
    k_buf = torch.zeros((B, Hq, buf_rows, D), dtype=torch.bfloat16, device="cuda")
    v_buf = torch.zeros_like(k_buf)
    tb.tb_offload_gather(k_host, v_host, idx, cnt, k_buf, v_buf)
    win = np.stack([np.broadcast_to(np.arange(L - W, L, dtype=np.int32), (Hq, W)) for L in L0])
    tb.tb_offload_gather(k_host, v_host, dev32(win), dev32(np.full((B, Hq), W, np.int32)), k_buf,
                         v_buf, slot0=cap, wrap=W)
    torch.cuda.synchronize()
    gi, gc = host(idx), host(cnt)
    kb = bits(k_buf)
    for b in range(B):
        for h in range(Hq):
            rows = gi[b, h, :gc[b, h]]
            assert np.array_equal(kb[b, h, :gc[b, h]], kc[b, h // (Hq // Hkv), rows])
            for t in range(L0[b] - W, L0[b]):
                assert np.array_equal(kb[b, h, cap + t % W], kc[b, h // (Hq // Hkv), t])

    iota = dev32(np.broadcast_to(np.arange(cap, dtype=np.int32), (B, Hq, cap)).copy())
    full = dev32(np.full(B, buf_rows, np.int32))
    out = torch.zeros((B, Hq, D), device="cuda")
    ws = tb.new_workspace(tb.tb_attn_workspace_bytes(B, Hq, cap, W, D))
    g_q = dev(q, torch.bfloat16)
    for j in range(I):
        kn = normal_bf16(rng, (B, Hkv, D))
        vn = normal_bf16(rng, (B, Hkv, D))
        tb.tb_offload_append(dev(kn, torch.bfloat16), dev(vn, torch.bfloat16), g_wk, k_host, v_host,
                             kp, ctx, plen, k_buf, v_buf, W)
        tb.tb_sparse_decode_attn(g_q, k_buf, v_buf, iota, cnt, out, ws, ctx_len=full, window=W)
        torch.cuda.synchronize()
        for b in range(B):
            kc[b, :, L0[b] + j] = kn[b]
            vc[b, :, L0[b] + j] = vn[b]
        assert host(ctx).tolist() == (L0 + j + 1).tolist()
        assert host(plen).tolist() == (L0 + j + 1).tolist()
        # oracle: the shared list plus this step's window
        Lj = L0 + j + 1
        lists = [[np.union1d(gi[b, h, :gc[b, h]], np.arange(Lj[b] - W, Lj[b])) for h in range(Hq)]
                 for b in range(B)]
        n = max(len(x) for row in lists for x in row)
        ref_idx = np.zeros((B, Hq, n), np.int32)
        ref_cnt = np.zeros((B, Hq), np.int32)
        for b in range(B):
            for h in range(Hq):
                ref_idx[b, h, :len(lists[b][h])] = lists[b][h]
                ref_cnt[b, h] = len(lists[b][h])
        ref = orc.sparse_attention(q, kc, vc, ref_idx, ref_cnt)
        assert_attn_close(host(out), ref, "offload step %d" % j)
    # host cache and projections of the appended tokens
    assert np.array_equal(k_host.view(torch.int16).numpy().view(np.uint16), kc)
    assert np.array_equal(v_host.view(torch.int16).numpy().view(np.uint16), vc)
    ref_kp = np.full((B, Hkv, Lmax, dp), 0, np.uint16)
    for b in range(B):
        orc.project_keys(kc[b:b + 1], wk, ref_kp[b:b + 1], np.array([L0[b]], np.int32), I)
    got = bits(kp)
    for b in range(B):
        sl = slice(L0[b], L0[b] + I)
        assert_rel(bits_to_f32_f16(got[b, :, sl]), bits_to_f32_f16(ref_kp[b, :, sl]), 2e-3, "kp")


def test_offload_long_context_shape(tb, orc):
    # the per-layer shape the offload benchmark times: 256K context, B 1,
    # 32 query / 8 KV heads, D 128, sink 64, window 256, budget 7872,
    # radius 2, an interval of 16 steps, the heavy-tailed keys. Queries are
    # predicted and the list selected on the GPU (shared with the oracle, as
    # above); every gathered row, every step's attention on every head, the
    # host cache and the appended projections are checked.
    cfg = CONFIGS[4]
    B, Hq, Hkv, D, dp, g = cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.dp, cfg.g
    S, W, K, r, I, L = cfg.S, cfg.W, cfg.K, cfg.r, cfg.interval, cfg.L
    Lmax = L + I
    say("offload long context", "generating")
    inp = make_layer(cfg, seed=2, Lmax=Lmax, direction_fn=oracle_direction(orc, cfg), n_spans=0,
                     heavy=True)
    kc, vc, wk = inp["kc"], inp["vc"], inp["wk"]
    L0 = inp["ctx_len"].astype(np.int32)
    say("offload long context", "pinning")
    k_host, v_host = pinned(kc), pinned(vc)
    g_wk = dev(wk, torch.bfloat16)
    kp = torch.zeros((B, Hkv, Lmax, dp), dtype=torch.float16, device="cuda")
    kd = dev(kc, torch.bfloat16)
    tb.tb_project_keys(kd, g_wk, kp, dev32(np.zeros(B, np.int32)), int(L0.max()))
    torch.cuda.synchronize()
    del kd
    qhat = torch.empty((B, cfg.n_out), device="cuda")
    tb.tb_predict_queries(dev(inp["x"], torch.bfloat16), dev(inp["w1"], torch.bfloat16),
                          dev(inp["w2"], torch.bfloat16), qhat,
                          tb.new_workspace(tb.tb_predict_workspace_bytes(B, cfg.E, cfg.Eh,
                                                                         cfg.n_out)))
    ctx, plen = dev32(L0), dev32(L0)
    scores = torch.empty((B, Hq, Lmax), device="cuda")
    cap = S + K
    idx = torch.zeros((B, Hq, cap), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((B, Hq), dtype=torch.int32, device="cuda")
    tb.tb_score_select(qhat, kp, ctx, plen, scores, S, W, K, r, idx, cnt,
                       tb.new_workspace(tb.tb_select_workspace_bytes(B, Hq, Lmax)),
                       mode=tb.TB_NF_FILL | tb.TB_SEL_OMIT_WINDOW)
    buf_rows = cap + W
    k_buf = torch.zeros((B, Hq, buf_rows, D), dtype=torch.bfloat16, device="cuda")
    v_buf = torch.zeros_like(k_buf)
    say("offload long context", "gather")
    win = np.stack([np.broadcast_to(np.arange(Lb - W, Lb, dtype=np.int32), (Hq, W)) for Lb in L0])
    tb.tb_offload_gather(k_host, v_host, dev32(win), dev32(np.full((B, Hq), W, np.int32)), k_buf,
                         v_buf, slot0=cap, wrap=W)
    tb.tb_offload_gather(k_host, v_host, idx, cnt, k_buf, v_buf)
    torch.cuda.synchronize()
    gi, gc = host(idx), host(cnt)
    assert (gc == S + K).all(), gc
    kb, vb = bits(k_buf), bits(v_buf)
    for b in range(B):
        for h in range(Hq):
            rows = gi[b, h, :gc[b, h]]
            assert np.array_equal(kb[b, h, :gc[b, h]], kc[b, h // g, rows]), ("K rows", b, h)
            assert np.array_equal(vb[b, h, :gc[b, h]], vc[b, h // g, rows]), ("V rows", b, h)
            wr = np.arange(L0[b] - W, L0[b])
            assert np.array_equal(kb[b, h, cap + wr % W], kc[b, h // g, wr]), ("K window", b, h)
            assert np.array_equal(vb[b, h, cap + wr % W], vc[b, h // g, wr]), ("V window", b, h)

    iota = dev32(np.broadcast_to(np.arange(cap, dtype=np.int32), (B, Hq, cap)).copy())
    full = dev32(np.full(B, buf_rows, np.int32))
    out = torch.zeros((B, Hq, D), device="cuda")
    ws = tb.new_workspace(tb.tb_attn_workspace_bytes(B, Hq, cap, W, D))
    g_q = dev(inp["q"], torch.bfloat16)
    rng = rng_for(81)
    kn = normal_bf16(rng, (I, B, Hkv, D))
    vn = normal_bf16(rng, (I, B, Hkv, D))
    for j in range(I):
        tb.tb_offload_append(dev(kn[j], torch.bfloat16), dev(vn[j], torch.bfloat16), g_wk, k_host,
                             v_host, kp, ctx, plen, k_buf, v_buf, W)
        tb.tb_sparse_decode_attn(g_q, k_buf, v_buf, iota, cnt, out, ws, ctx_len=full, window=W)
        torch.cuda.synchronize()
        for b in range(B):
            kc[b, :, L0[b] + j] = kn[j, b]
            vc[b, :, L0[b] + j] = vn[j, b]
        assert host(ctx).tolist() == (L0 + j + 1).tolist()
        assert host(plen).tolist() == (L0 + j + 1).tolist()
        Lj = L0 + j + 1
        ref_idx = np.zeros((B, Hq, cap + W), np.int32)
        ref_cnt = np.zeros((B, Hq), np.int32)
        for b in range(B):
            for h in range(Hq):
                lst = np.union1d(gi[b, h, :gc[b, h]], np.arange(Lj[b] - W, Lj[b]))
                ref_idx[b, h, :len(lst)] = lst
                ref_cnt[b, h] = len(lst)
        ref = orc.sparse_attention(inp["q"], kc, vc, ref_idx, ref_cnt)
        assert_attn_close(host(out), ref, "offload long context step %d" % j)
    say("offload long context", "host cache and projections")
    for b in range(B):
        sl = slice(int(L0[b]) - 2, int(L0[b]) + I)
        assert np.array_equal(k_host[b, :, sl].view(torch.int16).numpy().view(np.uint16), kc[b, :, sl])
        assert np.array_equal(v_host[b, :, sl].view(torch.int16).numpy().view(np.uint16), vc[b, :, sl])
    assert np.array_equal(k_host.view(torch.int16).numpy().view(np.uint16), kc)
    ref_kp = np.zeros((B, Hkv, Lmax, dp), np.uint16)
    for b in range(B):
        orc.project_keys(kc[b:b + 1], wk, ref_kp[b:b + 1], np.array([L0[b]], np.int32), I)
    got = bits(kp)
    for b in range(B):
        sl = slice(int(L0[b]), int(L0[b]) + I)
        assert_rel(bits_to_f32_f16(got[b, :, sl]), bits_to_f32_f16(ref_kp[b, :, sl]), 2e-3, "kp")
    del k_buf, v_buf, kp, scores
    torch.cuda.empty_cache()
