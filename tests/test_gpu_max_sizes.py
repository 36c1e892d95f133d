"""GPU parity at the largest sizes the entry points accept or are sized for:
a selection over a 2^24-token context (the largest Lmax: 8192 chunks, the
threshold kernel's chunk table full) with radius 2 on a Gaussian head and a
tie-heavy head; tb_score_select over a 2^24-token projected-key cache with the
largest query group (8 heads per KV head), bitwise equal to tb_score +
tb_select, its scores within 2e-3 of a float64 evaluation at sampled
positions and its lists equal to the oracle's on the same scores; and sparse
attention over 2^19-entry index lists (2048 splits merged per head)."""
import numpy as np
import pytest
import torch

from synthetic import normal_bf16, rng_for
from gpu_util import assert_attn_close, dev, dev32, host, say

pytestmark = pytest.mark.gpu

LMAX = 1 << 24


@pytest.fixture(scope="module")
def tb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import learned_kv_cache_amd as tb
    tb.lib()
    return tb


def _same_lists(gi, gc, ri, rc, what):
    assert np.array_equal(gc, rc), what
    for b in range(rc.shape[0]):
        for h in range(rc.shape[1]):
            n = rc[b, h]
            assert np.array_equal(gi[b, h, :n], ri[b, h, :n]), (what, b, h)


def test_select_at_largest_context(tb, orc):
    S, W, K, r = 64, 256, 120000, 2
    rng = rng_for(81)
    s = rng.standard_normal((1, 2, LMAX)).astype(np.float32)
    s[0, 1] = np.round(s[0, 1] * 2.0)           # few distinct values: long runs of ties
    L = np.array([LMAX], np.int32)
    P = np.array([LMAX - 5], np.int32)           # projection lagging by a few tokens
    cap = S + W + K
    say("max select: oracle")
    ri, rc = orc.select(s, L, P, S, W, K, r, cap)
    say("max select: gpu")
    idx = torch.full((1, 2, cap), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((1, 2), -7, dtype=torch.int32, device="cuda")
    ws = tb.new_workspace(tb.tb_select_workspace_bytes(1, 2, LMAX))
    tb.tb_select(dev32(s), dev32(L), dev32(P), S, W, K, r, idx, cnt, ws)
    torch.cuda.synchronize()
    _same_lists(host(idx), host(cnt), ri, rc, "select 2^24")


def test_score_select_at_largest_context_and_group(tb, orc):
    B, Hq, Hkv, dp = 1, 8, 1, 16
    S, W, K, r = 64, 256, 7872, 1
    gen = torch.Generator(device="cuda")
    gen.manual_seed(82)
    kp = (torch.randn((B, Hkv, LMAX, dp), generator=gen, device="cuda") * 0.5).to(torch.float16)
    qh = torch.randn((B, Hq * dp), generator=gen, device="cuda")
    ctx = dev32(np.array([LMAX], np.int32))
    cap = S + W + K
    ws = tb.new_workspace(tb.tb_select_workspace_bytes(B, Hq, LMAX))
    res = []
    for fused in (False, True):
        say("max score_select: fused" if fused else "max score_select: separate")
        scores = torch.full((B, Hq, LMAX), -3.5, device="cuda")
        idx = torch.full((B, Hq, cap), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((B, Hq), -7, dtype=torch.int32, device="cuda")
        if fused:
            tb.tb_score_select(qh, kp, ctx, ctx, scores, S, W, K, r, idx, cnt, ws)
        else:
            tb.tb_score(qh, kp, ctx, scores)
            tb.tb_select(scores, ctx, ctx, S, W, K, r, idx, cnt, ws)
        torch.cuda.synchronize()
        res.append((scores, host(idx), host(cnt)))
        if not fused:
            del scores
    (s0, i0, c0), (s1, i1, c1) = res
    assert torch.equal(s0.view(torch.int32), s1.view(torch.int32)), "scores differ"
    _same_lists(i1, c1, i0, c0, "fused vs separate")
    # scores against a float64 evaluation at sampled positions (every head)
    rng = rng_for(82, 1)
    pos = np.unique(np.concatenate([rng.integers(0, LMAX, 4000), [0, 1, LMAX - 2, LMAX - 1]]))
    rows = kp[0, 0, torch.from_numpy(pos).cuda()].float().cpu().numpy().astype(np.float64)
    q = host(qh).reshape(Hq, dp).astype(np.float64)
    ref = q @ rows.T                                  # [Hq, npos]
    got = s1[0][:, torch.from_numpy(pos).cuda()].cpu().numpy().astype(np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=1, keepdims=True))
    assert np.all(np.abs(got - ref) <= 2e-3 * np.maximum(np.abs(ref), rms)), "scores off"
    # lists of two heads against the oracle's selection on the same scores
    say("max score_select: oracle")
    s_host = s1[:, :2].contiguous().cpu().numpy()
    del res, s0, s1
    L = np.array([LMAX], np.int32)
    ri, rc = orc.select(s_host, L, L, S, W, K, r, cap)
    _same_lists(i1[:, :2], c1[:, :2], ri, rc, "oracle")


def test_attention_over_largest_lists(tb, orc):
    B, Hq, Hkv, Lmax, D = 1, 4, 1, 1 << 20, 128
    cap = 1 << 19
    rng = rng_for(83)
    say("max attention: inputs")
    kc = normal_bf16(rng, (B, Hkv, Lmax, D))
    vc = normal_bf16(rng, (B, Hkv, Lmax, D))
    q = normal_bf16(rng, (B, Hq, D))
    idx = np.zeros((B, Hq, cap), np.int32)
    for h in range(Hq):
        idx[0, h] = np.sort(rng.choice(Lmax, cap, replace=False)).astype(np.int32)
    cnt = np.array([[cap, cap, cap - 77, 1]], np.int32)   # ragged tail, a single entry
    say("max attention: oracle")
    ref = orc.sparse_attention(q, kc, vc, idx, cnt)
    say("max attention: gpu")
    out = torch.full((B, Hq, D), float("nan"), device="cuda")
    ws = tb.new_workspace(tb.tb_attn_workspace_bytes(B, Hq, cap, 0, D))
    tb.tb_sparse_decode_attn(dev(q, torch.bfloat16), dev(kc, torch.bfloat16),
                             dev(vc, torch.bfloat16), dev32(idx), dev32(cnt), out, ws)
    torch.cuda.synchronize()
    assert_attn_close(host(out), ref, "attention 2^19 entries")
