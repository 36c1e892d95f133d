"""tb_sparse_decode_attn_noalloc: the attention without a workspace (its
partials and arrival counters in the library's fixed per-GPU array) must give
exactly what tb_sparse_decode_attn gives with a caller workspace (the same
kernels), call after call, with calls of different shapes sharing the array
(the second call smaller than the first), and the oracle's result within the
attention tolerance. Calls beyond the array's capacity are rejected before
anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

from synthetic import normal_bf16, rng_for
from gpu_util import assert_attn_close, dev, dev32, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import learned_kv_cache_amd as tb
    tb.lib()
    return tb


def _case(seed, B, Hq, Hkv, L, D, cap):
    rng = rng_for(90, seed, B, Hq, L, D, cap)
    q = normal_bf16(rng, (B, Hq, D))
    kc = normal_bf16(rng, (B, Hkv, L, D))
    vc = normal_bf16(rng, (B, Hkv, L, D))
    idx = np.zeros((B, Hq, cap), np.int32)
    cnt = np.zeros((B, Hq), np.int32)
    for b in range(B):
        for h in range(Hq):
            n = cap if (b + h) % 3 == 0 else int(rng.integers(0, cap + 1))
            idx[b, h, :n] = np.sort(rng.choice(L, n, replace=False))
            cnt[b, h] = n
    return q, kc, vc, idx, cnt


def _run_both(tb, orc, q, kc, vc, idx, cnt, ctx=None, window=0, what=""):
    B, Hq, D = q.shape
    cap = idx.shape[-1]
    dq, dk, dv = dev(q, torch.bfloat16), dev(kc, torch.bfloat16), dev(vc, torch.bfloat16)
    di, dc = dev32(idx), dev32(cnt)
    dctx = None if ctx is None else dev32(ctx)
    want = torch.full((B, Hq, D), float("nan"), device="cuda")
    ws = tb.new_workspace(tb.tb_attn_workspace_bytes(B, Hq, cap, window if ctx is not None else 0, D))
    tb.tb_sparse_decode_attn(dq, dk, dv, di, dc, want, ws, ctx_len=dctx, window=window)
    got = torch.full((B, Hq, D), float("nan"), device="cuda")
    tb.tb_sparse_decode_attn_noalloc(dq, dk, dv, di, dc, got, ctx_len=dctx, window=window)
    torch.cuda.synchronize()
    g, w = host(got), host(want)
    assert np.array_equal(g.view(np.uint32), w.view(np.uint32)), what
    if ctx is None:
        assert_attn_close(g, orc.sparse_attention(q, kc, vc, idx, cnt), what)
    return g


def test_noalloc_equals_workspace_call_on_two_calls_of_different_shapes(tb, orc):
    # first call: the C2 single-layer shape (32 heads, 32 splits per head)
    say("noalloc: C2-shaped call")
    big = _case(0, 1, 32, 8, 65536, 128, 8192)
    _run_both(tb, orc, *big, what="C2-shaped")
    # second call, smaller: other heads, head dim and split count share the
    # array the first call used (its counters must be found at zero)
    say("noalloc: smaller call")
    small = _case(1, 2, 8, 2, 3000, 64, 300)
    _run_both(tb, orc, *small, what="smaller")
    # the smaller shape again with the implicit window, then the big one again
    say("noalloc: window, then the C2 shape again")
    q, kc, vc, idx, cnt = small
    ctx = np.full(q.shape[0], kc.shape[2], np.int32)
    _run_both(tb, orc, q, kc, vc, idx, cnt, ctx=ctx, window=40, what="window")
    _run_both(tb, orc, *big, what="C2-shaped again")


def test_noalloc_repeated_calls_bitwise(tb, orc):
    say("noalloc: repeated calls")
    q, kc, vc, idx, cnt = _case(2, 1, 16, 4, 20000, 128, 4000)
    B, Hq, D = q.shape
    dq, dk, dv = dev(q, torch.bfloat16), dev(kc, torch.bfloat16), dev(vc, torch.bfloat16)
    di, dc = dev32(idx), dev32(cnt)
    outs = []
    for _ in range(5):
        o = torch.full((B, Hq, D), float("nan"), device="cuda")
        tb.tb_sparse_decode_attn_noalloc(dq, dk, dv, di, dc, o)
        outs.append(o)
    torch.cuda.synchronize()
    first = host(outs[0])
    assert_attn_close(first, orc.sparse_attention(q, kc, vc, idx, cnt), "repeat")
    for o in outs[1:]:
        assert np.array_equal(host(o).view(np.uint32), first.view(np.uint32))


def test_noalloc_rejects_calls_beyond_the_array(tb):
    say("noalloc: oversize rejected")
    L = tb.lib()
    # 64 sequences x 32 heads x 128 splits x 130 floats: far beyond 8 MiB
    B, Hq, Hkv, Lmax, D, cap = 64, 32, 8, 65536, 128, 32768
    fake = ctypes.c_void_p(0x10000)
    st = L.tb_sparse_decode_attn_noalloc(fake, fake, fake, fake, fake, cap, None, 0, B, Hq, Hkv,
                                         Lmax, D, ctypes.c_float(0.1), fake, None)
    assert st == tb.TB_ERR_UNSUPPORTED_SHAPE
    assert b"fixed scratch" in L.tb_last_error_detail()
