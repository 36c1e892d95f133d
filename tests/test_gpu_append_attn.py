"""The decode step's append and attention in one launch (tb_append_attn)
against tb_append_kv followed by tb_sparse_decode_attn on copies of the same
state: output, caches, projected keys and lengths bit for bit, step after
step (steps that project the pending keys included), with ragged lengths,
lengths the append refuses (a full cache, a projected length past the
context), no window, D 64 and 128, and the 256K per-layer shape of the
interval workload; the workspace's arrival counters are zero after every
call; and steps captured in a graph, replayed with eager calls between."""
import numpy as np
import pytest
import torch

from synthetic import normal_bf16, normal_f16, rng_for, xavier_bf16
from gpu_util import bits, dev, dev32, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import learned_kv_cache_amd as tb
    tb.lib()
    return tb


def _pad(n):
    return (n + 255) // 256 * 256


def _run(tb, seed, B, Hq, Hkv, Lmax, D, dp, ctx0, proj0, cap, window, n_p, steps):
    say("append_attn", seed, B, Hq, Hkv, Lmax, D, dp, ctx0, proj0, cap, window, n_p, steps)
    rng = rng_for(71, seed)
    kc = dev(normal_bf16(rng, (B, Hkv, Lmax, D)), torch.bfloat16)
    vc = dev(normal_bf16(rng, (B, Hkv, Lmax, D)), torch.bfloat16)
    kp = dev(normal_f16(rng, (B, Hkv, Lmax, dp), std=0.5), torch.float16)
    wk = dev(xavier_bf16(rng, dp, D, lead=(Hkv,)), torch.bfloat16)
    q = dev(normal_bf16(rng, (B, Hq, D)), torch.bfloat16)
    # the interval's list: ascending positions below the first step's window
    idx = np.zeros((B, Hq, cap), np.int32)
    cnt = np.zeros((B, Hq), np.int32)
    for b in range(B):
        top = max(0, min(int(ctx0[b]), Lmax) - window)
        for h in range(Hq):
            n = int(rng.integers(0, min(cap, top) + 1)) if h % 3 else min(cap, top)
            idx[b, h, :n] = np.sort(rng.choice(top, n, replace=False)) if n else []
            cnt[b, h] = n
    idx, cnt = dev32(idx), dev32(cnt)
    st = {k: [t, t.clone()] for k, t in (("kc", kc), ("vc", vc), ("kp", kp))}
    ctx = [dev32(np.asarray(ctx0, np.int32)), dev32(np.asarray(ctx0, np.int32))]
    proj = [dev32(np.asarray(proj0, np.int32)), dev32(np.asarray(proj0, np.int32))]
    nbytes = tb.tb_attn_workspace_bytes(B, Hq, cap, window, D)
    ws = [tb.new_workspace(nbytes), tb.new_workspace(nbytes)]
    nsplit = (cap + window + 255) // 256
    part_bytes = _pad(B * Hq * nsplit * (D + 2) * 4)
    out = [torch.full((B, Hq, D), float("nan"), device="cuda") for _ in range(2)]
    for step in range(steps):
        kn = dev(normal_bf16(rng, (B, Hkv, D)), torch.bfloat16)
        vn = dev(normal_bf16(rng, (B, Hkv, D)), torch.bfloat16)
        tb.tb_append_attn(kn, vn, st["kc"][0], st["vc"][0], st["kp"][0], wk, ctx[0], proj[0], n_p,
                          q, idx, cnt, out[0], ws[0], window=window)
        tb.tb_append_kv(kn, vn, st["kc"][1], st["vc"][1], st["kp"][1], wk, ctx[1], proj[1], n_p)
        tb.tb_sparse_decode_attn(q, st["kc"][1], st["vc"][1], idx, cnt, out[1], ws[1],
                                 ctx_len=ctx[1], window=window)
        torch.cuda.synchronize()
        assert host(ctx[0]).tolist() == host(ctx[1]).tolist(), step
        assert host(proj[0]).tolist() == host(proj[1]).tolist(), step
        assert np.array_equal(host(out[0]).view(np.uint32), host(out[1]).view(np.uint32)), step
        # the per-head and per-sequence arrival counters are back to zero
        assert int(ws[0][-B * Hq * 4:].count_nonzero()) == 0, step
        assert int(ws[0][part_bytes:part_bytes + B * 4].count_nonzero()) == 0, step
    for k in st:
        assert np.array_equal(bits(st[k][0]), bits(st[k][1])), k
    return host(ctx[0]), host(proj[0])


def test_append_attn_matches_separate_calls(tb):
    # sequence 2 fills its cache on the way; sequence 3's projected length
    # lies past its context (the append refuses it every step)
    c, p = _run(tb, 1, 4, 8, 2, 4000, 128, 32, [3000, 1500, 3995, 2000], [3000, 1490, 3995, 2005],
                256, 64, 4, 12)
    assert c.tolist() == [3012, 1512, 4000, 2000] and p.tolist() == [3012, 1509, 3999, 2005]


def test_append_attn_small_shapes(tb):
    _run(tb, 2, 2, 4, 4, 3000, 64, 16, [10, 2999], [10, 2990], 64, 0, 1, 5)     # no window
    _run(tb, 3, 1, 6, 2, 2100, 64, 32, [700], [690], 300, 300, 16, 9)
    _run(tb, 4, 3, 12, 4, 5000, 128, 16, [4000, 0, 4500], [3990, 0, 4499], 512, 128, 8, 4)


def test_append_attn_interval_layer_shape(tb):
    # one layer of the 256K interval workload: 32 query heads, 8 KV heads,
    # sink + budget rows in the list, a 256-row window, projection every 16
    _run(tb, 5, 1, 32, 8, 262144, 128, 32, [262000], [261990], 7936, 256, 16, 3)


def test_append_attn_graph_replays(tb):
    """Steps of the fused call captured in a graph and replayed from the same
    starting lengths, with eager calls between replays: every replay gives
    the eager run's output, lengths and cache rows."""
    B, Hq, Hkv, Lmax, D, dp, cap, window, n_p, steps = 2, 8, 2, 3000, 128, 32, 256, 64, 4, 6
    say("append_attn graph", B, Hq, Lmax, steps)
    rng = rng_for(71, 9)
    kc = dev(normal_bf16(rng, (B, Hkv, Lmax, D)), torch.bfloat16)
    vc = dev(normal_bf16(rng, (B, Hkv, Lmax, D)), torch.bfloat16)
    kp = dev(normal_f16(rng, (B, Hkv, Lmax, dp), std=0.5), torch.float16)
    wk = dev(xavier_bf16(rng, dp, D, lead=(Hkv,)), torch.bfloat16)
    q = dev(normal_bf16(rng, (B, Hq, D)), torch.bfloat16)
    idx = np.zeros((B, Hq, cap), np.int32)
    for b in range(B):
        for h in range(Hq):
            idx[b, h] = np.sort(rng.choice(2000, cap, replace=False))
    idx, cnt = dev32(idx), dev32(np.full((B, Hq), cap, np.int32))
    kn = [dev(normal_bf16(rng, (B, Hkv, D)), torch.bfloat16) for _ in range(steps)]
    vn = [dev(normal_bf16(rng, (B, Hkv, D)), torch.bfloat16) for _ in range(steps)]
    lens0 = dev32(np.array([[2500, 2998], [2497, 2990]], np.int32))   # [ctx, proj] x B
    lens = lens0.clone()
    ws = tb.new_workspace(tb.tb_attn_workspace_bytes(B, Hq, cap, window, D))
    outs = [torch.zeros(B, Hq, D, device="cuda") for _ in range(steps)]

    def run():
        lens.copy_(lens0)
        for j in range(steps):
            tb.tb_append_attn(kn[j], vn[j], kc, vc, kp, wk, lens[0], lens[1], n_p, q, idx, cnt,
                              outs[j], ws, window=window)

    run()
    torch.cuda.synchronize()
    ref = ([host(o).copy() for o in outs], host(lens).copy(), bits(kc).copy(), bits(kp).copy())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            run()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for j in range(steps):
            assert np.array_equal(host(outs[j]).view(np.uint32), ref[0][j].view(np.uint32)), (rep, j)
        assert np.array_equal(host(lens), ref[1]), rep
        assert np.array_equal(bits(kc), ref[2]) and np.array_equal(bits(kp), ref[3]), rep
        run()   # eager work between replays
        torch.cuda.synchronize()
