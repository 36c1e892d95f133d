"""GPU parity: every libtb entry point against the oracle on the same seeded
inputs, through the C ABI. Tolerances: projected keys, predicted queries and
scores within 2e-3 relative (to max(|ref|, row rms)); selections bit-exact
when both sides see the same scores; attention within 1e-2 abs + 2e-2 rel."""
import numpy as np
import pytest
import torch

from synthetic import (CONFIGS, bits_to_f32_bf16, bits_to_f32_f16, integer_scores, normal_bf16,
                       normal_f16, rng_for, xavier_bf16)
from synthetic.workload import make_layer
from gpu_util import (assert_attn_close, assert_rel, bits, check_selection_band, dev, dev32, host,
                      say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import learned_kv_cache_amd as tb
    tb.lib()
    return tb


# ------------------------------------------------------------------ projection

@pytest.mark.parametrize("B,Hkv,L,D,dp,pos0,ntok", [
    (1, 2, 300, 64, 16, [0], 300),
    (2, 2, 333, 64, 32, [5, 310], 40),         # second row runs past Lmax
    (1, 8, 4099, 128, 32, [0], 4099),
    (3, 4, 1000, 128, 16, [999, 17, 640], 16),
    (1, 8, 64, 128, 32, [63], 1),
    (2, 2, 6000, 64, 16, [100, 3000], 4000),   # bulk path; second row runs past Lmax
    (1, 4, 2048, 128, 16, [0], 2048),          # bulk path, exactly one batch multiple
])
def test_project_keys(tb, orc, B, Hkv, L, D, dp, pos0, ntok):
    say("project", B, Hkv, L, D, dp, pos0, ntok)
    rng = rng_for(50, B, Hkv, L, D, dp)
    kc = normal_bf16(rng, (B, Hkv, L, D))
    wk = xavier_bf16(rng, dp, D, lead=(Hkv,))
    ref = np.full((B, Hkv, L, dp), 0x7E00, np.uint16)
    orc.project_keys(kc, wk, ref, np.array(pos0, np.int32), ntok)
    kp = dev(np.full((B, Hkv, L, dp), 0x7E00, np.uint16), torch.float16)
    tb.tb_project_keys(dev(kc, torch.bfloat16), dev(wk, torch.bfloat16), kp,
                       dev32(np.array(pos0, np.int32)), ntok)
    torch.cuda.synchronize()
    got = bits(kp)
    untouched = ref == 0x7E00
    assert np.array_equal(got[untouched], ref[untouched])
    for b in range(B):
        lo, hi = pos0[b], min(L, pos0[b] + ntok)
        assert_rel(bits_to_f32_f16(got[b, :, lo:hi]), bits_to_f32_f16(ref[b, :, lo:hi]), 2e-3,
                   "project b=%d" % b)


def test_project_bulk_equals_small_batches(tb):
    # the whole-context path (>= 2048 tokens per call) and the per-step path
    # (a few tokens per call) give the same bits
    rng = rng_for(51)
    B, Hkv, L, D, dp = 2, 8, 9000, 128, 32
    kc = dev(normal_bf16(rng, (B, Hkv, L, D)), torch.bfloat16)
    wk = dev(xavier_bf16(rng, dp, D, lead=(Hkv,)), torch.bfloat16)
    a = torch.zeros((B, Hkv, L, dp), dtype=torch.float16, device="cuda")
    b = torch.zeros_like(a)
    tb.tb_project_keys(kc, wk, a, dev32(np.array([0, 0], np.int32)), L)
    for p0 in range(0, L, 1500):
        tb.tb_project_keys(kc, wk, b, dev32(np.array([p0, p0], np.int32)), min(1500, L - p0))
    torch.cuda.synchronize()
    assert np.array_equal(bits(a), bits(b))


# ------------------------------------------------------------------ predictor

@pytest.mark.parametrize("B,E,Eh,nout", [(1, 512, 128, 128), (3, 512, 128, 128),
                                          (1, 4096, 1024, 1024), (8, 4096, 1024, 1024),
                                          (4, 3584, 896, 896), (17, 1024, 256, 64)])
def test_predict_queries(tb, orc, B, E, Eh, nout):
    say("predict", B, E, Eh, nout)
    rng = rng_for(51, B, E, Eh, nout)
    x = normal_bf16(rng, (B, E))
    w1 = xavier_bf16(rng, Eh, E)
    w2 = xavier_bf16(rng, nout, Eh)
    _, ref = orc.predict_queries(x, w1, w2)
    q = torch.full((B, nout), float("nan"), device="cuda")
    ws = tb.new_workspace(tb.tb_predict_workspace_bytes(B, E, Eh, nout))
    tb.tb_predict_queries(dev(x, torch.bfloat16), dev(w1, torch.bfloat16), dev(w2, torch.bfloat16),
                          q, ws)
    torch.cuda.synchronize()
    assert_rel(host(q), ref, 2e-3, "predict")


# ------------------------------------------------------------------ scoring

@pytest.mark.parametrize("B,Hq,Hkv,L,dp,P,ns,slot", [
    (1, 8, 2, 300, 16, [300], 1, 0),
    (1, 32, 8, 65536, 32, [65536], 1, 0),
    (2, 28, 4, 5000, 32, [5000, 1234], 2, 1),
    (3, 8, 8, 777, 16, [1, 777, 513], 1, 0),
    (1, 16, 2, 2048, 32, [0], 1, 0),
])
def test_score(tb, orc, B, Hq, Hkv, L, dp, P, ns, slot):
    say("score", B, Hq, Hkv, L, dp, P, ns, slot)
    rng = rng_for(52, B, Hq, L, dp)
    kp = normal_f16(rng, (B, Hkv, L, dp), std=0.5)
    qh = rng.standard_normal((B, ns * Hq * dp)).astype(np.float32)
    Pn = np.array(P, np.int32)
    ref = orc.score(qh, kp, Pn, Hq, n_slots=ns, slot=slot)
    s = torch.full((B, Hq, L), float("nan"), device="cuda")
    tb.tb_score(dev32(qh), dev(kp, torch.float16), dev32(Pn), s, n_slots=ns, slot=slot)
    torch.cuda.synchronize()
    got = host(s)
    for b in range(B):
        assert np.isnan(got[b, :, P[b]:]).all()
        if P[b]:
            assert_rel(got[b, :, :P[b]], ref[b, :, :P[b]], 2e-3, "score b=%d" % b)


# ------------------------------------------------------------------ selection

def run_select(tb, scores, L, P, S, W, K, r, cap=None, ws=None, dilate=False, omit=False):
    B, Hq, Lmax = scores.shape
    imp = (2 * r + 1) * K if dilate else K
    cap = cap or min(Lmax, S + (0 if omit else W) + imp)
    idx = torch.full((B, Hq, cap), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, Hq), -7, dtype=torch.int32, device="cuda")
    if ws is None:
        ws = tb.new_workspace(tb.tb_select_workspace_bytes(B, Hq, Lmax))
    mode = (tb.TB_NF_DILATE if dilate else tb.TB_NF_FILL) | (tb.TB_SEL_OMIT_WINDOW if omit else 0)
    tb.tb_select(dev32(scores), dev32(np.asarray(L, np.int32)), dev32(np.asarray(P, np.int32)),
                 S, W, K, r, idx, cnt, ws, mode=mode)
    torch.cuda.synchronize()
    return host(idx), host(cnt), ws


def assert_same_selection(orc, tb, scores, L, P, S, W, K, r, what, ws=None, dilate=False):
    say("select", what, scores.shape, S, W, K, r, "dilate" if dilate else "fill")
    cap = min(scores.shape[-1], S + W + ((2 * r + 1) * K if dilate else K))
    ri, rc = orc.select(scores, np.asarray(L, np.int32), np.asarray(P, np.int32), S, W, K, r, cap,
                        dilate=dilate)
    gi, gc, ws = run_select(tb, scores, L, P, S, W, K, r, cap, ws, dilate=dilate)
    assert np.array_equal(gc, rc), what
    for b in range(rc.shape[0]):
        for h in range(rc.shape[1]):
            n = rc[b, h]
            assert np.array_equal(gi[b, h, :n], ri[b, h, :n]), (what, b, h)
    return ws


@pytest.mark.parametrize("r", [0, 1, 2])
def test_select_c1_shapes(tb, orc, r):
    rng = rng_for(53, r)
    s = rng.standard_normal((1, 8, 300)).astype(np.float32)
    assert_same_selection(orc, tb, s, [300], [300], 4, 16, 32, r, "c1 r=%d" % r)


@pytest.mark.parametrize("r", [1, 2])
def test_select_c2_shapes(tb, orc, r):
    rng = rng_for(54, r)
    s = rng.standard_normal((1, 32, 65536)).astype(np.float32)
    assert_same_selection(orc, tb, s, [65536], [65536], 64, 256, 7872, r, "c2 r=%d" % r)



def test_select_c4_shape_heavy_tail(tb, orc):
    # 256K context, radius 2, one percent of positions per head shifted up by
    # 2.5 score standard deviations (the long-context workload's heavy tail)
    rng = rng_for(65)
    L = 262144
    s = rng.standard_normal((1, 32, L)).astype(np.float32)
    for h in range(32):
        pos = rng.integers(64, L - 256, size=L // 100)
        s[0, h, pos] += 2.5
    assert_same_selection(orc, tb, s, [L], [L], 64, 256, 7872, 2, "c4 heavy tail")


def test_select_c3_batch(tb, orc):
    # the 32-layer workload's batch of 8 sequences: 256 segments in one call
    rng = rng_for(66)
    s = rng.standard_normal((8, 32, 65536)).astype(np.float32)
    L = [65536, 65000, 64000, 50000, 65536, 30000, 65535, 40001]
    assert_same_selection(orc, tb, s, L, L, 64, 256, 7872, 1, "c3 batch")

def test_select_tie_heavy_and_large_candidate_groups(tb, orc):
    rng = rng_for(55)
    # integer scores: few distinct values, the band around the budget's key holds thousands of ties
    s = integer_scores(rng, (2, 4, 20000), -3, 4)
    s[:, :, ::7] = -0.0
    assert_same_selection(orc, tb, s, [20000, 15001], [20000, 14900], 16, 64, 3000, 1, "ints r1")
    assert_same_selection(orc, tb, s, [20000, 15001], [20000, 14900], 16, 64, 3000, 2, "ints r2")
    # all equal: one bin holds all of E (candidate list beyond LDS)
    z = np.zeros((1, 2, 30000), np.float32)
    assert_same_selection(orc, tb, z, [30000], [30000], 8, 32, 12000, 1, "all-equal")


def test_select_edge_cases(tb, orc):
    rng = rng_for(56)
    s = rng.standard_normal((3, 4, 1000)).astype(np.float32)
    L = [1000, 400, 60]
    assert_same_selection(orc, tb, s, L, L, 8, 32, 10000, 1, "budget >= |E|")
    assert_same_selection(orc, tb, s, L, L, 8, 32, 0, 1, "budget 0")
    assert_same_selection(orc, tb, s, [30, 40, 39], [30, 40, 39], 8, 32, 5, 1, "L <= S + W")
    assert_same_selection(orc, tb, s, L, [500, 100, 60], 8, 32, 100, 2, "projection lag")
    assert_same_selection(orc, tb, s, [1, 1, 2], [1, 1, 2], 0, 0, 1, 0, "tiny")
    pm = np.full((1, 1, 12), -0.0, np.float32)
    pm[0, 0, 5] = 0.0
    assert_same_selection(orc, tb, pm, [12], [12], 2, 2, 1, 0, "+0 above -0")


def test_select_bad_lengths_flagged(tb, orc):
    s = np.zeros((2, 2, 100), np.float32)
    gi, gc, _ = run_select(tb, s, [100, 101], [100, 50], 4, 8, 10, 1)
    assert (gc[1] == -1).all() and (gc[0] == 22).all()


def test_select_workspace_reuse(tb, orc):
    rng = rng_for(57)
    B, Hq, Lmax = 2, 8, 9000
    ws = tb.new_workspace(tb.tb_select_workspace_bytes(B, Hq, Lmax))
    for i in range(3):
        s = rng.standard_normal((B, Hq, Lmax)).astype(np.float32)
        ws = assert_same_selection(orc, tb, s, [9000, 7777], [9000, 7700], 16, 64, 900, 1,
                                   "reuse %d" % i, ws)
        assert int(ws[: B * Hq * 4].count_nonzero()) == 0   # arrival counters back at zero


def _sample_positions(e0, e1, Lmax):
    """Eligible positions whose pooled keys the band estimate samples: every
    stride-th token from e0 + stride // 2, stride = ceil((Lmax - e0) / 8192)
    (e0 = the sink size)."""
    stride = max(1, -(-(Lmax - e0) // 8192))
    return np.arange(e0 + stride // 2, e1, stride), stride


def _band_missed(ws, scores, L, S, W, K, r):
    """Per segment: whether the key band left in the selection workspace
    misses the budget's key, i.e. with A eligible tokens whose pooled key32
    lies above the band and C inside it, need - A falls outside [0, C]."""
    B, Hq, Lmax = scores.shape
    up = lambda x: (x + 255) // 256 * 256
    info = host(ws[up(B * Hq * 4): up(B * Hq * 4) + B * Hq * 8].view(torch.int32))
    info = (info.astype(np.int64) & 0xFFFFFFFF).reshape(-1, 2)
    out = []
    for b in range(B):
        e0, e1 = S, max(S, L[b] - W)
        need = min(K, e1 - e0)
        for h in range(Hq):
            u = scores[b, h, e0:e1].view(np.uint32).astype(np.int64)
            key = np.where(u >> 31, u ^ 0xFFFFFFFF, u ^ 0x80000000)
            pooled = key.copy()
            for d in range(1, r + 1):
                pooled[d:] = np.maximum(pooled[d:], key[:-d])
                pooled[:-d] = np.maximum(pooled[:-d], key[d:])
            tlo, thi = info[b * Hq + h, 0], info[b * Hq + h, 1]
            A = int((pooled > thi).sum())
            C = int(((pooled >= tlo) & (pooled <= thi)).sum())
            out.append(not (0 <= need - A <= C))
    return np.array(out)


def _around(pos, r, lo, hi):
    """Positions within r of any of pos, clipped to [lo, hi)."""
    p = (pos[:, None] + np.arange(-r, r + 1)[None, :]).ravel()
    return np.unique(p[(p >= lo) & (p < hi)])


@pytest.mark.parametrize("r", [0, 1, 2])
def test_select_band_miss_takes_exact_path(tb, orc, r):
    """Scores built so that the sampled tokens misrepresent the segment: in
    head 0 every sampled token outranks every other token (the band sits far
    above the budget's key), in head 1 every token within r of a sampled one
    is below all the others, so every sampled pooled key is low (the band sits
    far below it). Head 2 is plain noise. The result must still equal the
    oracle's, and heads 0 and 1 must have taken the exact fallback."""
    rng = rng_for(58, r)
    B, Hq, L, S, W, K = 1, 3, 70000, 16, 64, 4000
    s = rng.standard_normal((B, Hq, L)).astype(np.float32)
    pos, stride = _sample_positions(S, L - W, L)
    assert stride > 2 * r + 1
    s[0, 0, pos] += 100.0
    s[0, 1, _around(pos, r, S, L - W)] -= 100.0
    ws = assert_same_selection(orc, tb, s, [L], [L], S, W, K, r, "band miss r=%d" % r)
    assert _band_missed(ws, s, [L], S, W, K, r).tolist() == [True, True, False]


def test_select_band_miss_with_ties(tb, orc):
    rng = rng_for(59)
    B, Hq, L, S, W, K = 1, 2, 70000, 8, 32, 2500
    for r in (0, 1, 2):
        s = integer_scores(rng, (B, Hq, L), -3, 4)
        pos, _ = _sample_positions(S, L - W, L)
        s[0, 0, pos] = 9.0
        s[0, 1, _around(pos, r, S, L - W)] = -9.0
        assert_same_selection(orc, tb, s, [L], [L], S, W, K, r, "band miss ties r=%d" % r)


@pytest.mark.parametrize("r", [0, 1])
def test_select_threshold_staging_beyond_prefetched_slots(tb, orc, r):
    """With at most 32 chunks per segment the threshold launch fetches each
    chunk's first 96 candidate slots with the chunk counts and reads the rest
    afterwards. Tie-heavy scores put every token of one score value in the
    band (hundreds of candidates per chunk, a few thousand per segment, inside
    the LDS limit); the lists must equal the oracle's, and the workspace must
    show chunks beyond the prefetched slots."""
    rng = rng_for(60, r)
    B, Hq, L, S, W, K = 1, 2, 20000, 16, 64, 5000
    s = integer_scores(rng, (B, Hq, L), -3, 4)
    ws = assert_same_selection(orc, tb, s, [L], [L], S, W, K, r, "staging r=%d" % r)
    up = lambda x: (x + 255) // 256 * 256
    nseg, nchunks = B * Hq, -(-L // 2048)
    off = up(nseg * 4) + up(nseg * 8) + up(nseg * 12)   # counters, band, bin info
    cc = host(ws[off: off + nseg * nchunks * 4].view(torch.int32)).reshape(nseg, nchunks)
    assert nchunks <= 32
    assert (cc.max(axis=1) > 96).all() and (cc.sum(axis=1) <= 8192).all(), cc


def test_select_threshold_candidates_beyond_lds(tb, orc):
    """At most 32 chunks but more candidates than the threshold launch holds
    in LDS (three score values, about 20 K tokens tied on the budget's one):
    the candidates are then read from global memory, not staged; the lists
    must still equal the oracle's."""
    rng = rng_for(61)
    B, Hq, L, S, W, K = 1, 2, 60000, 16, 64, 30000
    s = integer_scores(rng, (B, Hq, L), -1, 2)
    ws = assert_same_selection(orc, tb, s, [L], [L], S, W, K, 0, "candidates beyond LDS")
    up = lambda x: (x + 255) // 256 * 256
    nseg, nchunks = B * Hq, -(-L // 2048)
    off = up(nseg * 4) + up(nseg * 8) + up(nseg * 12)   # counters, band, bin info
    cc = host(ws[off: off + nseg * nchunks * 4].view(torch.int32)).reshape(nseg, nchunks)
    assert nchunks <= 32 and (cc.sum(axis=1) > 8192).all(), cc.sum(axis=1)


# ------------------------------------------------- selection, dilation mode

@pytest.mark.parametrize("r", [0, 1, 2])
def test_select_dilate_c1_shapes(tb, orc, r):
    rng = rng_for(60, r)
    s = rng.standard_normal((1, 8, 300)).astype(np.float32)
    assert_same_selection(orc, tb, s, [300], [300], 4, 16, 32, r, "dilate c1 r=%d" % r, dilate=True)


def test_select_dilate_c2_shape(tb, orc):
    rng = rng_for(61)
    s = rng.standard_normal((1, 32, 65536)).astype(np.float32)
    assert_same_selection(orc, tb, s, [65536], [65536], 64, 256, 7872, 1, "dilate c2",
                          dilate=True)
    assert_same_selection(orc, tb, s, [65536], [65536], 64, 256, 7872, 2, "dilate c2 r=2",
                          dilate=True)


def test_select_dilate_c4_shape_heavy_tail(tb, orc):
    # the 256K-context segment with radius 2 and its heavy tail (one percent of
    # positions per head shifted up by 2.5), a full-length and a ragged sequence
    rng = rng_for(67)
    L = 262144
    s = rng.standard_normal((2, 32, L)).astype(np.float32)
    for b in range(2):
        for h in range(32):
            pos = rng.integers(64, L - 256, size=L // 100)
            s[b, h, pos] += 2.5
    assert_same_selection(orc, tb, s, [L, 200001], [L, 199990], 64, 256, 7872, 2,
                          "dilate c4 heavy tail", dilate=True)


def test_select_dilate_ties_edges_and_max_radius(tb, orc):
    rng = rng_for(62)
    s = integer_scores(rng, (2, 4, 20000), -3, 4)
    s[:, :, ::7] = -0.0
    for r in (1, 2):
        assert_same_selection(orc, tb, s, [20000, 15001], [20000, 14900], 16, 64, 900, r,
                              "dilate ints r%d" % r, dilate=True)
    e = rng.standard_normal((3, 4, 1000)).astype(np.float32)
    L = [1000, 400, 60]
    assert_same_selection(orc, tb, e, L, L, 8, 32, 10000, 1, "dilate budget >= |E|", dilate=True)
    assert_same_selection(orc, tb, e, L, L, 8, 32, 0, 1, "dilate budget 0", dilate=True)
    assert_same_selection(orc, tb, e, L, [500, 100, 60], 8, 32, 40, 2, "dilate projection lag",
                          dilate=True)
    assert_same_selection(orc, tb, e, [1, 1, 2], [1, 1, 2], 0, 0, 1, 3, "dilate tiny", dilate=True)
    # radius 64 spans chunk boundaries: centres next to every 2048-token edge
    m = rng.uniform(-1, 0, (1, 2, 9000)).astype(np.float32)
    m[:, :, [2047, 2048, 4095, 6144, 8191, 100, 8900]] = 5.0
    assert_same_selection(orc, tb, m, [9000], [9000], 16, 32, 7, 64, "dilate r=64 chunk edges",
                          dilate=True)
    assert_same_selection(orc, tb, m, [9000], [9000], 16, 32, 150, 64, "dilate r=64 overlap",
                          dilate=True)


def test_select_dilate_band_miss(tb, orc):
    rng = rng_for(63)
    B, Hq, L, S, W, K = 1, 2, 70000, 16, 64, 3000
    s = rng.standard_normal((B, Hq, L)).astype(np.float32)
    pos, _ = _sample_positions(S, L - W, L)
    s[0, 0, pos] += 100.0
    s[0, 1, pos] -= 100.0
    assert_same_selection(orc, tb, s, [L], [L], S, W, K, 2, "dilate band miss", dilate=True)


def test_select_dilate_omit_window(tb, orc):
    rng = rng_for(64)
    B, Hq, L, S, W, K, r = 2, 4, 6000, 8, 64, 500, 2
    s = rng.standard_normal((B, Hq, L)).astype(np.float32)
    Ls = np.array([6000, 4321], np.int32)
    gi, gc, _ = run_select(tb, s, Ls, Ls, S, W, K, r, dilate=True, omit=True)
    ri, rc = orc.select(s, Ls, Ls, S, W, K, r, dilate=True)
    for b in range(B):
        for h in range(Hq):
            ref = ri[b, h, :rc[b, h]]
            ref = ref[ref < Ls[b] - W]
            assert np.array_equal(gi[b, h, :gc[b, h]], ref), (b, h)


# ------------------------------------------------------------------ attention

# the last two: more split partials per head than one merge pass takes (32
# at D = 128, 64 at D = 64)
@pytest.mark.parametrize("B,Hq,Hkv,L,D,cap", [(1, 8, 2, 300, 64, 52), (2, 32, 8, 5000, 128, 700),
                                              (1, 28, 4, 3000, 128, 3000), (1, 4, 1, 600, 64, 513),
                                              (1, 8, 2, 30000, 128, 20000),
                                              (1, 4, 2, 40000, 64, 33000)])
def test_attention_random_sets(tb, orc, B, Hq, Hkv, L, D, cap):
    say("attn", B, Hq, Hkv, L, D, cap)
    rng = rng_for(58, B, Hq, L, D, cap)
    q = normal_bf16(rng, (B, Hq, D))
    kc = normal_bf16(rng, (B, Hkv, L, D))
    vc = normal_bf16(rng, (B, Hkv, L, D))
    idx = np.zeros((B, Hq, cap), np.int32)
    cnt = np.zeros((B, Hq), np.int32)
    for b in range(B):
        for h in range(Hq):
            n = int(rng.integers(0, cap + 1)) if (b + h) % 5 else cap
            if (b + h) % 11 == 3:
                n = 0
            sel = np.sort(rng.choice(L, n, replace=False)).astype(np.int32)
            idx[b, h, :n] = sel
            cnt[b, h] = n
    ref = orc.sparse_attention(q, kc, vc, idx, cnt)
    out = torch.full((B, Hq, D), float("nan"), device="cuda")
    ws = tb.new_workspace(tb.tb_attn_workspace_bytes(B, Hq, cap, 0, D))
    for rep in range(2):                        # the arrival counters reset themselves
        tb.tb_sparse_decode_attn(dev(q, torch.bfloat16), dev(kc, torch.bfloat16),
                                 dev(vc, torch.bfloat16), dev32(idx), dev32(cnt), out, ws)
        torch.cuda.synchronize()
        assert_attn_close(host(out), ref, "attn rep %d" % rep)


def test_attention_dense_equals_full_budget(tb, orc):
    say("attn dense")
    rng = rng_for(59)
    B, Hq, Hkv, L, D = 1, 8, 2, 4000, 128
    q = normal_bf16(rng, (B, Hq, D))
    kc = normal_bf16(rng, (B, Hkv, L, D))
    vc = normal_bf16(rng, (B, Hkv, L, D))
    idx = np.broadcast_to(np.arange(L, dtype=np.int32), (B, Hq, L)).copy()
    cnt = np.full((B, Hq), L, np.int32)
    out = torch.zeros((B, Hq, D), device="cuda")
    ws = tb.new_workspace(tb.tb_attn_workspace_bytes(B, Hq, L, 0, D))
    tb.tb_sparse_decode_attn(dev(q, torch.bfloat16), dev(kc, torch.bfloat16),
                             dev(vc, torch.bfloat16), dev32(idx), dev32(cnt), out, ws)
    torch.cuda.synchronize()
    # dense causal attention, last query row, fp64 CPU library routine
    kk = torch.from_numpy(np.repeat(bits_to_f32_bf16(kc), 4, axis=1)).double()
    vv = torch.from_numpy(np.repeat(bits_to_f32_bf16(vc), 4, axis=1)).double()
    qq = torch.from_numpy(bits_to_f32_bf16(q)).double()[:, :, None]
    dense = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)[:, :, 0].numpy()
    assert_attn_close(host(out), dense, "dense")


def test_attention_repeatable_bitwise_at_c2_shape(tb, orc):
    """The split partials are handed between workgroups through agent-scope
    atomics and an arrival counter; repeated launches must give bitwise
    identical outputs (the merge order is fixed), and match the oracle."""
    say("attn repeat c2 shape")
    rng = rng_for(60)
    B, Hq, Hkv, L, D, cap = 1, 32, 8, 65536, 128, 8192
    q = normal_bf16(rng, (B, Hq, D))
    kc = normal_bf16(rng, (B, Hkv, L, D))
    vc = normal_bf16(rng, (B, Hkv, L, D))
    idx = np.zeros((B, Hq, cap), np.int32)
    for h in range(Hq):
        idx[0, h] = np.sort(rng.choice(L, cap, replace=False))
    cnt = np.full((B, Hq), cap, np.int32)
    cnt[0, 5] = 1000
    ref = orc.sparse_attention(q, kc, vc, idx, cnt)
    dq, dk, dv = dev(q, torch.bfloat16), dev(kc, torch.bfloat16), dev(vc, torch.bfloat16)
    di, dc = dev32(idx), dev32(cnt)
    ws = tb.new_workspace(tb.tb_attn_workspace_bytes(B, Hq, cap, 0, D))
    outs = []
    for rep in range(20):
        out = torch.full((B, Hq, D), float("nan"), device="cuda")
        tb.tb_sparse_decode_attn(dq, dk, dv, di, dc, out, ws)
        outs.append(out)
    torch.cuda.synchronize()
    first = host(outs[0])
    assert_attn_close(first, ref, "attn c2 shape")
    for rep, o in enumerate(outs[1:], 1):
        assert np.array_equal(host(o).view(np.uint32), first.view(np.uint32)), rep
    # the arrival counters (one per head, at the end of the workspace) are back to zero
    assert int(ws[-B * Hq * 4:].count_nonzero()) == 0


@pytest.mark.parametrize("B,E,Eh,nout,Hkv,L,D,dp,ntok", [(1, 4096, 1024, 1024, 8, 4096, 128, 32, 1),
                                                        (3, 512, 128, 128, 2, 300, 64, 16, 16)])
def test_predict_project_fused_equals_separate(tb, orc, B, E, Eh, nout, Hkv, L, D, dp, ntok):
    say("predict+project fused", B, E, Eh, Hkv, L, ntok)
    rng = rng_for(61, B, E, L)
    x = dev(normal_bf16(rng, (B, E)), torch.bfloat16)
    w1 = dev(xavier_bf16(rng, Eh, E), torch.bfloat16)
    w2 = dev(xavier_bf16(rng, nout, Eh), torch.bfloat16)
    kc = dev(normal_bf16(rng, (B, Hkv, L, D)), torch.bfloat16)
    wk = dev(xavier_bf16(rng, dp, D, lead=(Hkv,)), torch.bfloat16)
    pos0 = dev32((L - ntok - np.arange(B)).astype(np.int32))
    ws = tb.new_workspace(tb.tb_predict_workspace_bytes(B, E, Eh, nout))
    q1 = torch.empty(B, nout, device="cuda")
    kp1 = torch.zeros(B, Hkv, L, dp, dtype=torch.float16, device="cuda")
    tb.tb_predict_queries(x, w1, w2, q1, ws)
    tb.tb_project_keys(kc, wk, kp1, pos0, ntok)
    q2 = torch.empty(B, nout, device="cuda")
    kp2 = torch.zeros(B, Hkv, L, dp, dtype=torch.float16, device="cuda")
    tb.tb_predict_project(x, w1, w2, q2, ws, kc, wk, kp2, pos0, ntok)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2)
    assert torch.equal(kp1.view(torch.int16), kp2.view(torch.int16))
