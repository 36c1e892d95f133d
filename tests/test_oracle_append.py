"""Pins for the oracle's decode-step cache append with batched key projection
(TokenButler summary, "Inference strategy": the newest token joins the
retained cache; "Optimizations": the key projection runs once per batch of
new tokens). Pinned by: the appended rows equal the inputs bit for bit and no
other row changes; the projection schedule in closed form (after m appends
from P = L0, proj_len = L0 + floor(m / n_p) n_p); the projected rows equal one
bulk projection of the final cache (the projection itself is pinned in
test_oracle_project_score); a full cache or out-of-range lengths leave
everything unchanged; a projection lag is caught up at the first trigger."""
import numpy as np

from synthetic import normal_bf16, rng_for, xavier_bf16


def setup(B=3, Hkv=2, Lmax=64, D=64, dp=16, seed=0):
    rng = rng_for(90, seed)
    kc = normal_bf16(rng, (B, Hkv, Lmax, D))
    vc = normal_bf16(rng, (B, Hkv, Lmax, D))
    wk = xavier_bf16(rng, dp, D, lead=(Hkv,))
    kp = np.full((B, Hkv, Lmax, dp), 0x7E00, np.uint16)
    return rng, kc, vc, wk, kp


def test_rows_copied_and_schedule_closed_form(orc):
    rng, kc, vc, wk, kp = setup()
    B, Hkv, Lmax, D = kc.shape
    L0 = np.array([5, 17, 30], np.int32)
    ctx, proj = L0.copy(), L0.copy()
    kc0, vc0 = kc.copy(), vc.copy()
    news = []
    n_p = 4
    for m in range(1, 11):
        kn = normal_bf16(rng, (B, Hkv, D))
        vn = normal_bf16(rng, (B, Hkv, D))
        news.append((kn, vn))
        orc.append_kv(kn, vn, kc, vc, kp, wk, ctx, proj, n_p)
        assert (ctx == L0 + m).all()
        assert (proj == L0 + (m // n_p) * n_p).all()
    for b in range(B):
        for m, (kn, vn) in enumerate(news):
            assert np.array_equal(kc[b, :, L0[b] + m], kn[b])
            assert np.array_equal(vc[b, :, L0[b] + m], vn[b])
        rest = np.ones(Lmax, bool)
        rest[L0[b]:L0[b] + len(news)] = False
        assert np.array_equal(kc[b, :, rest], kc0[b, :, rest])
        assert np.array_equal(vc[b, :, rest], vc0[b, :, rest])
    # projected rows equal one bulk projection of the final cache
    ref = np.full_like(kp, 0x7E00)
    orc.project_keys(kc, wk, ref, L0, 8)
    assert np.array_equal(kp, ref)


def test_full_cache_and_bad_lengths_unchanged(orc):
    rng, kc, vc, wk, kp = setup(B=3)
    B, Hkv, Lmax, D = kc.shape
    ctx = np.array([Lmax, 10, 7], np.int32)
    proj = np.array([0, 11, -1], np.int32)     # full; proj > ctx; proj < 0
    before = [a.copy() for a in (kc, vc, kp, ctx, proj)]
    orc.append_kv(normal_bf16(rng, (B, Hkv, D)), normal_bf16(rng, (B, Hkv, D)), kc, vc, kp, wk,
                  ctx, proj, 1)
    for a, b in zip((kc, vc, kp, ctx, proj), before):
        assert np.array_equal(a, b)


def test_projection_lag_caught_up_and_every_step(orc):
    rng, kc, vc, wk, kp = setup(B=2)
    B, Hkv, Lmax, D = kc.shape
    ctx = np.array([20, 9], np.int32)
    proj = np.array([12, 9], np.int32)         # b=0 lags by 8 tokens
    orc.append_kv(normal_bf16(rng, (B, Hkv, D)), normal_bf16(rng, (B, Hkv, D)), kc, vc, kp, wk,
                  ctx, proj, 4)
    assert ctx.tolist() == [21, 10] and proj.tolist() == [21, 9]
    ref = np.full_like(kp, 0x7E00)
    orc.project_keys(kc, wk, ref, np.array([12, 0], np.int32), 9)
    assert np.array_equal(kp[0], ref[0])
    assert (kp[1] == 0x7E00).all()
    # n_p = 1 projects the new token every step
    orc.append_kv(normal_bf16(rng, (B, Hkv, D)), normal_bf16(rng, (B, Hkv, D)), kc, vc, kp, wk,
                  ctx, proj, 1)
    assert ctx.tolist() == [22, 11] and proj.tolist() == [22, 11]
