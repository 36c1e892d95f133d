"""Pins for the oracle's key projection ("Core architecture": key projection,
a learned matrix per consumer layer; "Inference strategy": projection done for
a batch of new tokens) and scoring (predicted query . projected key)."""
import numpy as np

from synthetic import (bf16_bits, bits_to_f32_bf16, bits_to_f32_f16, normal_bf16,
                       normal_f16, rng_for, xavier_bf16)


def test_projection_one_hot_rows(orc):
    # K row t = e_{i(t)}  =>  kp[t, c] = fp16(Wk[c, i(t)])  (Wk is [dp, D])
    B, Hkv, L, D, dp = 1, 2, 40, 64, 16
    rng = np.random.default_rng(5)
    it = rng.integers(0, D, size=(B, Hkv, L))
    kf = np.zeros((B, Hkv, L, D), np.float32)
    for j in range(Hkv):
        kf[0, j, np.arange(L), it[0, j]] = 1.0
    wk = xavier_bf16(rng, dp, D, lead=(Hkv,))
    kp = np.zeros((B, Hkv, L, dp), np.uint16)
    orc.project_keys(bf16_bits(kf), wk, kp, np.zeros(B, np.int32), L)
    wv = bits_to_f32_bf16(wk)
    for j in range(Hkv):
        expect = wv[j][:, it[0, j]].T.astype(np.float16).view(np.uint16)
        assert np.array_equal(kp[0, j], expect)


def test_projection_window_and_bounds(orc):
    B, Hkv, L, D, dp = 2, 1, 30, 64, 16
    rng = np.random.default_rng(6)
    kc = normal_bf16(rng, (B, Hkv, L, D))
    wk = xavier_bf16(rng, dp, D, lead=(Hkv,))
    kp = np.full((B, Hkv, L, dp), 0xBEEF, np.uint16)
    pos0 = np.array([5, 26], np.int32)           # second batch row runs past L
    orc.project_keys(kc, wk, kp, pos0, 8)
    full = np.zeros_like(kp)
    orc.project_keys(kc, wk, full, np.zeros(B, np.int32), L)
    for b, (lo, hi) in enumerate(((5, 13), (26, 30))):
        assert np.array_equal(kp[b, :, lo:hi], full[b, :, lo:hi])
        assert (kp[b, :, :lo] == 0xBEEF).all() and (kp[b, :, hi:] == 0xBEEF).all()


def test_projection_dense_vs_numpy(orc):
    rng = rng_for(1, 92)
    B, Hkv, L, D, dp = 1, 2, 50, 128, 32
    kc = normal_bf16(rng, (B, Hkv, L, D))
    wk = xavier_bf16(rng, dp, D, lead=(Hkv,))
    kp = np.zeros((B, Hkv, L, dp), np.uint16)
    orc.project_keys(kc, wk, kp, np.zeros(B, np.int32), L)
    ref = np.einsum("bjtd,jcd->bjtc", bits_to_f32_bf16(kc).astype(np.float64),
                    bits_to_f32_bf16(wk).astype(np.float64))
    assert np.array_equal(kp, ref.astype(np.float16).view(np.uint16))


def test_score_one_hot_query_and_gqa(orc):
    # q_hat[h] = e_c(h) => scores[h, t] = kp[h // g, t, c(h)] exactly
    B, Hq, Hkv, L, dp = 1, 8, 2, 33, 16
    rng = np.random.default_rng(7)
    kp = normal_f16(rng, (B, Hkv, L, dp))
    ch = rng.integers(0, dp, Hq)
    q = np.zeros((B, Hq, dp), np.float32)
    q[0, np.arange(Hq), ch] = 1.0
    s = orc.score(q.reshape(B, -1), kp, np.array([L], np.int32), Hq)
    kv = bits_to_f32_f16(kp)
    for h in range(Hq):
        assert np.array_equal(s[0, h], kv[0, h // 4, :, ch[h]])


def test_score_slots_lengths_scaling(orc):
    B, Hq, Hkv, L, dp, ns = 2, 4, 2, 20, 16, 3
    rng = np.random.default_rng(8)
    kp = normal_f16(rng, (B, Hkv, L, dp))
    q = rng.standard_normal((B, ns, Hq, dp)).astype(np.float32)
    P = np.array([20, 11], np.int32)
    for slot in range(ns):
        s = orc.score(q.reshape(B, -1), kp, P, Hq, n_slots=ns, slot=slot)
        ref = np.einsum("bhc,bhtc->bht", q[:, slot].astype(np.float64),
                        np.repeat(bits_to_f32_f16(kp).astype(np.float64), 2, axis=1))
        for b in range(B):
            np.testing.assert_allclose(s[b, :, :P[b]], ref[b, :, :P[b]], rtol=1e-6, atol=1e-6)
            assert np.isnan(s[b, :, P[b]:]).all()
    s1 = orc.score(q.reshape(B, -1), kp, P, Hq, n_slots=ns, slot=1)
    s2 = orc.score((2 * q).reshape(B, -1), kp, P, Hq, n_slots=ns, slot=1)
    assert np.array_equal(s2[0], 2 * s1[0])
