"""Pins for the oracle's decode attention over the selected set (TokenButler
summary, "Significance": attend to the selected tokens of the retained full
cache). Checked against torch's scaled_dot_product_attention in float64 on the
CPU (dense causal last row; masked subsets), hand-worked closed forms in
tests/golden/attn_hand.json, and the single-token and equal-logit cases."""
import json
import os

import numpy as np
import torch

from synthetic import bf16_bits, bits_to_f32_bf16, normal_bf16

HERE = os.path.dirname(os.path.abspath(__file__))


def _sdpa(q, k, v, mask=None):
    # q [B,Hq,D], k/v [B,Hkv,L,D] (float values); GQA by repeating KV heads
    B, Hq, D = q.shape
    g = Hq // k.shape[1]
    kk = torch.from_numpy(np.repeat(k, g, axis=1)).double()
    vv = torch.from_numpy(np.repeat(v, g, axis=1)).double()
    qq = torch.from_numpy(q).double()[:, :, None, :]
    m = None if mask is None else torch.from_numpy(mask)[:, :, None, :]
    return torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=m)[:, :, 0].numpy()


def test_dense_equals_sdpa(orc):
    rng = np.random.default_rng(21)
    B, Hq, Hkv, L, D = 2, 8, 2, 150, 64
    q = normal_bf16(rng, (B, Hq, D))
    k = normal_bf16(rng, (B, Hkv, L, D))
    v = normal_bf16(rng, (B, Hkv, L, D))
    idx = np.broadcast_to(np.arange(L, dtype=np.int32), (B, Hq, L)).copy()
    cnt = np.full((B, Hq), L, np.int32)
    out = orc.sparse_attention(q, k, v, idx, cnt)
    ref = _sdpa(bits_to_f32_bf16(q), bits_to_f32_bf16(k), bits_to_f32_bf16(v))
    np.testing.assert_allclose(out, ref, rtol=1e-6, atol=1e-6)


def test_subset_equals_masked_sdpa(orc):
    rng = np.random.default_rng(22)
    B, Hq, Hkv, Lmax, D = 1, 4, 1, 90, 128
    q = normal_bf16(rng, (B, Hq, D))
    k = normal_bf16(rng, (B, Hkv, Lmax, D))
    v = normal_bf16(rng, (B, Hkv, Lmax, D))
    cap = 40
    idx = np.zeros((B, Hq, cap), np.int32)
    cnt = np.zeros((B, Hq), np.int32)
    mask = np.zeros((B, Hq, Lmax), bool)
    for h in range(Hq):
        sel = np.sort(rng.choice(Lmax, 10 + 7 * h, replace=False))
        idx[0, h, :len(sel)] = sel
        cnt[0, h] = len(sel)
        mask[0, h, sel] = True
    out = orc.sparse_attention(q, k, v, idx, cnt)
    ref = _sdpa(bits_to_f32_bf16(q), bits_to_f32_bf16(k), bits_to_f32_bf16(v), mask)
    np.testing.assert_allclose(out, ref, rtol=1e-6, atol=1e-6)


def test_single_token_returns_its_value(orc):
    rng = np.random.default_rng(23)
    q = normal_bf16(rng, (1, 2, 64))
    k = normal_bf16(rng, (1, 1, 10, 64))
    v = normal_bf16(rng, (1, 1, 10, 64))
    idx = np.array([[[7], [3]]], np.int32)
    out = orc.sparse_attention(q, k, v, idx, np.array([[1, 1]], np.int32))
    vf = bits_to_f32_bf16(v)
    assert np.array_equal(out[0, 0], vf[0, 0, 7]) and np.array_equal(out[0, 1], vf[0, 0, 3])


def test_golden_hand_cases(orc):
    g = json.load(open(os.path.join(HERE, "golden", "attn_hand.json")))
    for c in g["cases"]:
        D = c["D"]
        k = bf16_bits(np.array(c["k"], np.float32))[None, None]
        v = bf16_bits(np.array(c["v"], np.float32))[None, None]
        q = bf16_bits(np.array(c["q"], np.float32))[None, None]
        F = np.array(c["F"], np.int32)[None, None]
        out = orc.sparse_attention(q, k, v, F, np.array([[F.shape[-1]]], np.int32), c["scale"])
        np.testing.assert_allclose(out[0, 0], c["out"], rtol=1e-7, atol=1e-7)
