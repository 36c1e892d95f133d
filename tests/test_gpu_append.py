"""GPU parity of the decode-step cache append with batched projection
(tb_append_kv) against the oracle, step by step: lengths exactly, K/V rows
bit for bit, projected rows within 2e-3 of the oracle and bit-identical to a
projection of the final cache by tb_project_keys."""
import numpy as np
import pytest
import torch

from synthetic import bits_to_f32_f16, normal_bf16, rng_for, xavier_bf16
from gpu_util import assert_rel, bits, dev, dev32, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import learned_kv_cache_amd as tb
    tb.lib()
    return tb


@pytest.mark.parametrize("D,dp,n_p", [(128, 32, 4), (64, 16, 1), (128, 16, 16)])
def test_append_matches_oracle(tb, orc, D, dp, n_p):
    say("append", D, dp, n_p)
    rng = rng_for(70, D, dp, n_p)
    B, Hkv, Lmax = 4, 4, 300
    kc = normal_bf16(rng, (B, Hkv, Lmax, D))
    vc = normal_bf16(rng, (B, Hkv, Lmax, D))
    wk = xavier_bf16(rng, dp, D, lead=(Hkv,))
    kp = np.full((B, Hkv, Lmax, dp), 0x7E00, np.uint16)
    ctx = np.array([5, 100, 297, 300], np.int32)     # the last cache is full
    proj = np.array([5, 92, 297, 0], np.int32)       # sequence 1 lags by 8
    g_kc, g_vc = dev(kc, torch.bfloat16), dev(vc, torch.bfloat16)
    g_kp = dev(kp, torch.float16)
    g_wk = dev(wk, torch.bfloat16)
    g_ctx, g_proj = dev32(ctx), dev32(proj)
    proj0 = proj.copy()
    for step in range(20):
        kn = normal_bf16(rng, (B, Hkv, D))
        vn = normal_bf16(rng, (B, Hkv, D))
        orc.append_kv(kn, vn, kc, vc, kp, wk, ctx, proj, n_p)
        tb.tb_append_kv(dev(kn, torch.bfloat16), dev(vn, torch.bfloat16), g_kc, g_vc, g_kp, g_wk,
                        g_ctx, g_proj, n_p)
        torch.cuda.synchronize()
        assert host(g_ctx).tolist() == ctx.tolist(), step
        assert host(g_proj).tolist() == proj.tolist(), step
    assert np.array_equal(bits(g_kc), kc) and np.array_equal(bits(g_vc), vc)
    got = bits(g_kp)
    untouched = kp == 0x7E00
    assert np.array_equal(got[untouched], kp[untouched])
    again = torch.full_like(g_kp, float("nan"))
    tb.tb_project_keys(g_kc, g_wk, again, dev32(np.zeros(B, np.int32)), Lmax)
    torch.cuda.synchronize()
    again = bits(again)
    for b in range(B):
        lo, hi = proj0[b], proj[b]
        if hi > lo:
            assert_rel(bits_to_f32_f16(got[b, :, lo:hi]), bits_to_f32_f16(kp[b, :, lo:hi]), 2e-3,
                       "append kp b=%d" % b)
            assert np.array_equal(got[b, :, lo:hi], again[b, :, lo:hi])
