"""Pins for the oracle's distillation loss (TokenButler summary, "Training":
the predictor is trained by distilling the frozen model's masked causal
attention distribution, minimizing the cross entropy between the teacher's
attention logits and the predictor's logits, at a subset of query positions
so the cost is O(R L)). Pinned by closed forms (uniform logits give log n;
a student whose logits equal the teacher's gives the teacher's entropy;
a one-hot teacher gives logsumexp(s) - s_j), by library routines on small
inputs (scipy softmax / log_softmax of logits computed with numpy), and by
invariants (tokens after the query position and other KV heads' rows do not
matter)."""
import numpy as np
from scipy.special import log_softmax, logsumexp, softmax
from scipy.stats import entropy

from synthetic import bits_to_f32_bf16, bits_to_f32_f16, f16_bits, normal_bf16, rng_for


def f16(a):
    return f16_bits(np.asarray(a, np.float32))


def make(rng, B=2, R=3, Hq=4, Hkv=2, Lmax=40, D=16, dp=8):
    q = normal_bf16(rng, (B, R, Hq, D))
    kc = normal_bf16(rng, (B, Hkv, Lmax, D))
    qhat = rng.standard_normal((B, R, Hq, dp)).astype(np.float32)
    kp = f16(rng.standard_normal((B, Hkv, Lmax, dp)))
    pos = rng.integers(0, Lmax, size=(B, R)).astype(np.int32)
    return q, kc, qhat, kp, pos


def test_library_routines_small(orc):
    rng = rng_for(100)
    q, kc, qhat, kp, pos = make(rng)
    B, R, Hq, D = q.shape
    Hkv, dp = kc.shape[1], kp.shape[-1]
    got = orc.distill_loss(q, kc, qhat, kp, pos)
    qf, kf = bits_to_f32_bf16(q).astype(np.float64), bits_to_f32_bf16(kc).astype(np.float64)
    kpf = bits_to_f32_f16(kp).astype(np.float64)
    g = Hq // Hkv
    for b in range(B):
        for r in range(R):
            i = pos[b, r]
            for h in range(Hq):
                z = kf[b, h // g, :i + 1] @ qf[b, r, h] / np.sqrt(D)
                s = kpf[b, h // g, :i + 1] @ qhat[b, r, h].astype(np.float64)
                ref = -(softmax(z) * log_softmax(s)).sum()
                assert abs(got[b, r, h] - ref) <= 1e-6 * max(1.0, abs(ref)), (b, r, h)


def test_uniform_logits_give_log_n(orc):
    rng = rng_for(101)
    q, kc, qhat, kp, pos = make(rng)
    kc[:] = kc[:, :, :1]          # every key row the same: uniform teacher
    kp[:] = kp[:, :, :1]          # every projected row the same: uniform student
    got = orc.distill_loss(q, kc, qhat, kp, pos)
    expect = np.log(pos.astype(np.float64) + 1)[:, :, None]
    assert np.allclose(got, np.broadcast_to(expect, got.shape), rtol=1e-6, atol=1e-6)


def test_student_equal_to_teacher_gives_entropy(orc):
    # D = dp, kp = k (bf16 values are exact in fp16 at these magnitudes) and
    # qhat = q / sqrt(D) exactly: s_t = z_t, so the loss is H(p)
    rng = rng_for(102)
    q, kc, _, _, pos = make(rng, D=16, dp=16)
    kp = f16(bits_to_f32_bf16(kc))
    qhat = (bits_to_f32_bf16(q) / 4.0).astype(np.float32)
    got = orc.distill_loss(q, kc, qhat, kp, pos)
    qf, kf = bits_to_f32_bf16(q).astype(np.float64), bits_to_f32_bf16(kc).astype(np.float64)
    B, R, Hq, D = q.shape
    g = Hq // kc.shape[1]
    for b in range(B):
        for r in range(R):
            for h in range(Hq):
                z = kf[b, h // g, :pos[b, r] + 1] @ qf[b, r, h] / 4.0
                assert abs(got[b, r, h] - entropy(softmax(z))) < 1e-6


def test_one_hot_teacher(orc):
    rng = rng_for(103)
    q, kc, qhat, kp, pos = make(rng, B=1, R=2, Hq=2, Hkv=1, Lmax=30)
    pos[:] = [[20, 29]]
    q[:] = 0
    q[..., 0] = 0x4300               # bf16 128.0
    kc[..., 0] = 0                    # only token j carries the first channel
    j = 7
    kc[0, 0, j, 0] = 0x4300
    got = orc.distill_loss(q, kc, qhat, kp, pos)
    kpf = bits_to_f32_f16(kp).astype(np.float64)
    for r in range(2):
        for h in range(2):
            s = kpf[0, 0, :pos[0, r] + 1] @ qhat[0, r, h].astype(np.float64)
            assert abs(got[0, r, h] - (logsumexp(s) - s[j])) < 1e-5


def test_causal_and_head_locality(orc):
    rng = rng_for(104)
    q, kc, qhat, kp, pos = make(rng, Lmax=50)
    pos[:] = [[10, 20, 30], [5, 25, 49]]
    base = orc.distill_loss(q, kc, qhat, kp, pos)
    # rows after every query position of sequence 0 do not matter
    kc2, kp2 = kc.copy(), kp.copy()
    kc2[0, :, 31:] = normal_bf16(rng, kc2[0, :, 31:].shape)
    kp2[0, :, 31:] = f16(rng.standard_normal(kp2[0, :, 31:].shape))
    assert np.array_equal(orc.distill_loss(q, kc2, qhat, kp2, pos)[0], base[0])
    # KV head 1 of sequence 1 changes only query heads 2, 3 of sequence 1
    kc3 = kc.copy()
    kc3[1, 1] = normal_bf16(rng, kc3[1, 1].shape)
    got = orc.distill_loss(q, kc3, qhat, kp, pos)
    assert np.array_equal(got[0], base[0]) and np.array_equal(got[1, :, :2], base[1, :, :2])
    assert not np.array_equal(got[1, :, 2:], base[1, :, 2:])
