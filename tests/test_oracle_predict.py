"""Pins for the oracle's query predictor (a two-layer MLP with SiLU between,
"Core architecture": query prediction). The MLP is written in C loops; these
tests check it against structure the definition fixes (one-hot and permutation
weights expose any transposed operand or index slip), against SiLU's closed
form via the identity logistic(z) = (1 + tanh(z/2)) / 2, against exact
scaling laws, and against numpy's float64 matmul on dense random inputs."""
import math

import numpy as np
import torch

from synthetic import bf16_bits, bits_to_f32_bf16, rng_for, xavier_bf16, normal_bf16


def silu_tanh(z):
    return z * (1.0 + np.tanh(z / 2.0)) / 2.0


def bf16_round(v):
    return bf16_bits(np.asarray(v, np.float64).astype(np.float32))


def test_identity_and_permutation_weights(orc):
    # E = Eh = 64, W1 = I, W2 = a permutation: q_hat[n] = bf16(silu(x[pi(n)]))
    E = 64
    rng = np.random.default_rng(3)
    x = normal_bf16(rng, (1, E), std=3.0)
    w1 = bf16_bits(np.eye(E, dtype=np.float32))
    perm = rng.permutation(E)
    w2 = bf16_bits(np.eye(E, dtype=np.float32)[perm])
    h, q = orc.predict_queries(x, w1, w2)
    xv = bits_to_f32_bf16(x[0]).astype(np.float64)
    h_expect = bf16_round(silu_tanh(xv))
    assert np.array_equal(h[0], h_expect)
    assert np.array_equal(q[0], bits_to_f32_bf16(h_expect)[perm])


def test_silu_known_values(orc):
    # z chosen bf16-exact; expected values from the tanh form of the logistic
    zs = np.array([0.0, 1.0, -1.0, 2.0, -2.0, 8.0, -8.0, 0.5], np.float32)
    E = len(zs)
    w1 = bf16_bits(np.eye(E, dtype=np.float32))
    w2 = bf16_bits(np.eye(E, dtype=np.float32))
    h, q = orc.predict_queries(bf16_bits(zs[None]), w1, w2)
    assert q[0, 0] == 0.0
    # silu(1) = 1 * logistic(1) = 0.731058..., silu(-1) = -0.268941...
    assert abs(q[0, 1] - 0.7310585786) < 2 ** -8
    assert abs(q[0, 2] + 0.2689414214) < 2 ** -9
    assert np.array_equal(h[0], bf16_round(silu_tanh(zs.astype(np.float64))))
    # silu(z) - silu(-z) = z (before rounding): check within bf16 rounding
    for a, b, z in ((1, 2, 1.0), (3, 4, 2.0), (5, 6, 8.0)):
        assert abs((q[0, a] - q[0, b]) - z) <= 2 * abs(z) * 2 ** -8


def test_w1_rows_index_outputs(orc):
    # non-square: E = 48 inputs, Eh = 32 outputs; W1[j, pi(j)] = 2^(j % 3)
    E, Eh = 48, 32
    rng = np.random.default_rng(4)
    pi = rng.choice(E, Eh, replace=False)
    w1f = np.zeros((Eh, E), np.float32)
    w1f[np.arange(Eh), pi] = 2.0 ** (np.arange(Eh) % 3)
    x = normal_bf16(rng, (2, E))
    w2 = bf16_bits(np.eye(Eh, dtype=np.float32))
    h, q = orc.predict_queries(x, bf16_bits(w1f), w2)
    xv = bits_to_f32_bf16(x).astype(np.float64)
    z = xv[:, pi] * (2.0 ** (np.arange(Eh) % 3))[None]
    assert np.array_equal(h, bf16_round(silu_tanh(z)))


def test_scaling_and_batch_independence(orc):
    rng = rng_for(1, 90)
    E, Eh, N = 128, 32, 48
    x = normal_bf16(rng, (3, E))
    w1 = xavier_bf16(rng, Eh, E)
    w2 = xavier_bf16(rng, N, Eh)
    h, q = orc.predict_queries(x, w1, w2)
    w2x2 = bf16_bits(bits_to_f32_bf16(w2) * 2)          # exact doubling
    _, q2 = orc.predict_queries(x, w1, w2x2)
    assert np.array_equal(q2, 2 * q)
    for b in range(3):
        hb, qb = orc.predict_queries(x[b:b + 1], w1, w2)
        assert np.array_equal(hb[0], h[b]) and np.array_equal(qb[0], q[b])


def test_dense_random_vs_numpy(orc):
    rng = rng_for(1, 91)
    B, E, Eh, N = 2, 512, 128, 128
    x = normal_bf16(rng, (B, E))
    w1 = xavier_bf16(rng, Eh, E)
    w2 = xavier_bf16(rng, N, Eh)
    h, q = orc.predict_queries(x, w1, w2)
    z = bits_to_f32_bf16(x).astype(np.float64) @ bits_to_f32_bf16(w1).astype(np.float64).T
    h_ref = bf16_round(silu_tanh(z))
    assert np.array_equal(h, h_ref)
    q_ref = bits_to_f32_bf16(h_ref).astype(np.float64) @ bits_to_f32_bf16(w2).astype(np.float64).T
    np.testing.assert_allclose(q, q_ref, rtol=1e-6, atol=1e-7)
