"""Seeded generators. Every tensor is drawn in float32 or float64 and rounded
to its storage format (bfloat16 / float16, round-to-nearest-even) by torch's
or numpy's own casts; 16-bit tensors are returned as raw uint16 bit patterns so
that both the GPU library and the CPU oracle read identical bytes.
"""
import numpy as np
import torch

__all__ = [
    "rng_for", "bf16_bits", "bits_to_f32_bf16", "f16_bits", "bits_to_f32_f16",
    "normal_bf16", "xavier_bf16", "normal_f16", "span_starts", "add_direction_bf16",
    "ragged_lengths", "integer_scores",
]

BASE_SEED = 20260101


def rng_for(cid, *path):
    """A numpy Generator for one (config, tensor kind, ...) slice, so that any
    slice can be regenerated on its own."""
    ss = np.random.SeedSequence([BASE_SEED + int(cid)] + [int(p) for p in path])
    return np.random.default_rng(ss)


def bf16_bits(a):
    """float32/float64 array -> uint16 bfloat16 bits (torch's RNE cast)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bits_to_f32_bf16(bits):
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32)


def f16_bits(a):
    return np.ascontiguousarray(a, dtype=np.float64).astype(np.float16).view(np.uint16)


def bits_to_f32_f16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def normal_bf16(rng, shape, mean=0.0, std=1.0):
    return bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
                     + np.float32(mean))


def xavier_bf16(rng, fan_out, fan_in, lead=()):
    """Xavier-uniform (gain 1) weight of shape lead + (fan_out, fan_in)."""
    bound = np.sqrt(6.0 / (fan_in + fan_out))
    w = rng.uniform(-bound, bound, size=tuple(lead) + (fan_out, fan_in))
    return bf16_bits(w.astype(np.float32))


def normal_f16(rng, shape, std=1.0):
    return f16_bits(rng.standard_normal(shape) * std)


def span_starts(rng, n, length, lo, hi, taken=None):
    """n non-overlapping spans [s, s+length) with lo <= s and s+length <= hi,
    by seeded rejection sampling; `taken` (a bool array) marks used positions."""
    if taken is None:
        taken = np.zeros(hi + length + 1, dtype=bool)
    out = []
    tries = 0
    while len(out) < n:
        tries += 1
        if tries > 100000:
            raise RuntimeError("cannot place spans")
        s = int(rng.integers(lo, hi - length + 1))
        if taken[s:s + length].any():
            continue
        taken[s:s + length] = True
        out.append(s)
    return out


def add_direction_bf16(rows_bits, direction, alpha):
    """rows <- bf16(rows + alpha * direction / |direction|), rows given as
    bf16 bits [n, D], direction a float64 [D] vector supplied by the caller."""
    d = np.asarray(direction, dtype=np.float64)
    d = d / np.linalg.norm(d)
    vals = bits_to_f32_bf16(rows_bits).astype(np.float64) + alpha * d
    return bf16_bits(vals.astype(np.float32))


def ragged_lengths(rng, B, lo, hi):
    return (lo + rng.integers(0, hi - lo + 1, size=B)).astype(np.int32)


def integer_scores(rng, shape, lo=-3, hi=4):
    """Tie-heavy scores: small integers stored as float32."""
    return rng.integers(lo, hi, size=shape).astype(np.float32)
