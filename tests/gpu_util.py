"""Helpers for the GPU parity tests: moving generator bit patterns to the
device, tolerance checks, and the selection band used when scores computed on
the two sides differ in their last bits."""
import sys

import numpy as np
import torch


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(bits, dtype):
    """uint16 bit patterns (numpy) -> GPU tensor of a 16-bit dtype."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dtype)
    return t.cuda()


def dev32(a, dtype=None):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host(t):
    return t.detach().cpu().numpy()


def assert_rel(gpu, ref, rtol, what=""):
    """|gpu - ref| <= rtol * max(|ref|, rms of ref over the last axis)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    bound = rtol * np.maximum(np.abs(ref), rms)
    err = np.abs(gpu - ref)
    bad = err > bound
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: %d elements off; first at %s: gpu=%r ref=%r bound=%r"
                             % (what, bad.sum(), tuple(i), gpu[tuple(i)], ref[tuple(i)],
                                bound[tuple(i)]))


def assert_attn_close(gpu, ref, what=""):
    """|gpu - ref| <= 1e-2 + 2e-2 |ref| elementwise."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    bad = np.abs(gpu - ref) > 1e-2 + 2e-2 * np.abs(ref)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: %d elements off; first at %s: gpu=%r ref=%r"
                             % (what, bad.sum(), tuple(i), gpu[tuple(i)], ref[tuple(i)]))


def rank_scores(s, e0, e1, r):
    """For each eligible t in [e0, e1): the score of its best centre within
    distance r (highest score, lowest position on ties). numpy, any size."""
    n = e1 - e0
    x = s[e0:e1].astype(np.float64)
    best = x.copy()
    for d in range(1, r + 1):
        left = np.full(n, -np.inf)
        left[d:] = x[:-d]
        right = np.full(n, -np.inf)
        right[:-d] = x[d:]
        best = np.maximum(best, np.maximum(left, right))
    return best


def check_selection_band(gpu_idx, gpu_cnt, ref_idx, ref_cnt, ref_scores, L, P, S, W, K, r,
                         rel=1e-3, what="", window_in_list=True):
    """Equal counts; sink and window in both; any token in the symmetric
    difference has an oracle rank score within rel of the K-th rank score."""
    B, Hq = ref_cnt.shape
    for b in range(B):
        Lb, Pb = int(L[b]), int(P[b])
        e0, e1 = S, max(S, min(Lb - W, Pb))
        for h in range(Hq):
            assert gpu_cnt[b, h] == ref_cnt[b, h], (what, b, h, gpu_cnt[b, h], ref_cnt[b, h])
            g = set(gpu_idx[b, h, :gpu_cnt[b, h]].tolist())
            o = set(ref_idx[b, h, :ref_cnt[b, h]].tolist())
            fixed = set(range(min(S, Lb)))
            if window_in_list:
                fixed |= set(range(max(0, Lb - W), Lb))
            assert fixed <= g and fixed <= o
            diff = g ^ o
            if not diff:
                continue
            rs = rank_scores(ref_scores[b, h], e0, e1, r)
            chosen = [t for t in o if e0 <= t < e1]
            sK = min(rs[t - e0] for t in chosen)
            rms = float(np.sqrt(np.mean(ref_scores[b, h, e0:e1].astype(np.float64) ** 2)))
            guard = rel * (abs(sK) if abs(sK) >= rms else rms)
            for t in diff:
                assert e0 <= t < e1, (what, b, h, t)
                assert abs(rs[t - e0] - sK) <= guard, (what, b, h, t, rs[t - e0], sK)
    return True
