"""Seeded single-layer decode workloads (numpy, uint16 bit patterns for bf16).

make_layer(cfg, ...) draws, for one consumer layer and the producer that feeds
it: the producer hidden state x, the MLP weights, the KV cache, the key
projection, the decode query and the per-sequence lengths; optionally it plants
high-affinity token spans. A planted row moves along a direction supplied by
the caller (the head's predicted query mapped back through the projection),
so this module stays free of the method's own arithmetic.
"""
import numpy as np

from .gen import (add_direction_bf16, normal_bf16, ragged_lengths, rng_for,
                  span_starts, xavier_bf16)

# tensor-kind tags for rng_for(cid, kind, layer, b)
T_X, T_W1, T_W2, T_WK, T_K, T_V, T_Q, T_LEN, T_SPAN, T_HEAVY = range(10)


def make_layer(cfg, layer=0, seed=0, L=None, B=None, direction_fn=None,
               n_spans=None, span_len=None, alpha=None, Lmax=None, heavy=False):
    """Inputs of one decode step of one consumer layer.

    Returns a dict of numpy arrays: x [B,E], w1 [Eh,E], w2 [Nout,Eh],
    kc/vc [B,Hkv,Lmax,D], wk [Hkv,dp,D], q [B,Hq,D] (bf16 bits, uint16) and
    ctx_len [B] (int32), plus 'spans': list of (b, head, start, length).

    direction_fn(inputs) -> float64 [B, Hq, D], when given, is used to plant
    spans: each span row of KV head h // g becomes bf16(k + alpha * v / |v|).
    With heavy=True (and cfg.heavy_frac > 0) it also draws the heavy tail of
    the long-context workload first: for every query head, heavy_frac of the
    positions in [S, L_b - W) (drawn with replacement) get their KV head's key
    moved by heavy_shift along that head's direction.
    """
    B = cfg.B if B is None else B
    L = cfg.L if L is None else L
    Lmax = L if Lmax is None else Lmax
    Hq, Hkv, D, E, Eh, dp = cfg.Hq, cfg.Hkv, cfg.D, cfg.E, cfg.Eh, cfg.dp
    cid = cfg.cid * 1000 + seed
    out = {}
    out["x"] = normal_bf16(rng_for(cid, T_X, layer), (B, E))
    out["w1"] = xavier_bf16(rng_for(cid, T_W1, layer // cfg.producer_stride), Eh, E)
    out["w2"] = xavier_bf16(rng_for(cid, T_W2, layer // cfg.producer_stride), cfg.n_out, Eh)
    out["wk"] = xavier_bf16(rng_for(cid, T_WK, layer), dp, D, lead=(Hkv,))
    kc = np.empty((B, Hkv, Lmax, D), np.uint16)
    vc = np.empty((B, Hkv, Lmax, D), np.uint16)
    for b in range(B):
        kc[b] = normal_bf16(rng_for(cid, T_K, layer, b), (Hkv, Lmax, D))
        vc[b] = normal_bf16(rng_for(cid, T_V, layer, b), (Hkv, Lmax, D))
    out["kc"], out["vc"] = kc, vc
    out["q"] = normal_bf16(rng_for(cid, T_Q, layer), (B, Hq, D))
    if cfg.ragged:
        out["ctx_len"] = ragged_lengths(rng_for(cid, T_LEN), B, L // 2, L)
    else:
        out["ctx_len"] = np.full(B, L, np.int32)
    out["spans"] = []
    n_spans = cfg.n_spans if n_spans is None else n_spans
    span_len = cfg.span_len if span_len is None else span_len
    alpha = cfg.alpha if alpha is None else alpha
    dirs = None
    g = Hq // Hkv
    if direction_fn is not None and heavy and cfg.heavy_frac > 0:
        dirs = np.asarray(direction_fn(out), np.float64)     # [B, Hq, D]
        for b in range(B):
            Lb = int(out["ctx_len"][b])
            n = int(cfg.heavy_frac * (Lb - cfg.W - cfg.S))
            for h in range(Hq):
                rng = rng_for(cid, T_HEAVY, layer, b, h)
                pos = rng.integers(cfg.S, Lb - cfg.W, size=n)
                kv = h // g
                kc[b, kv, pos] = add_direction_bf16(kc[b, kv, pos], dirs[b, h], cfg.heavy_shift)
    if direction_fn is not None and n_spans > 0:
        if dirs is None:
            dirs = np.asarray(direction_fn(out), np.float64)     # [B, Hq, D]
        rng = rng_for(cid, T_SPAN, layer)
        for b in range(B):
            Lb = int(out["ctx_len"][b])
            lo, hi = cfg.S + cfg.r, Lb - cfg.W - cfg.r
            taken = [np.zeros(Lmax + span_len + 1, bool) for _ in range(Hkv)]
            for j in range(n_spans):
                h = j % Hq
                kv = h // g
                s0 = span_starts(rng, 1, span_len, lo, hi, taken[kv])[0]
                rows = kc[b, kv, s0:s0 + span_len]
                kc[b, kv, s0:s0 + span_len] = add_direction_bf16(rows, dirs[b, h], alpha)
                out["spans"].append((b, h, s0, span_len))
    return out
