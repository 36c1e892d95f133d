"""ORACLE (test infrastructure only): ctypes wrapper around tb_oracle.c plus
the decode-step and prediction-interval compositions.

Only tests/, the smoke check and the benchmark's cpu_baseline leg may import
this module. Every function takes and returns numpy arrays; 16-bit storage
formats travel as uint16 bit patterns.

Method source: "TokenButler" technical summary -- "Core architecture" (query
prediction, key projection, scoring), "Inference strategy" (sink, circular
local window and important buffers; batched key projection; prediction
interval; neighbour fetching) and "Significance" (attend to the selected
tokens of the retained full cache).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tb_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libtb_oracle.so")
_lib = None

_u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_c_int = ctypes.c_int


# AddressSanitizer + UndefinedBehaviorSanitizer build (CPU runs of the pins)
SANITIZE_FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                  "-fno-omit-frame-pointer"]


def build(path=None, extra_flags=()):
    """Compile the oracle with gcc (strict IEEE: no contraction, no fast-math;
    OpenMP over independent outputs, which leaves every result unchanged).
    `path` and `extra_flags` make another build of it (e.g. SANITIZE_FLAGS)."""
    path = path or _LIB_PATH
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-ffp-contract=off", "-fopenmp",
           "-fPIC", "-shared"] + list(extra_flags) + ["-o", path + ".tmp", _SRC, "-lm"]
    subprocess.check_call(cmd)
    os.replace(path + ".tmp", path)


def num_threads():
    """Threads the oracle's parallel loops use (OMP_NUM_THREADS, else all cores)."""
    return int(lib().orc_num_threads())


def lib():
    """Load the oracle library, rebuilding it when the source is newer. The
    environment variable TB_ORACLE_LIB names another build of the same source
    to load instead (the sanitizer run uses it); that one is never rebuilt."""
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("TB_ORACLE_LIB")
    if not path:
        path = _LIB_PATH
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
            build()
    L = ctypes.CDLL(path)
    L.orc_num_threads.restype = ctypes.c_int
    L.orc_num_threads.argtypes = []
    L.orc_bf16_bits.restype = ctypes.c_uint16
    L.orc_bf16_bits.argtypes = [ctypes.c_double]
    L.orc_f16_bits.restype = ctypes.c_uint16
    L.orc_f16_bits.argtypes = [ctypes.c_double]
    L.orc_bf16_value.restype = ctypes.c_double
    L.orc_bf16_value.argtypes = [ctypes.c_uint16]
    L.orc_f16_value.restype = ctypes.c_double
    L.orc_f16_value.argtypes = [ctypes.c_uint16]
    L.orc_predict_queries.restype = None
    L.orc_predict_queries.argtypes = [_u16p, _u16p, _u16p, _u16p, _f32p,
                                      _c_int, _c_int, _c_int, _c_int]
    L.orc_project_keys.restype = None
    L.orc_project_keys.argtypes = [_u16p, _u16p, _u16p, _i32p, _c_int,
                                   _c_int, _c_int, _c_int, _c_int, _c_int]
    L.orc_append_kv.restype = None
    L.orc_append_kv.argtypes = [_u16p, _u16p, _u16p, _u16p, _u16p, _u16p, _i32p, _i32p,
                                _c_int, _c_int, _c_int, _c_int, _c_int, _c_int]
    L.orc_distill_loss.restype = None
    L.orc_distill_loss.argtypes = [_u16p, _u16p, _f32p, _u16p, _i32p, _c_int, _c_int, _c_int,
                                   _c_int, _c_int, _c_int, _c_int, ctypes.c_double, _f32p]
    L.orc_score.restype = None
    L.orc_score.argtypes = [_f32p, _c_int, _c_int, _u16p, _i32p, _f32p,
                            _c_int, _c_int, _c_int, _c_int, _c_int]
    for fn in (L.orc_select, L.orc_select_dilate):
        fn.restype = ctypes.c_int
        fn.argtypes = [_f32p, _i32p, _i32p, _c_int, _c_int, _c_int,
                       _c_int, _c_int, _c_int, _c_int, _i32p, _i32p, _c_int]
    L.orc_sparse_attention.restype = None
    L.orc_sparse_attention.argtypes = [_u16p, _u16p, _u16p, _i32p, _i32p, _c_int,
                                       _c_int, _c_int, _c_int, _c_int, _c_int,
                                       ctypes.c_double, _f32p]
    _lib = L
    return L


def _u16(a):
    return np.ascontiguousarray(a, dtype=np.uint16)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


# --- storage formats -------------------------------------------------------

def bf16_bits(v):
    return int(lib().orc_bf16_bits(float(v)))


def f16_bits(v):
    return int(lib().orc_f16_bits(float(v)))


def bf16_value(b):
    return lib().orc_bf16_value(int(b))


def f16_value(b):
    return lib().orc_f16_value(int(b))


# --- stages ----------------------------------------------------------------

def predict_queries(x, w1, w2):
    """q_hat = bf16(SiLU(x W1^T)) W2^T.  x [B,E], w1 [Eh,E], w2 [Nout,Eh] (bf16
    bits). Returns (h bits [B,Eh], q_hat float32 [B,Nout])."""
    x, w1, w2 = _u16(x), _u16(w1), _u16(w2)
    B, E = x.shape
    Eh, Nout = w1.shape[0], w2.shape[0]
    assert w1.shape == (Eh, E) and w2.shape == (Nout, Eh)
    h = np.zeros((B, Eh), np.uint16)
    q = np.zeros((B, Nout), np.float32)
    lib().orc_predict_queries(x, w1, w2, h, q, B, E, Eh, Nout)
    return h, q


def project_keys(kc, wk, kp, pos0, ntok):
    """kp[b, j, t] = fp16(K[b, j, t] . Wk[j]^T) for t in [pos0[b], pos0[b]+ntok).
    kc [B,Hkv,Lmax,D] bf16 bits, wk [Hkv,dp,D] bf16 bits, kp [B,Hkv,Lmax,dp]
    fp16 bits, updated in place (returned)."""
    kc, wk = _u16(kc), _u16(wk)
    assert kp.dtype == np.uint16 and kp.flags.c_contiguous
    B, Hkv, Lmax, D = kc.shape
    dp = wk.shape[1]
    assert wk.shape == (Hkv, dp, D) and kp.shape == (B, Hkv, Lmax, dp)
    lib().orc_project_keys(kc, wk, kp, _i32(pos0), int(ntok), B, Hkv, Lmax, D, dp)
    return kp


def append_kv(k_new, v_new, kc, vc, kp, wk, ctx_len, proj_len, n_p):
    """Append one token's K/V rows per sequence at ctx_len and project the
    pending keys once n_p of them have accumulated. Updates kc, vc, kp,
    ctx_len and proj_len in place (numpy arrays: uint16 bit patterns for
    bf16 / fp16, int32 lengths)."""
    B, Hkv, Lmax, D = kc.shape
    dp = wk.shape[1]
    for a in (kc, vc, kp, ctx_len, proj_len):
        assert a.flags["C_CONTIGUOUS"] and a.flags["WRITEABLE"]
    assert kc.dtype == vc.dtype == kp.dtype == np.uint16
    assert ctx_len.dtype == proj_len.dtype == np.int32
    lib().orc_append_kv(_u16(k_new), _u16(v_new), kc, vc, kp, _u16(wk), ctx_len, proj_len,
                        B, Hkv, Lmax, D, dp, int(n_p))


def distill_loss(q, kc, qhat, kp, pos, scale=None):
    """Cross entropy between the teacher's causal attention distribution and
    the predictor's logits at R query positions: loss [B, R, Hq] fp32.
    q [B,R,Hq,D] bf16 bits, kc [B,Hkv,Lmax,D] bf16 bits, qhat [B,R,Hq,dp]
    fp32, kp [B,Hkv,Lmax,dp] fp16 bits, pos [B,R] int32."""
    q, kc, kp = _u16(q), _u16(kc), _u16(kp)
    qhat = np.ascontiguousarray(qhat, dtype=np.float32)
    B, R, Hq, D = q.shape
    _, Hkv, Lmax, _ = kc.shape
    dp = kp.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    loss = np.zeros((B, R, Hq), np.float32)
    lib().orc_distill_loss(q, kc, qhat, kp, _i32(pos), B, R, Hq, Hkv, Lmax, D, dp, float(scale),
                           loss)
    return loss


def score(qhat, kp, proj_len, Hq, n_slots=1, slot=0, fill=np.nan):
    """scores[b, h, t] = q_hat[b, slot, h] . kp[b, h // g, t] for t < P_b;
    other positions hold `fill`. qhat float32 [B, n_slots*Hq*dp]."""
    kp = _u16(kp)
    B, Hkv, Lmax, dp = kp.shape
    q = np.ascontiguousarray(qhat, dtype=np.float32).reshape(B, n_slots * Hq * dp)
    s = np.full((B, Hq, Lmax), fill, np.float32)
    lib().orc_score(q, n_slots, slot, kp, _i32(proj_len), s, B, Hq, Hkv, Lmax, dp)
    return s


def select(scores, ctx_len, proj_len, S, W, K, r, cap=None, dilate=False):
    """Fixed-budget important buffer (greedy neighbour fill) unioned with sink
    and window; with dilate=True the top-K centres widened by +-r beyond the
    budget instead. Returns (idx int32 [B,Hq,cap] ascending, -1 past count;
    count int32 [B,Hq])."""
    s = np.ascontiguousarray(scores, dtype=np.float32)
    B, Hq, Lmax = s.shape
    if cap is None:
        cap = min(Lmax, S + W + ((2 * r + 1) * K if dilate else K))
    idx = np.full((B, Hq, cap), -1, np.int32)
    cnt = np.zeros((B, Hq), np.int32)
    fn = lib().orc_select_dilate if dilate else lib().orc_select
    st = fn(s, _i32(ctx_len), _i32(proj_len), B, Hq, Lmax,
            int(S), int(W), int(K), int(r), idx, cnt, int(cap))
    if st != 0:
        raise ValueError("oracle select: status %d" % st)
    return idx, cnt


def sparse_attention(q, kc, vc, idx, count, scale=None):
    """out[b,h] = softmax over t in F of (q.k_t * scale) weighted sum of v_t."""
    q, kc, vc = _u16(q), _u16(kc), _u16(vc)
    B, Hkv, Lmax, D = kc.shape
    Hq = q.shape[1]
    idx = _i32(idx)
    cap = idx.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((B, Hq, D), np.float32)
    lib().orc_sparse_attention(q, kc, vc, idx, _i32(count), cap, B, Hq, Hkv, Lmax, D,
                               float(scale), out)
    return out


# --- compositions ------------------------------------------------------------

def decode_step(x, w1, w2, kc, vc, wk, kp, q, ctx_len, proj_len, pos0, ntok,
                S, W, K, r, cap=None, scale=None):
    """One decode step of a single consumer layer: predict, project the pending
    tokens, score, select, attend. kp is updated in place. Returns a dict."""
    Hq = q.shape[1]
    h, qhat = predict_queries(x, w1, w2)
    if ntok > 0:
        project_keys(kc, wk, kp, pos0, ntok)
    s = score(qhat, kp, proj_len, Hq)
    idx, cnt = select(s, ctx_len, proj_len, S, W, K, r, cap)
    out = sparse_attention(q, kc, vc, idx, cnt, scale)
    return dict(h=h, qhat=qhat, scores=s, idx=idx, count=cnt, out=out)


def interval_attended(important, ctx_len0, step, S, W):
    """Attended sets at step j of a prediction interval: the sink, the window
    of the current length L_b + j (the circular buffer of the most recent W
    tokens), and the important tokens chosen at the interval start. Returns
    a list over b of lists over h of ascending int64 arrays."""
    res = []
    for b, row in enumerate(important):
        L = int(ctx_len0[b]) + int(step)
        out = []
        for imp in row:
            keep = set(range(0, min(S, L)))
            keep.update(range(max(0, L - W), L))
            keep.update(int(t) for t in imp)
            out.append(np.array(sorted(keep), dtype=np.int64))
        res.append(out)
    return res


def important_only(scores, ctx_len, proj_len, S, W, K, r):
    """The important buffer alone (no sink / window union), per (b, h), as
    sorted lists: the selection minus the sink and window ranges."""
    idx, cnt = select(scores, ctx_len, proj_len, S, W, K, r)
    B, Hq, _ = idx.shape
    res = []
    for b in range(B):
        L = int(ctx_len[b])
        row = []
        for h in range(Hq):
            t = idx[b, h, :cnt[b, h]]
            t = t[(t >= S) & (t < L - W)]
            row.append(t.astype(np.int64))
        res.append(row)
    return res
