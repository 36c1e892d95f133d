"""libtb: the TokenButler decode-time hot path on MI355X (gfx950).

Thin ctypes binding over the C ABI declared in include/tb.h. Every function
has the C name, takes torch tensors already resident on the GPU, checks
dtype / device / shape / contiguity, and passes raw pointers plus the current
HIP stream. All arithmetic happens in the HIP kernels of libtb.so; if the
library is missing, loading fails loudly -- there is no fallback.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtb.so")

TB_OK = 0
TB_ERR_INVALID_ARGUMENT = 1
TB_ERR_UNSUPPORTED_SHAPE = 2
TB_ERR_WORKSPACE_TOO_SMALL = 3
TB_ERR_HIP = 4
TB_NF_FILL = 0
TB_NF_DILATE = 1
TB_SEL_OMIT_WINDOW = 0x100
TB_SEL_DEFER_LIST = 0x200
TB_SEL_DEFER_SELECT = 0x400

_lib = None
_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t


class TBError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__("libtb status %d (%s): %s" % (status, status_string(status), detail))
        self.status = status


def lib():
    """Load libtb.so (built in-tree by learned_kv_cache_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libtb.so not built: run __graft_entry__.build() "
                          "(or python -m learned_kv_cache_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    L.tb_status_string.restype = ctypes.c_char_p
    L.tb_status_string.argtypes = [_i]
    L.tb_last_error_detail.restype = ctypes.c_char_p
    L.tb_last_error_detail.argtypes = []
    L.tb_abi_version.restype = _i
    L.tb_predict_workspace_bytes.restype = _sz
    L.tb_predict_workspace_bytes.argtypes = [_i, _i, _i, _i]
    L.tb_predict_queries.restype = _i
    L.tb_predict_queries.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _sz, _vp]
    L.tb_predict_project.restype = _i
    L.tb_predict_project.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _sz, _vp, _vp, _vp,
                                     _vp, _i, _i, _i, _i, _i, _vp]
    L.tb_project_keys.restype = _i
    L.tb_project_keys.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]
    L.tb_append_kv.restype = _i
    L.tb_append_kv.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]
    L.tb_offload_gather.restype = _i
    L.tb_offload_gather.argtypes = [_vp, _vp, _i, _i, _i, _i, _vp, _vp, _i, _i, _vp, _vp, _i, _i, _i,
                                    _vp]
    L.tb_offload_append.restype = _i
    L.tb_offload_append.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp,
                                    _vp, _i, _i, _i, _vp]
    L.tb_distill_workspace_bytes.restype = _sz
    L.tb_distill_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]
    L.tb_distill_loss.restype = _i
    L.tb_distill_loss.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i,
                                  ctypes.c_float, _vp, _vp, _sz, _vp]
    L.tb_score.restype = _i
    L.tb_score.argtypes = [_vp, _i, _i, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]
    L.tb_select_workspace_bytes.restype = _sz
    L.tb_select_workspace_bytes.argtypes = [_i, _i, _i]
    L.tb_select.restype = _i
    L.tb_select.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _i, _vp,
                            _sz, _vp]
    L.tb_score_select.restype = _i
    L.tb_score_select.argtypes = [_vp, _i, _i, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i,
                                  _i, _i, _i, _vp, _vp, _i, _vp, _sz, _vp]
    L.tb_select_attn.restype = _i
    L.tb_select_attn.argtypes = [_vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _i, _vp,
                                 _sz, _vp, _vp, _vp, _i, ctypes.c_float, _vp, _vp, _sz, _vp]
    L.tb_append_attn.restype = _i
    L.tb_append_attn.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _i,
                                 _i, _i, _i, _i, _i, _i, ctypes.c_float, _vp, _vp, _sz, _vp]
    L.tb_attn_workspace_bytes.restype = _sz
    L.tb_attn_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]
    L.tb_sparse_decode_attn.restype = _i
    L.tb_sparse_decode_attn.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _vp, _i, _i, _i, _i, _i, _i,
                                        ctypes.c_float, _vp, _vp, _sz, _vp]
    L.tb_probe_stream_read.restype = _i
    L.tb_probe_stream_read.argtypes = [_vp, _sz, _vp, _i, _vp]
    L.tb_probe_row_gather_sink_words.restype = _sz
    L.tb_probe_row_gather_sink_words.argtypes = [_i, _i, _i]
    L.tb_probe_row_gather.restype = _i
    L.tb_probe_row_gather.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]
    L.tb_sparse_decode_attn_noalloc.restype = _i
    L.tb_sparse_decode_attn_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _vp, _i, _i, _i, _i,
                                                _i, _i, ctypes.c_float, _vp, _vp]
    _lib = L
    return L


def status_string(s):
    return lib().tb_status_string(int(s)).decode()


def _check(status):
    if status != TB_OK:
        raise TBError(status, lib().tb_last_error_detail().decode())


def _ptr(t, dtype, name, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims, got shape %s" % (name, ndim, tuple(t.shape)))
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ws(workspace):
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    return ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()


def new_workspace(nbytes, device="cuda"):
    """A zero-filled workspace of at least nbytes (calls leave what must start at zero zeroed)."""
    return torch.zeros(max(int(nbytes), 16), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- predictor

def tb_predict_workspace_bytes(B, E, Eh, n_out):
    return int(lib().tb_predict_workspace_bytes(B, E, Eh, n_out))


def tb_predict_queries(x, w1, w2, qhat, workspace, stream=None):
    """qhat[B, n_out] = bf16(SiLU(x w1^T)) w2^T. x [B,E] bf16, w1 [Eh,E] bf16,
    w2 [n_out,Eh] bf16, qhat fp32 (any shape with B*n_out elements)."""
    B, E = x.shape
    Eh, n_out = w1.shape[0], w2.shape[0]
    if tuple(w1.shape) != (Eh, E) or tuple(w2.shape) != (n_out, Eh) or qhat.numel() != B * n_out:
        raise ValueError("tb_predict_queries: shape mismatch")
    wp, wn = _ws(workspace)
    _check(lib().tb_predict_queries(_ptr(x, torch.bfloat16, "x", 2), _ptr(w1, torch.bfloat16, "w1", 2),
                                    _ptr(w2, torch.bfloat16, "w2", 2), _ptr(qhat, torch.float32, "qhat"),
                                    B, E, Eh, n_out, wp, wn, _stream(stream)))
    return qhat


def tb_predict_project(x, w1, w2, qhat, workspace, k_cache, wk, kp, pos0, n_tokens, stream=None):
    """tb_predict_queries and tb_project_keys in one call (one launch fewer)."""
    B, E = x.shape
    Eh, n_out = w1.shape[0], w2.shape[0]
    Bk, Hkv, Lmax, D = k_cache.shape
    dp = wk.shape[1]
    if (tuple(w1.shape) != (Eh, E) or tuple(w2.shape) != (n_out, Eh) or qhat.numel() != B * n_out
            or Bk != B or tuple(wk.shape) != (Hkv, dp, D) or tuple(kp.shape) != (B, Hkv, Lmax, dp)
            or pos0.numel() != B):
        raise ValueError("tb_predict_project: shape mismatch")
    wp, wn = _ws(workspace)
    _check(lib().tb_predict_project(_ptr(x, torch.bfloat16, "x", 2), _ptr(w1, torch.bfloat16, "w1", 2),
                                    _ptr(w2, torch.bfloat16, "w2", 2), _ptr(qhat, torch.float32, "qhat"),
                                    B, E, Eh, n_out, wp, wn, _ptr(k_cache, torch.bfloat16, "k_cache", 4),
                                    _ptr(wk, torch.bfloat16, "wk", 3), _ptr(kp, torch.float16, "kp", 4),
                                    _ptr(pos0, torch.int32, "pos0"), int(n_tokens), Hkv, Lmax, D, dp,
                                    _stream(stream)))
    return qhat, kp


# ---------------------------------------------------------------- projection

def tb_project_keys(k_cache, wk, kp, pos0, n_tokens, stream=None):
    """kp[b, j, t] = fp16(k_cache[b, j, t] wk[j]^T) for t in [pos0[b], pos0[b] + n_tokens)."""
    B, Hkv, Lmax, D = k_cache.shape
    dp = wk.shape[1]
    if tuple(wk.shape) != (Hkv, dp, D) or tuple(kp.shape) != (B, Hkv, Lmax, dp) or pos0.numel() != B:
        raise ValueError("tb_project_keys: shape mismatch")
    _check(lib().tb_project_keys(_ptr(k_cache, torch.bfloat16, "k_cache", 4),
                                 _ptr(wk, torch.bfloat16, "wk", 3), _ptr(kp, torch.float16, "kp", 4),
                                 _ptr(pos0, torch.int32, "pos0"), int(n_tokens), B, Hkv, Lmax, D, dp,
                                 _stream(stream)))
    return kp


def tb_append_kv(k_new, v_new, k_cache, v_cache, kp, wk, ctx_len, proj_len, n_p, stream=None):
    """Write one token's K/V per sequence at ctx_len[b]; project the pending
    keys once n_p have accumulated; advance ctx_len / proj_len in place."""
    B, Hkv, Lmax, D = k_cache.shape
    dp = wk.shape[1]
    if (tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D)
            or tuple(v_cache.shape) != (B, Hkv, Lmax, D) or tuple(wk.shape) != (Hkv, dp, D)
            or tuple(kp.shape) != (B, Hkv, Lmax, dp) or ctx_len.numel() != B
            or proj_len.numel() != B):
        raise ValueError("tb_append_kv: shape mismatch")
    _check(lib().tb_append_kv(_ptr(k_new, torch.bfloat16, "k_new", 3),
                              _ptr(v_new, torch.bfloat16, "v_new", 3),
                              _ptr(k_cache, torch.bfloat16, "k_cache", 4),
                              _ptr(v_cache, torch.bfloat16, "v_cache", 4),
                              _ptr(kp, torch.float16, "kp", 4), _ptr(wk, torch.bfloat16, "wk", 3),
                              _ptr(ctx_len, torch.int32, "ctx_len"),
                              _ptr(proj_len, torch.int32, "proj_len"), B, Hkv, Lmax, D, dp,
                              int(n_p), _stream(stream)))


def _host_ptr(t, name):
    if not isinstance(t, torch.Tensor) or t.is_cuda or not t.is_pinned():
        raise ValueError("%s must be a pinned host tensor" % name)
    if t.dtype != torch.bfloat16 or not t.is_contiguous() or t.dim() != 4:
        raise ValueError("%s must be a contiguous 4-d bfloat16 tensor" % name)
    return ctypes.c_void_p(t.data_ptr())


def tb_offload_gather(k_host, v_host, idx, count, k_buf, v_buf, slot0=0, wrap=0, stream=None):
    """Copy the listed rows of the pinned host cache into the per-query-head
    device buffers: slot slot0 + i (or slot0 + t % wrap when wrap > 0)."""
    B, Hkv, Lmax, D = k_host.shape
    Bq, Hq, buf_rows, Db = k_buf.shape
    cap = idx.shape[-1]
    if (tuple(v_host.shape) != (B, Hkv, Lmax, D) or (Bq, Db) != (B, D)
            or tuple(v_buf.shape) != tuple(k_buf.shape) or tuple(idx.shape) != (B, Hq, cap)
            or tuple(count.shape) != (B, Hq)):
        raise ValueError("tb_offload_gather: shape mismatch")
    _check(lib().tb_offload_gather(_host_ptr(k_host, "k_host"), _host_ptr(v_host, "v_host"), B, Hkv,
                                   Lmax, D, _ptr(idx, torch.int32, "idx", 3),
                                   _ptr(count, torch.int32, "count", 2), cap, Hq,
                                   _ptr(k_buf, torch.bfloat16, "k_buf", 4),
                                   _ptr(v_buf, torch.bfloat16, "v_buf", 4), buf_rows, int(slot0),
                                   int(wrap), _stream(stream)))


def tb_offload_append(k_new, v_new, wk, k_host, v_host, kp, ctx_len, proj_len, k_buf, v_buf,
                      window, stream=None):
    """One decode step of the offloaded cache: new rows to the host cache and
    the window slots, the new key projected into kp, lengths advanced."""
    B, Hkv, Lmax, D = k_host.shape
    dp = wk.shape[1]
    Hq, buf_rows = k_buf.shape[1], k_buf.shape[2]
    if (tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D)
            or tuple(wk.shape) != (Hkv, dp, D) or tuple(kp.shape) != (B, Hkv, Lmax, dp)
            or tuple(k_buf.shape) != (B, Hq, buf_rows, D) or tuple(v_buf.shape) != tuple(k_buf.shape)):
        raise ValueError("tb_offload_append: shape mismatch")
    _check(lib().tb_offload_append(_ptr(k_new, torch.bfloat16, "k_new", 3),
                                   _ptr(v_new, torch.bfloat16, "v_new", 3),
                                   _ptr(wk, torch.bfloat16, "wk", 3), _host_ptr(k_host, "k_host"),
                                   _host_ptr(v_host, "v_host"), _ptr(kp, torch.float16, "kp", 4),
                                   _ptr(ctx_len, torch.int32, "ctx_len"),
                                   _ptr(proj_len, torch.int32, "proj_len"), B, Hkv, Lmax, D, dp,
                                   _ptr(k_buf, torch.bfloat16, "k_buf", 4),
                                   _ptr(v_buf, torch.bfloat16, "v_buf", 4), Hq, buf_rows,
                                   int(window), _stream(stream)))


def tb_distill_workspace_bytes(B, R, Hq, Hkv, Lmax):
    return int(lib().tb_distill_workspace_bytes(B, R, Hq, Hkv, Lmax))


def tb_distill_loss(q, k_cache, qhat, kp, pos, loss, workspace, scale=None, stream=None):
    """loss[b, r, h] = cross entropy between softmax(scale q.k_t) and the
    predictor's logits qhat.kp_t over the causal tokens t <= pos[b, r]."""
    B, R, Hq, D = q.shape
    _, Hkv, Lmax, _ = k_cache.shape
    dp = kp.shape[-1]
    if (tuple(k_cache.shape) != (B, Hkv, Lmax, D) or tuple(qhat.shape) != (B, R, Hq, dp)
            or tuple(kp.shape) != (B, Hkv, Lmax, dp) or tuple(pos.shape) != (B, R)
            or tuple(loss.shape) != (B, R, Hq)):
        raise ValueError("tb_distill_loss: shape mismatch")
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    wp, wn = _ws(workspace)
    _check(lib().tb_distill_loss(_ptr(q, torch.bfloat16, "q", 4), _ptr(k_cache, torch.bfloat16, "k_cache", 4),
                                 _ptr(qhat, torch.float32, "qhat", 4), _ptr(kp, torch.float16, "kp", 4),
                                 _ptr(pos, torch.int32, "pos", 2), B, R, Hq, Hkv, Lmax, D, dp,
                                 ctypes.c_float(scale), _ptr(loss, torch.float32, "loss", 3), wp, wn,
                                 _stream(stream)))
    return loss


# ---------------------------------------------------------------- scoring

def tb_score(qhat, kp, proj_len, scores, n_slots=1, slot=0, stream=None):
    """scores[b, h, t] = qhat[b, slot, h] . kp[b, h // g, t] for t < proj_len[b]."""
    B, Hkv, Lmax, dp = kp.shape
    Hq = scores.shape[1]
    if tuple(scores.shape) != (B, Hq, Lmax) or qhat.numel() != B * n_slots * Hq * dp:
        raise ValueError("tb_score: shape mismatch")
    _check(lib().tb_score(_ptr(qhat, torch.float32, "qhat"), int(n_slots), int(slot),
                          _ptr(kp, torch.float16, "kp", 4), _ptr(proj_len, torch.int32, "proj_len"),
                          _ptr(scores, torch.float32, "scores", 3), B, Hq, Hkv, Lmax, dp,
                          _stream(stream)))
    return scores


# ---------------------------------------------------------------- selection

def tb_select_workspace_bytes(B, Hq, Lmax):
    return int(lib().tb_select_workspace_bytes(B, Hq, Lmax))


def tb_select(scores, ctx_len, proj_len, sink, window, budget, radius, idx, count, workspace,
              mode=TB_NF_FILL, stream=None):
    """Sink U window U fixed-budget important tokens (neighbour fill), ascending.
    mode: TB_NF_FILL or TB_NF_DILATE, optionally | TB_SEL_OMIT_WINDOW."""
    B, Hq, Lmax = scores.shape
    cap = idx.shape[-1]
    if tuple(idx.shape) != (B, Hq, cap) or tuple(count.shape) != (B, Hq):
        raise ValueError("tb_select: shape mismatch")
    wp, wn = _ws(workspace)
    _check(lib().tb_select(_ptr(scores, torch.float32, "scores", 3), _ptr(ctx_len, torch.int32, "ctx_len"),
                           _ptr(proj_len, torch.int32, "proj_len"), B, Hq, Lmax, int(sink), int(window),
                           int(budget), int(radius), int(mode), _ptr(idx, torch.int32, "idx", 3),
                           _ptr(count, torch.int32, "count", 2), cap, wp, wn, _stream(stream)))
    return idx, count


def tb_score_select(qhat, kp, ctx_len, proj_len, scores, sink, window, budget, radius, idx, count,
                    workspace, mode=TB_NF_FILL, n_slots=1, slot=0, stream=None):
    """tb_score followed by tb_select (same results) with the selection's band
    sampled inside the scoring launch."""
    B, Hkv, Lmax, dp = kp.shape
    Hq = scores.shape[1]
    cap = idx.shape[-1]
    if tuple(scores.shape) != (B, Hq, Lmax) or qhat.numel() != B * n_slots * Hq * dp:
        raise ValueError("tb_score_select: shape mismatch")
    if tuple(idx.shape) != (B, Hq, cap) or tuple(count.shape) != (B, Hq):
        raise ValueError("tb_score_select: shape mismatch")
    wp, wn = _ws(workspace)
    _check(lib().tb_score_select(_ptr(qhat, torch.float32, "qhat"), int(n_slots), int(slot),
                                 _ptr(kp, torch.float16, "kp", 4), _ptr(ctx_len, torch.int32, "ctx_len"),
                                 _ptr(proj_len, torch.int32, "proj_len"),
                                 _ptr(scores, torch.float32, "scores", 3), B, Hq, Hkv, Lmax, dp,
                                 int(sink), int(window), int(budget), int(radius), int(mode),
                                 _ptr(idx, torch.int32, "idx", 3), _ptr(count, torch.int32, "count", 2),
                                 cap, wp, wn, _stream(stream)))
    return idx, count


def tb_select_attn(ctx_len, proj_len, sink, window, budget, radius, idx, count, sel_workspace, q,
                   k_cache, v_cache, out, attn_workspace, mode=TB_NF_FILL | TB_SEL_DEFER_LIST,
                   scale=None, stream=None):
    """After a selection with TB_SEL_DEFER_LIST: write its list and attend over it."""
    B, Hq, cap = idx.shape
    Hkv, Lmax, D = k_cache.shape[1], k_cache.shape[2], k_cache.shape[3]
    if (tuple(count.shape) != (B, Hq) or tuple(k_cache.shape) != (B, Hkv, Lmax, D)
            or tuple(v_cache.shape) != (B, Hkv, Lmax, D) or tuple(q.shape) != (B, Hq, D)
            or tuple(out.shape) != (B, Hq, D)):
        raise ValueError("tb_select_attn: shape mismatch")
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    sp, sn = _ws(sel_workspace)
    ap, an = _ws(attn_workspace)
    _check(lib().tb_select_attn(_ptr(ctx_len, torch.int32, "ctx_len"), _ptr(proj_len, torch.int32, "proj_len"),
                                B, Hq, Hkv, Lmax, int(sink), int(window), int(budget), int(radius),
                                int(mode), _ptr(idx, torch.int32, "idx", 3), _ptr(count, torch.int32, "count", 2),
                                cap, sp, sn, _ptr(q, torch.bfloat16, "q", 3),
                                _ptr(k_cache, torch.bfloat16, "k_cache", 4),
                                _ptr(v_cache, torch.bfloat16, "v_cache", 4), D, ctypes.c_float(scale),
                                _ptr(out, torch.float32, "out", 3), ap, an, _stream(stream)))
    return idx, out


# ---------------------------------------------------------------- attention

def tb_attn_workspace_bytes(B, Hq, cap, window, D):
    return int(lib().tb_attn_workspace_bytes(B, Hq, cap, window, D))


def tb_sparse_decode_attn(q, k_cache, v_cache, idx, count, out, workspace, scale=None,
                          ctx_len=None, window=0, stream=None):
    """out[b, h] = softmax-weighted sum of v over the positions idx[b, h, :count[b, h]]
    plus, with ctx_len given, the local window of the last `window` positions."""
    B, Hkv, Lmax, D = k_cache.shape
    Hq = q.shape[1]
    cap = idx.shape[-1]
    if (tuple(q.shape) != (B, Hq, D) or tuple(v_cache.shape) != (B, Hkv, Lmax, D)
            or tuple(idx.shape) != (B, Hq, cap) or tuple(out.shape) != (B, Hq, D)):
        raise ValueError("tb_sparse_decode_attn: shape mismatch")
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    ctx = None if ctx_len is None else _ptr(ctx_len, torch.int32, "ctx_len")
    wp, wn = _ws(workspace)
    _check(lib().tb_sparse_decode_attn(_ptr(q, torch.bfloat16, "q", 3), _ptr(k_cache, torch.bfloat16, "k_cache", 4),
                                       _ptr(v_cache, torch.bfloat16, "v_cache", 4), _ptr(idx, torch.int32, "idx", 3),
                                       _ptr(count, torch.int32, "count", 2), cap, ctx, int(window),
                                       B, Hq, Hkv, Lmax, D, float(scale), _ptr(out, torch.float32, "out", 3),
                                       wp, wn, _stream(stream)))
    return out


def tb_append_attn(k_new, v_new, k_cache, v_cache, kp, wk, ctx_len, proj_len, n_p, q, idx, count,
                   out, workspace, window=0, scale=None, stream=None):
    """tb_append_kv then tb_sparse_decode_attn(ctx_len=ctx_len, window=window) in one launch."""
    B, Hkv, Lmax, D = k_cache.shape
    dp = wk.shape[1]
    Hq = q.shape[1]
    cap = idx.shape[-1]
    if (tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D)
            or tuple(v_cache.shape) != (B, Hkv, Lmax, D) or tuple(wk.shape) != (Hkv, dp, D)
            or tuple(kp.shape) != (B, Hkv, Lmax, dp) or ctx_len.numel() != B
            or proj_len.numel() != B or tuple(q.shape) != (B, Hq, D)
            or tuple(idx.shape) != (B, Hq, cap) or tuple(count.shape) != (B, Hq)
            or tuple(out.shape) != (B, Hq, D)):
        raise ValueError("tb_append_attn: shape mismatch")
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    wp, wn = _ws(workspace)
    _check(lib().tb_append_attn(_ptr(k_new, torch.bfloat16, "k_new", 3),
                                _ptr(v_new, torch.bfloat16, "v_new", 3),
                                _ptr(k_cache, torch.bfloat16, "k_cache", 4),
                                _ptr(v_cache, torch.bfloat16, "v_cache", 4),
                                _ptr(kp, torch.float16, "kp", 4), _ptr(wk, torch.bfloat16, "wk", 3),
                                _ptr(ctx_len, torch.int32, "ctx_len"),
                                _ptr(proj_len, torch.int32, "proj_len"), int(n_p),
                                _ptr(q, torch.bfloat16, "q", 3), _ptr(idx, torch.int32, "idx", 3),
                                _ptr(count, torch.int32, "count", 2), cap, int(window), B, Hq, Hkv,
                                Lmax, D, dp, float(scale), _ptr(out, torch.float32, "out", 3), wp,
                                wn, _stream(stream)))
    return out


def tb_sparse_decode_attn_noalloc(q, k_cache, v_cache, idx, count, out, scale=None, ctx_len=None,
                                  window=0, stream=None):
    """tb_sparse_decode_attn without a workspace: the library's fixed per-GPU
    scratch array holds the partials (calls that overlap on one GPU race)."""
    B, Hkv, Lmax, D = k_cache.shape
    Hq = q.shape[1]
    cap = idx.shape[-1]
    if (tuple(q.shape) != (B, Hq, D) or tuple(v_cache.shape) != (B, Hkv, Lmax, D)
            or tuple(idx.shape) != (B, Hq, cap) or tuple(out.shape) != (B, Hq, D)):
        raise ValueError("tb_sparse_decode_attn_noalloc: shape mismatch")
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    ctx = None if ctx_len is None else _ptr(ctx_len, torch.int32, "ctx_len")
    _check(lib().tb_sparse_decode_attn_noalloc(
        _ptr(q, torch.bfloat16, "q", 3), _ptr(k_cache, torch.bfloat16, "k_cache", 4),
        _ptr(v_cache, torch.bfloat16, "v_cache", 4), _ptr(idx, torch.int32, "idx", 3),
        _ptr(count, torch.int32, "count", 2), cap, ctx, int(window), B, Hq, Hkv, Lmax, D,
        float(scale), _ptr(out, torch.float32, "out", 3), _stream(stream)))
    return out


def tb_probe_stream_read(src, sink, stream=None):
    """Read every byte of src once (bandwidth probe); one XOR word per workgroup to sink."""
    if not src.is_cuda or not src.is_contiguous() or (src.numel() * src.element_size()) % 16:
        raise ValueError("src must be a contiguous GPU tensor of a multiple of 16 bytes")
    _check(lib().tb_probe_stream_read(ctypes.c_void_p(src.data_ptr()),
                                      src.numel() * src.element_size(),
                                      _ptr(sink, torch.int32, "sink", 1), sink.numel(),
                                      _stream(stream)))


def tb_probe_row_gather_sink_words(B, Hq, cap):
    return int(lib().tb_probe_row_gather_sink_words(B, Hq, cap))


def tb_probe_row_gather(k_cache, v_cache, idx, count, sink, stream=None):
    """Request the K/V rows the sparse attention over (idx, count) reads (bandwidth probe)."""
    B, Hkv, Lmax, D = k_cache.shape
    _, Hq, cap = idx.shape
    _check(lib().tb_probe_row_gather(_ptr(k_cache, torch.bfloat16, "k_cache", 4),
                                     _ptr(v_cache, torch.bfloat16, "v_cache", 4),
                                     _ptr(idx, torch.int32, "idx", 3),
                                     _ptr(count, torch.int32, "count", 2), cap, B, Hq, Hkv, Lmax,
                                     D, _ptr(sink, torch.int32, "sink", 1), sink.numel(),
                                     _stream(stream)))
