"""The C ABI library: it loads, exports every function include/tb.h declares,
and its host-side validation rejects bad arguments before anything is
enqueued (these calls never reach the GPU, so they run on the CPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tb.h")


@pytest.fixture(scope="module")
def tb():
    import learned_kv_cache_amd as tb
    if not os.path.exists(tb.LIB_PATH):
        from learned_kv_cache_amd import build
        build.build()
    return tb


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tb_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(tb):
    names = declared_functions()
    assert len(names) == 24
    lib = ctypes.CDLL(tb.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version(tb):
    L = tb.lib()
    assert L.tb_abi_version() == 1
    assert tb.status_string(0) == "ok"
    assert tb.status_string(3) == "workspace too small"
    assert tb.status_string(99) == "unknown status"


def test_workspace_queries(tb):
    assert tb.tb_predict_workspace_bytes(1, 4096, 1024, 1024) == 8 * 1 * 1024 * 4
    assert tb.tb_predict_workspace_bytes(1, 100, 1024, 1024) == 0
    s = tb.tb_select_workspace_bytes(1, 32, 65536)
    assert s >= 32 * (65536 * 8 + 65536 // 8)   # candidate slots + bitmap per segment
    a = tb.tb_attn_workspace_bytes(1, 32, 8192, 0, 128)
    assert a >= 32 * 32 * 130 * 4
    assert tb.tb_attn_workspace_bytes(1, 32, 8192, 256, 128) > a


FAKE = 0x10000          # aligned, never dereferenced: validation fails first
MIS = 0x10002


def test_validation_rejects_before_launch(tb):
    L = tb.lib()
    vp = ctypes.c_void_p
    # null pointers
    assert L.tb_predict_queries(None, vp(FAKE), vp(FAKE), vp(FAKE), 1, 512, 128, 128, vp(FAKE), 1 << 20, None) == 1
    assert L.tb_score(None, 1, 0, vp(FAKE), vp(FAKE), vp(FAKE), 1, 8, 2, 300, 16, None) == 1
    # misaligned
    assert L.tb_project_keys(vp(MIS), vp(FAKE), vp(FAKE), vp(FAKE), 1, 1, 2, 300, 64, 16, None) == 1
    assert b"aligned" in L.tb_last_error_detail()
    # unsupported shapes
    assert L.tb_project_keys(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 1, 1, 2, 300, 96, 16, None) == 2
    # append: n_p < 1, unsupported dp, null pointer
    ap = lambda n_p, dp, first=vp(FAKE): (first, vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE),
                                          vp(FAKE), vp(FAKE), 1, 2, 300, 64, dp, n_p, None)
    assert L.tb_append_kv(*ap(0, 16)) == 1
    assert L.tb_append_kv(*ap(4, 8)) == 2
    assert L.tb_append_kv(*ap(4, 16, None)) == 1
    # offload: bad slot range, unsupported D, unpinned (unregistered) host memory
    og = lambda D, slot0, wrap, host=vp(FAKE): (host, vp(FAKE), 1, 2, 300, D, vp(FAKE), vp(FAKE), 64,
                                                8, vp(FAKE), vp(FAKE), 100, slot0, wrap, None)
    assert L.tb_offload_gather(*og(128, 100, 0)) == 1
    assert L.tb_offload_gather(*og(128, 50, 60)) == 1
    assert L.tb_offload_gather(*og(96, 0, 0)) == 2
    import torch
    if not torch.cuda.is_available():
        # every other argument passes validation here, so only run where no
        # kernel could be launched should the pinned-memory check let it by
        buf = ctypes.create_string_buffer(4096 + 16)
        plain = vp((ctypes.addressof(buf) + 15) & ~15)
        assert L.tb_offload_gather(*og(128, 0, 0, plain)) == 1
        assert b"pinned" in L.tb_last_error_detail()
    assert L.tb_score(vp(FAKE), 1, 0, vp(FAKE), vp(FAKE), vp(FAKE), 1, 18, 2, 300, 16, None) == 2
    assert L.tb_score(vp(FAKE), 1, 0, vp(FAKE), vp(FAKE), vp(FAKE), 1, 9, 2, 300, 16, None) == 1
    assert L.tb_predict_queries(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 1, 500, 128, 128, vp(FAKE), 1 << 20, None) == 2
    # selection: negative budget, radius too large, cap too small, workspace too small, DILATE
    ws = 1 << 30
    args = lambda S, W, K, r, mode, cap, wsb: (vp(FAKE), vp(FAKE), vp(FAKE), 1, 8, 300, S, W, K, r, mode,
                                               vp(FAKE), vp(FAKE), cap, vp(FAKE), wsb, None)
    assert L.tb_select(*args(4, 16, -1, 1, 0, 52, ws)) == 1
    assert L.tb_select(*args(4, 16, 32, 65, 0, 52, ws)) == 2
    assert L.tb_select(*args(4, 16, 32, 1, 0, 51, ws)) == 1
    assert L.tb_select(*args(4, 16, 32, 1, 0, 52, 100)) == 3
    assert L.tb_select(*args(4, 16, 32, 1, 1, 115, ws)) == 1   # DILATE needs S + W + (2r+1)K
    assert L.tb_select(*args(4, 16, 32, 1, 2, 300, ws)) == 1   # unknown neighbour mode
    # attention: D unsupported, workspace too small, Hq % Hkv
    A = lambda Hq, D, wsb, win=0: (vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 64, None, win, 1, Hq,
                                   2, 300, D, ctypes.c_float(0.1), vp(FAKE), vp(FAKE), wsb, None)
    assert L.tb_sparse_decode_attn(*A(8, 96, ws)) == 2
    assert L.tb_sparse_decode_attn(*A(8, 64, 16)) == 3
    assert L.tb_sparse_decode_attn(*A(9, 64, ws)) == 1
    assert L.tb_sparse_decode_attn(*A(8, 64, ws, -1)) == 1
    # the fused append + attention: the union of both calls' checks
    AA = lambda Hq, D, dp, wsb, n_p=4, win=16: (vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE),
                                                vp(FAKE), vp(FAKE), vp(FAKE), n_p, vp(FAKE),
                                                vp(FAKE), vp(FAKE), 64, win, 1, Hq, 2, 300, D, dp,
                                                ctypes.c_float(0.1), vp(FAKE), vp(FAKE), wsb, None)
    assert L.tb_append_attn(*AA(8, 96, 32, ws)) == 2
    assert L.tb_append_attn(*AA(8, 64, 24, ws)) == 2
    assert L.tb_append_attn(*AA(8, 64, 16, 16)) == 3
    assert L.tb_append_attn(*AA(9, 64, 16, ws)) == 1
    assert L.tb_append_attn(*AA(8, 64, 16, ws, 0)) == 1
    assert L.tb_append_attn(*AA(8, 64, 16, ws, 4, -1)) == 1
    assert L.tb_select(*args(4, 16, 32, 1, 0x400, 52, ws)) == 1   # unknown mode bit
    assert L.tb_select(*args(4, 16, 32, 1, 0x201, 115, ws)) == 1  # deferred list with dilation
    # list + attention after a deferred selection: its checks reject before launch
    SA = lambda mode, D, wsa: (vp(FAKE), vp(FAKE), 1, 8, 2, 300, 4, 16, 32, 1, mode, vp(FAKE),
                               vp(FAKE), 52, vp(FAKE), ws, vp(FAKE), vp(FAKE), vp(FAKE), D,
                               ctypes.c_float(0.1), vp(FAKE), vp(FAKE), wsa, None)
    assert L.tb_select_attn(*SA(0, 64, ws)) == 1             # mode without the deferral flag
    assert L.tb_select_attn(*SA(0x200, 96, ws)) == 2         # unsupported D
    assert L.tb_select_attn(*SA(0x200, 64, 16)) == 3         # attention workspace too small
    # score + select in one call: the checks of both
    SS = lambda q, Hq, dp, K, r, cap, wsb: (q, 1, 0, vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 1, Hq, 2,
                                            300, dp, 4, 16, K, r, 0, vp(FAKE), vp(FAKE), cap, vp(FAKE),
                                            wsb, None)
    assert L.tb_score_select(*SS(None, 8, 16, 32, 1, 52, ws)) == 1
    assert L.tb_score_select(*SS(vp(MIS), 8, 16, 32, 1, 52, ws)) == 1
    assert L.tb_score_select(*SS(vp(FAKE), 9, 16, 32, 1, 52, ws)) == 1     # Hq % Hkv
    assert L.tb_score_select(*SS(vp(FAKE), 18, 16, 32, 1, 52, ws)) == 2    # group of 9
    assert L.tb_score_select(*SS(vp(FAKE), 8, 24, 32, 1, 52, ws)) == 2     # d' = 24
    assert L.tb_score_select(*SS(vp(FAKE), 8, 16, -1, 1, 52, ws)) == 1
    assert L.tb_score_select(*SS(vp(FAKE), 8, 16, 32, 65, 52, ws)) == 2
    assert L.tb_score_select(*SS(vp(FAKE), 8, 16, 32, 1, 51, ws)) == 1
    assert L.tb_score_select(*SS(vp(FAKE), 8, 16, 32, 1, 52, 100)) == 3


def test_binding_rejects_cpu_tensors(tb):
    import torch
    x = torch.zeros(1, 512, dtype=torch.bfloat16)
    w1 = torch.zeros(128, 512, dtype=torch.bfloat16)
    w2 = torch.zeros(128, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        tb.tb_predict_queries(x, w1, w2, torch.zeros(1, 128), torch.zeros(16, dtype=torch.uint8))


BIG = 2 ** 31 - 1


def test_workspace_queries_at_extreme_sizes(tb):
    # every size query returns 0 for sizes its call rejects and never wraps
    # around (the sanitizer run of this file checks the arithmetic itself)
    L = tb.lib()
    assert L.tb_select_workspace_bytes(1, 1, BIG) == 0            # Lmax > 2^24
    assert L.tb_select_workspace_bytes(BIG, BIG, 1) == 0          # B * Hq > 65535
    assert L.tb_select_workspace_bytes(1, 65535, 1 << 24) > 65535 * (1 << 24) * 8
    assert L.tb_attn_workspace_bytes(1, 1, BIG, BIG, 128) == 0    # cap + window > INT_MAX
    assert L.tb_attn_workspace_bytes(BIG, BIG, 1, 0, 128) == 0    # grid beyond INT_MAX
    assert L.tb_attn_workspace_bytes(1, 1, 1, 0, BIG) == 0        # D unsupported
    a = L.tb_attn_workspace_bytes(1, 1, BIG - 300, 256, 64)
    assert a >= (BIG - 44) // 256 * 66 * 4
    assert L.tb_distill_workspace_bytes(1, 1, 1, 1, BIG) == 0     # Lmax > 2^30
    assert L.tb_distill_workspace_bytes(BIG, 1, 8, 8, 1000) == 0  # B * Hkv > 65535
    assert L.tb_distill_workspace_bytes(1, BIG, 32, 8, 1000) == 0  # R * Hq > 2^24
    assert L.tb_predict_workspace_bytes(BIG, 4096, 1024, 1024) == 0
    assert L.tb_predict_workspace_bytes(1, 4096, BIG - 127, 1024) == 0
    assert L.tb_probe_row_gather_sink_words(BIG, BIG, BIG) == 0


def test_calls_with_extreme_sizes_are_rejected(tb):
    import torch
    if torch.cuda.is_available():
        pytest.skip("runs only where no kernel could be launched")
    L = tb.lib()
    vp = ctypes.c_void_p
    # attention: cap + window beyond INT_MAX, grid beyond INT_MAX, huge workspace claimed
    A = lambda B, Hq, cap, win, ctx: (vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), cap, ctx,
                                      win, B, Hq, 1, 300, 64, ctypes.c_float(0.1), vp(FAKE),
                                      vp(FAKE), 2 ** 62, None)
    assert L.tb_sparse_decode_attn(*A(1, 8, BIG, BIG, vp(FAKE))) == 2
    assert L.tb_sparse_decode_attn(*A(BIG, BIG, 64, 0, None)) == 2
    N = lambda B, Hq, cap, win: (vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), cap, vp(FAKE),
                                 win, B, Hq, 1, 300, 64, ctypes.c_float(0.1), vp(FAKE), None)
    assert L.tb_sparse_decode_attn_noalloc(*N(1, 8, BIG, BIG)) == 2
    assert L.tb_sparse_decode_attn_noalloc(*N(BIG, BIG, 64, 0)) == 2
    # distillation: B * Hkv, R * Hq and Lmax beyond the supported range
    Dl = lambda B, R, Hq, Hkv, Lmax: (vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), B, R, Hq,
                                      Hkv, Lmax, 128, 32, ctypes.c_float(0.1), vp(FAKE), vp(FAKE),
                                      2 ** 62, None)
    assert L.tb_distill_loss(*Dl(BIG, 1, 8, 8, 1000)) == 1
    assert L.tb_distill_loss(*Dl(1, BIG, 32, 8, 1000)) == 1
    assert L.tb_distill_loss(*Dl(1, 4, 32, 8, BIG)) == 2
    # selection over more than 2^24 tokens, over more than 65535 segments
    S = lambda B, Hq, Lmax: (vp(FAKE), vp(FAKE), vp(FAKE), B, Hq, Lmax, 4, 16, 32, 1, 0, vp(FAKE),
                             vp(FAKE), 52, vp(FAKE), 2 ** 62, None)
    assert L.tb_select(*S(1, 8, BIG)) == 2
    assert L.tb_select(*S(BIG, BIG, 300)) == 1
    # prediction: B or Eh beyond the supported range
    assert L.tb_predict_queries(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), BIG, 4096, 1024, 1024,
                                vp(FAKE), 2 ** 62, None) == 1
    assert L.tb_predict_queries(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 1, 4096, BIG - 127, 1024,
                                vp(FAKE), 2 ** 62, None) in (1, 2)
    # probes
    assert L.tb_probe_row_gather(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), BIG, BIG, BIG, 1, 300,
                                 64, vp(FAKE), 2 ** 62, None) == 2
