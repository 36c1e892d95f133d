"""Decode-step throughput of the TokenButler hot path on one MI355X.

A step is one pass of the whole path over one batch: predict the importance
queries (producer MLP), project the newest token's key, score every cached
token, select sink + window + fixed budget with neighbour fill, and run
sparse decode attention. Workload: Llama-3.1-8B-shaped single consumer layer,
B=1, L=65536, 32 query / 8 KV heads, head dim 128, E=4096, Eh=1024, d'=32,
sink 64, window 256, budget 7872, radius 1, 64 planted 8-token spans.

Inputs are resident in HBM before the timed region; R replicas of every
per-step input are rotated so that each step reads cold memory (the working
set of one step fits in the 256 MiB MALL). The timed steps replay a HIP graph
that holds R consecutive steps (one per replica), as a serving loop would;
the same steps issued call by call are timed too ("eager"). The step's calls
are tb_predict_project, tb_score_select with the list deferred, and
tb_select_attn (the list written by the attention workgroups, which then
attend over it). The dominant kernel (that compaction + attention launch)
is timed live with HIP events on its launch stream, over back-to-back graph
replays of it alone.

Prints one JSON line. Run with --gpus 1 only.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np

METRIC = "sparse decode steps/s at 64K ctx, 8K budget; achieved HBM GB/s vs peak"
PEAK_HBM_GBS = 8000.0
# the step's dominant kernel: its committed traffic record and its sources,
# for the split selection (threshold + list + attention) and for the deferred
# list (compaction + attention)
TRAFFIC_FILES = {"select": os.path.join(ROOT, "profiles", "split_attn_c2_traffic.txt"),
                 "list": os.path.join(ROOT, "profiles", "compact_attn_c2_traffic.txt")}
KERNEL_SRCS = {k: [os.path.join(ROOT, "learned_kv_cache_amd", "csrc", f)
                   for f in (first, "select_impl.h", "attn_impl.h")]
               for k, first in (("select", "select_attn_hist.hip"), ("list", "select_attn.hip"))}


def kernel_source_hash(defer="select"):
    h = hashlib.sha256()
    for f in KERNEL_SRCS[defer]:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class FenceFreeEvent:
    """A timing event of the HIP runtime torch uses, created with
    hipEventDisableSystemFence: recording it writes no caches back and
    invalidates none, so the work timed between two of them runs as it does
    between kernels (events recorded with the default system-scope fence add
    about 3 us around a single launch on this part)."""
    _hip = None

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            path = None
            for line in open("/proc/self/maps"):
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
            if path is None:
                raise RuntimeError("the HIP runtime is not loaded")
            h = ctypes.CDLL(path)
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                              ctypes.c_void_p]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = h
        return cls._hip

    def __init__(self):
        self.e = ctypes.c_void_p()
        if self._lib().hipEventCreateWithFlags(ctypes.byref(self.e), 0x20000000):
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream):
        if self._lib().hipEventRecord(self.e, ctypes.c_void_p(stream.cuda_stream)):
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end):
        ms = ctypes.c_float()
        if self._lib().hipEventElapsedTime(ctypes.byref(ms), self.e, end.e):
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.e:
            self._hip.hipEventDestroy(self.e)


def planting_direction(inp, cfg):
    """Key direction that raises head h's score fastest (Wk^T q_hat_h), from a
    float64 numpy evaluation of the predictor on the host; only used to build
    the planted spans of the synthetic workload."""
    from synthetic import bits_to_f32_bf16
    x = bits_to_f32_bf16(inp["x"]).astype(np.float64)
    w1 = bits_to_f32_bf16(inp["w1"]).astype(np.float64)
    w2 = bits_to_f32_bf16(inp["w2"]).astype(np.float64)
    z = x @ w1.T
    h = z / (1.0 + np.exp(-z))
    qh = (h @ w2.T).reshape(x.shape[0], cfg.Hq, cfg.dp)
    wk = np.repeat(bits_to_f32_bf16(inp["wk"]).astype(np.float64), cfg.g, axis=0)
    return np.einsum("bhc,hcd->bhd", qh, wk)


def traffic_record(defer="select"):
    """HBM bytes per launch of the step's dominant kernel from the committed
    rocprofv3 PMC summary, if it was taken on the kernel's current sources."""
    path = TRAFFIC_FILES[defer]
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    if (rec.get("kernel_source_sha256_16") != kernel_source_hash(defer)
            or "traffic_bytes_per_launch" not in rec):
        return None
    return float(rec["traffic_bytes_per_launch"])


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, cfg, seconds):
    """The oracle (plain C, fp64, OpenMP over independent heads and hidden
    units) on full decode steps of the same workload, repeated for about
    `seconds` of wall time on the host's cores."""
    import oracle as orc
    B, L = 1, cfg.L
    kp = np.zeros((B, cfg.Hkv, L, cfg.dp), np.uint16)
    orc.project_keys(inp["kc"], inp["wk"], kp, np.zeros(B, np.int32), L - 1)   # setup, untimed
    ctx = inp["ctx_len"]
    n = 0
    t0 = time.perf_counter()
    while True:
        orc.decode_step(inp["x"], inp["w1"], inp["w2"], inp["kc"], inp["vc"], inp["wk"], kp,
                        inp["q"], ctx, ctx, (ctx - 1).astype(np.int32), 1, cfg.S, cfg.W, cfg.K,
                        cfg.r, cap=cfg.cap)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    threads = orc.num_threads()
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count()
    return {"value": n / el, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "nproc": nproc,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "sample": "%d full decode steps of the same workload (predict, project 1 token, "
                      "score 65536 tokens x 32 heads, select, attend), C with OpenMP over heads "
                      "and hidden units on %d threads, %.1f s" % (n, threads, el)}


def run_interval(cfg, args, emit=True):
    """Prediction-interval pipeline over all layers of a multi-layer workload:
    once per interval, run every producer's predictor, score and select every
    consumer layer (the window left out of the list); then I decode steps,
    each appending one token's K/V per sequence to every layer (which projects
    the pending keys once N_p of them have accumulated) and running sparse
    attention on every layer with the sliding window, both in one launch per
    layer (tb_append_attn; --append separate: tb_append_kv for every layer,
    then tb_sparse_decode_attn for every layer). Every
    interval starts from the same lengths (the appended rows are rewritten).
    steps/s = I / interval time, with each interval replayed from one HIP
    graph of the whole interval (the same intervals issued call by call are
    timed too: eager_steps_per_s). The caches are generated on the GPU
    (torch.randn, bf16): they are far larger than the 256 MiB MALL."""
    import torch
    import learned_kv_cache_amd as tb
    from synthetic import rng_for
    from synthetic.workload import T_LEN

    B, Hq, Hkv, D, dp, E, Eh = cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.dp, cfg.E, cfg.Eh
    I, Np, nl = cfg.interval, cfg.n_proj, cfg.layers
    npro = (nl + cfg.producer_stride - 1) // cfg.producer_stride
    Lmax = cfg.L + I
    if cfg.ragged:
        L0 = (cfg.L // 2 + rng_for(cfg.cid, T_LEN).integers(0, cfg.L // 2 + 1, size=B)).astype(np.int32)
    else:
        L0 = np.full(B, cfg.L, np.int32)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20260101 + cfg.cid)
    log("allocating %d layers of K/V [%d, %d, %d, %d] bf16 on the GPU" % (nl, B, Hkv, Lmax, D))

    def randn(*shape, std=1.0):
        return (torch.randn(*shape, generator=gen, device="cuda") * std).to(torch.bfloat16)

    def xavier(o, i, lead=()):
        bnd = (6.0 / (i + o)) ** 0.5
        return ((torch.rand(*lead, o, i, generator=gen, device="cuda") * 2 - 1) * bnd).to(torch.bfloat16)

    K = [randn(B, Hkv, Lmax, D) for _ in range(nl)]
    V = [randn(B, Hkv, Lmax, D) for _ in range(nl)]
    Wk = [xavier(dp, D, (Hkv,)) for _ in range(nl)]
    Q = [randn(B, Hq, D) for _ in range(nl)]
    X = [randn(B, E) for _ in range(npro)]
    W1 = [xavier(Eh, E) for _ in range(npro)]
    W2 = [xavier(Hq * dp, Eh) for _ in range(npro)]
    ws_p = tb.new_workspace(tb.tb_predict_workspace_bytes(B, E, Eh, Hq * dp))
    qhat = [torch.empty(B, Hq * dp, device="cuda") for _ in range(npro)]
    ctx0 = torch.from_numpy(L0).cuda()
    if cfg.heavy_frac > 0:
        # heavy tail: a fraction of positions per query head gets keys moved
        # along that head's predicted-query direction by heavy_shift score std
        for p in range(npro):
            tb.tb_predict_queries(X[p], W1[p], W2[p], qhat[p], ws_p)
        for l in range(nl):
            qh = qhat[l // cfg.producer_stride].view(B, Hq, dp)
            wk = Wk[l].float().repeat_interleave(cfg.g, 0)                 # [Hq, dp, D]
            v = torch.einsum("bhc,hcd->bhd", qh, wk)
            v = v / v.norm(dim=-1, keepdim=True)
            for b in range(B):
                n = int(cfg.heavy_frac * (int(L0[b]) - cfg.W - cfg.S))
                for h in range(Hq):
                    pos = torch.randint(cfg.S, int(L0[b]) - cfg.W, (n,), generator=gen, device="cuda")
                    kv = h // cfg.g
                    K[l][b, kv, pos] = (K[l][b, kv, pos].float() + cfg.heavy_shift * v[b, h]).to(torch.bfloat16)
    # projected keys of the whole context; the decode steps append after it
    Kp = [torch.zeros(B, Hkv, Lmax, dp, dtype=torch.float16, device="cuda") for _ in range(nl)]
    zero = torch.zeros(B, dtype=torch.int32, device="cuda")
    for l in range(nl):
        tb.tb_project_keys(K[l], Wk[l], Kp[l], zero, int(L0.max()))
    torch.cuda.synchronize()
    scores = torch.empty(B, Hq, Lmax, device="cuda")
    cap = cfg.S + cfg.K
    idx = [torch.zeros(B, Hq, cap, dtype=torch.int32, device="cuda") for _ in range(nl)]
    cnt = [torch.zeros(B, Hq, dtype=torch.int32, device="cuda") for _ in range(nl)]
    out = torch.empty(B, Hq, D, device="cuda")
    ws_s = tb.new_workspace(tb.tb_select_workspace_bytes(B, Hq, Lmax))
    ws_a = tb.new_workspace(tb.tb_attn_workspace_bytes(B, Hq, cap, cfg.W, D))
    # per-layer device lengths [layer, (ctx, proj), B], reset at every interval
    lens0 = torch.from_numpy(np.stack([np.stack([L0, L0])] * nl)).cuda()
    lens = lens0.clone()
    k_new = [randn(B, Hkv, D) for _ in range(I)]
    v_new = [randn(B, Hkv, D) for _ in range(I)]
    mode = tb.TB_NF_FILL | tb.TB_SEL_OMIT_WINDOW
    stream = torch.cuda.current_stream()
    fused = args.append == "fused"

    def interval(attn_ev=None, app_ev=None):
        lens.copy_(lens0)
        for p in range(npro):
            tb.tb_predict_queries(X[p], W1[p], W2[p], qhat[p], ws_p)
        for l in range(nl):
            tb.tb_score_select(qhat[l // cfg.producer_stride], Kp[l], ctx0, ctx0, scores, cfg.S,
                               cfg.W, cfg.K, cfg.r, idx[l], cnt[l], ws_s, mode=mode)
        for j in range(I):
            if fused:
                # each layer's append and attention in one launch
                if attn_ev is not None:
                    attn_ev[j][0].record(stream)
                for l in range(nl):
                    tb.tb_append_attn(k_new[j], v_new[j], K[l], V[l], Kp[l], Wk[l], lens[l, 0],
                                      lens[l, 1], Np, Q[l], idx[l], cnt[l], out, ws_a, window=cfg.W)
                if attn_ev is not None:
                    attn_ev[j][1].record(stream)
                continue
            if app_ev is not None:
                app_ev[j][0].record(stream)
            for l in range(nl):
                tb.tb_append_kv(k_new[j], v_new[j], K[l], V[l], Kp[l], Wk[l], lens[l, 0], lens[l, 1],
                                Np)
            if attn_ev is not None:
                app_ev[j][1].record(stream)
                attn_ev[j][0].record(stream)
            for l in range(nl):
                tb.tb_sparse_decode_attn(Q[l], K[l], V[l], idx[l], cnt[l], out, ws_a,
                                         ctx_len=lens[l, 0], window=cfg.W)
            if attn_ev is not None:
                attn_ev[j][1].record(stream)

    log("warmup interval")
    interval()
    torch.cuda.synchronize()
    n_int = max(1, args.intervals)
    mk = lambda: [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(I)] for _ in range(n_int)]
    evs, aevs = mk(), mk()
    iev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_int)]
    log("timing %d intervals of %d steps" % (n_int, I))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(n_int):
        iev[k][0].record(stream)
        interval(evs[k], aevs[k])
        iev[k][1].record(stream)
    torch.cuda.synchronize()
    el_eager = time.perf_counter() - t0
    eager_ms = [a.elapsed_time(b) / I for a, b in iev]
    attn_us = float(np.mean([a.elapsed_time(b) for row in evs for a, b in row])) * 1e3 / nl
    # the same intervals replayed from one HIP graph of a whole interval
    log("capturing one interval in a graph")
    g_int = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_int, stream=stream):
        interval()
    g_int.replay()
    torch.cuda.synchronize()
    log("timing %d graph-replayed intervals" % n_int)
    gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_int)]
    t0 = time.perf_counter()
    for a, b in gev:
        a.record(stream)
        g_int.replay()
        b.record(stream)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    graph_ms = [a.elapsed_time(b) / I for a, b in gev]
    pct = lambda v: {"p10": round(float(np.percentile(v, 10)), 4),
                     "p50": round(float(np.percentile(v, 50)), 4),
                     "p90": round(float(np.percentile(v, 90)), 4), "intervals": len(v)}
    if fused:
        append = {"fused_with_attention": True, "n_p": Np}
    else:
        app = np.array([[a.elapsed_time(b) * 1e3 / nl for a, b in row] for row in aevs])
        proj_step = Np - 1 if Np <= I else None   # the step whose appends project the batch
        append = {"us_per_layer_call": round(float(np.median(app)), 2),
                  "us_per_layer_call_projecting": (round(float(np.median(app[:, proj_step])), 2)
                                                   if proj_step is not None else None),
                  "n_p": Np}
    # compulsory gather bytes of one layer's attention launch at the first step
    gi, gc = idx[0].cpu().numpy(), cnt[0].cpu().numpy()
    rows = 0
    for b in range(B):
        Lb = int(L0[b]) + 1
        win = set(range(max(0, Lb - cfg.W), Lb))
        for kvh in range(Hkv):
            u = set(win)
            for h in range(kvh * cfg.g, (kvh + 1) * cfg.g):
                u.update(gi[b, h, :gc[b, h]].tolist())
            rows += len(u)
    attn_bytes = rows * 2 * D * 2
    achieved = attn_bytes / (attn_us * 1e-6) / 1e9
    steps = n_int * I
    res = {
        "metric": METRIC, "value": steps / el, "unit": "steps/s", "n_gpus": 1, "steps": steps,
        "warmup": I, "ms_per_step": el / steps * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (device-generated)",
        "config": {"workload": "%s: B=%d L=%s layers=%d Hq=%d Hkv=%d D=%d E=%d Eh=%d d'=%d sink=%d "
                               "window=%d budget=%d radius=%d interval=%d projection batch=%d"
                               % (cfg.name, B, "ragged %d..%d" % (L0.min(), L0.max()) if cfg.ragged
                                  else str(cfg.L), nl, Hq, Hkv, D, E, Eh, dp, cfg.S, cfg.W, cfg.K,
                                  cfg.r, I, Np),
                   "global_batch": B, "seq_len": int(L0.max())},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": None,
                     "kernel": ("append + sparse decode attention gather (one layer, one step, "
                                "one launch)" if fused else
                                "sparse decode attention gather (one layer, one step)"),
                     "bytes_per_launch": attn_bytes, "avg_launch_us": attn_us},
        "append": append,
        "eager_steps_per_s": n_int * I / el_eager,
        "ms_per_step_graph": pct(graph_ms),
        "ms_per_step_eager": pct(eager_ms),
    }
    # compulsory bytes of one interval: every layer's union gather at every
    # step, plus the K' read, predictor weights and projections once
    kp_bytes = nl * int(L0.sum()) * Hkv * dp * 2
    mlp_bytes = npro * (E * Eh + Eh * Hq * dp) * 2
    proj_bytes = nl * B * Hkv * I * (D * 2 + dp * 2)
    interval_bytes = I * nl * attn_bytes + kp_bytes + mlp_bytes + proj_bytes
    res["compulsory_bytes_per_step"] = interval_bytes / I
    res["gbps"] = interval_bytes / (el / n_int) / 1e9
    res["frac_of_peak"] = res["gbps"] / PEAK_HBM_GBS
    if emit:
        print(json.dumps(res), flush=True)
    del K, V, Kp, Wk, Q
    return res


def run_offload(cfg, args):
    """CPU-offload decoding on the 256K-context shape: every layer's full K/V
    cache in pinned host memory (read over the host link), K' and the
    per-query-head sink + important + circular-window buffers in HBM. One
    interval per layer: score and select (window left out), gather the
    selected rows from host memory into the buffers; then I steps, each
    appending the new token (host cache, window slot, K') and attending over
    the buffers. Compared with dense decoding over the same offloaded cache:
    every step fetches all L rows of every KV head over the host link, then
    attends over them."""
    import torch
    import learned_kv_cache_amd as tb

    B, Hq, Hkv, D, dp = cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.dp
    I, nl = cfg.interval, max(1, args.offload_layers)
    n_int = max(1, args.intervals)
    L = cfg.L
    Lmax = L + I * (n_int + 1)
    cap = cfg.S + cfg.K
    W = cfg.W
    buf_rows = cap + W
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20260101 + cfg.cid)

    def randn(*shape, std=1.0):
        return (torch.randn(*shape, generator=gen, device="cuda") * std).to(torch.bfloat16)

    log("building %d layers: K/V [%d, %d, %d, %d] bf16 in pinned host memory" % (nl, B, Hkv, Lmax, D))
    kh, vh, kp, wk, kb, vb, qs = [], [], [], [], [], [], []
    zero = torch.zeros(B, dtype=torch.int32, device="cuda")
    for l in range(nl):
        kd, vd = randn(B, Hkv, Lmax, D), randn(B, Hkv, Lmax, D)
        w = randn(Hkv, dp, D, std=D ** -0.5)
        p_ = torch.zeros(B, Hkv, Lmax, dp, dtype=torch.float16, device="cuda")
        tb.tb_project_keys(kd, w, p_, zero, L)
        hk = torch.empty(kd.shape, dtype=torch.bfloat16, pin_memory=True)
        hv = torch.empty(vd.shape, dtype=torch.bfloat16, pin_memory=True)
        hk.copy_(kd)
        hv.copy_(vd)
        del kd, vd
        kh.append(hk), vh.append(hv), kp.append(p_), wk.append(w)
        kb.append(torch.zeros(B, Hq, buf_rows, D, dtype=torch.bfloat16, device="cuda"))
        vb.append(torch.zeros(B, Hq, buf_rows, D, dtype=torch.bfloat16, device="cuda"))
        qs.append(randn(B, Hq, D))
    torch.cuda.synchronize()
    lens = torch.full((nl, 2, B), L, dtype=torch.int32, device="cuda")
    win = torch.arange(L - W, L, dtype=torch.int32, device="cuda").expand(B, Hq, W).contiguous()
    wcnt = torch.full((B, Hq), W, dtype=torch.int32, device="cuda")
    for l in range(nl):
        tb.tb_offload_gather(kh[l], vh[l], win, wcnt, kb[l], vb[l], slot0=cap, wrap=W)
    qhat = torch.randn(B, Hq * dp, generator=gen, device="cuda")
    scores = torch.empty(B, Hq, Lmax, device="cuda")
    idx = torch.zeros(B, Hq, cap, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(B, Hq, dtype=torch.int32, device="cuda")
    ws_s = tb.new_workspace(tb.tb_select_workspace_bytes(B, Hq, Lmax))
    ws_a = tb.new_workspace(tb.tb_attn_workspace_bytes(B, Hq, cap, W, D))
    iota = torch.arange(cap, dtype=torch.int32, device="cuda").expand(B, Hq, cap).contiguous()
    full = torch.full((B,), buf_rows, dtype=torch.int32, device="cuda")
    out = torch.empty(B, Hq, D, device="cuda")
    k_new = [randn(B, Hkv, D) for _ in range(I)]
    v_new = [randn(B, Hkv, D) for _ in range(I)]
    mode = tb.TB_NF_FILL | tb.TB_SEL_OMIT_WINDOW
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def interval(rec):
        for l in range(nl):
            ctx, pl = lens[l, 0], lens[l, 1]
            e = [ev() for _ in range(3)]
            e[0].record()
            tb.tb_score_select(qhat, kp[l], ctx, pl, scores, cfg.S, W, cfg.K, cfg.r, idx, cnt, ws_s,
                               mode=mode)
            e[1].record()
            tb.tb_offload_gather(kh[l], vh[l], idx, cnt, kb[l], vb[l])
            e[2].record()
            rec["select"].append(e[:2])
            rec["gather"].append(e[1:])
        for j in range(I):
            e = [ev() for _ in range(3)]
            e[0].record()
            for l in range(nl):
                tb.tb_offload_append(k_new[j], v_new[j], wk[l], kh[l], vh[l], kp[l], lens[l, 0],
                                     lens[l, 1], kb[l], vb[l], W)
            e[1].record()
            for l in range(nl):
                tb.tb_sparse_decode_attn(qs[l], kb[l], vb[l], iota, cnt, out, ws_a, ctx_len=full,
                                         window=W)
            e[2].record()
            rec["append"].append(e[:2])
            rec["attn"].append(e[1:])

    log("warmup interval")
    interval({"select": [], "gather": [], "append": [], "attn": []})
    torch.cuda.synchronize()
    rec = {"select": [], "gather": [], "append": [], "attn": []}
    log("timing %d intervals of %d steps over %d layers" % (n_int - 1, I, nl))
    t0 = time.perf_counter()
    for _ in range(n_int - 1):
        interval(rec)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms = lambda k: float(np.mean([a.elapsed_time(b) for a, b in rec[k]]))
    gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
    gather_bytes = int(gc.sum()) * 2 * D * 2
    union = 0
    for kvh in range(Hkv):
        su = set()
        for h in range(kvh * cfg.g, (kvh + 1) * cfg.g):
            su.update(gi[0, h, :gc[0, h]].tolist())
        union += len(su)
    steps = (n_int - 1) * I
    # dense decoding over the offloaded cache, one layer: fetch all rows of
    # every KV head over the host link, attend over them
    log("dense comparison: fetching %d rows x %d KV heads over the host link" % (L, Hkv))
    dk = torch.empty(B, Hkv, L, D, dtype=torch.bfloat16, device="cuda")
    dv = torch.empty_like(dk)
    didx = torch.arange(L, dtype=torch.int32, device="cuda").expand(B, Hkv, L).contiguous()
    dcnt = torch.full((B, Hkv), L, dtype=torch.int32, device="cuda")
    aidx = torch.arange(L, dtype=torch.int32, device="cuda").expand(B, Hq, L).contiguous()
    acnt = torch.full((B, Hq), L, dtype=torch.int32, device="cuda")
    ws_d = tb.new_workspace(tb.tb_attn_workspace_bytes(B, Hq, L, 0, D))
    dres = []
    for rep in range(3):
        e = [ev() for _ in range(3)]
        e[0].record()
        tb.tb_offload_gather(kh[0], vh[0], didx, dcnt, dk, dv)
        e[1].record()
        tb.tb_sparse_decode_attn(qs[0], dk, dv, aidx, acnt, out, ws_d)
        e[2].record()
        dres.append(e)
    torch.cuda.synchronize()
    dense_fetch = float(np.mean([e[0].elapsed_time(e[1]) for e in dres[1:]]))
    dense_attn = float(np.mean([e[1].elapsed_time(e[2]) for e in dres[1:]]))
    dense_bytes = B * Hkv * L * 2 * D * 2
    per_step_layer = el / steps / nl
    res = {
        "metric": "offloaded decode steps/s at 256K ctx, 8K budget; host-link GB/s",
        "value": steps / el, "unit": "steps/s (all %d layers)" % nl, "n_gpus": 1, "steps": steps,
        "warmup": I, "ms_per_step": el / steps * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (device-generated, copied to pinned host memory)",
        "config": {"workload": "%s, CPU offload: B=%d L=%d layers=%d Hq=%d Hkv=%d D=%d sink=%d window=%d "
                               "budget=%d radius=%d interval=%d" % (cfg.name, B, L, nl, Hq, Hkv, D,
                                                                   cfg.S, W, cfg.K, cfg.r, I),
                   "global_batch": B, "seq_len": L},
        "per_layer_ms": {"select": round(ms("select"), 4), "gather": round(ms("gather"), 4),
                         "append_step": round(ms("append") / nl, 4),
                         "attention_step": round(ms("attn") / nl, 4),
                         "per_step_amortised": round(per_step_layer * 1e3, 4)},
        "gather": {"rows_per_head_total": int(gc.sum()), "union_rows": union,
                   "bytes": gather_bytes, "gbps": gather_bytes / ms("gather") / 1e6},
        "dense_offload_per_layer_ms": {"fetch": round(dense_fetch, 3), "attention": round(dense_attn, 3),
                                       "bytes": dense_bytes,
                                       "fetch_gbps": dense_bytes / dense_fetch / 1e6},
        "speedup_vs_dense_offload": (dense_fetch + dense_attn) / (per_step_layer * 1e3),
    }
    print(json.dumps(res), flush=True)


def run_distill(cfg, args):
    """The distillation loss on the 64K single-layer shape: R query positions
    per sequence taken from the late context (the last quarter, always
    including the final token), every query head, the causal tokens up to
    each position. Reports the time per call against HBM (K and K' read
    once per row group) and against bf16 MFMA (teacher logits)."""
    import torch
    import learned_kv_cache_amd as tb

    B, Hq, Hkv, D, dp, L = cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.dp, cfg.L
    R = args.distill_positions
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20260101 + cfg.cid)
    rn = lambda *sh: torch.randn(*sh, generator=gen, device="cuda").to(torch.bfloat16)
    reps = []
    for i in range(args.replicas):
        reps.append(dict(q=rn(B, R, Hq, D), kc=rn(B, Hkv, L, D),
                         qhat=torch.randn(B, R, Hq, dp, generator=gen, device="cuda"),
                         kp=torch.randn(B, Hkv, L, dp, generator=gen, device="cuda").half()))
    pos_np = np.sort(np.random.default_rng(20260101).integers(3 * L // 4, L, size=(B, R)), axis=1)
    pos_np[:, -1] = L - 1
    pos = torch.from_numpy(pos_np.astype(np.int32)).cuda()
    loss = torch.empty(B, R, Hq, device="cuda")
    ws = tb.new_workspace(tb.tb_distill_workspace_bytes(B, R, Hq, Hkv, L))
    for r_ in reps:
        tb.tb_distill_loss(r_["q"], r_["kc"], r_["qhat"], r_["kp"], pos, loss, ws)
    torch.cuda.synchronize()
    n = 10 * len(reps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        r_ = reps[i % len(reps)]
        tb.tb_distill_loss(r_["q"], r_["kc"], r_["qhat"], r_["kp"], pos, loss, ws)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / n
    toks = int((pos_np.astype(np.int64) + 1).sum()) * Hq
    flops = 2 * toks * (D + dp)
    ng = -(-R * (Hq // Hkv) // 256)
    last = int(pos_np.max()) + 1
    hbm = B * Hkv * ng * last * (D + dp) * 2
    res = {
        "metric": "distillation-loss calls/s at 64K ctx, %d query positions" % R,
        "value": 1e6 / us, "unit": "calls/s", "n_gpus": 1, "steps": n, "warmup": len(reps),
        "ms_per_step": us / 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (device-generated)",
        "config": {"workload": "distillation loss: B=%d L=%d R=%d positions in the last quarter "
                               "Hq=%d Hkv=%d D=%d d'=%d, %d rotated replicas"
                               % (B, L, R, Hq, Hkv, D, dp, len(reps)),
                   "global_batch": B, "seq_len": L},
        "hbm": {"bytes": hbm, "gbps": hbm / us / 1e3, "frac": hbm / us / 1e3 / PEAK_HBM_GBS},
        "mfma": {"flops": flops, "tflops": flops / us / 1e6, "frac_of_bf16_dense": flops / us / 1e6 / 2500.0},
    }
    print(json.dumps(res), flush=True)


def measure_ceilings(tb, reps, idx, cnt, cfg, union_rows, row_bytes, stream, capture):
    """Bandwidth ceilings of this part in the same process: a plain streaming
    read of 2 GiB, and a gather of exactly the K/V rows the step's attention
    reads (its launch shape, K and V rows requested together, no arithmetic),
    over the rotated replicas."""
    import torch
    R = len(reps)
    nbytes = 2 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    tb.tb_probe_stream_read(buf, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 10
    e0.record(stream)
    for _ in range(n):
        tb.tb_probe_stream_read(buf, sink)
    e1.record(stream)
    torch.cuda.synchronize()
    read_us = e0.elapsed_time(e1) * 1e3 / n
    del buf
    B, Hq, cap = idx.shape
    gsink = torch.zeros(tb.tb_probe_row_gather_sink_words(B, Hq, cap), dtype=torch.int32,
                        device="cuda")

    def one(i):
        r = reps[i % R]
        tb.tb_probe_row_gather(r["kc"], r["vc"], idx, cnt, gsink)
    g = capture(one, R)
    g.replay()
    torch.cuda.synchronize()
    n = 50
    e0.record(stream)
    for _ in range(n):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    gather_us = e0.elapsed_time(e1) * 1e3 / (n * R)
    gather_bytes = union_rows * row_bytes
    return {"stream_read": {"bytes": nbytes, "us": round(read_us, 2),
                            "gbps": nbytes / read_us / 1e3,
                            "frac": nbytes / read_us / 1e3 / PEAK_HBM_GBS},
            "attention_row_gather": {"bytes": gather_bytes, "us": round(gather_us, 2),
                                     "gbps": gather_bytes / gather_us / 1e3,
                                     "frac": gather_bytes / gather_us / 1e3 / PEAK_HBM_GBS,
                                     "note": "the step's attention rows (per-head lists, union "
                                             "bytes counted), its launch shape, no arithmetic"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-intervals", action="store_true",
                    help="skip the C3 and C5 interval lines of the default run")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured streaming-read and row-gather ceilings")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--append", choices=("fused", "separate"), default="fused",
                    help="interval steps: each layer's K/V append and attention in one launch "
                         "(tb_append_attn) or as tb_append_kv then tb_sparse_decode_attn")
    ap.add_argument("--defer", choices=("select", "list"), default="select",
                    help="the step's selection: split across the two calls "
                         "(TB_SEL_DEFER_SELECT; the attention launch finds the threshold) or "
                         "the list deferred (TB_SEL_DEFER_LIST)")
    ap.add_argument("--stages", action="store_true",
                    help="also time the other call sequences' stages (list written by the "
                         "selection, separate score and select)")
    ap.add_argument("--core-only", action="store_true",
                    help="time the decode step only (no whole-context projection), e.g. under a "
                         "profiler")
    ap.add_argument("--dilate", action="store_true",
                    help="also time the dilation reading of neighbour fetching on the same scores "
                         "(its attention launches are of the same kernel, so they are kept out of "
                         "the default run and its kernel trace)")
    ap.add_argument("--config", type=int, default=2,
                    help="2: the single-layer decode step (default); 3, 4, 5: the multi-layer "
                         "prediction-interval workloads")
    ap.add_argument("--intervals", type=int, default=5)
    ap.add_argument("--offload", action="store_true",
                    help="CPU-offload decoding on the 256K-context shape (with --config 4)")
    ap.add_argument("--offload-layers", type=int, default=4)
    ap.add_argument("--distill", action="store_true",
                    help="time the distillation loss on the 64K single-layer shape")
    ap.add_argument("--distill-positions", type=int, default=64)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 1 GiB device copy (for PMC byte-counter calibration) and exit")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only; --gpus %d is not supported (this path does not "
              "shard across GPUs)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import learned_kv_cache_amd as tb
    from synthetic import CONFIGS
    from synthetic.workload import make_layer

    torch.cuda.set_device(0)
    # all work on one non-default stream (graph capture needs one)
    torch.cuda.set_stream(torch.cuda.Stream())
    if args.copy_calibration:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty(n, dtype=torch.uint8, device="cuda")
        a.fill_(1)
        torch.cuda.synchronize()
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))
        return

    if args.distill:
        run_distill(CONFIGS[2], args)
        return
    if args.offload:
        run_offload(CONFIGS[4 if args.config == 2 else args.config], args)
        return
    if args.config != 2:
        run_interval(CONFIGS[args.config], args)
        return
    cfg = CONFIGS[2]
    B, L, R = 1, cfg.L, max(1, args.replicas)
    log("generating inputs (%s)" % cfg.name)
    inp = make_layer(cfg, seed=0, direction_fn=lambda d: planting_direction(d, cfg))

    def dev16(a, dt):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(dt).cuda()

    log("uploading %d replicas" % R)
    reps = []
    base = {k: dev16(inp[k], torch.bfloat16) for k in ("x", "w1", "w2", "kc", "vc", "wk", "q")}
    zeros = torch.zeros(B, dtype=torch.int32, device="cuda")
    for i in range(R):
        r = {k: (v if i == 0 else v.clone()) for k, v in base.items()}
        r["kp"] = torch.zeros((B, cfg.Hkv, L, cfg.dp), dtype=torch.float16, device="cuda")
        tb.tb_project_keys(r["kc"], r["wk"], r["kp"], zeros, L - 1)   # the cache before this step
        reps.append(r)
    torch.cuda.synchronize()

    # whole-context key projection (the prefill step before the decode path),
    # timed over the rotated replicas
    pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(0 if args.core_only else 3 * R)]
    for i, (e0, e1) in enumerate(pev):
        r_ = reps[i % R]
        e0.record()
        tb.tb_project_keys(r_["kc"], r_["wk"], r_["kp"], zeros, L - 1)
        e1.record()
    torch.cuda.synchronize()
    prefill = None
    if pev:
        proj_us = float(np.mean([a.elapsed_time(b) for a, b in pev[R:]])) * 1e3
        proj_bytes = B * cfg.Hkv * (L - 1) * (cfg.D * 2 + cfg.dp * 2) + cfg.Hkv * cfg.dp * cfg.D * 2
        prefill = {"tokens": (L - 1) * B, "kv_heads": cfg.Hkv, "us": round(proj_us, 2),
                   "bytes": proj_bytes, "gbps": proj_bytes / proj_us / 1e3,
                   "frac": proj_bytes / proj_us / 1e3 / PEAK_HBM_GBS}

    ctx = torch.full((B,), L, dtype=torch.int32, device="cuda")
    pos_new = torch.full((B,), L - 1, dtype=torch.int32, device="cuda")
    qhat = torch.empty((B, cfg.n_out), device="cuda")
    scores = torch.empty((B, cfg.Hq, L), device="cuda")
    cap = cfg.cap
    idx = torch.zeros((B, cfg.Hq, cap), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((B, cfg.Hq), dtype=torch.int32, device="cuda")
    out = torch.zeros((B, cfg.Hq, cfg.D), device="cuda")
    ws_p = tb.new_workspace(tb.tb_predict_workspace_bytes(B, cfg.E, cfg.Eh, cfg.n_out))
    ws_s = tb.new_workspace(tb.tb_select_workspace_bytes(B, cfg.Hq, L))
    ws_a = tb.new_workspace(tb.tb_attn_workspace_bytes(B, cfg.Hq, cap, 0, cfg.D))

    # Pre-marshalled C ABI calls (same entry points as the binding, without
    # per-call Python argument checks, so the host keeps ahead of the GPU).
    # Validate every argument set once through the checked binding first.
    tb.tb_predict_project(reps[0]["x"], reps[0]["w1"], reps[0]["w2"], qhat, ws_p, reps[0]["kc"],
                          reps[0]["wk"], reps[0]["kp"], pos_new, 1)
    tb.tb_score(qhat, reps[0]["kp"], ctx, scores)
    tb.tb_select(scores, ctx, ctx, cfg.S, cfg.W, cfg.K, cfg.r, idx, cnt, ws_s)
    tb.tb_score_select(qhat, reps[0]["kp"], ctx, ctx, scores, cfg.S, cfg.W, cfg.K, cfg.r, idx, cnt,
                       ws_s)
    tb.tb_sparse_decode_attn(reps[0]["q"], reps[0]["kc"], reps[0]["vc"], idx, cnt, out, ws_a)
    split = args.defer == "select"
    defer = tb.TB_NF_FILL | (tb.TB_SEL_DEFER_SELECT if split else tb.TB_SEL_DEFER_LIST)
    tb.tb_score_select(qhat, reps[0]["kp"], ctx, ctx, scores, cfg.S, cfg.W, cfg.K, cfg.r, idx, cnt,
                       ws_s, mode=defer)
    tb.tb_select_attn(ctx, ctx, cfg.S, cfg.W, cfg.K, cfg.r, idx, cnt, ws_s, reps[0]["q"],
                      reps[0]["kc"], reps[0]["vc"], out, ws_a, mode=defer)
    torch.cuda.synchronize()

    L_ = tb.lib()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    nb = lambda w: w.numel()
    calls = []
    for r in reps:
        calls.append([
            (L_.tb_predict_project, (P(r["x"]), P(r["w1"]), P(r["w2"]), P(qhat), B, cfg.E, cfg.Eh,
                                     cfg.n_out, P(ws_p), nb(ws_p), P(r["kc"]), P(r["wk"]),
                                     P(r["kp"]), P(pos_new), 1, cfg.Hkv, L, cfg.D, cfg.dp, sp)),
            (L_.tb_score_select, (P(qhat), 1, 0, P(r["kp"]), P(ctx), P(ctx), P(scores), B, cfg.Hq,
                                  cfg.Hkv, L, cfg.dp, cfg.S, cfg.W, cfg.K, cfg.r, defer, P(idx),
                                  P(cnt), cap, P(ws_s), nb(ws_s), sp)),
            (L_.tb_select_attn, (P(ctx), P(ctx), B, cfg.Hq, cfg.Hkv, L, cfg.S, cfg.W, cfg.K, cfg.r,
                                 defer, P(idx), P(cnt), cap, P(ws_s), nb(ws_s), P(r["q"]),
                                 P(r["kc"]), P(r["vc"]), cfg.D,
                                 ctypes.c_float(1.0 / np.sqrt(cfg.D)), P(out), P(ws_a), nb(ws_a),
                                 sp)),
        ])

    def run_step(i, ev=None):
        c = calls[i % R]
        for j, (fn, a) in enumerate(c):
            if ev is not None and j == len(c) - 1:   # the list + attention
                ev[0].record(stream)
            st = fn(*a)
            if st:
                raise RuntimeError("libtb call failed: %s" % L_.tb_last_error_detail().decode())
        if ev is not None:
            ev[1].record(stream)

    log("warmup %d" % args.warmup)
    for i in range(args.warmup):
        run_step(i)
    torch.cuda.synchronize()

    K = args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    log("timing %d eager steps" % K)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        run_step(i, evs[i])
    torch.cuda.synchronize()
    eager_elapsed = time.perf_counter() - t0
    attn_ms = [a.elapsed_time(b) for a, b in evs]
    attn_avg_s = float(np.mean(attn_ms)) / 1e3

    def capture(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                fn(i)
        return g

    full, rem = divmod(K, R)
    g_all = capture(run_step, R)
    g_rem = capture(run_step, rem) if rem else None
    for _ in range(max(1, args.warmup // R)):
        g_all.replay()
    torch.cuda.synchronize()
    log("timing %d graph-replayed steps" % K)
    t0 = time.perf_counter()
    for _ in range(full):
        g_all.replay()
    if g_rem is not None:
        g_rem.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # per-step time distribution: one more pass of replays, each bracketed by events
    rev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(min(full, 100))]
    for a, b in rev:
        a.record(stream)
        g_all.replay()
        b.record(stream)
    torch.cuda.synchronize()
    step_pct = None
    if rev:
        per = np.array([a.elapsed_time(b) * 1e3 / R for a, b in rev])
        step_pct = {"p10": round(float(np.percentile(per, 10)), 2),
                    "p50": round(float(np.percentile(per, 50)), 2),
                    "p90": round(float(np.percentile(per, 90)), 2), "replays": len(rev)}

    # the dominant kernel alone: a graph of one compaction + attention launch
    # per replica (tb_select_attn on the selection state the last step left),
    # replayed back to back between two events on its stream, so the average
    # is the launch's own duration (no host gaps between launches). With the
    # split selection the attention launch consumes its state (it clears the
    # histograms), so it cannot be replayed alone: its duration is the mean of
    # fence-free events recorded around it on its stream over whole eager
    # steps, issued behind a GPU spin long enough that the host stays ahead of
    # the GPU (no host gaps inside the events).
    attn_eager_avg_s = attn_avg_s
    n_attn = K
    g_attn = None
    if split:
        n_attn = min(K, 600)
        evs2 = [(FenceFreeEvent(), FenceFreeEvent()) for _ in range(n_attn)]
        torch.cuda.synchronize()
        torch.cuda._sleep(int(2.4e9 * (n_attn * 40e-6 + 5e-3)))   # cycles at ~2.4 GHz
        for i in range(n_attn):
            run_step(i, evs2[i])
        torch.cuda.synchronize()
        attn_avg_s = float(np.mean([a.elapsed_time(b) for a, b in evs2])) / 1e3
    else:
        def attn_only(i):
            fn, a = calls[i % R][-1]
            if fn(*a):
                raise RuntimeError(L_.tb_last_error_detail().decode())
        g_attn = capture(attn_only, R)
        g_attn.replay()
        ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n_attn = max(1, min(200, K // R)) * R
        torch.cuda.synchronize()
        ea.record(stream)
        for _ in range(n_attn // R):
            g_attn.replay()
        eb.record(stream)
        torch.cuda.synchronize()
        attn_avg_s = ea.elapsed_time(eb) / 1e3 / n_attn

    # algorithmic bytes of one attention launch: each distinct (kv head, token)
    # row of the g heads' attended sets, K and V, bf16 -- counted from idx
    gi = idx.cpu().numpy()
    gc = cnt.cpu().numpy()
    union_rows = 0
    per_head_rows = int(gc.sum())
    for kvh in range(cfg.Hkv):
        s = set()
        for h in range(kvh * cfg.g, (kvh + 1) * cfg.g):
            s.update(gi[0, h, :gc[0, h]].tolist())
        union_rows += len(s)
    row_bytes = 2 * cfg.D * 2
    attn_bytes = union_rows * row_bytes + cfg.Hq * cfg.D * (2 + 4) + gc.size * 4 + per_head_rows * 4
    achieved = attn_bytes / attn_avg_s / 1e9

    # compulsory bytes of the whole step (for the step-level GB/s)
    kp_bytes = L * cfg.Hkv * cfg.dp * 2
    mlp_bytes = (cfg.E * cfg.Eh + cfg.Eh * cfg.n_out) * 2
    proj_bytes = cfg.Hkv * (cfg.D * 2 + cfg.dp * cfg.D * 2 + cfg.dp * 2)
    step_bytes = union_rows * row_bytes + kp_bytes + mlp_bytes + proj_bytes
    step_s = elapsed / K

    # each stage alone, as a graph of that stage over the R replicas: the
    # step's three calls always; with --stages also the other call sequence
    # on the same inputs (the list written by the selection, then the
    # attention launch over it) and the separate score and select calls
    # (the attention call consumes the selection's state, so the span is timed
    # as the two calls together and score+select as the difference)
    names = [("predict+project", calls, (0,)), ("score+select+attention", calls, (1, 2))]
    if not split:
        names.append(("list+attention", calls, (2,)))
    if args.stages:
        sep = [[(L_.tb_score, (P(qhat), 1, 0, P(r["kp"]), P(ctx), P(scores), B, cfg.Hq, cfg.Hkv,
                               L, cfg.dp, sp)),
                (L_.tb_select, (P(scores), P(ctx), P(ctx), B, cfg.Hq, L, cfg.S, cfg.W, cfg.K,
                                cfg.r, tb.TB_NF_FILL, P(idx), P(cnt), cap, P(ws_s), nb(ws_s),
                                sp))] for r in reps]
        lst = [[(L_.tb_score_select, (P(qhat), 1, 0, P(r["kp"]), P(ctx), P(ctx), P(scores), B,
                                      cfg.Hq, cfg.Hkv, L, cfg.dp, cfg.S, cfg.W, cfg.K, cfg.r,
                                      tb.TB_NF_FILL, P(idx), P(cnt), cap, P(ws_s), nb(ws_s), sp)),
                (L_.tb_sparse_decode_attn, (P(r["q"]), P(r["kc"]), P(r["vc"]), P(idx), P(cnt),
                                            cap, None, 0, B, cfg.Hq, cfg.Hkv, L, cfg.D,
                                            ctypes.c_float(1.0 / np.sqrt(cfg.D)), P(out), P(ws_a),
                                            nb(ws_a), sp))] for r in reps]
        names += [("score+select, list written", lst, (0,)), ("attention", lst, (1,)),
                  ("score", sep, (0,)), ("select", sep, (1,))]
    stages = {}
    n_rep = 50
    for n, cl, js in names:
        def one(i, js=js, cl=cl):
            for j in js:
                fn, a = cl[i % R][j]
                if fn(*a):
                    raise RuntimeError(L_.tb_last_error_detail().decode())
        g = capture(one, R)
        g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n_rep):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        stages[n] = round(e0.elapsed_time(e1) * 1e3 / (n_rep * R), 2)
    if split:
        stages["threshold+list+attention"] = round(attn_avg_s * 1e6, 2)
    stages["score+select"] = round(stages["score+select+attention"] -
                                   (attn_avg_s * 1e6 if split else stages["list+attention"]), 2)
    # the last stage graphs leave the step's selection state in place again
    for i in range(R):
        run_step(i)
    torch.cuda.synchronize()

    ceilings = None
    if not args.no_ceilings:
        ceilings = measure_ceilings(tb, reps, idx, cnt, cfg, union_rows, row_bytes, stream, capture)

    dilate = None
    if args.dilate:
        # the other reading of neighbour fetching (neighbours beyond the budget),
        # on the same scores: its list sizes, bytes and times beside the fill mode
        cap_d = min(L, cfg.S + cfg.W + (2 * cfg.r + 1) * cfg.K)
        idx_d = torch.zeros((B, cfg.Hq, cap_d), dtype=torch.int32, device="cuda")
        cnt_d = torch.zeros((B, cfg.Hq), dtype=torch.int32, device="cuda")
        out_d = torch.zeros((B, cfg.Hq, cfg.D), device="cuda")
        ws_ad = tb.new_workspace(tb.tb_attn_workspace_bytes(B, cfg.Hq, cap_d, 0, cfg.D))
        tb.tb_select(scores, ctx, ctx, cfg.S, cfg.W, cfg.K, cfg.r, idx_d, cnt_d, ws_s,
                     mode=tb.TB_NF_DILATE)
        torch.cuda.synchronize()
        dcalls = []
        for r_ in reps:
            dcalls.append([
                (L_.tb_select, (P(scores), P(ctx), P(ctx), B, cfg.Hq, L, cfg.S, cfg.W, cfg.K, cfg.r,
                                tb.TB_NF_DILATE, P(idx_d), P(cnt_d), cap_d, P(ws_s), nb(ws_s), sp)),
                (L_.tb_sparse_decode_attn, (P(r_["q"]), P(r_["kc"]), P(r_["vc"]), P(idx_d), P(cnt_d),
                                            cap_d, None, 0, B, cfg.Hq, cfg.Hkv, L, cfg.D,
                                            ctypes.c_float(1.0 / np.sqrt(cfg.D)), P(out_d), P(ws_ad),
                                            nb(ws_ad), sp)),
            ])
        dil_us = []
        for j in range(2):
            def one_d(i, j=j):
                fn, a = dcalls[i % R][j]
                if fn(*a):
                    raise RuntimeError(L_.tb_last_error_detail().decode())
            gd = capture(one_d, R)
            gd.replay()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(20):
                gd.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            dil_us.append(e0.elapsed_time(e1) * 1e3 / (20 * R))
        di, dc = idx_d.cpu().numpy(), cnt_d.cpu().numpy()
        d_union = 0
        for kvh in range(cfg.Hkv):
            su = set()
            for h in range(kvh * cfg.g, (kvh + 1) * cfg.g):
                su.update(di[0, h, :dc[0, h]].tolist())
            d_union += len(su)
        d_bytes = d_union * row_bytes + cfg.Hq * cfg.D * (2 + 4) + dc.size * 4 + int(dc.sum()) * 4
        dilate = {"attended_per_head_mean": float(dc.mean()), "union_rows": d_union,
                  "per_head_rows": int(dc.sum()), "attn_bytes": d_bytes,
                  "select_us": round(dil_us[0], 2), "attention_us": round(dil_us[1], 2),
                  "attention_gbps": d_bytes / dil_us[1] / 1e3,
                  "fill_attended_per_head_mean": float(gc.mean()), "fill_attn_bytes": attn_bytes}

    traffic = traffic_record(args.defer)
    res = {
        "metric": METRIC,
        "value": K / elapsed,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s: B=%d L=%d Hq=%d Hkv=%d D=%d E=%d Eh=%d d'=%d sink=%d "
                               "window=%d budget=%d radius=%d, predictor every step, %d planted "
                               "8-token spans, %d rotated input replicas"
                               % (cfg.name, B, L, cfg.Hq, cfg.Hkv, cfg.D, cfg.E, cfg.Eh, cfg.dp,
                                  cfg.S, cfg.W, cfg.K, cfg.r, cfg.n_spans, R),
                   "global_batch": B, "seq_len": L},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": ("threshold + list + sparse decode attention gather "
                                "(split_attn_kernel<128>)" if split else
                                "list compaction + sparse decode attention gather "
                                "(compact_attn_kernel<128>)"),
                     "bytes_per_launch": attn_bytes, "avg_launch_us": attn_avg_s * 1e6,
                     "launches_timed": n_attn,
                     "avg_launch_us_eager_events": attn_eager_avg_s * 1e6},
        "eager_steps_per_s": K / eager_elapsed,
        "step_us": step_pct,
        "step_gbps": step_bytes / step_s / 1e9,
        "step_compulsory_bytes": step_bytes,
        "attended_rows": {"union": union_rows, "per_head": per_head_rows},
        **({"dilate_mode": dilate} if dilate else {}),
        **({"prefill_projection": prefill} if prefill else {}),
    }
    res["stages_us"] = stages
    # the target span, score + select + attention: its compulsory bytes are
    # the K' read and the union gather
    span_us = stages["score+select+attention"]
    span_bytes = kp_bytes + union_rows * row_bytes
    res["score_select_attn"] = {"us": round(span_us, 2), "bytes": span_bytes,
                                "gbps": span_bytes / span_us / 1e3,
                                "frac": span_bytes / span_us / 1e3 / PEAK_HBM_GBS}
    if ceilings:
        res["ceilings"] = ceilings
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle), ~%.0f s" % args.cpu_seconds)
        res["cpu_baseline"] = cpu_baseline(inp, cfg, args.cpu_seconds)
    if not args.no_intervals:
        # the multi-layer prediction-interval workloads on the Llama-3.1-8B
        # (C3) and Qwen2.5-7B (C5) shapes, after the single-layer step's
        # buffers are released
        del calls, reps, base, g_all, g_rem, g_attn
        import gc
        gc.collect()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        res["interval_workloads"] = {}
        for cid in (3, 5):
            a2 = argparse.Namespace(**vars(args))
            a2.intervals = 3
            r_ = run_interval(CONFIGS[cid], a2, emit=False)
            res["interval_workloads"]["C%d" % cid] = {
                "workload": r_["config"]["workload"], "steps_per_s": r_["value"],
                "ms_per_step_graph": r_["ms_per_step_graph"],
                "compulsory_bytes_per_step": r_["compulsory_bytes_per_step"],
                "gbps": r_["gbps"], "frac_of_peak": r_["frac_of_peak"],
                "attention_gbps_per_launch": r_["roofline"]["achieved"]}
            gc.collect()
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
