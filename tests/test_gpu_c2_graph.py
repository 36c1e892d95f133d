"""GPU parity of the full-size single-layer decode step (Llama-3.1-8B-shaped
layer, 64K context, budget 7872, radius 1, planted spans) in the launch
configuration the benchmark times: tb_predict_project (predictor + the
newest key's projection in one launch), tb_score_select with the list
deferred (scoring with the selection's band sampled in the same launch, then
the selection up to its threshold) and tb_select_attn (the list written by the
attention workgroups, which attend over it) captured in one HIP graph and
replayed. Every replay,
with the outputs poisoned before it, is checked against the oracle's step
on the same seeded inputs (predicted queries, sampled projected-key rows,
scores, selection with the near-tie band rule, attention)."""
import numpy as np
import pytest
import torch

from synthetic import CONFIGS
from synthetic.workload import make_layer
from gpu_util import bits, dev, dev32, host, say
from workloads import oracle_direction, oracle_step
from test_gpu_e2e import compare_step

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import learned_kv_cache_amd as tb
    tb.lib()
    return tb


def test_c2_step_graph_replays_match_oracle(tb, orc):
    cfg = CONFIGS[2]
    say("c2 graph step: generating")
    inp = make_layer(cfg, seed=0, direction_fn=oracle_direction(orc, cfg))
    say("c2 graph step: oracle")
    o = oracle_step(orc, cfg, inp)
    B, L = 1, cfg.L
    x, w1, w2 = (dev(inp[k], torch.bfloat16) for k in ("x", "w1", "w2"))
    kc, vc, wk, q = (dev(inp[k], torch.bfloat16) for k in ("kc", "vc", "wk", "q"))
    kp = torch.zeros((B, cfg.Hkv, L, cfg.dp), dtype=torch.float16, device="cuda")
    # the cache before this step is projected (setup, as in the benchmark)
    tb.tb_project_keys(kc, wk, kp, dev32(np.zeros(B, np.int32)), L - 1)
    ctx = dev32(np.full(B, L, np.int32))
    pos_new = dev32(np.full(B, L - 1, np.int32))
    cap = cfg.S + cfg.W + cfg.K
    qhat = torch.empty((B, cfg.n_out), device="cuda")
    scores = torch.empty((B, cfg.Hq, L), device="cuda")
    idx = torch.empty((B, cfg.Hq, cap), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, cfg.Hq), dtype=torch.int32, device="cuda")
    out = torch.empty((B, cfg.Hq, cfg.D), device="cuda")
    ws_p = tb.new_workspace(tb.tb_predict_workspace_bytes(B, cfg.E, cfg.Eh, cfg.n_out))
    ws_s = tb.new_workspace(tb.tb_select_workspace_bytes(B, cfg.Hq, L))
    ws_a = tb.new_workspace(tb.tb_attn_workspace_bytes(B, cfg.Hq, cap, 0, cfg.D))

    def step():
        tb.tb_predict_project(x, w1, w2, qhat, ws_p, kc, wk, kp, pos_new, 1)
        defer = tb.TB_NF_FILL | tb.TB_SEL_DEFER_LIST
        tb.tb_score_select(qhat, kp, ctx, ctx, scores, cfg.S, cfg.W, cfg.K, cfg.r, idx, cnt, ws_s,
                           mode=defer)
        tb.tb_select_attn(ctx, ctx, cfg.S, cfg.W, cfg.K, cfg.r, idx, cnt, ws_s, q, kc, vc, out,
                          ws_a, mode=defer)

    def poison():
        qhat.fill_(float("nan"))
        scores.fill_(float("nan"))
        idx.fill_(-7)
        cnt.fill_(-1)
        out.fill_(float("nan"))

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step()                                  # eager warm-up on the capture stream
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            step()
        rows = list(range(0, L, 997)) + [L - 1]
        for rep in range(3):
            poison()
            g.replay()
            torch.cuda.synchronize()
            say("c2 graph step: replay", rep)
            got = dict(qhat=host(qhat), kp=bits(kp), scores=host(scores), idx=host(idx),
                       count=host(cnt), out=host(out), dev=dict(q=q, kc=kc, vc=vc))
            compare_step(tb, orc, cfg, inp, got, o, kp_rows=rows)
