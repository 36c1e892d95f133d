"""A whole decode step (predict + project, score, select, sparse attention)
captured in a HIP graph through torch.cuda.CUDAGraph replays to bitwise the
results of the same calls issued eagerly. Between replays, eager calls on a
second input set share every workspace, so state a call leaves behind (the
arrival counters, the sample and candidate buffers) is exercised too."""
import numpy as np
import pytest
import torch

from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import learned_kv_cache_amd as tb
    tb.lib()
    return tb


B, Hq, Hkv, D, E, Eh, DP = 2, 32, 8, 128, 4096, 1024, 32
LMAX, S, W, K, R = 20000, 64, 256, 2000, 1
CAP = S + W + K


def make_inputs(seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    rn = lambda *s, std=1.0: (torch.randn(*s, generator=g, device="cuda") * std).to(torch.bfloat16)
    return dict(x=rn(B, E), w1=rn(Eh, E, std=E ** -0.5), w2=rn(Hq * DP, Eh, std=Eh ** -0.5),
                kc=rn(B, Hkv, LMAX, D), vc=rn(B, Hkv, LMAX, D), wk=rn(Hkv, DP, D, std=D ** -0.5),
                q=rn(B, Hq, D))


class Step:
    def __init__(self, tb, inp, ws):
        self.tb, self.inp, self.ws = tb, inp, ws
        self.ctx = torch.tensor([LMAX, 13001], dtype=torch.int32, device="cuda")
        self.pos = self.ctx - 1
        self.kp = torch.zeros((B, Hkv, LMAX, DP), dtype=torch.float16, device="cuda")
        tb.tb_project_keys(inp["kc"], inp["wk"], self.kp, torch.zeros(B, dtype=torch.int32,
                                                                      device="cuda"), LMAX - 1)
        self.qhat = torch.empty((B, Hq * DP), device="cuda")
        self.scores = torch.empty((B, Hq, LMAX), device="cuda")
        self.idx = torch.full((B, Hq, CAP), -1, dtype=torch.int32, device="cuda")
        self.cnt = torch.zeros((B, Hq), dtype=torch.int32, device="cuda")
        self.out = torch.zeros((B, Hq, D), device="cuda")

    def __call__(self):
        tb, i, ws = self.tb, self.inp, self.ws
        tb.tb_predict_project(i["x"], i["w1"], i["w2"], self.qhat, ws["p"], i["kc"], i["wk"],
                              self.kp, self.pos, 1)
        tb.tb_score(self.qhat, self.kp, self.ctx, self.scores)
        tb.tb_select(self.scores, self.ctx, self.ctx, S, W, K, R, self.idx, self.cnt, ws["s"])
        tb.tb_sparse_decode_attn(i["q"], i["kc"], i["vc"], self.idx, self.cnt, self.out, ws["a"])

    def result(self):
        cnt = self.cnt.cpu().numpy()
        idx = self.idx.cpu().numpy()
        L = self.ctx.cpu().numpy()
        sc = self.scores.cpu().numpy().view(np.uint32)   # written below ctx_len only
        return dict(qhat=self.qhat.cpu().numpy().view(np.uint32),
                    kp=self.kp.cpu().numpy().view(np.uint16),
                    scores=np.concatenate([sc[b, :, :L[b]].ravel() for b in range(B)]), cnt=cnt,
                    idx=[idx[b, h, :cnt[b, h]] for b in range(B) for h in range(Hq)],
                    out=self.out.cpu().numpy().view(np.uint32))


def assert_same(a, b, what):
    for k in a:
        if k == "idx":
            assert all(np.array_equal(x, y) for x, y in zip(a[k], b[k])), (what, k)
        else:
            assert np.array_equal(a[k], b[k]), (what, k)


def test_graph_replay_matches_eager(tb):
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        ws = dict(p=tb.new_workspace(tb.tb_predict_workspace_bytes(B, E, Eh, Hq * DP)),
                  s=tb.new_workspace(tb.tb_select_workspace_bytes(B, Hq, LMAX)),
                  a=tb.new_workspace(tb.tb_attn_workspace_bytes(B, Hq, CAP, 0, D)))
        step_a = Step(tb, make_inputs(71), ws)
        step_b = Step(tb, make_inputs(72), ws)
        step_a()
        torch.cuda.synchronize()
        ref_a = step_a.result()
        step_b()
        torch.cuda.synchronize()
        ref_b = step_b.result()
        assert (ref_a["cnt"] == S + W + K).all()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step_a()
    torch.cuda.synchronize()
    for rep in range(3):
        say("graph replay", rep)
        with torch.cuda.stream(stream):
            step_a.scores.fill_(float("nan"))
            step_a.out.zero_()
            g.replay()
        torch.cuda.synchronize()
        assert_same(step_a.result(), ref_a, "replay %d" % rep)
        with torch.cuda.stream(stream):
            step_b()
        torch.cuda.synchronize()
        assert_same(step_b.result(), ref_b, "eager after replay %d" % rep)
