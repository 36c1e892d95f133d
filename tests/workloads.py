"""Test-side helpers: oracle-derived planting directions and the one-layer
decode-step protocol shared by the CPU and GPU tests."""
import numpy as np

from synthetic import bits_to_f32_bf16, CONFIGS
from synthetic.workload import make_layer


def oracle_direction(orc, cfg):
    """v_h = Wk[h // g]^T q_hat_h with q_hat from the oracle's predictor: the
    key direction that raises head h's score fastest."""
    def fn(inp):
        _, qhat = orc.predict_queries(inp["x"], inp["w1"], inp["w2"])
        B = qhat.shape[0]
        qh = qhat.reshape(B, cfg.Hq, cfg.dp).astype(np.float64)
        wk = bits_to_f32_bf16(inp["wk"]).astype(np.float64)          # [Hkv, dp, D]
        wk_h = np.repeat(wk, cfg.g, axis=0)                          # [Hq, dp, D]
        return np.einsum("bhc,hcd->bhd", qh, wk_h)
    return fn


def oracle_step(orc, cfg, inp, K=None, r=None):
    """One decode step of one layer, oracle side: the cache of every token but
    the newest is already projected; the step projects the newest token,
    predicts, scores, selects and attends."""
    B = inp["x"].shape[0]
    L = inp["ctx_len"]
    Lmax = inp["kc"].shape[2]
    kp = np.zeros((B, cfg.Hkv, Lmax, cfg.dp), np.uint16)
    orc.project_keys(inp["kc"], inp["wk"], kp, np.zeros(B, np.int32), int(L.max()) - 1)
    res = orc.decode_step(inp["x"], inp["w1"], inp["w2"], inp["kc"], inp["vc"], inp["wk"],
                          kp, inp["q"], L, L, (L - 1).astype(np.int32), 1,
                          cfg.S, cfg.W, cfg.K if K is None else K, cfg.r if r is None else r,
                          cap=min(Lmax, cfg.S + cfg.W + (cfg.K if K is None else K)))
    res["kp"] = kp
    return res


def recovered(res, spans):
    ok = []
    for (b, h, s0, n) in spans:
        F = set(res["idx"][b, h, :res["count"][b, h]].tolist())
        ok.append(all(t in F for t in range(s0, s0 + n)))
    return ok
