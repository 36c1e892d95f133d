"""Planted-span retrieval at 300 tokens (TokenButler summary, "Contributions"
and "Results": a synthetic co-referential retrieval task at 300 tokens where
the method is near-oracle). Stand-in: three 4-token spans whose keys are moved
along their head's predicted-query direction by 3 score standard deviations;
a span is recovered when every token of it is in its head's attended set."""
import numpy as np

from synthetic import CONFIGS
from synthetic.workload import make_layer
from workloads import oracle_direction, oracle_step, recovered

C1 = CONFIGS[1]


def test_fixed_seed_recovers_all_spans(orc):
    inp = make_layer(C1, seed=0, direction_fn=oracle_direction(orc, C1))
    assert len(inp["spans"]) == 3
    res = oracle_step(orc, C1, inp)
    assert all(recovered(res, inp["spans"])), inp["spans"]
    # the budget is respected while doing so
    assert (res["count"] <= C1.S + C1.W + C1.K).all()


def test_recovery_rate_and_neighbour_fetching(orc):
    n_seeds = 60
    full = {0: 0, 1: 0}
    for seed in range(n_seeds):
        inp = make_layer(C1, seed=seed, direction_fn=oracle_direction(orc, C1))
        for r in (0, 1):
            res = oracle_step(orc, C1, inp, r=r)
            full[r] += all(recovered(res, inp["spans"]))
    rate = {r: full[r] / n_seeds for r in full}
    print("planted-span full recovery rate over %d seeds: %s" % (n_seeds, rate))
    # neighbour fetching exists to cover multi-token entities
    assert rate[1] > rate[0]
    assert rate[1] >= 0.6
