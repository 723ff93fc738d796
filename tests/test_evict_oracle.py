"""Pins of the eviction-order oracle (oracle/evict_oracle.py) against what the
pages and the mathematics fix:
  * hand-worked orders and scores (tests/golden/evict_hand.json), before and
    past a turning point;
  * the order-preserving property of Appendix A.1: past the turning point the
    ranking of blocks that are not accessed never changes with time, while a
    non-exponential decay (a power law) does reorder them;
  * textbook special cases: equal costs and single accesses past the turning
    point give LRU order; a turning point beyond every idle time gives the
    order of cost x accesses;
  * Eq. 10 as printed, and the turning point s ln(lambda) where the weight
    leaves 1;
  * the cost is Eq. 5's dT_B (its own oracle is pinned in
    tests/test_latency_oracle.py).
A planted mistake (decay sign, frequency ignored, wrong tie-break, turning
point at s / lambda) fails at least one of these.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import EvictOracle, block_cost, delta_b, lambda_from_lifespan, weight

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = json.load(open(os.path.join(HERE, "golden", "evict_hand.json")))
S2 = 1.0 / math.log(2.0)   # time scale for which the weight is min(1, lambda * 2^-x)


def _oracle(ex):
    o = EvictOracle(GOLD["k"], S2, ex["lambda"])
    for bid, l1, q1, n, t in ex["blocks"]:
        o.insert(bid, l1, q1, 0.0)
        o.blocks[bid][1] = n          # accesses and last access as written in the example
        o.blocks[bid][2] = t
    return o


@pytest.mark.parametrize("ex", GOLD["examples"], ids=lambda e: e["name"])
def test_hand_worked_orders(ex):
    o = _oracle(ex)
    for (bid, *_), c in zip(ex["blocks"], ex["costs"]):
        assert o.blocks[bid][0] == c
    for at in ex["at"]:
        for bid, frac in at["scores"].items():
            assert o.score(int(bid), at["now"]) == pytest.approx(float(Fraction(frac)), rel=1e-12)
        o2 = _oracle(ex)
        order = [o2.pop(at["now"])[0] for _ in range(len(ex["blocks"]))]
        assert order == at["eviction_order"]


def test_eq10_as_printed():
    for e in GOLD["eq10"]:
        want = math.e ** 2 if e["lambda"] == "e^2" else float(Fraction(e["lambda"]))
        assert lambda_from_lifespan(e["tau"], e["tau0"], e["alpha"], e["beta"]) == pytest.approx(want, rel=1e-15)


def test_turning_point_is_s_ln_lambda():
    for s, lam in ((2.0, 4.0), (0.5, 9.0), (3.0, 1.0)):
        xt = s * math.log(lam)
        assert weight(xt, s, lam) == pytest.approx(1.0, rel=1e-15)
        assert weight(max(xt - 1e-9, 0.0), s, lam) == 1.0
        assert weight(xt + s, s, lam) == pytest.approx(math.exp(-1.0), rel=1e-12)
    assert weight(0.0, 2.0, 0.5) == 0.5              # lambda < 1: already decaying at x = 0


def _random_oracle(rng, n, lam, s, t_now):
    k = [10.0, 0.4, 0.2, 0.05, 0.06]
    o = EvictOracle(k, s, lam)
    for b in range(n):
        o.insert(b, float(rng.integers(0, 300)), float(rng.integers(0, 40)), 0.0)
        o.blocks[b][1] = int(rng.integers(1, 6))
        o.blocks[b][2] = float(rng.uniform(0.0, t_now))
    return o


def test_order_preserved_past_the_turning_point():
    rng = np.random.default_rng(0)
    s, lam = 5.0, 2.0
    o = _random_oracle(rng, 200, lam, s, 50.0)
    t1 = 50.0 + s * math.log(lam) + 1e-6        # every block past its turning point
    r1 = sorted(o.blocks, key=lambda b: (o.score(b, t1), b))
    for t2 in (t1 + 3.7, t1 + 40.0, t1 + 400.0):
        r2 = sorted(o.blocks, key=lambda b: (o.score(b, t2), b))
        assert r2 == r1


def test_power_law_decay_does_reorder():
    # the same blocks with a non-exponential decay 1 / (1 + x) change order with
    # time: the property above is not vacuous (Appendix A.1's lemma)
    a = (1.0, 0.0)     # cost 1, last access at 0
    b = (3.0, -5.0)    # cost 3, last access at -5
    pl = lambda c, tb, t: c / (1.0 + t - tb)
    assert pl(*a, 0.0) > pl(*b, 0.0) and pl(*a, 100.0) < pl(*b, 100.0)
    ex = lambda c, tb, t: c * math.exp(-(t - tb) / 4.0)
    assert (ex(*a, 0.0) < ex(*b, 0.0)) == (ex(*a, 100.0) < ex(*b, 100.0))


def test_lru_special_case():
    # equal costs, one access each, every block past its turning point: the
    # least recently used block goes first
    rng = np.random.default_rng(1)
    o = EvictOracle([0.0, 1.0, 1.0, 0.0, 1.0], 2.0, 1.0)
    times = rng.permutation(50).astype(float)
    for b, t in enumerate(times):
        o.insert(b, 3, 1, 0.0)
        o.blocks[b][2] = t
    order = [o.pop(60.0)[0] for _ in range(50)]
    assert order == list(np.argsort(times, kind="stable"))


def test_cost_times_frequency_before_the_turning_point():
    rng = np.random.default_rng(2)
    o = _random_oracle(rng, 100, 1e12, 1.0, 10.0)    # turning point ~27.6: nothing decays by t = 10
    expect = sorted(o.blocks, key=lambda b: (o.blocks[b][0] * o.blocks[b][1], b))
    assert [o.pop(10.0)[0] for _ in range(100)] == expect


def test_ties_go_to_the_smaller_id():
    o = EvictOracle([0.0, 1.0, 1.0, 0.0, 1.0], 1.0, 1e12)   # no decay yet: scores are exact integers
    for b, (l1, n) in {8: (2, 1), 3: (0, 3), 5: (2, 1), 1: (4, 1)}.items():
        o.insert(b, l1, 0, 0.0)
        o.blocks[b][1] = n
    # costs 3, 1, 3, 5 -> scores 3, 3, 3, 5
    assert [o.pop(1.0)[0] for _ in range(4)] == [3, 5, 8, 1]


def test_cost_is_eq5_floored_at_zero():
    k = [5.0, 0.3, 0.2, 0.01, 0.02]
    for l1, q1 in ((0, 0), (10, 3), (200, 17)):
        assert block_cost(k, l1, q1) == pytest.approx(0.02 * (l1 + 2 * q1) + (0.3 - 0.2 + 0.02), rel=1e-12)
        assert block_cost(k, l1, q1) == pytest.approx(float(delta_b(k, l1, q1)), rel=1e-15)
    assert block_cost([0.0, 0.1, 0.5, 0.0, 0.01], 0, 0) == 0.0          # negative dT_B counts as 0


def test_touch_counts_and_refreshes():
    o = EvictOracle([0.0, 1.0, 1.0, 0.0, 1.0], S2, 1.0)
    o.insert(1, 0, 0, 0.0)     # cost 1
    o.insert(2, 0, 0, 0.0)
    o.touch(2, 1.0)            # two accesses, last at 1
    assert o.score(1, 2.0) == pytest.approx(0.25) and o.score(2, 2.0) == pytest.approx(1.0)
    assert o.pop(2.0) == (1, pytest.approx(0.25))
