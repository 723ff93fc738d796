"""The native eviction index (include/msa_evict.h) against the O(n) oracle
(oracle/evict_oracle.py) on seeded random traces of inserts, hits,
repositions, removals, lambda changes (Eq. 10) and evictions, host only.

Where several blocks score within rounding of each other either may be
evicted, so each native eviction is checked to be a minimum of the oracle's
scores (within 1e-9 relative) and then applied to both; ties that are exact
must go to the smaller id.  Also: the hand-worked orders of
tests/golden/evict_hand.json, the O(n) scan agrees with the heap, and
argument errors.
"""
import json
import math
import os

import numpy as np
import pytest

import kv_cache_attention_msa_amd as msa
from oracle import EvictOracle, lambda_from_lifespan

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = json.load(open(os.path.join(HERE, "golden", "evict_hand.json")))
K = [12.0, 0.4, 0.2, 0.05, 0.06]


def _check_pick(o, now, block, score):
    ref = o.scores(now)
    lo = min(ref.values())
    assert ref[block] <= lo + 1e-9 * abs(lo) + 1e-300, (block, ref[block], lo)
    assert score == pytest.approx(ref[block], rel=1e-9, abs=1e-300)
    exact = [b for b, v in ref.items() if v == lo]
    if len(exact) > 1 and ref[block] == lo:
        assert block == min(exact)


@pytest.mark.parametrize("seed,s,lam", [(0, 5.0, 3.0), (1, 2.0, 1.0), (2, 10.0, 0.5), (3, 1.0, 50.0)])
def test_random_trace_matches_oracle(seed, s, lam):
    rng = np.random.default_rng(seed)
    model = msa.LatencyModel.from_coefficients(K)
    idx = msa.EvictIndex(model, s, lam)
    o = EvictOracle(K, s, lam)
    now, next_id, pops = 0.0, 0, 0
    try:
        for step in range(3000):
            now += float(rng.exponential(0.3))
            r = rng.random()
            live = list(o.blocks)
            if r < 0.35 or len(live) < 5:
                l1, q1 = float(rng.integers(0, 400)), float(rng.integers(0, 50))
                idx.insert(next_id, l1, q1, now)
                o.insert(next_id, l1, q1, now)
                next_id += 1
            elif r < 0.65:
                b = int(rng.choice(live))
                idx.touch(b, now)
                o.touch(b, now)
            elif r < 0.72:
                b = int(rng.choice(live))
                l1, q1 = float(rng.integers(0, 400)), float(rng.integers(0, 50))
                idx.set_position(b, l1, q1)
                o.set_position(b, l1, q1)
            elif r < 0.75:
                b = int(rng.choice(live))
                idx.remove(b)
                o.remove(b)
            elif r < 0.78:
                tau = float(rng.uniform(0, 20))
                lam2 = lambda_from_lifespan(tau, 5.0, 8.0, 4.0)
                assert msa.lambda_from_lifespan(tau, 5.0, 8.0, 4.0) == pytest.approx(lam2, rel=1e-15)
                idx.set_lambda(lam2, now)
                o.set_lambda(lam2)
            else:
                sb, ss = idx.scan_min(now)
                b, sc = idx.pop(now)
                _check_pick(o, now, sb, ss)
                _check_pick(o, now, b, sc)
                o.remove(b)
                pops += 1
            assert len(idx) == len(o.blocks)
        # drain
        while len(o.blocks):
            now += 0.5
            sb, ss = idx.scan_min(now)
            b, sc = idx.pop(now)
            assert (sb, ss) == (b, pytest.approx(sc, rel=1e-12))
            _check_pick(o, now, b, sc)
            o.remove(b)
        assert pops > 300
    finally:
        idx.close()


@pytest.mark.parametrize("ex", GOLD["examples"], ids=lambda e: e["name"])
def test_hand_worked_orders(ex):
    model = msa.LatencyModel.from_coefficients(GOLD["k"])
    s2 = 1.0 / math.log(2.0)
    for at in ex["at"]:
        idx = msa.EvictIndex(model, s2, ex["lambda"])
        try:
            # replay each block's history: inserted at its last access time and
            # touched n - 1 times there
            for bid, l1, q1, n, t in sorted(ex["blocks"], key=lambda b: b[4]):
                idx.insert(bid, l1, q1, t)
                for _ in range(n - 1):
                    idx.touch(bid, t)
            assert [idx.pop(at["now"])[0] for _ in ex["blocks"]] == at["eviction_order"]
        finally:
            idx.close()


def test_lambda_growth_moves_blocks_back_before_their_turning_points():
    # lambda 0.5: every block decays from its last access.  Raising lambda to
    # 100 puts the turning point at ln 100 ~ 4.6: blocks accessed less than
    # that ago are back at full weight, and the one with the lowest cost x
    # accesses among them must be evicted first.
    k = [0.0, 1.0, 1.0, 0.0, 1.0]          # cost = l1 + 2 q1 + 1
    idx = msa.EvictIndex(msa.LatencyModel.from_coefficients(k), 1.0, 0.5)
    o = EvictOracle(k, 1.0, 0.5)
    try:
        for b, l1, t in ((2, 4, 5.0), (1, 0, 10.0), (3, 1, 10.1)):     # costs 5, 1, 2
            idx.insert(b, l1, 0, t)
            o.insert(b, l1, 0, t)
        idx.set_lambda(100.0, 10.1)
        o.set_lambda(100.0)
        order = []
        while len(idx):
            b, sc = idx.pop(10.1)
            _check_pick(o, 10.1, b, sc)
            o.remove(b)
            order.append(b)
        assert order == [1, 3, 2]    # scores 1, 2 and 5 * 100 e^-5.1 ~ 3.05
    finally:
        idx.close()


def test_eq10_native_matches_printed_form():
    for e in GOLD["eq10"]:
        want = math.e ** 2 if e["lambda"] == "e^2" else float(e["lambda"])
        assert msa.lambda_from_lifespan(e["tau"], e["tau0"], e["alpha"], e["beta"]) == pytest.approx(want, rel=1e-15)


def test_argument_errors():
    model = msa.LatencyModel.from_coefficients(K)
    with pytest.raises(msa.MsaError):
        msa.EvictIndex(model, 0.0, 1.0)
    with pytest.raises(msa.MsaError):
        msa.EvictIndex(model, 1.0, -1.0)
    idx = msa.EvictIndex(model, 1.0, 2.0)
    try:
        with pytest.raises(msa.MsaError):
            idx.pop(0.0)                       # empty
        idx.insert(1, 3, 0, 5.0)
        with pytest.raises(msa.MsaError):
            idx.insert(1, 3, 0, 5.0)           # already present
        with pytest.raises(msa.MsaError):
            idx.touch(1, 4.0)                  # time went back
        with pytest.raises(msa.MsaError):
            idx.touch(2, 6.0)                  # absent
        with pytest.raises(msa.MsaError):
            idx.insert(3, -1, 0, 6.0)          # negative position
        with pytest.raises(msa.MsaError):
            msa.lambda_from_lifespan(1.0, 0.0, 0.0, 1.0)
        assert len(idx) == 1
    finally:
        idx.close()
