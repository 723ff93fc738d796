"""CPU oracle for the eviction order of cached KV blocks -- test
infrastructure only.

Nothing in the product path may import, call or link this module; the tests,
the package smoke check and the benchmark's CPU-baseline and sweep legs may.

What the pages give (AsymCache / Multi-Segment Attention paper): the eviction
policy weighs a block's hit rate against the position-aware cost of
recomputing it (abstract); that cost is dT_B of Eq. 5 (Figure 6 caption);
the frequency term is a piecewise exponential function with a turning point
(Figure 8 caption); lambda rescales the frequency term, which moves the
turning point, and follows the average block lifespan tau by Eq. 10,
lambda <- exp((tau - tau0) / beta - tau / alpha) (Figure 10 caption); only an
exponential decay keeps the order of blocks that are not accessed unchanged
over time (Appendix A.1), which is what lets an O(log n) structure replace an
O(n) rescoring scan (Figure 9's axes).  The formula that combines these is cut
off on the pages.

Reading taken (stated again in the design notes):

    score_b(t) = c_b * n_b * w(t - t_b),   w(x) = min(1, lambda * exp(-x / s))

with c_b = max(dT_B(l1_b, q1_b), 0) from the Eq. 5 oracle, n_b the number of
accesses (insertion + hits), t_b the last access, s a decay time scale; the
lowest score is evicted first, ties going to the smaller block id.  The
turning point is x* = s ln(lambda).

This module scores every block on every eviction (O(n)) -- plainly, with no
heap and no time-invariant keys.
"""
from __future__ import annotations

import math

from .latency_oracle import delta_b


def block_cost(k, l1, q1):
    """Recomputation cost of a block with l1 cached and q1 recomputed blocks
    before it (Eq. 5), floored at 0."""
    return max(float(delta_b(k, l1, q1)), 0.0)


def weight(x, s, lam):
    """Piecewise exponential weight of a block idle for time x: 1 up to the
    turning point s ln(lambda), lambda * exp(-x / s) after it."""
    return min(1.0, lam * math.exp(-x / s))


def score(c, n, t_last, now, s, lam):
    return c * n * weight(now - t_last, s, lam)


def lambda_from_lifespan(tau, tau0, alpha, beta):
    """Eq. 10."""
    return math.exp((tau - tau0) / beta - tau / alpha)


class EvictOracle:
    """Blocks as plain records; every eviction rescans them all."""

    def __init__(self, k, s, lam):
        self.k, self.s, self.lam = list(k), float(s), float(lam)
        self.blocks = {}   # id -> [cost, accesses, last access]

    def insert(self, block, l1, q1, now):
        assert block not in self.blocks
        self.blocks[block] = [block_cost(self.k, l1, q1), 1, float(now)]

    def touch(self, block, now):
        b = self.blocks[block]
        b[1] += 1
        b[2] = float(now)

    def set_position(self, block, l1, q1):
        self.blocks[block][0] = block_cost(self.k, l1, q1)

    def remove(self, block):
        del self.blocks[block]

    def set_lambda(self, lam):
        self.lam = float(lam)

    def score(self, block, now):
        c, n, t = self.blocks[block]
        return score(c, n, t, now, self.s, self.lam)

    def scores(self, now):
        return {b: self.score(b, now) for b in self.blocks}

    def argmin(self, now):
        """(block, score) that the next eviction takes: lowest score, then smallest id."""
        best = None
        for b in sorted(self.blocks):
            sc = self.score(b, now)
            if best is None or sc < best[1]:
                best = (b, sc)
        return best

    def pop(self, now):
        b, sc = self.argmin(now)
        del self.blocks[b]
        return b, sc
