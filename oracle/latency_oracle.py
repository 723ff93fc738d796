"""CPU oracle for the Eq. 5 latency model -- test infrastructure only.

Nothing in the product path may import, call or link this module; the tests,
the package smoke check and the benchmark's CPU-baseline leg may.

What the pages give (AsymCache / Multi-Segment Attention paper, Figure 6
caption, Eq. 5): a request's context is four regions in position order -- l1
cached blocks, q1 blocks recomputed this step, l2 cached blocks, q2 new blocks
-- and the cost of recomputing one more block instead of keeping it cached is

    dT_B = T(l1, q1 + 1, l2 - 1, q2) - T(l1, q1, l2, q2) = k5 (l1 + 2 q1) + (k2 - k3 + k5),

with coefficients k that depend on the hardware.  T itself is not printed.

Reading taken: the plainest T whose difference is exactly Eq. 5,

    T = k1 + k2 (q1 + q2) + k3 (l1 + l2) + k4 q2 (l1 + q1 + l2 + q2) + k5 q1 (l1 + q1),

i.e. a fixed cost, a cost per computed block, a cost per cached block read, the
new blocks attending to the whole context, and the recomputed blocks attending
to the prefix and to themselves (they sit before l2).  Units are blocks (the
eviction unit), so "+1" moves one block.  The coefficients are fitted to
measured times by least squares; with ``relative`` the residuals are taken
relative to the measured time (rows scaled by 1/T), which suits timings whose
noise grows with their size.

Adaptive chunk size (the pages' adaptive chunking scheduler, named in the
abstract for hardware utilisation; the rule itself is not given).  Reading
taken: for the next step of a request with l1, q1, l2 blocks of context and
``remaining`` new blocks, take the largest chunk c in [1, remaining] whose
modelled step time T(l1, q1, l2, c) fits a per-step budget (1 if none does).

Pins (``tests/test_latency_oracle.py``): the difference of T equals Eq. 5 as
printed, exact recovery of known coefficients, exact interpolation through
five points, detection of a grid that cannot determine all five, and the
chunk rule against the closed-form root of its quadratic.
"""
from __future__ import annotations

import numpy as np


def model_terms(l1, q1, l2, q2):
    """The five terms of T for arrays of (l1, q1, l2, q2); shape [n, 5]."""
    l1, q1, l2, q2 = (np.asarray(x, dtype=np.float64) for x in (l1, q1, l2, q2))
    return np.stack([np.ones_like(l1), q1 + q2, l1 + l2, q2 * (l1 + q1 + l2 + q2), q1 * (l1 + q1)], axis=-1)


def latency(k, l1, q1, l2, q2):
    """T(l1, q1, l2, q2) for coefficients k[0..4] = k1..k5."""
    return model_terms(l1, q1, l2, q2) @ np.asarray(k, dtype=np.float64)


def delta_b(k, l1, q1):
    """Eq. 5: cost of recomputing one more block instead of keeping it cached."""
    k = np.asarray(k, dtype=np.float64)
    return k[4] * (np.asarray(l1, dtype=np.float64) + 2 * np.asarray(q1, dtype=np.float64)) + (k[1] - k[2] + k[4])


def fit_latency(samples, relative=True):
    """Least-squares k1..k5 from rows (l1, q1, l2, q2, T).

    Returns (k, rms) where rms is the root-mean-square residual (relative to T
    when ``relative``).  Raises ValueError when the samples cannot determine
    all five coefficients."""
    s = np.asarray(samples, dtype=np.float64).reshape(-1, 5)
    A = model_terms(s[:, 0], s[:, 1], s[:, 2], s[:, 3])
    t = s[:, 4]
    w = 1.0 / t if relative else np.ones_like(t)
    Aw, tw = A * w[:, None], t * w
    if len(s) < 5 or np.linalg.matrix_rank(Aw / np.linalg.norm(Aw, axis=0).clip(min=1e-300)) < 5:
        raise ValueError("the samples do not determine all five coefficients")
    k, *_ = np.linalg.lstsq(Aw, tw, rcond=None)
    r = Aw @ k - tw
    return k, float(np.sqrt(np.mean(r * r)))


def chunk_blocks(k, l1, q1, l2, remaining, budget):
    """Largest c in [1, remaining] with T(l1, q1, l2, c) <= budget, else 1."""
    fits = [c for c in range(1, int(remaining) + 1) if latency(k, l1, q1, l2, c) <= budget]
    return max(fits) if fits else 1
