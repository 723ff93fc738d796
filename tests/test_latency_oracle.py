"""Pins for the Eq. 5 latency-model oracle (``oracle.latency_oracle``).

The pages print only the difference dT_B (Eq. 5, Figure 6 caption), so the
reconstructed T is pinned by that printed difference; the fit is pinned by
exact recovery and exact interpolation, which do not depend on how least
squares is computed.
"""
import itertools

import numpy as np
import pytest

from oracle.latency_oracle import chunk_blocks, delta_b, fit_latency, latency, model_terms


def eq5_as_printed(k, l1, q1):
    k1, k2, k3, k4, k5 = k
    return k5 * (l1 + 2 * q1) + (k2 - k3 + k5)


@pytest.mark.parametrize("seed", range(5))
def test_difference_of_T_is_eq5(seed):
    rng = np.random.default_rng(seed)
    k = rng.uniform(-2, 3, size=5)
    l1, q1, q2 = rng.integers(0, 400, size=3)
    l2 = int(rng.integers(1, 400))
    lhs = latency(k, l1, q1 + 1, l2 - 1, q2) - latency(k, l1, q1, l2, q2)
    assert lhs == pytest.approx(eq5_as_printed(k, l1, q1), rel=1e-12, abs=1e-9)
    assert delta_b(k, l1, q1) == pytest.approx(eq5_as_printed(k, l1, q1), rel=1e-12, abs=1e-12)


def test_terms_for_a_hand_example():
    # l1=3, q1=2, l2=5, q2=4: context 14 blocks; q2 attends 14, q1 attends 3+2
    assert model_terms(3, 2, 5, 4).tolist() == [1, 6, 8, 4 * 14, 2 * 5]


def _grid():
    pts = list(itertools.product([0, 16, 64, 256], [0, 8, 32], [0, 16, 128], [4, 32]))
    return np.array(pts, dtype=np.float64)


@pytest.mark.parametrize("relative", [True, False])
def test_exact_recovery(relative):
    k = np.array([12.0, 0.8, 0.05, 0.003, 0.004])
    g = _grid()
    T = latency(k, *g.T)
    kf, rms = fit_latency(np.column_stack([g, T]), relative=relative)
    np.testing.assert_allclose(kf, k, rtol=1e-9)
    assert rms < 1e-9


def test_interpolates_five_points():
    pts = np.array([[0, 0, 0, 1], [10, 0, 0, 1], [0, 0, 0, 9], [0, 5, 0, 1], [4, 3, 7, 2]], dtype=np.float64)
    T = np.array([3.0, 5.0, 4.0, 11.0, 40.0])
    k, rms = fit_latency(np.column_stack([pts, T]), relative=False)
    np.testing.assert_allclose(model_terms(*pts.T) @ k, T, rtol=1e-12)
    assert rms < 1e-12


def test_noisy_fit_close():
    rng = np.random.default_rng(3)
    k = np.array([12.0, 0.8, 0.05, 0.003, 0.004])
    g = _grid()
    T = latency(k, *g.T) * (1 + 0.01 * rng.standard_normal(len(g)))
    kf, rms = fit_latency(np.column_stack([g, T]))
    assert 0.003 < rms < 0.02
    assert abs(kf[4] - k[4]) / k[4] < 0.1 and abs(kf[3] - k[3]) / k[3] < 0.1


def test_undetermined_grid_rejected():
    g = _grid()
    g = g[g[:, 1] == 0]                 # no recomputed blocks: k5 cannot be seen
    T = latency([1, 1, 1, 1, 1], *g.T)
    with pytest.raises(ValueError):
        fit_latency(np.column_stack([g, T]))
    with pytest.raises(ValueError):
        fit_latency(np.zeros((4, 5)) + 1)


def test_chunk_rule_is_the_root_of_its_quadratic():
    # T(l1, q1, l2, c) = k1 + k2 (q1 + c) + k3 (l1 + l2) + k4 c (l1 + q1 + l2 + c) + k5 q1 (l1 + q1)
    # is k4 c^2 + b c + a; the rule must return floor of the larger root of T = budget.
    k = [30.0, 0.2, 0.19, 0.07, 0.07]
    l1, q1, l2, budget = 100, 10, 50, 900.0
    a = k[0] + k[1] * q1 + k[2] * (l1 + l2) + k[4] * q1 * (l1 + q1) - budget
    b = k[1] + k[3] * (l1 + q1 + l2)
    root = (-b + np.sqrt(b * b - 4 * k[3] * a)) / (2 * k[3])
    assert chunk_blocks(k, l1, q1, l2, 10_000, budget) == int(np.floor(root))
    assert chunk_blocks(k, l1, q1, l2, 5, budget) == 5                 # capped by what is left
    assert chunk_blocks(k, l1, q1, l2, 10_000, 1.0) == 1               # nothing fits: still progress
    sizes = [chunk_blocks(k, l1, q1, l2, 10_000, t) for t in (200, 400, 800, 1600)]
    assert sizes == sorted(sizes)                                      # a larger budget never shrinks it
