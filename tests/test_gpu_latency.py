"""Calibration of the Eq. 5 latency model on the GPU (timing, so loose checks only)."""
import numpy as np
import pytest

from kv_cache_attention_msa_amd import calibrate as C

pytestmark = pytest.mark.gpu


def test_small_grid_calibrates():
    print("[latency] small grid, batch 2", flush=True)
    grid = {"l1": (0, 64), "q1": (0, 8), "l2": (0, 32), "q2": (1, 8)}
    samples = C.measure_grid(grid=grid, batch=2, reps=5, warmup=2, seed=3)
    assert samples.shape == (16, 5)
    assert (samples[:, 4] > 0).all()
    model = C.calibrate(samples)
    pred = np.array([model(*r[:4]) for r in samples])
    assert np.isfinite(model.k).all() and (pred > 0).all()
    assert model.rms < 0.5
