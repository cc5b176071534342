"""Synthetic-input checks (CPU only): exact-accumulation grid and calibration."""

import numpy as np
import pytest

import oracle
from helpers import grid_ok
from workloads import (bf16_representable, make_decode_windows, make_layer_0p5b, make_layer_2b,
                       make_random_small, make_stress_layer, make_tiny)
from workloads.gen import stress_layer_mean


def test_tiny_grid_and_rate():
    wl = make_tiny()
    assert (wl.T, wl.d, wl.F, wl.dtype, wl.tile_w, wl.cap) == (64, 256, 1024, "f32", 128, 16)
    grid_ok(wl)
    z = oracle.gate(wl.x, wl.wg_t)
    p = (z > 0).mean()
    n = z.size
    assert abs(p - 0.03) < 3.3 * np.sqrt(0.03 * 0.97 / n) + 0.004  # binomial 99.9% + model slack
    assert np.array_equal(z, oracle.matmul_rows(wl.x, np.arange(wl.T), wl.wg_t))


def test_0p5b_grid_and_rate():
    wl = make_layer_0p5b()
    assert (wl.T, wl.d, wl.F, wl.dtype, wl.tile_w, wl.cap) == (4096, 1024, 4096, "bf16", 128, 8)
    grid_ok(wl)
    z = oracle.gate(wl.x[:512], wl.wg_t)
    p = (z > 0).mean()
    assert abs(p - 0.01) < 0.0015
    rows = np.array([0, 100, 511])
    np.testing.assert_array_equal(z[rows], oracle.matmul_rows(wl.x, rows, wl.wg_t))


def test_2b_grid_dead_and_mean():
    wl = make_layer_2b()
    assert (wl.T, wl.d, wl.F, wl.dtype, wl.tile_w, wl.cap) == (8192, 2048, 8192, "bf16", 256, 16)
    grid_ok(wl)
    dead = wl.meta["dead"]
    assert len(dead) == 1638 and np.isneginf(wl.wg_t[dead, -1]).all()
    assert np.isfinite(wl.wg_t[:, -1]).sum() == 8192 - 1638
    z = oracle.gate(wl.x[:2048], wl.wg_t)
    n = (z > 0).sum(1)
    assert not np.isnan(z).any()
    assert not (z[:, dead] > 0).any()
    assert 24.0 < n.mean() < 34.0          # mean ~29 active neurons per token
    assert np.median(n) < 5                 # heavy tail: most tokens nearly inactive
    assert np.percentile(n, 99) > 200


def test_decode_windows():
    for T in (1, 8, 64):
        ws = make_decode_windows(T, max_windows=4)
        assert len(ws) == 4 and all(w.T == T for w in ws)
        base = make_layer_2b()
        np.testing.assert_array_equal(ws[1].x, base.x[T:2 * T])


@pytest.mark.parametrize("layer", [0, 23])
def test_stress_layer(layer):
    wl = make_stress_layer(layer, T=2048)
    grid_ok(wl)
    z = oracle.gate(wl.x, wl.wg_t)
    n = (z > 0).sum(1)
    stress = wl.meta["stress_rows"]
    normal = np.setdiff1d(np.arange(wl.T), stress)
    m = stress_layer_mean(layer)
    assert abs(n[normal].mean() - m) < 0.15 * m + 2
    frac = n[stress] / wl.F
    assert np.all(frac > 0.03) and np.all(frac < 0.33)


def test_stress_layer_means_profile():
    ms = [stress_layer_mean(l) for l in range(24)]
    assert ms[0] == 10.0 and ms[-1] == 60.0 and all(a <= b for a, b in zip(ms, ms[1:]))


def test_random_small_grid():
    for s in range(3):
        grid_ok(make_random_small(100, 64, 256, 64, 4, active_frac=0.1, seed=s, jitter=0.5))


def test_seed_streams_independent_of_shape():
    a = make_stress_layer(3, T=64)
    b = make_stress_layer(3, T=128)
    np.testing.assert_array_equal(a.wg_t[:, :-1], b.wg_t[:, :-1])
    np.testing.assert_array_equal(a.wd, b.wd)


def test_continuous_mode():
    """Continuous mode: same shapes and bias structure, values representable
    in the storage type but off the grid; grid mode is unchanged by it."""
    from workloads import make_random_small
    g = make_random_small(64, 128, 512, 128, 8, "bf16", active_frac=0.05, seed=5, jitter=0.5)
    c = make_random_small(64, 128, 512, 128, 8, "bf16", active_frac=0.05, seed=5, jitter=0.5, mode="continuous")
    assert c.x.shape == g.x.shape and c.wg_t.shape == g.wg_t.shape
    assert bf16_representable(c.x) and bf16_representable(c.wg_t) and bf16_representable(c.wd)
    off = c.x[:, :-1] * 16 - np.rint(c.x[:, :-1] * 16)
    assert np.abs(off).max() > 0.1                       # not on the 2^-4 grid
    np.testing.assert_array_equal(c.x[:, -1], g.x[:, -1])  # same jitter column
    np.testing.assert_array_equal(c.wg_t[:, -1], g.wg_t[:, -1])  # same biases
    assert abs(c.wg_t[:, :-1].std() * np.sqrt(128) - 1) < 0.05
    f = make_random_small(32, 64, 256, 64, 4, "f32", seed=6, mode="continuous")
    assert not bf16_representable(f.x)                    # fp32 layers keep full fp32 values
    g2 = make_random_small(64, 128, 512, 128, 8, "bf16", active_frac=0.05, seed=5, jitter=0.5)
    np.testing.assert_array_equal(g.x, g2.x)
