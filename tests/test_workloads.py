"""Synthetic-input checks (CPU only): exact-accumulation grid and calibration."""

import numpy as np
import pytest

import oracle
from workloads import (bf16_representable, make_decode_windows, make_layer_0p5b, make_layer_2b,
                       make_random_small, make_stress_layer, make_tiny)
from workloads.gen import stress_layer_mean


def _grid_ok(wl):
    """Every partial sum of x_t . w_j stays below 2^7 and every product is a multiple of 2^-17.

    Bound: |sum_k<d-1 x_k w_k| <= ||x_t[:-1]|| ||w_j[:-1]|| (Cauchy-Schwarz), plus |x_t,last * w_j,last|.
    """
    x = wl.x.astype(np.float64)
    for w in (wl.wg_t, wl.wu_t):
        w = w.astype(np.float64)
        fin = np.isfinite(w[:, -1])
        nx = np.sqrt((x[:, :-1] ** 2).sum(1)).max()
        nw = np.sqrt((w[:, :-1] ** 2).sum(1)).max()
        bias = np.abs(x[:, -1]).max() * np.abs(w[fin, -1]).max()
        assert nx * nw + bias < 128.0, (wl.name, nx, nw, bias)
    # grids: x body on 2^-4, weights on 2^-10, last column of x >= 2^-3 and bf16,
    # finite biases bf16 (or 2^-10 grid for fp32) with magnitude >= 1
    assert np.all(np.rint(wl.x[:, :-1] * 16) == wl.x[:, :-1] * 16)
    for w in (wl.wg_t[:, :-1], wl.wu_t, wl.wd):
        assert np.all(np.rint(w * 1024) == w * 1024)
    assert np.all(wl.x[:, -1] >= 0.125)
    fb = wl.wg_t[np.isfinite(wl.wg_t[:, -1]), -1]
    assert np.all(np.abs(fb) >= 1.0)
    if wl.dtype == "bf16":
        assert bf16_representable(wl.x) and bf16_representable(wl.wu_t) and bf16_representable(wl.wd)
        assert bf16_representable(wl.wg_t[np.isfinite(wl.wg_t)])
    else:
        assert np.all(np.rint(fb * 1024) == fb * 1024)


def test_tiny_grid_and_rate():
    wl = make_tiny()
    assert (wl.T, wl.d, wl.F, wl.dtype, wl.tile_w, wl.cap) == (64, 256, 1024, "f32", 128, 16)
    _grid_ok(wl)
    z = oracle.gate(wl.x, wl.wg_t)
    p = (z > 0).mean()
    n = z.size
    assert abs(p - 0.03) < 3.3 * np.sqrt(0.03 * 0.97 / n) + 0.004  # binomial 99.9% + model slack
    assert np.array_equal(z, oracle.matmul_rows(wl.x, np.arange(wl.T), wl.wg_t))


def test_0p5b_grid_and_rate():
    wl = make_layer_0p5b()
    assert (wl.T, wl.d, wl.F, wl.dtype, wl.tile_w, wl.cap) == (4096, 1024, 4096, "bf16", 128, 8)
    _grid_ok(wl)
    z = oracle.gate(wl.x[:512], wl.wg_t)
    p = (z > 0).mean()
    assert abs(p - 0.01) < 0.0015
    rows = np.array([0, 100, 511])
    np.testing.assert_array_equal(z[rows], oracle.matmul_rows(wl.x, rows, wl.wg_t))


def test_2b_grid_dead_and_mean():
    wl = make_layer_2b()
    assert (wl.T, wl.d, wl.F, wl.dtype, wl.tile_w, wl.cap) == (8192, 2048, 8192, "bf16", 256, 16)
    _grid_ok(wl)
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
    _grid_ok(wl)
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
        _grid_ok(make_random_small(100, 64, 256, 64, 4, active_frac=0.1, seed=s, jitter=0.5))


def test_seed_streams_independent_of_shape():
    a = make_stress_layer(3, T=64)
    b = make_stress_layer(3, T=128)
    np.testing.assert_array_equal(a.wg_t[:, :-1], b.wg_t[:, :-1])
    np.testing.assert_array_equal(a.wd, b.wd)
