"""Pins for the CPU oracle (CPU only).

Each test checks the oracle against something other than itself: a
hand-worked example, an independent pure-Python brute force, exhaustive
enumeration, closed forms, invariants, or a library routine (numpy fp64
matmul; torch's bf16 conversion).
"""

import itertools
import json
import os

import numpy as np
import pytest

import oracle
from oracle import brute
from workloads import make_random_small

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32(a):
    return np.asarray(a, np.float32)


# ------------------------------------------------------------ hand-worked example
def test_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    e = g["expect"]
    x, wg, wu, wd = (_f32(g[k]) for k in ("x", "wg_t", "wu_t", "wd"))
    w, cap = g["tile_w"], g["cap"]
    z = oracle.matmul_rows(x, np.arange(2), wg)
    np.testing.assert_array_equal(z, np.asarray(e["z"], np.float64))
    tw = oracle.pack_twell(z, w, cap, "f32")
    np.testing.assert_array_equal(tw.cnt, np.asarray(e["cnt"]))
    for t in range(2):
        for b in range(2):
            m = min(tw.cnt[t, b], cap)
            assert list(tw.idx[t, b, :m]) == e["idx_kept"][t][b]
            assert list(tw.val[t, b, :m]) == e["val_kept"][t][b]
    row_ovf, rows, n = oracle.partition_overflow(tw.cnt, cap)
    assert list(row_ovf) == e["row_ovf"] and list(rows) == e["ovf_rows"] and n == 1
    np.testing.assert_array_equal(oracle.dense_backup(z, rows, "f32"), np.asarray(e["dense_backup"], np.float64))
    np.testing.assert_array_equal(oracle.ffn_active(z, x, wu, wd), np.asarray(e["y_hybrid"], np.float64))
    np.testing.assert_array_equal(oracle.ffn_twell(tw, x, wu, wd, skip_overflow=True),
                                  np.asarray(e["y_fused_only"], np.float64))
    # the brute force agrees with the same hand values
    yb = brute.ffn(x.tolist(), wg.tolist(), wu.tolist(), wd.tolist())
    np.testing.assert_array_equal(np.asarray(yb), np.asarray(e["y_hybrid"], np.float64))


# ------------------------------------------------------------ exhaustive single tile
def test_exhaustive_8wide_tile_all_caps():
    """All 2^8 activity patterns of one 8-wide tile x capacities 1..8."""
    pats = np.arange(256)
    bits = ((pats[:, None] >> np.arange(8)[None, :]) & 1).astype(bool)
    # active -> a distinct positive value, inactive -> negative, zero or NaN (all inactive)
    inactive_fill = np.array([-1.0, 0.0, -0.0, np.nan, -np.inf])
    z = np.where(bits, 1.0 + np.arange(8)[None, :] * 0.25,
                 inactive_fill[np.arange(256)[:, None] % 5 + 0 * np.arange(8)[None, :]])
    for cap in range(1, 9):
        tw = oracle.pack_twell(z, 8, cap, "exact")
        row_ovf, rows, n = oracle.partition_overflow(tw.cnt, cap)
        for p in range(256):
            set_cols = [c for c in range(8) if (p >> c) & 1]
            assert tw.cnt[p, 0] == len(set_cols)
            m = min(len(set_cols), cap)
            assert list(tw.idx[p, 0, :m]) == set_cols[:cap]
            assert list(tw.val[p, 0, :m]) == [1.0 + 0.25 * c for c in set_cols[:cap]]
            assert row_ovf[p] == (1 if len(set_cols) > cap else 0)
        assert list(rows) == [p for p in range(256) if bin(p).count("1") > cap]


# ------------------------------------------------------------ brute force on tiny inputs
@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("w", [4, 8])
def test_against_brute_force(seed, w):
    rng = np.random.default_rng(1000 + seed)
    T = int(rng.integers(1, 5))
    d = int(rng.integers(2, 9))
    F = w * int(rng.integers(1, 32 // w + 1))
    x = _f32(rng.integers(-8, 9, (T, d)) / 4)
    wg = _f32(rng.integers(-8, 9, (F, d)) / 8)
    wu = _f32(rng.integers(-8, 9, (F, d)) / 8)
    wd = _f32(rng.integers(-8, 9, (F, d)) / 8)
    zb = brute.matmul_nt(x.tolist(), wg.tolist())
    z = oracle.matmul_rows(x, np.arange(T), wg)
    np.testing.assert_array_equal(z, np.asarray(zb))
    for cap in range(1, w + 1):
        for vd in ("f32", "bf16"):
            tw = oracle.pack_twell(z, w, cap, vd)
            pb = brute.pack(zb, w, cap, vd)
            for t in range(T):
                for b in range(F // w):
                    n, vals, cols = pb[t][b]
                    assert tw.cnt[t, b] == n
                    m = min(n, cap)
                    assert list(tw.idx[t, b, :m]) == cols
                    assert list(tw.val[t, b, :m]) == vals
                    # unused slots are zero
                    assert not tw.idx[t, b, m:].any() and not tw.val[t, b, m:].any()
            _, rows, _ = oracle.partition_overflow(tw.cnt, cap)
            assert list(rows) == brute.overflow_rows(pb, cap)
    for hr in (None, "bf16"):
        yb = np.asarray(brute.ffn(x.tolist(), wg.tolist(), wu.tolist(), wd.tolist(), hr))
        y = oracle.ffn_active(z, x, wu, wd, hr)
        np.testing.assert_allclose(y, yb, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------ rounding vs library routines
def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    a = rng.standard_normal(200000).astype(np.float32) * np.float32(3.0) ** rng.integers(-30, 30, 200000)
    # exact ties: upper 16 bits arbitrary, lower half exactly 0x8000
    ties = (rng.integers(0, 2 ** 15, 5000).astype(np.uint32) << 16 | 0x8000).view(np.float32)
    special = np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 3.3895314e38, 1e-40, -1e-40], np.float32)
    a = np.concatenate([a, ties[np.isfinite(ties)], special]).astype(np.float32)
    want = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    got = oracle.store_round(a.astype(np.float64), "bf16").astype(np.float32)
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
    # NaN stays NaN (payloads are not compared: torch canonicalises them)
    assert np.isnan(oracle.store_round(np.array([np.nan]), "bf16")).all()


def test_f32_rounding_matches_numpy():
    rng = np.random.default_rng(8)
    a = rng.standard_normal(100000) * 10.0 ** rng.integers(-20, 20, 100000)
    np.testing.assert_array_equal(oracle.store_round(a, "f32"), a.astype(np.float32).astype(np.float64))


# ------------------------------------------------------------ dense == sparse, invariants
@pytest.mark.parametrize("seed,w,cap,frac", [(0, 32, 4, 0.05), (1, 64, 8, 0.1), (2, 128, 16, 0.02),
                                             (3, 32, 2, 0.2)])
def test_dense_equals_sparse_bitwise_and_invariants(seed, w, cap, frac):
    wl = make_random_small(T=37, d=64, F=4 * w, tile_w=w, cap=cap, active_frac=frac, seed=seed, jitter=0.5)
    rows = np.arange(wl.T)
    z = oracle.matmul_rows(wl.x, rows, wl.wg_t)
    u = oracle.matmul_rows(wl.x, rows, wl.wu_t)
    for hr in (None, "bf16"):
        yd = oracle.ffn_dense(z, u, wl.wd, hr)
        ys = oracle.ffn_active(z, wl.x, wl.wu_t, wl.wd, hr)
        assert np.array_equal(yd, ys), "dense and sparse sums must agree bit for bit"
    tw = oracle.pack_twell(z, w, cap, "bf16")
    row_ovf, ovf_rows, n_ovf = oracle.partition_overflow(tw.cnt, cap)
    nnz = int((z > 0).sum())
    assert int(tw.cnt.sum()) == nnz                               # nonzero conservation
    dense = oracle.dense_backup(z, ovf_rows, "bf16")
    assert int(tw.cnt[row_ovf == 0].sum()) + int((dense > 0).sum()) == nnz  # hybrid conservation
    ok = row_ovf == 0
    h_stored = oracle.store_round(np.where(z > 0, z, 0.0), "bf16")
    np.testing.assert_array_equal(oracle.unpack_twell(tw)[ok], h_stored[ok])  # round trip
    # overflow tiles keep the cap lowest active columns
    for t, b in zip(*np.nonzero(tw.cnt > cap)):
        cols = np.nonzero(z[t, b * w:(b + 1) * w] > 0)[0][:cap]
        np.testing.assert_array_equal(tw.idx[t, b], cols)
    # fused-only output: non-overflow rows equal the full sum, overflow rows are 0
    yf = oracle.ffn_twell(tw, wl.x, wl.wu_t, wl.wd, skip_overflow=True)
    ys = oracle.ffn_active(z, wl.x, wl.wu_t, wl.wd, "bf16")
    assert np.array_equal(yf[ok], ys[ok])
    assert not yf[~ok].any()


@pytest.mark.parametrize("seed", [0, 1])
def test_numpy_library_crosscheck(seed):
    wl = make_random_small(T=50, d=128, F=512, tile_w=128, cap=8, active_frac=0.05, seed=seed)
    z = oracle.matmul_rows(wl.x, np.arange(wl.T), wl.wg_t)
    np.testing.assert_array_equal(z, oracle.gate(wl.x, wl.wg_t))  # exact on the grid
    y = oracle.ffn_active(z, wl.x, wl.wu_t, wl.wd)
    yn = oracle.ffn_numpy(wl.x, wl.wg_t, wl.wu_t, wl.wd)
    np.testing.assert_allclose(y, yn, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------ closed forms
def test_closed_form_all_dead():
    wl = make_random_small(T=20, d=64, F=256, tile_w=64, cap=4, active_frac=0.5, seed=3)
    wl.wg_t[:, -1] = -np.inf
    ref = oracle.reference(wl)
    assert not ref.tw.cnt.any() and not ref.y_exact.any() and not ref.y_fused.any()
    assert not np.isnan(ref.z).any()


def test_closed_form_single_active_neuron():
    wl = make_random_small(T=40, d=64, F=256, tile_w=64, cap=4, active_frac=0.5, seed=4)
    j = 77
    wl.wg_t[:, -1] = -np.inf
    wl.wg_t[j, -1] = 1.0
    ref = oracle.reference(wl)
    zj = ref.z[:, j]
    act = zj > 0
    assert act.any() and (~act).any()
    uj = wl.x.astype(np.float64) @ wl.wu_t[j].astype(np.float64)
    want = np.where(act, zj, 0.0)[:, None] * uj[:, None] * wl.wd[j].astype(np.float64)[None, :]
    np.testing.assert_allclose(ref.y_exact, want, rtol=1e-14, atol=0)
    assert (ref.tw.cnt.sum(1) == act).all()
    assert (ref.tw.idx[act, j // 64, 0] == j % 64).all()


def test_closed_form_cap_equals_tile_all_active():
    wl = make_random_small(T=16, d=64, F=128, tile_w=32, cap=32, active_frac=0.5, seed=5)
    wl.wg_t[:, -1] = 64.0  # every pre-activation strictly positive
    ref = oracle.reference(wl)
    assert (ref.tw.cnt == 32).all()
    assert (ref.tw.idx == np.arange(32)[None, None, :]).all()
    np.testing.assert_array_equal(ref.tw.val.reshape(16, 128), oracle.store_round(ref.z, "bf16"))
    np.testing.assert_allclose(ref.y_exact, oracle.ffn_numpy(wl.x, wl.wg_t, wl.wu_t, wl.wd), rtol=1e-12)


def test_closed_form_identity_up_down():
    """F = d, W_u = W_d = I  ->  y = ReLU(x W_g) * x."""
    wl = make_random_small(T=24, d=64, F=64, tile_w=32, cap=32, active_frac=0.3, seed=6)
    eye = np.eye(64, dtype=np.float32)
    ref = oracle.reference(type(wl)(wl.name, wl.T, 64, 64, "bf16", 32, 32, wl.x, wl.wg_t, eye, eye))
    want = np.where(ref.z > 0, ref.z, 0.0) * wl.x.astype(np.float64)
    np.testing.assert_array_equal(ref.y_exact, want)


def test_reference_rows_subset_consistent():
    """Sampled-row reference equals the full reference restricted to those rows."""
    wl = make_random_small(T=64, d=64, F=256, tile_w=64, cap=4, active_frac=0.08, seed=9, jitter=0.5)
    full = oracle.reference(wl)
    rows = np.array([3, 17, 18, 40, 63])
    sub = oracle.reference(wl, rows)
    np.testing.assert_array_equal(sub.tw.cnt, full.tw.cnt[rows])
    np.testing.assert_array_equal(sub.y_exact, full.y_exact[rows])


@pytest.mark.parametrize("w,cap", list(itertools.product([32, 256], [1, 16])))
def test_nan_and_signed_zero_inactive(w, cap):
    z = np.full((3, w), -1.0)
    z[0, 0] = 0.0
    z[0, 1] = -0.0
    z[0, 2] = np.nan
    z[1, 5] = 1e-30
    z[2, w - 1] = 2.0
    tw = oracle.pack_twell(z, w, cap, "f32")
    assert tw.cnt[:, 0].tolist() == [0, 1, 1]
    assert tw.idx[1, 0, 0] == 5 and tw.idx[2, 0, 0] == w - 1


# ------------------------------------------------------------ gate activation statistics
@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("w", [4, 8, 32])
def test_gate_stats_against_brute_force(seed, w):
    rng = np.random.default_rng(2000 + seed)
    T = int(rng.integers(1, 7))
    F = w * int(rng.integers(1, 5))
    z = rng.integers(-6, 7, (T, F)) / 4.0
    cnt, l1 = oracle.gate_stats(z, w)
    cb, lb = brute.gate_stats(z.tolist(), w)
    assert list(cnt) == cb
    np.testing.assert_array_equal(l1, np.asarray(lb))


@pytest.mark.parametrize("w,cap", [(32, 4), (64, 8), (256, 16)])
def test_gate_stats_against_twell(w, cap):
    """Counts conserve the TwELL true counts; with cap = tile width and exact
    storage every active value is stored, so each tile's stored values sum to l1."""
    wl = make_random_small(T=48, d=64, F=512, tile_w=w, cap=cap, active_frac=0.1, seed=11, jitter=0.5)
    z = oracle.gate(wl.x, wl.wg_t)
    cnt, l1 = oracle.gate_stats(z, w)
    tw = oracle.pack_twell(z, w, cap, "bf16")
    assert cnt.sum() == tw.cnt.sum()
    full = oracle.pack_twell(z, w, w, "exact")
    np.testing.assert_array_equal(cnt, (oracle.unpack_twell(full) > 0).sum(0))
    np.testing.assert_allclose(l1, full.val.sum(2), rtol=1e-14, atol=0)
    assert (l1 >= 0).all() and ((l1 > 0) == (tw.cnt > 0)).all()


def test_gate_stats_closed_forms():
    T, F, w = 5, 64, 16
    cnt, l1 = oracle.gate_stats(np.full((T, F), -1.0), w)
    assert not cnt.any() and not l1.any()
    cnt, l1 = oracle.gate_stats(np.full((T, F), 0.5), w)
    assert (cnt == T).all() and (l1 == 0.5 * w).all()
    z = np.full((T, F), -2.0)
    z[:, 7] = np.arange(1, T + 1)  # one live neuron, the rest dead
    z[0, 9] = np.nan
    z[1, 9] = -0.0
    z[2, 9] = 0.0
    cnt, l1 = oracle.gate_stats(z, w)
    assert cnt[7] == T and cnt.sum() == T
    np.testing.assert_array_equal(l1[:, 0], np.arange(1, T + 1))
    assert not l1[:, 1:].any()


# ------------------------------------------------------------ hybrid <-> dense conversions
def test_hybrid_to_dense_hand_example():
    """w = 4, cap = 2: row 0 fits (2 and 1 actives), row 1 overflows (3 actives
    in tile 0), row 2 overflows too; max_ovf = 1 serves only row 1."""
    h = np.array([[0.0, 1.5, 0.0, 2.0, 0.0, 0.0, 0.0, 3.0],
                  [4.0, 5.0, 6.0, 0.0, 0.0, 0.0, 7.0, 0.0],
                  [0.0, 1.0, 1.0, 1.0, 0.0, 0.0, 0.0, 0.0]])
    tw = oracle.pack_twell(h, 4, 2, "f32")
    row_ovf, rows, n = oracle.partition_overflow(tw.cnt, 2)
    assert list(row_ovf) == [0, 1, 1] and list(rows) == [1, 2] and n == 2
    dense = oracle.dense_backup(h, rows, "f32")
    out = oracle.hybrid_to_dense(tw, rows, dense, max_ovf=1)
    np.testing.assert_array_equal(out[0], h[0])
    np.testing.assert_array_equal(out[1], h[1])
    # row 2 is not served: only its first two actives of tile 0 survive
    np.testing.assert_array_equal(out[2], [0.0, 1.0, 1.0, 0.0, 0.0, 0.0, 0.0, 0.0])


@pytest.mark.parametrize("w,cap", [(32, 2), (64, 8), (256, 16)])
def test_dense_hybrid_round_trip(w, cap):
    """dense -> hybrid -> dense gives back max(H, 0) exactly when every
    overflow row is served (TwELL keeps a fitting row whole, the dense backup
    keeps an overflow row whole); negative and NaN entries come back as 0."""
    rng = np.random.default_rng(w + cap)
    T, F = 40, 512
    h = oracle.store_round(rng.standard_normal((T, F)) * (rng.random((T, F)) < 0.08), "bf16")
    h[3, :200] = np.abs(h[3, :200]) + 0.5  # a heavy row
    h = oracle.store_round(h, "bf16")
    h[5, 7] = np.nan
    tw = oracle.pack_twell(h, w, cap, "bf16")
    _, rows, n = oracle.partition_overflow(tw.cnt, cap)
    assert n > 0
    dense = oracle.dense_backup(h, rows, "bf16")
    out = oracle.hybrid_to_dense(tw, rows, dense, max_ovf=n)
    want = np.where(h > 0, h, 0.0)
    np.testing.assert_array_equal(out, want)


def test_compact_hybrid_hand_example():
    """Same matrix as the hybrid-to-dense example: row 0 fits (entries at
    columns 1, 3, 7), rows 1 and 2 overflow; max_ovf = 1 holds row 1 densely."""
    h = np.array([[0.0, 1.5, 0.0, 2.0, 0.0, 0.0, 0.0, 3.0],
                  [4.0, 5.0, 6.0, 0.0, 0.0, 0.0, 7.0, 0.0],
                  [0.0, 1.0, 1.0, 1.0, 0.0, 0.0, 0.0, 0.0]])
    tw = oracle.pack_twell(h, 4, 2, "f32")
    row_ovf, rows, n = oracle.partition_overflow(tw.cnt, 2)
    c = oracle.compact_hybrid(tw, row_ovf, rows, oracle.dense_backup(h, rows, "f32"), max_ovf=1)
    assert list(c["row_ptr"]) == [0, 3, 3, 3]
    assert list(c["col"]) == [1, 3, 7] and list(c["val"]) == [1.5, 2.0, 3.0]
    assert list(c["ovf_rows"]) == [1, 2] and c["n_ovf"] == 2 and not c["complete"]
    np.testing.assert_array_equal(c["dense"], h[1:2])
    out = oracle.compact_to_dense(c, 3, 8)
    np.testing.assert_array_equal(out[:2], h[:2])
    assert not out[2].any()  # row 2 is held nowhere


@pytest.mark.parametrize("w,cap", [(32, 2), (256, 16)])
def test_compact_round_trip_and_conservation(w, cap):
    rng = np.random.default_rng(7 * w + cap)
    T, F = 60, 512
    h = rng.standard_normal((T, F)) * (rng.random((T, F)) < 0.06)
    h[4, :300] = np.abs(h[4, :300]) + 1.0
    h = oracle.store_round(h, "bf16")
    tw = oracle.pack_twell(h, w, cap, "bf16")
    row_ovf, rows, n = oracle.partition_overflow(tw.cnt, cap)
    c = oracle.compact_hybrid(tw, row_ovf, rows, oracle.dense_backup(h, rows, "bf16"), max_ovf=n)
    assert c["complete"]
    np.testing.assert_array_equal(oracle.compact_to_dense(c, T, F), np.where(h > 0, h, 0.0))
    # entries held compactly = positives of the rows that fit
    fit = row_ovf == 0
    assert c["row_ptr"][-1] == int((h[fit] > 0).sum())
    for t in range(T):
        cs = c["col"][c["row_ptr"][t]:c["row_ptr"][t + 1]]
        assert (np.diff(cs) > 0).all()


# ------------------------------------------------------------ backward pass
def _np_forward(x, wg_t, wu_t, wd):
    """An independent fp64 forward for finite differences: ReLU(x W_g) * (x W_u), then W_d."""
    z = x @ wg_t.T
    return (np.where(z > 0, z, 0.0) * (x @ wu_t.T)) @ wd


def _small_problem(seed):
    rng = np.random.default_rng(seed)
    T, d, F = 3, 8, 16
    x = _f32(rng.integers(-4, 5, (T, d)) / 4)
    wg = _f32(rng.integers(-4, 5, (F, d)) / 8)
    wu = _f32(rng.integers(-4, 5, (F, d)) / 8)
    wd = _f32(rng.integers(-4, 5, (F, d)) / 8)
    dy = rng.integers(-3, 4, (T, d)) / 2.0
    # a ones column and a 1/64 bias keep every z off 0 (other terms are multiples of 1/32)
    x[:, -1] = 1.0
    wg[:, -1] = _f32(np.full(F, 1 / 64) + rng.integers(-2, 3, F) / 8)
    return x, wg, wu, wd, dy


@pytest.mark.parametrize("seed", range(3))
def test_backward_finite_differences(seed):
    """Every gradient entry against central differences of sum(y * dy) of an
    independent numpy forward (fp64, h = ReLU(z) unrounded); the active set
    does not change for the step used (|z| is far from 0 on the grid)."""
    x, wg, wu, wd, dy = _small_problem(seed)
    z = x.astype(np.float64) @ wg.astype(np.float64).T
    assert np.min(np.abs(z)) >= 1.0 / 64  # grid values: no sign change within eps
    dx, dwg, dwu, dwd = oracle.ffn_backward(z, x, wg, wu, wd, dy, None)
    base = [a.astype(np.float64) for a in (x, wg, wu, wd)]
    loss = lambda p: float((_np_forward(*p) * dy).sum())  # noqa: E731
    eps = 1e-4
    for which, grad in ((0, dx), (1, dwg), (2, dwu), (3, dwd)):
        fd = np.zeros_like(grad)
        for i in np.ndindex(grad.shape):
            p = [a.copy() for a in base]
            p[which][i] += eps
            lp = loss(p)
            p[which][i] -= 2 * eps
            lm = loss(p)
            fd[i] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-7, err_msg=f"parameter {which}")


def test_backward_matrix_form():
    """Library cross-check: the same gradients as dense matrix products (numpy
    fp64 matmuls) on a random layer, with the stored (bf16) h."""
    wl = make_random_small(T=40, d=64, F=256, tile_w=64, cap=8, active_frac=0.1, seed=12, jitter=0.5)
    rng = np.random.default_rng(3)
    dy = rng.standard_normal((wl.T, wl.d))
    z = oracle.gate(wl.x, wl.wg_t)
    dx, dwg, dwu, dwd = oracle.ffn_backward(z, wl.x, wl.wg_t, wl.wu_t, wl.wd, dy, "bf16")
    x = wl.x.astype(np.float64)
    H = oracle.store_round(np.where(z > 0, z, 0.0), "bf16")
    U = x @ wl.wu_t.astype(np.float64).T
    G = dy @ wl.wd.astype(np.float64).T
    DU, DZ = G * H, G * U * (z > 0)
    np.testing.assert_allclose(dx, DU @ wl.wu_t.astype(np.float64) + DZ @ wl.wg_t.astype(np.float64), rtol=1e-10,
                               atol=1e-10)
    np.testing.assert_allclose(dwd, (H * U).T @ dy, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(dwu, DU.T @ x, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(dwg, DZ.T @ x, rtol=1e-10, atol=1e-10)


def test_backward_single_neuron_closed_form():
    """One active neuron j: dW_d[j] = sum_t (h_t u_t) dy_t, every other
    neuron's gradients 0, dx_t = g_t (h_t W_u[j] + u_t W_g[j])."""
    wl = make_random_small(T=10, d=64, F=128, tile_w=64, cap=4, active_frac=0.5, seed=4)
    j = 37
    wl.wg_t[:, -1] = -np.inf
    wl.wg_t[j, -1] = 2.0
    z = oracle.gate(wl.x, wl.wg_t)
    rng = np.random.default_rng(5)
    dy = rng.standard_normal((wl.T, wl.d))
    dx, dwg, dwu, dwd = oracle.ffn_backward(z, wl.x, wl.wg_t, wl.wu_t, wl.wd, dy, None)
    act = z[:, j] > 0
    assert act.any()
    others = np.arange(wl.F) != j
    assert not dwd[others].any() and not dwu[others].any() and not dwg[others].any()
    x = wl.x.astype(np.float64)
    u = x @ wl.wu_t[j].astype(np.float64)
    g = dy @ wl.wd[j].astype(np.float64)
    h = np.where(act, z[:, j], 0.0)
    np.testing.assert_allclose(dwd[j], ((h * u)[:, None] * dy).sum(0), rtol=1e-12)
    want_dx = np.where(act[:, None], g[:, None] * (h[:, None] * wl.wu_t[j].astype(np.float64)
                                                    + u[:, None] * wl.wg_t[j].astype(np.float64)), 0.0)
    np.testing.assert_allclose(dx, want_dx, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------ magnitude sums (tie band, y tolerance)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_abs_sums_against_brute_force(seed):
    """sum_k |x_k w_jk| with mixed signs, against pure-Python loops."""
    rng = np.random.default_rng(100 + seed)
    x = rng.standard_normal((3, 7)).astype(np.float32)
    w = rng.standard_normal((5, 7)).astype(np.float32)
    m = oracle.abs_sums(x, w)
    for t in range(3):
        for j in range(5):
            s = 0.0
            for k in range(7):
                s += abs(float(x[t, k]) * float(w[j, k]))
            assert m[t, j] == pytest.approx(s, rel=1e-15, abs=0.0)


def test_abs_sums_closed_forms():
    """Non-negative operands: the magnitude sum is the dot product itself;
    gamma(2048) at fp32's unit 2^-23 is 2^-12 / (1 - 2^-12) = 1/4095."""
    rng = np.random.default_rng(7)
    x = np.abs(rng.standard_normal((4, 16))).astype(np.float32)
    w = np.abs(rng.standard_normal((6, 16))).astype(np.float32)
    np.testing.assert_allclose(oracle.abs_sums(x, w), oracle.gate(x, w), rtol=1e-15)
    assert oracle.gamma(2048) == pytest.approx(1.0 / 4095.0, rel=1e-15)
    assert oracle.gamma(1, 2.0 ** -24) == pytest.approx(2.0 ** -24 / (1 - 2.0 ** -24), rel=1e-15)


def test_tie_band_bounds_fp32_orders():
    """Continuous bf16-valued inputs: fp32 sums of x.w in several orders all
    lie within gamma(d) * sum|x w| of the fp64 value (the tie band is a valid
    bound on summation-order effects)."""
    import torch
    rng = np.random.default_rng(9)
    d = 512
    x = torch.from_numpy(rng.standard_normal((8, d)).astype(np.float32)).bfloat16().float().numpy()
    w = torch.from_numpy((rng.standard_normal((64, d)) / np.sqrt(d)).astype(np.float32)).bfloat16().float().numpy()
    z = oracle.gate(x, w)
    band = oracle.gamma(d) * oracle.abs_sums(x, w)
    prods = x[:, None, :] * w[None, :, :]            # exact in fp32 (bf16 x bf16)
    fwd = np.zeros((8, 64), np.float32)
    for k in range(d):
        fwd = fwd + prods[:, :, k]
    rev = np.zeros((8, 64), np.float32)
    for k in reversed(range(d)):
        rev = rev + prods[:, :, k]
    pair = prods.sum(axis=2, dtype=np.float32)
    for s in (fwd, rev, pair):
        assert (np.abs(s.astype(np.float64) - z) <= band).all()
    assert (fwd != rev).any()  # the orders do differ: the check is not vacuous
