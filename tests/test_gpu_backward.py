"""GPU parity of the sparse FFN's backward pass (twell_ffn_backward) against
the oracle's ffn_backward (fp64, stored bf16 h), through the C ABI.

dx per row and each weight-gradient row per neuron must be within 1e-4 of the
oracle in relative L2 norm (fp32 dot products and sums over up to a few
thousand terms, against fp64 -- the same bar as the forward's stored-h check);
rows and neurons without entries must be exactly 0; repeated calls must give
the same bits."""

import numpy as np
import pytest

import oracle
from helpers import say, to_device
from workloads import make_layer_0p5b, make_layer_2b, make_random_small

pytestmark = pytest.mark.gpu

RTOL = 1e-4


def _run(wl, dy, max_ovf=None, max_entries=None, calls=2):
    import torch
    import unstructured_sparse_transformer_amd as tw
    dt, x, wg, wu, wd = to_device(wl)
    if max_ovf is None:
        max_ovf = wl.T
    hy = tw.Hybrid.empty(wl.T, wl.F, wl.tile_w, wl.cap, dt, max_ovf)
    tw.twell_pack_gate_hybrid(x, wg, hy)
    if max_entries is None:
        max_entries = min(wl.T * wl.F, 1 << 20)
    ws = tw.backward_workspace(wl.T, wl.F, wl.d, max_entries)
    ws.fill_(0xCD)
    dyd = torch.from_numpy(np.ascontiguousarray(dy, dtype=np.float32)).to("cuda")
    outs = []
    for _ in range(calls):
        dx = torch.full((wl.T, wl.d), float("nan"), dtype=torch.float32, device="cuda")
        g = [torch.full((wl.F, wl.d), float("nan"), dtype=torch.float32, device="cuda") for _ in range(3)]
        tw.twell_ffn_backward(hy, x, wg, wu, wd, dyd, dx, g[0], g[1], g[2], max_entries, ws)
        outs.append([dx] + g)
    torch.cuda.synchronize()
    status = tw.backward_status(ws)
    host = [[a.cpu().numpy() for a in o] for o in outs]
    return host, status, int(hy.n_ovf.item())


def _rel_ok(got, want, label):
    got = got.astype(np.float64)
    assert np.isfinite(got).all(), f"{label}: non-finite"
    num = np.linalg.norm(got - want, axis=1)
    den = np.linalg.norm(want, axis=1)
    zero = den == 0
    assert not got[zero].any(), f"{label}: rows without entries must be exactly 0"
    bad = ~zero & (num > RTOL * den)
    assert not bad.any(), f"{label}: {bad.sum()} rows off, max rel {np.max(num[~zero] / den[~zero]):.3g}"


def _check(wl, dy, host, z, label, drop_rows=()):
    if len(drop_rows):
        z = z.copy()
        z[list(drop_rows)] = -1.0  # rows that contribute nothing
    want = oracle.ffn_backward(z, wl.x, wl.wg_t, wl.wu_t, wl.wd, dy, wl.dtype)
    for name, got, w in zip(("dx", "dW_g", "dW_u", "dW_d"), host[-1], want):
        _rel_ok(got, w, f"{label} {name}")
    for k, o in enumerate(host[:-1]):
        for a, b in zip(o, host[-1]):
            np.testing.assert_array_equal(a, b, err_msg=f"{label}: call {k} differs")


BW_CASES = [
    # (T, d, F, w, cap, frac, jitter, dead)
    (300, 128, 512, 128, 8, 0.05, 0.5, 0),     # ragged T
    (257, 64, 384, 128, 4, 0.08, 0.5, 0),      # F not a multiple of 256, d = 64
    (100, 256, 1024, 32, 4, 0.1, 0.5, 0),      # w = 32
    (100, 256, 1024, 64, 2, 0.1, 0.5, 30),     # w = 64, dead neurons
    (64, 2048, 512, 256, 16, 0.05, 0.5, 0),    # d = 2048
    (512, 256, 1024, 128, 3, 0.4, 0.2, 0),     # nearly every row overflows
    (1, 128, 256, 32, 2, 0.3, 0.3, 0),         # T = 1
]


@pytest.mark.parametrize("case", BW_CASES, ids=[f"T{c[0]}_d{c[1]}_F{c[2]}_w{c[3]}_c{c[4]}" for c in BW_CASES])
def test_backward_shapes(gpu_lib, case):
    T, d, F, w, cap, frac, jit, dead = case
    wl = make_random_small(T, d, F, w, cap, "bf16", active_frac=frac, seed=T + d + 7, jitter=jit, n_dead=dead)
    rng = np.random.default_rng(T + F)
    dy = rng.standard_normal((T, d)).astype(np.float32)
    say(f"case backward {wl.name}")
    host, status, n_ovf = _run(wl, dy)
    assert status[1] == 0
    _check(wl, dy, host, oracle.gate(wl.x, wl.wg_t), wl.name)


def test_backward_overflow_rows_not_held(gpu_lib):
    """Overflow rows past max_ovf contribute nothing (dx row 0)."""
    wl = make_random_small(96, 128, 512, 128, 2, "bf16", active_frac=0.1, seed=31, jitter=0.6)
    dy = np.random.default_rng(1).standard_normal((wl.T, wl.d)).astype(np.float32)
    say("case backward with max_ovf below n_ovf")
    z = oracle.gate(wl.x, wl.wg_t)
    tw_ = oracle.pack_twell(z, wl.tile_w, wl.cap, wl.dtype)
    _, rows, n = oracle.partition_overflow(tw_.cnt, wl.cap)
    assert n > 4
    host, status, n_ovf = _run(wl, dy, max_ovf=3)
    assert n_ovf == n
    _check(wl, dy, host, z, "max_ovf=3", drop_rows=rows[3:])
    assert not host[-1][0][rows[3:]].any()


def test_backward_too_many_entries(gpu_lib):
    """max_entries below the entry count: status says so, outputs are zero."""
    wl = make_random_small(64, 128, 512, 128, 8, "bf16", active_frac=0.1, seed=3, jitter=0.5)
    dy = np.ones((wl.T, wl.d), np.float32)
    say("case backward with too small an entry bound")
    host, status, _ = _run(wl, dy, max_entries=10, calls=1)
    assert status[1] == 1 and status[0] > 10
    for a in host[-1]:
        assert not a.any()


def test_backward_layer_0p5b(gpu_lib):
    wl = make_layer_0p5b()
    dy = np.random.default_rng(2).standard_normal((wl.T, wl.d)).astype(np.float32)
    say(f"case backward layer_0p5b T={wl.T} d={wl.d} F={wl.F}")
    host, status, _ = _run(wl, dy, calls=1)
    assert status[1] == 0
    _check(wl, dy, host, oracle.gate(wl.x, wl.wg_t), "0p5b")


def test_backward_layer_2b(gpu_lib):
    """The full 2B-like layer: 1638 dead neurons get zero weight gradients."""
    wl = make_layer_2b()
    dy = np.random.default_rng(4).standard_normal((wl.T, wl.d)).astype(np.float32)
    say(f"case backward layer_2b T={wl.T} d={wl.d} F={wl.F}")
    host, status, n_ovf = _run(wl, dy, max_ovf=1024, max_entries=1 << 20, calls=1)
    assert status[1] == 0
    say(f"  entries={status[0]} n_ovf={n_ovf}")
    _check(wl, dy, host, oracle.gate(wl.x, wl.wg_t), "2b")
    dead = wl.meta["dead"]
    for a in host[-1][1:]:
        assert not a[dead].any()
