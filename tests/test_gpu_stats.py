"""GPU parity of the gate activation statistics (twell_pack_gate_stats)
against the oracle's gate_stats.

Per-neuron active counts must match exactly (they are integers, and z is
exact in fp32 for grid-mode inputs).  The per (row, tile) sums of the positive
gate values are fp32 sums of at most w non-negative terms, so each is within
(w - 1) * 2^-24 relative of the exact sum (the standard bound for summing
non-negative numbers in any order); a tile without actives must be exactly 0.
The TwELL written alongside must be the same bits as twell_pack_gate's.
"""

import numpy as np
import pytest

import oracle
from helpers import say, to_device
from workloads import make_layer_0p5b, make_layer_2b, make_random_small, make_tiny

pytestmark = pytest.mark.gpu

PRESET = 5  # neuron_cnt is added to: start from a known non-zero value


def _run(wl, calls=1):
    import torch
    import unstructured_sparse_transformer_amd as tw
    dt, x, wg, _, _ = to_device(wl)
    n_b = wl.F // wl.tile_w
    ref_tw = tw.TwELL.empty(wl.T, wl.F, wl.tile_w, wl.cap, dt)
    tw.twell_pack_gate(x, wg, ref_tw)
    st_tw = tw.TwELL.empty(wl.T, wl.F, wl.tile_w, wl.cap, dt)
    st_tw.cnt.fill_(-7)
    st_tw.idx.fill_(0xAB)
    st_tw.val.fill_(-3.0)
    ncnt = torch.full((wl.F,), PRESET, dtype=torch.int32, device="cuda")
    l1s = []
    for _ in range(calls):
        l1 = torch.full((wl.T, n_b), float("nan"), dtype=torch.float32, device="cuda")
        tw.twell_pack_gate_stats(x, wg, st_tw, ncnt, l1)
        l1s.append(l1)
    torch.cuda.synchronize()
    for name in ("cnt", "idx"):
        assert torch.equal(getattr(st_tw, name), getattr(ref_tw, name)), name
    assert torch.equal(st_tw.val.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                       ref_tw.val.view(torch.int16 if dt == torch.bfloat16 else torch.int32))
    return ncnt.cpu().numpy().astype(np.int64), [a.cpu().numpy() for a in l1s]


def _check(wl, calls=1, label=""):
    ncnt, l1s = _run(wl, calls)
    z = oracle.gate(wl.x, wl.wg_t)
    cnt_ref, l1_ref = oracle.gate_stats(z, wl.tile_w)
    np.testing.assert_array_equal(ncnt - PRESET, calls * cnt_ref, err_msg=label)
    rtol = (wl.tile_w - 1) * 2.0 ** -24
    for l1 in l1s:
        assert not np.isnan(l1).any(), label
        np.testing.assert_allclose(l1, l1_ref, rtol=rtol, atol=0, err_msg=label)
        assert ((l1 == 0) == (l1_ref == 0)).all(), label
        np.testing.assert_array_equal(l1, l1s[0])  # fixed summation order: same bits
    say(f"  {label}: active={int(cnt_ref.sum())} dead={int((cnt_ref == 0).sum())}/{wl.F} "
        f"max l1 rel err={np.max(np.abs(l1s[0] - l1_ref) / np.maximum(l1_ref, 1e-300)):.2e}")
    return cnt_ref


def test_stats_tiny_fp32(gpu_lib):
    wl = make_tiny()
    say(f"case stats tiny T={wl.T} d={wl.d} F={wl.F} f32")
    _check(wl, label="tiny")


STATS_EDGE = [
    # (T, d, F, w, cap, dtype, frac, jitter, dead)
    (300, 128, 512, 128, 8, "bf16", 0.05, 0.5, 0),    # ragged T
    (257, 64, 384, 128, 4, "bf16", 0.08, 0.5, 0),     # F not a multiple of 256
    (100, 256, 1024, 32, 4, "bf16", 0.1, 0.5, 0),     # w = 32
    (100, 256, 1024, 64, 2, "bf16", 0.1, 0.5, 30),    # w = 64, dead neurons
    (130, 512, 2048, 256, 1, "bf16", 0.3, 0.5, 0),    # w = 256 (a tile spans two waves)
    (200, 256, 1024, 256, 64, "bf16", 0.3, 0.5, 0),   # large cap (general packing epilogue)
    (70, 2048, 512, 128, 8, "f32", 0.1, 0.5, 0),      # fp32
    (90, 192, 640, 64, 8, "f32", 0.2, 0.3, 5),        # fp32 odd shapes, dead neurons
    (96, 128, 512, 256, 48, "f32", 0.4, 0.5, 0),      # fp32, w = 256
    (50, 64, 64, 64, 8, "bf16", 0.1, 0.5, 0),         # F = 64: less than a workgroup's columns
    (1, 128, 256, 32, 2, "f32", 0.3, 0.3, 0),         # T = 1
]


@pytest.mark.parametrize("case", STATS_EDGE,
                         ids=[f"T{c[0]}_d{c[1]}_F{c[2]}_w{c[3]}_c{c[4]}_{c[5]}" for c in STATS_EDGE])
def test_stats_edge_shapes(gpu_lib, case):
    T, d, F, w, cap, dt, frac, jit, dead = case
    wl = make_random_small(T, d, F, w, cap, dt, active_frac=frac, seed=T + d + 1, jitter=jit, n_dead=dead)
    say(f"case stats edge {wl.name}")
    cnt = _check(wl, calls=2, label=wl.name)
    assert (cnt == 0).sum() >= dead


def test_stats_all_active(gpu_lib):
    """Every pre-activation positive: each neuron counts every row, and each
    tile's sum is the sum of its whole row segment."""
    wl = make_random_small(64, 128, 512, 64, 64, "bf16", active_frac=0.5, seed=8)
    wl.wg_t[:, -1] = 64.0
    say("case stats all active")
    cnt = _check(wl, label="all active")
    assert (cnt == wl.T).all()


def test_stats_layer_0p5b(gpu_lib):
    wl = make_layer_0p5b()
    say(f"case stats layer_0p5b T={wl.T} d={wl.d} F={wl.F}")
    _check(wl, label="0p5b")


def test_stats_layer_2b_dead_neurons(gpu_lib):
    """Full-size layer with 20% of the neurons dead by construction: those read 0."""
    wl = make_layer_2b()
    say(f"case stats layer_2b T={wl.T} d={wl.d} F={wl.F} (full oracle)")
    cnt = _check(wl, label="2b")
    assert (cnt[wl.meta["dead"]] == 0).all()


@pytest.mark.parametrize("name", ["tiny", "0p5b"])
def test_stats_gate_then_from_gate(gpu_lib, name):
    """twell_pack_gate_stats followed by twell_ffn_from_gate writes the same
    hybrid and y bits as twell_ffn_forward (the statistics change nothing else)."""
    import torch
    import unstructured_sparse_transformer_amd as tw
    wl = make_tiny() if name == "tiny" else make_layer_0p5b()
    say(f"case stats gate + twell_ffn_from_gate {wl.name}")
    dt, x, wg, wu, wd = to_device(wl)
    max_ovf = min(wl.T, 256)
    n_b = wl.F // wl.tile_w
    out = []
    for with_stats in (False, True):
        hy = tw.Hybrid.empty(wl.T, wl.F, wl.tile_w, wl.cap, dt, max_ovf)
        y = torch.full((wl.T, wl.d), float("nan"), dtype=torch.float32, device="cuda")
        ws = tw.hybrid_workspace(hy, wl.d)
        if with_stats:
            ncnt = torch.zeros(wl.F, dtype=torch.int32, device="cuda")
            l1 = torch.empty((wl.T, n_b), dtype=torch.float32, device="cuda")
            tw.twell_pack_gate_stats(x, wg, hy.ell, ncnt, l1)
            tw.twell_ffn_from_gate(x, wg, wu, wd, hy, y, ws)
        else:
            tw.twell_ffn_forward(x, wg, wu, wd, hy, y, ws)
        torch.cuda.synchronize()
        m = min(int(hy.n_ovf.item()), max_ovf)
        out.append([hy.ell.cnt, hy.ell.idx, hy.ell.val.view(torch.uint8) if dt == torch.bfloat16 else hy.ell.val,
                    hy.row_ovf, hy.n_ovf, hy.order, hy.ovf_rows[:m], hy.dense[:m].contiguous().view(torch.uint8),
                    y.view(torch.int32)])
    for a, b in zip(*out):
        assert torch.equal(a, b), f"{wl.name}: stats gate + from_gate differs from twell_ffn_forward"
    assert int(ncnt.sum().item()) == int((hy.ell.cnt.sum()).item()), f"{wl.name}: neuron counts vs TwELL counts"
