"""HIP-graph capture of the hot path through the C ABI.

One twell_ffn_decode call, and one batch step (twell_pack_gate then
twell_ffn_from_gate), are captured once into a graph and replayed several
times.  Before each replay a new input is copied into the captured x and the
captured outputs are poisoned; between replays the eager call runs on the same
input into buffers of its own, with synchronisations in between.  Every
replay's outputs (y, TwELL, overflow flags and list, dense backup, work order)
must equal the eager call's bit for bit.  The captured calls launch kernels
only: the counters they use are cleared by their own kernels, so the graphs
hold no memset nodes."""

import numpy as np
import pytest
import torch

from helpers import say, to_device
from workloads import make_decode_windows, make_layer_2b

pytestmark = pytest.mark.gpu


def _capture(fn):
    """Run fn once on a side stream (warm-up), then capture it into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _poison(hy, y):
    y.fill_(float("nan"))
    hy.ell.cnt.fill_(-7)
    hy.ell.val.fill_(-3.0)
    hy.ell.idx.fill_(0xAB)
    hy.row_ovf.fill_(-7)
    hy.n_ovf.fill_(-7)
    hy.order.fill_(-7)
    if hy.max_ovf:
        hy.ovf_rows.fill_(-7)
        hy.dense.fill_(-5.0)


def _assert_same(hy_g, y_g, hy_e, y_e, label):
    n = int(hy_e.n_ovf.item())
    m = min(n, hy_e.max_ovf)
    pairs = [("y", y_g, y_e), ("cnt", hy_g.ell.cnt, hy_e.ell.cnt), ("val", hy_g.ell.val, hy_e.ell.val),
             ("idx", hy_g.ell.idx, hy_e.ell.idx), ("row_ovf", hy_g.row_ovf, hy_e.row_ovf),
             ("n_ovf", hy_g.n_ovf, hy_e.n_ovf), ("order", hy_g.order, hy_e.order)]
    if m:
        pairs += [("ovf_rows", hy_g.ovf_rows[:m], hy_e.ovf_rows[:m]), ("dense", hy_g.dense[:m], hy_e.dense[:m])]
    for name, a, b in pairs:
        assert torch.equal(a, b), f"{label}: graph replay differs from the eager call in {name}"
    assert not torch.isnan(y_g).any(), f"{label}: replay left unwritten rows of y"
    return n


@pytest.mark.parametrize("T", [1, 8, 64])
def test_decode_graph_replay(gpu_lib, T):
    """twell_ffn_decode captured once, replayed on windows 1 and 2 of the 2B
    layer and on the three busiest of its first 64 windows (overflow rows occur
    there for T >= 8)."""
    tw = gpu_lib
    wins = make_decode_windows(T, max_windows=64)
    dt, x, wg, wu, wd = to_device(wins[0])
    hy = tw.Hybrid.empty(T, wins[0].F, wins[0].tile_w, wins[0].cap, dt, T)
    hy_e = tw.Hybrid.empty(T, wins[0].F, wins[0].tile_w, wins[0].cap, dt, T)
    ws = tw.decode_workspace(T, wins[0].F, wins[0].d, wins[0].tile_w)
    ws_e = tw.decode_workspace(T, wins[0].F, wins[0].d, wins[0].tile_w)
    y = torch.empty((T, wins[0].d), dtype=torch.float32, device="cuda")
    y_e = torch.empty_like(y)
    g = _capture(lambda: tw.twell_ffn_decode(x, wg, wu, wd, hy, y, ws))
    base = make_layer_2b()
    xs = torch.from_numpy(np.ascontiguousarray(base.x[: len(wins) * T])).to("cuda").to(dt)
    z = torch.matmul(xs.float(), wg.float().t())
    busy = torch.argsort((z > 0).reshape(len(wins), T, -1).sum((1, 2)), descending=True)[:3].tolist()
    n_seen = 0
    for i in sorted(set([1, 2] + busy)):
        say(f"case graph decode T={T} window={i}")
        xi = xs[i * T:(i + 1) * T]
        x.copy_(xi)
        _poison(hy, y)
        g.replay()
        torch.cuda.synchronize()
        _poison(hy_e, y_e)
        tw.twell_ffn_decode(xi.contiguous(), wg, wu, wd, hy_e, y_e, ws_e)
        torch.cuda.synchronize()
        n_seen += _assert_same(hy, y, hy_e, y_e, f"decode T={T} window={i}")
    if T >= 8:
        assert n_seen > 0


def test_batch_step_graph_replay(gpu_lib):
    """twell_pack_gate + twell_ffn_from_gate captured once on 2048 rows of the
    2B layer, replayed on other row blocks (each with overflow rows) and, in
    between, on all-zero rows (no active neuron, no overflow: no state of the
    earlier replays may leak into it)."""
    tw = gpu_lib
    T = 2048
    base = make_layer_2b()
    wl = base.rows(0, T)
    dt, x, wg, wu, wd = to_device(wl)
    hy = tw.Hybrid.empty(T, wl.F, wl.tile_w, wl.cap, dt, T)
    hy_e = tw.Hybrid.empty(T, wl.F, wl.tile_w, wl.cap, dt, T)
    ws = tw.hybrid_workspace(hy, wl.d)
    ws_e = tw.hybrid_workspace(hy_e, wl.d)
    y = torch.empty((T, wl.d), dtype=torch.float32, device="cuda")
    y_e = torch.empty_like(y)

    def step(xx, h, yy, w):
        tw.twell_pack_gate(xx, wg, h.ell)
        tw.twell_ffn_from_gate(xx, wg, wu, wd, h, yy, w)

    g = _capture(lambda: step(x, hy, y, ws))
    blocks = [torch.from_numpy(np.ascontiguousarray(base.x[b * T:(b + 1) * T])).to("cuda").to(dt) for b in (1, 3, 2)]
    inputs = [("block 1", blocks[0]), ("block 3", blocks[1]), ("zero rows", torch.zeros_like(x)),
              ("block 2", blocks[2])]
    n_ovf = {}
    for name, xb in inputs:
        say(f"case graph batch T={T} {name}")
        x.copy_(xb)
        _poison(hy, y)
        g.replay()
        torch.cuda.synchronize()
        _poison(hy_e, y_e)
        step(xb, hy_e, y_e, ws_e)
        torch.cuda.synchronize()
        n_ovf[name] = _assert_same(hy, y, hy_e, y_e, f"batch {name}")
    assert n_ovf["zero rows"] == 0 and all(n_ovf[k] > 0 for k in ("block 1", "block 3", "block 2"))
