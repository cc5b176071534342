"""twell_ffn_decode_noalloc (the decode path on the library's static scratch)
against twell_ffn_decode with a caller workspace, on three calls in a row
with shrinking inputs (T = 64, then 8, then 1), so stale scratch contents
from a larger call must not leak into a smaller one.

The no-alloc call keeps the four-kernel decode path (its partial rows fit
the 16 MiB scratch); twell_ffn_decode runs the two-kernel path, whose partial
rows per (row, gate workgroup) need a workspace that grows with T * F / 32 * d.
Both write the same TwELL, flags, overflow list, order and dense backup, bit
for bit; y is the same sum over the same terms in another order, so the two
y agree to fp32 rounding (per row, relative 1e-5) and each meets the
oracle's bar on its own (compare_decode)."""

import numpy as np
import pytest

from helpers import compare_decode, say, to_device
from workloads import make_layer_2b

pytestmark = pytest.mark.gpu


def _window_with_overflow(base, T, skip=()):
    """A window of T consecutive tokens holding the token with the lowest
    jitter value not in `skip` (lowest threshold: the most actives, so the
    window has an overflow row)."""
    order = np.argsort(base.x[:, base.d - 1], kind="stable")
    for t in order:
        i = int(t) // T
        if i not in skip:
            return i
    raise AssertionError("no window")


def _run(tw, wl, noalloc):
    import torch
    dt, x, wg, wu, wd = to_device(wl)
    hy = tw.Hybrid.empty(wl.T, wl.F, wl.tile_w, wl.cap, dt, wl.T)
    hy.ell.cnt.fill_(-7)
    hy.ell.idx.fill_(0xAB)
    hy.ell.val.fill_(-3.0)
    hy.row_ovf.fill_(-7)
    hy.n_ovf.fill_(-7)
    hy.order.fill_(-7)
    hy.ovf_rows.fill_(-7)
    hy.dense.fill_(-5.0)
    y = torch.full((wl.T, wl.d), float("nan"), dtype=torch.float32, device="cuda")
    if noalloc:
        tw.twell_ffn_decode_noalloc(x, wg, wu, wd, hy, y)
    else:
        ws = tw.decode_workspace(wl.T, wl.F, wl.d, wl.tile_w)
        ws.fill_(0xCD)
        tw.twell_ffn_decode(x, wg, wu, wd, hy, y, ws)
    torch.cuda.synchronize()
    return hy, y


def test_noalloc_matches_workspace_call(gpu_lib):
    import torch
    tw = gpu_lib
    base = make_layer_2b()
    for T in (64, 8, 1):
        i = _window_with_overflow(base, T)
        wl = base.rows(i * T, (i + 1) * T)
        say(f"case no-alloc decode T={T} window={i}")
        hy_s, y_s = _run(tw, wl, noalloc=True)
        hy_w, y_w = _run(tw, wl, noalloc=False)
        n = int(hy_w.n_ovf.item())
        m = min(n, wl.T)
        assert int(hy_s.n_ovf.item()) == n, f"T={T}: n_ovf differs"
        for name, a, b in (("cnt", hy_s.ell.cnt, hy_w.ell.cnt), ("idx", hy_s.ell.idx, hy_w.ell.idx),
                           ("val", hy_s.ell.val, hy_w.ell.val), ("row_ovf", hy_s.row_ovf, hy_w.row_ovf),
                           ("order", hy_s.order, hy_w.order), ("ovf_rows", hy_s.ovf_rows[:m], hy_w.ovf_rows[:m]),
                           ("dense", hy_s.dense[:m], hy_w.dense[:m])):
            assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), \
                f"T={T}: twell_ffn_decode_noalloc differs from twell_ffn_decode in {name}"
        ys, yw = y_s.double().cpu().numpy(), y_w.double().cpu().numpy()
        assert np.isfinite(ys).all() and np.isfinite(yw).all(), f"T={T}: non-finite y"
        num = np.linalg.norm(ys - yw, axis=1)
        den = np.linalg.norm(yw, axis=1)
        assert (num <= 1e-5 * den).all() and not ys[den == 0].any(), f"T={T}: y of the two paths differs"
        out = {
            "cnt": hy_s.ell.cnt.cpu().numpy(), "val": hy_s.ell.val.float().cpu().numpy(),
            "idx": hy_s.ell.idx.cpu().numpy(), "row_ovf": hy_s.row_ovf.cpu().numpy(), "n_ovf": n,
            "ovf_rows": hy_s.ovf_rows[:m].cpu().numpy(), "dense": hy_s.dense[:m].float().cpu().numpy(),
            "y": y_s.cpu().numpy(), "ys": [y_s.cpu().numpy()], "order": hy_s.order.cpu().numpy(),
            "max_ovf": wl.T,
        }
        compare_decode(wl, out, label=f"no-alloc T={T}")
        out["y"], out["ys"] = y_w.cpu().numpy(), [y_w.cpu().numpy()]
        compare_decode(wl, out, label=f"workspace T={T}")
        say(f"  n_ovf={n} entries={int(np.minimum(out['cnt'], wl.cap).sum())}: equal")
