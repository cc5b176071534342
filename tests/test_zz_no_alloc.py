"""twell_ffn_decode_noalloc (the decode path on the library's static scratch)
against twell_ffn_decode with a caller workspace, on calls in a row with
shrinking inputs (T = 64, then 8, then 1 at the 2B-like shape; T = 4, then 2
at d = 4096), so stale scratch contents from a larger call must not leak into
a smaller one.

For T <= 16 twell_ffn_decode runs the two-kernel organisation, whose partial
rows per (row, gate workgroup) grow with T * F / 32 * d; the no-alloc call
runs it too when that layout fits its 16 MiB scratch (T = 1 at the 2B-like
shape, both d = 4096 cases), else the chunked kernels (T = 8 there), as both
do for T > 16.  The two calls always write the same TwELL, flags, overflow
list, order and dense backup, bit for bit; y is the same bits when they took
the same kernels, else the same sum over the same terms in another order
(per row, relative 1e-5).  Each meets the oracle's bar on its own
(compare_decode)."""

import numpy as np
import pytest

from helpers import compare_decode, say, to_device
from workloads import make_layer_2b, make_random_small

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


def _same_kernels(wl):
    """Whether the no-alloc call takes twell_ffn_decode's organisation: the
    two-kernel one (T <= 16) needs z, flags and T * F / 32 partial rows of d
    floats in the 16 MiB scratch; for T > 16 both take the chunked kernels."""
    if wl.T > 16:
        return True
    up = lambda b: (b + 255) & ~255  # noqa: E731
    g = wl.F // 32
    return up(wl.T * wl.F * 4) + 256 + up(wl.T * g * 4) + up(wl.T * g * wl.d * 4) <= 16 << 20


def test_noalloc_matches_workspace_call(gpu_lib):
    base = make_layer_2b()
    cases = []
    for T in (64, 8, 1):
        i = _window_with_overflow(base, T)
        cases.append((f"T={T} window={i}", base.rows(i * T, (i + 1) * T)))
    for T in (4, 2):
        cases.append((f"d=4096 T={T}", make_random_small(T, 4096, 1024, 256, 2, "bf16", active_frac=0.1, seed=40 + T,
                                                         jitter=0.5)))
    for name, wl in cases:
        _compare(gpu_lib, name, wl)


def _compare(tw, name, wl):
    import torch
    say(f"case no-alloc decode {name} ({'same kernels' if _same_kernels(wl) else 'chunked kernels'})")
    hy_s, y_s = _run(tw, wl, noalloc=True)
    hy_w, y_w = _run(tw, wl, noalloc=False)
    n = int(hy_w.n_ovf.item())
    m = min(n, wl.T)
    assert int(hy_s.n_ovf.item()) == n, f"{name}: n_ovf differs"
    for key, a, b in (("cnt", hy_s.ell.cnt, hy_w.ell.cnt), ("idx", hy_s.ell.idx, hy_w.ell.idx),
                      ("val", hy_s.ell.val, hy_w.ell.val), ("row_ovf", hy_s.row_ovf, hy_w.row_ovf),
                      ("order", hy_s.order, hy_w.order), ("ovf_rows", hy_s.ovf_rows[:m], hy_w.ovf_rows[:m]),
                      ("dense", hy_s.dense[:m], hy_w.dense[:m])):
        assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), \
            f"{name}: twell_ffn_decode_noalloc differs from twell_ffn_decode in {key}"
    ys, yw = y_s.double().cpu().numpy(), y_w.double().cpu().numpy()
    assert np.isfinite(ys).all() and np.isfinite(yw).all(), f"{name}: non-finite y"
    if _same_kernels(wl):
        assert np.array_equal(ys, yw), f"{name}: y differs from twell_ffn_decode's with the same kernels"
    num = np.linalg.norm(ys - yw, axis=1)
    den = np.linalg.norm(yw, axis=1)
    assert (num <= 1e-5 * den).all() and not ys[den == 0].any(), f"{name}: y of the two paths differs"
    out = {
        "cnt": hy_s.ell.cnt.cpu().numpy(), "val": hy_s.ell.val.float().cpu().numpy(),
        "idx": hy_s.ell.idx.cpu().numpy(), "row_ovf": hy_s.row_ovf.cpu().numpy(), "n_ovf": n,
        "ovf_rows": hy_s.ovf_rows[:m].cpu().numpy(), "dense": hy_s.dense[:m].float().cpu().numpy(),
        "y": y_s.cpu().numpy(), "ys": [y_s.cpu().numpy()], "order": hy_s.order.cpu().numpy(),
        "max_ovf": wl.T,
    }
    compare_decode(wl, out, label=f"no-alloc {name}")
    out["y"], out["ys"] = y_w.cpu().numpy(), [y_w.cpu().numpy()]
    compare_decode(wl, out, label=f"workspace {name}")
    say(f"  n_ovf={n} entries={int(np.minimum(out['cnt'], wl.cap).sum())}: equal")
