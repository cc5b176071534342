"""Shared test helpers: run the HIP path through the binding and compare it
with the oracle.  Imported by the test modules only."""

from __future__ import annotations

import sys

import numpy as np

import oracle

# y tolerance: per row, ||y_gpu - y_ref||_2 <= 1e-2 ||y_ref||_2 against the oracle's
# exact-h sum (bf16 inputs, fp32 accumulation); rows without actives exactly 0.
Y_RTOL = 1e-2
# Tighter check against the oracle's stored-h sum for TwELL rows: the only
# differences left are fp32 rounding and summation order in the fused step.
Y_RTOL_STORED = 1e-4


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(wl):
    import torch
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    dev = "cuda"
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device=dev).to(dt)  # noqa: E731
    return dt, f(wl.x), f(wl.wg_t), f(wl.wu_t), f(wl.wd)


def _offset_views(hy, dt):
    """Re-point the TwELL buffers at views that start one element into larger
    allocations (val: 2 or 4 bytes, idx: 1 byte, cnt: 4 bytes off 16-byte
    alignment), so the kernels' scalar (unaligned) paths run."""
    import torch
    ell = hy.ell
    nv = ell.val.numel()
    ell.val = torch.empty(nv + 8, dtype=dt, device="cuda")[1:1 + nv].view(ell.val.shape)
    ell.idx = torch.empty(nv + 16, dtype=torch.uint8, device="cuda")[1:1 + nv].view(ell.idx.shape)
    nc = ell.cnt.numel()
    ell.cnt = torch.empty(nc + 4, dtype=torch.int32, device="cuda")[1:1 + nc].view(ell.cnt.shape)


def _poison(hy, T, d):
    import torch
    hy.ell.cnt.fill_(-7)
    hy.ell.idx.fill_(0xAB)
    hy.ell.val.fill_(-3.0)
    hy.row_ovf.fill_(-7)
    hy.n_ovf.fill_(-7)
    hy.order.fill_(-7)
    return torch.full((T, d), float("nan"), dtype=torch.float32, device="cuda")


def _check_forward(hy, y, hy1, y1, m):
    """twell_ffn_forward's (or pack_gate + twell_ffn_from_gate's) outputs equal
    the separate calls' bit for bit."""
    import torch
    for name, a, b in (("cnt", hy.ell.cnt, hy1.ell.cnt), ("idx", hy.ell.idx, hy1.ell.idx),
                       ("val", hy.ell.val, hy1.ell.val), ("row_ovf", hy.row_ovf, hy1.row_ovf),
                       ("n_ovf", hy.n_ovf, hy1.n_ovf), ("order", hy.order, hy1.order),
                       ("ovf_rows", hy.ovf_rows[:m], hy1.ovf_rows[:m]), ("dense", hy.dense[:m], hy1.dense[:m])):
        assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), \
            f"twell_ffn_forward differs from the separate calls in {name}"
    assert torch.equal(y.view(torch.int32), y1.view(torch.int32)), \
        "twell_ffn_forward differs from the separate calls in y"


def run_hip(wl, max_ovf=None, stream=None, unaligned=False):
    """Run pack_gate_hybrid + ffn_hybrid and (separately) ffn_fused; return host arrays.
    Also runs twell_ffn_forward into fresh buffers and checks that it writes the
    same bits as pack_gate_hybrid + ffn_hybrid."""
    import torch
    import unstructured_sparse_transformer_amd as tw
    dt, x, wg, wu, wd = to_device(wl)
    if max_ovf is None:
        max_ovf = wl.T
    hy = tw.Hybrid.empty(wl.T, wl.F, wl.tile_w, wl.cap, dt, max_ovf)
    if unaligned:
        _offset_views(hy, dt)
    # poison the outputs so stale memory cannot pass a check
    hy.ell.cnt.fill_(-7)
    hy.ell.idx.fill_(0xAB)
    hy.ell.val.fill_(-3.0)
    hy.row_ovf.fill_(-7)
    hy.n_ovf.fill_(-7)
    hy.order.fill_(-7)
    y = torch.full((wl.T, wl.d), float("nan"), dtype=torch.float32, device="cuda")
    yf = torch.full((wl.T, wl.d), float("nan"), dtype=torch.float32, device="cuda")
    yo = torch.full((wl.T, wl.d), float("nan"), dtype=torch.float32, device="cuda")
    ws = tw.hybrid_workspace(max_ovf, wl.F, wl.d, dt)
    tw.twell_pack_gate_hybrid(x, wg, hy, stream)
    tw.twell_ffn_hybrid(hy, x, wu, wd, y, ws, stream)
    tw.twell_ffn_fused(hy.ell, x, wu, wd, yf, stream)                 # ascending rows
    tw.twell_ffn_fused(hy.ell, x, wu, wd, yo, stream, order=hy.order)  # work order
    hy2 = tw.Hybrid.empty(wl.T, wl.F, wl.tile_w, wl.cap, dt, max_ovf)
    if unaligned:
        _offset_views(hy2, dt)
    y2 = _poison(hy2, wl.T, wl.d)
    tw.twell_ffn_forward(x, wg, wu, wd, hy2, y2, tw.hybrid_workspace(max_ovf, wl.F, wl.d, dt), stream)
    hy3 = tw.Hybrid.empty(wl.T, wl.F, wl.tile_w, wl.cap, dt, max_ovf)
    y3 = _poison(hy3, wl.T, wl.d)
    tw.twell_pack_gate(x, wg, hy3.ell, stream)
    tw.twell_ffn_from_gate(x, wg, wu, wd, hy3, y3, tw.hybrid_workspace(max_ovf, wl.F, wl.d, dt), stream)
    torch.cuda.synchronize()
    n_ovf = int(hy.n_ovf.item())
    m = min(n_ovf, max_ovf)
    _check_forward(hy2, y2, hy, y, m)
    _check_forward(hy3, y3, hy, y, m)
    return {
        "cnt": hy.ell.cnt.cpu().numpy(),
        "val": hy.ell.val.float().cpu().numpy(),
        "idx": hy.ell.idx.cpu().numpy(),
        "row_ovf": hy.row_ovf.cpu().numpy(),
        "n_ovf": n_ovf,
        "ovf_rows": hy.ovf_rows[:m].cpu().numpy(),
        "dense": hy.dense[:m].float().cpu().numpy(),
        "y": y.cpu().numpy(),
        "y_fused": yf.cpu().numpy(),
        "y_fused_order": yo.cpu().numpy(),
        "order": hy.order.cpu().numpy(),
        "max_ovf": max_ovf,
    }


def run_decode(wl, max_ovf=None, stream=None, unaligned=False, calls=1):
    """Run twell_ffn_decode `calls` times (poisoned outputs and workspace before
    the first); return host arrays of the last call plus every call's y."""
    import torch
    import unstructured_sparse_transformer_amd as tw
    dt, x, wg, wu, wd = to_device(wl)
    if max_ovf is None:
        max_ovf = wl.T
    hy = tw.Hybrid.empty(wl.T, wl.F, wl.tile_w, wl.cap, dt, max_ovf)
    if unaligned:
        _offset_views(hy, dt)
    hy.ell.cnt.fill_(-7)
    hy.ell.idx.fill_(0xAB)
    hy.ell.val.fill_(-3.0)
    hy.row_ovf.fill_(-7)
    hy.n_ovf.fill_(-7)
    hy.order.fill_(-7)
    if max_ovf:
        hy.ovf_rows.fill_(-7)
        hy.dense.fill_(-5.0)
    ws = tw.decode_workspace(wl.T, wl.F, wl.d, wl.tile_w)
    ws.fill_(0xCD)  # content is ignored on entry
    ys = []
    for _ in range(calls):
        y = torch.full((wl.T, wl.d), float("nan"), dtype=torch.float32, device="cuda")
        tw.twell_ffn_decode(x, wg, wu, wd, hy, y, ws, stream)
        ys.append(y)
    torch.cuda.synchronize()
    n_ovf = int(hy.n_ovf.item())
    m = min(n_ovf, max_ovf)
    return {
        "cnt": hy.ell.cnt.cpu().numpy(),
        "val": hy.ell.val.float().cpu().numpy(),
        "idx": hy.ell.idx.cpu().numpy(),
        "row_ovf": hy.row_ovf.cpu().numpy(),
        "n_ovf": n_ovf,
        "ovf_rows": hy.ovf_rows[:m].cpu().numpy(),
        "dense": hy.dense[:m].float().cpu().numpy(),
        "y": ys[-1].cpu().numpy(),
        "ys": [a.cpu().numpy() for a in ys],
        "order": hy.order.cpu().numpy(),
        "max_ovf": max_ovf,
    }


def compare_decode(wl, out, label=""):
    """TwELL, partition, dense backup and order as for the batch path; every
    row of y (overflow rows included) within Y_RTOL of the exact-h oracle and
    within Y_RTOL_STORED of the stored-h oracle; repeated calls bit-identical."""
    ref = compare(wl, out, check_y=False, label=label)
    y = out["y"].astype(np.float64)
    assert np.isfinite(y).all(), f"{label}: non-finite y"
    num, den = row_rel_err(y, ref.y_exact)
    zero = den == 0
    assert not y[zero].any(), f"{label}: rows without actives must be exactly 0"
    bad = ~zero & (num > Y_RTOL * den)
    assert not bad.any(), f"{label}: y rows off by more than {Y_RTOL}: {np.nonzero(bad)[0][:10]}"
    num2, den2 = row_rel_err(y, ref.y_stored)
    nz = den2 > 0
    assert (num2[nz] <= Y_RTOL_STORED * den2[nz]).all(), \
        f"{label}: y vs stored-h oracle: max rel {np.max(num2[nz] / den2[nz]):.3g}"
    for k, yk in enumerate(out["ys"][:-1]):
        np.testing.assert_array_equal(yk, out["y"], err_msg=f"{label}: call {k} differs from the last call")
    return ref


# Work classes of the fused step's schedule (the C header's definition):
# stored entries e >= 256, 192..255, 128..191, 64..127, 32..63, 16..31, 1..15, 0.
WORK_EDGES = (1, 16, 32, 64, 128, 192, 256)
ORDER_CHUNK = 16384


def check_order(wl, out, label=""):
    """hy.order: a permutation of the rows; per chunk of 16384 rows, work
    classes from the heaviest, ascending rows inside a class."""
    cnt = out["cnt"]
    ovf = (cnt > wl.cap).any(1)
    e = np.where(ovf, 0, np.minimum(cnt, wl.cap).sum(1))
    cls = np.searchsorted(np.array(WORK_EDGES), e, side="right")
    order = out["order"]
    assert np.array_equal(np.sort(order), np.arange(wl.T)), f"{label}: order is not a permutation"
    for c0 in range(0, wl.T, ORDER_CHUNK):
        rows = np.arange(c0, min(wl.T, c0 + ORDER_CHUNK))
        want = rows[np.lexsort((rows, -cls[rows]))]
        np.testing.assert_array_equal(order[rows], want, err_msg=f"{label}: work order")


def row_rel_err(a, b):
    num = np.linalg.norm(a - b, axis=1)
    den = np.linalg.norm(b, axis=1)
    return num, den


def compare(wl, out, ref=None, rows=None, check_y=True, label=""):
    """Assert GPU == oracle: TwELL bit-exact (counts, kept indices and values),
    partition and dense backup exact, y within the stated tolerance."""
    if ref is None:
        ref = oracle.reference(wl, rows)
    rows = ref.rows
    cnt = out["cnt"][rows]
    np.testing.assert_array_equal(cnt, ref.tw.cnt, err_msg=f"{label}: TwELL counts")
    # kept slots and the zero padding past min(cnt, cap), bit for bit
    np.testing.assert_array_equal(out["idx"][rows], ref.tw.idx, err_msg=f"{label}: TwELL indices")
    np.testing.assert_array_equal(out["val"][rows], ref.tw.val.astype(np.float32),
                                  err_msg=f"{label}: TwELL values")
    np.testing.assert_array_equal(out["row_ovf"][rows], ref.row_ovf, err_msg=f"{label}: row_ovf")
    check_order(wl, out, label)
    # the overflow list is a property of all rows: it must be exactly the ascending list
    # of rows whose GPU counts exceed cap (checked against the oracle's flags on `rows`)
    all_ovf = np.nonzero((out["cnt"] > wl.cap).any(1))[0]
    assert out["n_ovf"] == len(all_ovf), f"{label}: n_ovf {out['n_ovf']} vs {len(all_ovf)}"
    m = min(out["n_ovf"], out["max_ovf"])
    np.testing.assert_array_equal(out["ovf_rows"], all_ovf[:m], err_msg=f"{label}: ovf_rows")
    # dense backup rows for the overflow rows covered by `rows`
    pos = {int(t): i for i, t in enumerate(out["ovf_rows"])}
    for li in ref.ovf_local:
        t = int(rows[li])
        if t in pos:
            want = oracle.dense_backup(ref.z[li:li + 1], [0], wl.dtype)[0]
            np.testing.assert_array_equal(out["dense"][pos[t]], want.astype(np.float32),
                                          err_msg=f"{label}: dense backup row {t}")
    if not check_y:
        return ref
    y = out["y"][rows].astype(np.float64)
    yf = out["y_fused"][rows].astype(np.float64)
    assert np.isfinite(y).all() and np.isfinite(yf).all(), f"{label}: non-finite y"
    covered = np.array([(int(t) in pos) or not ref.row_ovf[i] for i, t in enumerate(rows)])
    num, den = row_rel_err(y, ref.y_exact)
    zero = den == 0
    assert not y[zero & covered].any(), f"{label}: rows without actives must be exactly 0"
    bad = covered & ~zero & (num > Y_RTOL * den)
    assert not bad.any(), f"{label}: y rows off by more than {Y_RTOL}: {np.nonzero(bad)[0][:10]} " \
                          f"max rel {np.max(num[~zero] / den[~zero]):.3g}"
    # the work order changes no bits
    np.testing.assert_array_equal(out["y_fused_order"][rows], out["y_fused"][rows],
                                  err_msg=f"{label}: fused result depends on the work order")
    # fused-only: overflow rows are 0, TwELL rows equal the hybrid's TwELL rows bit for bit
    ok = ref.row_ovf == 0
    assert not yf[~ok].any(), f"{label}: fused-only output must zero overflow rows"
    np.testing.assert_array_equal(yf[ok], y[ok], err_msg=f"{label}: fused vs hybrid TwELL rows")
    num2, den2 = row_rel_err(yf[ok], ref.y_stored[ok])
    nz = den2 > 0
    tight = num2[nz] <= Y_RTOL_STORED * den2[nz]
    assert tight.all(), f"{label}: fused y vs stored-h oracle: max rel {np.max(num2[nz] / den2[nz]):.3g}"
    return ref
