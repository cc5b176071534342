"""Shared test helpers: run the HIP path through the binding and compare it
with the oracle.  Imported by the test modules only."""

from __future__ import annotations

import sys

import numpy as np

import oracle
from workloads import bf16_representable

# y tolerance: per row, ||y_gpu - y_ref||_2 <= 1e-2 ||y_ref||_2 against the oracle's
# exact-h sum (bf16 inputs, fp32 accumulation); rows without actives exactly 0.
Y_RTOL = 1e-2
# Tighter check against the oracle's stored-h sum for TwELL rows: the only
# differences left are fp32 rounding and summation order in the fused step.
Y_RTOL_STORED = 1e-4


def grid_ok(wl):
    """The exactness grid: every product x_k (W_g)_jk is a multiple of 2^-17 and
    every partial sum of x_t . w_j stays below 2^7, so the gate's fp32 sums are
    exact in any order.

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
    ws = tw.hybrid_workspace(hy, wl.d)
    tw.twell_pack_gate_hybrid(x, wg, hy, stream)
    tw.twell_ffn_hybrid(hy, x, wu, wd, y, ws, stream)
    tw.twell_ffn_fused(hy.ell, x, wu, wd, yf, ws, stream)                 # ascending rows
    tw.twell_ffn_fused(hy.ell, x, wu, wd, yo, ws, stream, order=hy.order)  # work order
    hy2 = tw.Hybrid.empty(wl.T, wl.F, wl.tile_w, wl.cap, dt, max_ovf)
    if unaligned:
        _offset_views(hy2, dt)
    y2 = _poison(hy2, wl.T, wl.d)
    tw.twell_ffn_forward(x, wg, wu, wd, hy2, y2, tw.hybrid_workspace(hy2, wl.d), stream)
    hy3 = tw.Hybrid.empty(wl.T, wl.F, wl.tile_w, wl.cap, dt, max_ovf)
    y3 = _poison(hy3, wl.T, wl.d)
    tw.twell_pack_gate(x, wg, hy3.ell, stream)
    tw.twell_ffn_from_gate(x, wg, wu, wd, hy3, y3, tw.hybrid_workspace(hy3, wl.d), stream)
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
    row of y (overflow rows included) against the exact-h oracle as in
    check_y and within Y_RTOL_STORED of the stored-h oracle; repeated calls
    bit-identical."""
    ref = compare(wl, out, ref=oracle.reference(wl), check_y=False, label=label)
    y = out["y"].astype(np.float64)
    r_inf, r_bound = check_y_rows(wl, y, ref, np.ones(wl.T, bool), label)
    say(f"  {label}: max |dy| {r_inf:.2e} of ||y_ref||_inf, {r_bound:.2f} of the rounding bound")
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


# Elementwise y tolerance against ||y_ref,t||_inf (reported, and asserted).
Y_INF_RTOL = 1e-2


def y_elem_bound(wl, z, x, band=None):
    """Per-element bound on |y_gpu - y_exact| for rows x with exact gate z.

    Each term of y_t[k] is h_j u_j W_d[j,k] over the active neurons j.  On the
    GPU, h is the gate's fp32 sum (off by at most `band`, 0 on the exactness
    grid) stored in the activation type (unit us: 2^-8 for bf16, 2^-24 for
    fp32), so e_h = us (|h| + band) + band; u is an fp32 sum of d products, off
    by e_u = gamma(d) sum_k |x_k W_u[j,k]|; the product h*u, its rounding to the
    activation type in the overflow rows' dense GEMM, and the fp32 sum over up
    to F terms in any order multiply each term by at most 1 + c,
    c = (1 + us)(1 + 2^-23)(1 + gamma(F)) - 1.  Entries inside the tie band
    (|z| <= band) may be active on one side only; they are included with
    their true h (0 when z <= 0).  Then
        |dy_k| <= sum_j |W_d[j,k]| ((1 + c)(|h_j| + e_h)(|u_j| + e_u) - |h_j| |u_j|).
    """
    import scipy.sparse as sp
    us = 2.0 ** -8 if wl.dtype == "bf16" else 2.0 ** -24
    c = (1 + us) * (1 + 2.0 ** -23) * (1 + oracle.gamma(wl.F)) - 1
    act = z > 0
    if band is not None:
        act = act | (np.abs(z) <= band)
    t, j = np.nonzero(act)
    h = np.where(z[t, j] > 0, z[t, j], 0.0)
    u = np.empty(len(t))
    ua = np.empty(len(t))
    for a in range(0, len(t), 8192):  # u and sum|x w_u| per entry, in chunks
        xa = x[t[a:a + 8192]].astype(np.float64)
        wa = wl.wu_t[j[a:a + 8192]].astype(np.float64)
        u[a:a + 8192] = np.einsum("ij,ij->i", xa, wa)
        ua[a:a + 8192] = np.einsum("ij,ij->i", np.abs(xa), np.abs(wa))
    bj = band[t, j] if band is not None else 0.0
    e_h = us * (h + bj) + bj
    e_u = oracle.gamma(wl.d) * ua
    wts = (1 + c) * (h + e_h) * (np.abs(u) + e_u) - h * np.abs(u)
    m = sp.csr_matrix((wts, (t, j)), shape=z.shape)
    return np.asarray(m @ np.abs(wl.wd.astype(np.float64)))


def check_y_rows(wl, y, ref, covered, label, band=None):
    """y rows (fused, hybrid or decode) against the exact-h oracle: rows without
    actives exactly 0, per row ||dy||_2 <= Y_RTOL ||y_ref||_2, every element
    within the bound of y_elem_bound, and max |dy| <= Y_INF_RTOL ||y_ref||_inf.
    Returns (max |dy| / ||y_ref||_inf, max |dy| / bound)."""
    y = np.asarray(y, np.float64)
    assert np.isfinite(y).all(), f"{label}: non-finite y"
    num, den = row_rel_err(y, ref.y_exact)
    zero = den == 0
    assert not y[zero & covered].any(), f"{label}: rows without actives must be exactly 0"
    bad = covered & ~zero & (num > Y_RTOL * den)
    assert not bad.any(), f"{label}: y rows off by more than {Y_RTOL}: {np.nonzero(bad)[0][:10]} " \
                          f"max rel {np.max(num[~zero] / den[~zero]):.3g}"
    rows = covered & ~zero
    if not rows.any():
        return 0.0, 0.0
    err = np.abs(y[rows] - ref.y_exact[rows])
    bound = y_elem_bound(wl, ref.z[rows], wl.x[ref.rows[rows]], None if band is None else band[rows])
    over = err > bound
    assert not over.any(), f"{label}: y elements beyond the rounding bound: rows " \
                           f"{ref.rows[rows][np.nonzero(over.any(1))[0][:10]]}, max err/bound {np.max(err / np.maximum(bound, 1e-300)):.3g}"
    inf = np.abs(ref.y_exact[rows]).max(1)
    ratio = err.max(1) / inf
    assert (ratio <= Y_INF_RTOL).all(), f"{label}: max |dy| / ||y_ref||_inf = {ratio.max():.3g} > {Y_INF_RTOL}"
    with np.errstate(invalid="ignore", divide="ignore"):
        used = np.where(bound > 0, err / bound, 0.0).max()
    return float(ratio.max()), float(used)


def compare(wl, out, ref=None, rows=None, check_y=True, label="", y_rows=None):
    """Assert GPU == oracle: TwELL bit-exact (counts, kept indices and values),
    partition and dense backup exact, y within the stated tolerance.

    With y_rows, TwELL, flags, overflow list and dense backup are compared on
    `rows` (all rows by default) and y on y_rows only."""
    if ref is None:
        ref = oracle.reference(wl, rows, with_y=y_rows is None and check_y)
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
    ref_y = ref if y_rows is None else oracle.reference(wl, y_rows)
    rows = ref_y.rows
    y = out["y"][rows].astype(np.float64)
    yf = out["y_fused"][rows].astype(np.float64)
    assert np.isfinite(yf).all(), f"{label}: non-finite fused y"
    covered = np.array([(int(t) in pos) or not ref_y.row_ovf[i] for i, t in enumerate(rows)])
    r_inf, r_bound = check_y_rows(wl, y, ref_y, covered, label)
    say(f"  {label}: y rows {len(rows)}, max |dy| {r_inf:.2e} of ||y_ref||_inf, {r_bound:.2f} of the rounding bound")
    # the work order changes no bits
    np.testing.assert_array_equal(out["y_fused_order"][rows], out["y_fused"][rows],
                                  err_msg=f"{label}: fused result depends on the work order")
    # fused-only: overflow rows are 0, TwELL rows equal the hybrid's TwELL rows bit for bit
    ok = ref_y.row_ovf == 0
    assert not yf[~ok].any(), f"{label}: fused-only output must zero overflow rows"
    np.testing.assert_array_equal(yf[ok], y[ok], err_msg=f"{label}: fused vs hybrid TwELL rows")
    num2, den2 = row_rel_err(yf[ok], ref_y.y_stored[ok])
    nz = den2 > 0
    tight = num2[nz] <= Y_RTOL_STORED * den2[nz]
    assert tight.all(), f"{label}: fused y vs stored-h oracle: max rel {np.max(num2[nz] / den2[nz]):.3g}"
    return ref


# ---------------------------------------------------------------- continuous mode (off the exactness grid)
def tie_band(wl, x):
    """Per (row, neuron): the largest possible difference between the GPU's
    fp32 gate sum (any order, any rounding mode: unit 2^-23, d + 2 terms to
    cover the rounding of fp32 products) and the oracle's fp64 z (its own
    error included).  0 for dead neurons (z = -inf on both sides)."""
    wg = np.where(np.isfinite(wl.wg_t), wl.wg_t, 0.0)
    g = oracle.abs_sums(x, wg)
    band = (oracle.gamma(wl.d + 2) + oracle.gamma(wl.d, 2.0 ** -52)) * g
    dead = ~np.isfinite(wl.wg_t).all(1)
    band[:, dead] = 0.0
    return band


def _ulp(v, dtype):
    """Spacing of the storage type at |v| (bf16: 8 significant bits, fp32: 24)."""
    _, e = np.frexp(np.abs(v))
    return np.ldexp(1.0, e - (8 if dtype == "bf16" else 24))


def compare_continuous(wl, out, label="", fused=True):
    """GPU results on continuous (off-grid) inputs against the exact oracle.

    Let band = tie_band, D = {z > band} (active in any summation order) and
    M = {|z| <= band} (active or not, depending on the order).  Required:
    every kept TwELL entry lies in D or M, in ascending column order, with zero
    padding; each tile's count lies in [|D|, |D| + |M|]; a tile that fits keeps
    all of D, an overflowing tile every D column below its last kept one; each
    kept value is bf16 (fp32) of a sum within band of z, i.e. within
    us (|z| + band) + band of z, and within 1 ulp of the oracle's stored value
    where band < us/2 |z|; flags, list and order consistent with the GPU's own
    counts; dense backup rows 0 where z < -band and within the same value bound
    elsewhere; y as in check_y_rows with the band's entries in the bound.
    Returns the counts of entries whose activity or stored value differs from
    the oracle's (reported, not required to be 0)."""
    ref = oracle.reference(wl)
    z, T, F, w, cap = ref.z, wl.T, wl.F, wl.tile_w, wl.cap
    nb = F // w
    us = 2.0 ** -8 if wl.dtype == "bf16" else 2.0 ** -24
    band = tie_band(wl, wl.x)
    D = z > band
    M = np.abs(z) <= band
    cnt, idx, val = out["cnt"], out["idx"], out["val"]
    kept = np.arange(cap)[None, None, :] < np.minimum(cnt, cap)[:, :, None]
    assert (cnt >= 0).all(), f"{label}: negative counts"
    assert not idx[~kept].any() and not val[~kept].any(), f"{label}: TwELL padding not zero"
    if cap > 1:
        asc = (np.diff(idx.astype(np.int32), axis=2) > 0) | ~kept[:, :, 1:]
        assert asc.all(), f"{label}: kept indices not ascending"
    t, b, s = np.nonzero(kept)
    col = b * w + idx[t, b, s].astype(np.int64)
    K = np.zeros((T, F), bool)
    K[t, col] = True
    assert (D | M)[t, col].all(), f"{label}: a kept entry is inactive in every summation order"
    Dt = D.reshape(T, nb, w).sum(2)
    Mt = M.reshape(T, nb, w).sum(2)
    assert ((cnt >= Dt) & (cnt <= Dt + Mt)).all(), f"{label}: a tile count is outside [|D|, |D| + |M|]"
    missing = (D & ~K).reshape(T, nb, w)
    fit = cnt <= cap
    assert not missing[fit].any(), f"{label}: a fitting tile lost a certain active"
    if (~fit).any():
        last = np.full((T, nb), -1, np.int64)
        np.maximum.at(last, (t, b), idx[t, b, s].astype(np.int64))
        below = np.arange(w)[None, None, :] < last[:, :, None]
        assert not (missing & below & ~fit[:, :, None]).any(), \
            f"{label}: an overflowing tile skipped a certain active below its last kept column"
    v = val[t, b, s].astype(np.float64)
    zk, bk = z[t, col], band[t, col]
    assert (np.abs(v - zk) <= us * (np.abs(zk) + bk) + bk).all(), f"{label}: TwELL value beyond the band bound"
    vo = oracle.store_round(zk, wl.dtype)
    safe = bk < 0.5 * us * np.abs(zk)
    assert (np.abs(v - vo) <= _ulp(np.maximum(np.abs(v), np.abs(vo)), wl.dtype))[safe].all(), \
        f"{label}: a TwELL value is more than 1 ulp from the oracle's where the band allows none"
    # partition and order from the GPU's own counts
    ovf_gpu = (cnt > cap).any(1)
    np.testing.assert_array_equal(out["row_ovf"], ovf_gpu.astype(out["row_ovf"].dtype),
                                  err_msg=f"{label}: row_ovf vs the GPU's counts")
    check_order(wl, out, label)
    all_ovf = np.nonzero(ovf_gpu)[0]
    assert out["n_ovf"] == len(all_ovf), f"{label}: n_ovf"
    m = min(out["n_ovf"], out["max_ovf"])
    np.testing.assert_array_equal(out["ovf_rows"], all_ovf[:m], err_msg=f"{label}: ovf_rows")
    if m:
        r = out["ovf_rows"]
        dv = out["dense"].astype(np.float64)
        zr, br = z[r], band[r]
        assert not dv[zr < -br].any(), f"{label}: dense backup nonzero where every order gives z < 0"
        amb = zr >= -br
        assert (np.abs(dv - np.maximum(zr, 0.0)) <= us * (np.abs(zr) + br) + br)[amb].all(), \
            f"{label}: dense backup value beyond the band bound"
    # y: every row served when max_ovf >= n_ovf
    pos = set(int(q) for q in out["ovf_rows"])
    covered = np.array([(not ovf_gpu[q]) or (q in pos) for q in range(T)])
    y = out["y"].astype(np.float64)
    r_inf, r_bound = check_y_rows(wl, y, ref, covered, label, band=band)
    if fused:
        yf = out["y_fused"]
        assert not yf[ovf_gpu].any(), f"{label}: fused-only output must zero overflow rows"
        np.testing.assert_array_equal(yf[~ovf_gpu], out["y"][~ovf_gpu], err_msg=f"{label}: fused vs hybrid rows")
        np.testing.assert_array_equal(out["y_fused_order"], yf, err_msg=f"{label}: order changes fused bits")
    act_diff = int((K != (z > 0)).reshape(T, nb, w)[fit & (ref.tw.cnt <= cap)].sum())
    stats = {"band_entries": int(M.sum()), "count_diff_tiles": int((cnt != ref.tw.cnt).sum()),
             "activity_diff": act_diff, "value_diff": int((v != vo).sum()), "kept": int(len(v)),
             "ovf_flag_diff": int((ovf_gpu != ref.row_ovf.astype(bool)).sum()),
             "y_inf_ratio": r_inf, "y_bound_use": r_bound}
    say(f"  {label}: continuous mode {stats}")
    return stats
