"""CPU oracle for the ReLU-sparse gated FFN with TwELL packing and the
ELL + dense-backup hybrid.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``, never by the product library.  It
shares no code with the HIP path: plain scalar C loops (``twell_oracle.c``)
plus numpy's fp64 matmul as a library primitive, and pure-Python loops in
``oracle.brute`` for tiny cases.

What each function follows ("Sparser, Faster, Lighter Transformer Language
Models", gist.science summary page):

* ``gate`` / ``up``: the gate and up projections x.W_g and x.W_u of section 2.2.
* ``pack_twell``: section 2.1, ReLU then per-tile packing of nonzeros with
  tile-local indices (readings: active iff z > 0; ascending columns; true count
  kept, first ``cap`` entries stored, on overflow).
* ``partition_overflow`` / ``dense_backup``: section 2.3, rows whose count does
  not fit go to a dense backup matrix (reading: a row overflows iff any tile
  holds more than ``cap`` actives; backup rows in ascending token order).
* ``ffn_dense`` / ``ffn_twell`` / ``ffn_active``: section 2.2, y = (ReLU(x.W_g)
  * x.W_u) . W_d, accumulated over neurons in ascending order in fp64.
* ``gate_stats``: section 2.4's L1 activation penalty and dead neurons, as
  per-neuron active counts and per (row, tile) sums of the active gate values.
* ``ffn_backward``: the gradients of the FFN (section 2.4's training
  kernels), per active (row, neuron) in ascending order.
* ``abs_sums`` / ``gamma``: not results of the method but the magnitudes
  that bound summation-order rounding (the gate's tie band, y's tolerance).
* ``compact_hybrid`` / ``compact_to_dense``: section 2.3's compact storage of
  the hybrid (reading: exact entries per fitting row, dense overflow rows).
* ``hybrid_to_dense``: section 2.4's hybrid-to-dense conversion; the
  dense-to-hybrid direction is ``pack_twell`` + ``partition_overflow`` +
  ``dense_backup`` applied to a dense activation matrix.

Pins (tests/test_oracle.py): pure-Python brute force on tiny inputs, all 2^8
patterns of one 8-wide tile, a hand-worked example (tests/golden), closed forms
(all dead; one active neuron; dense tile; identity up/down), dense == sparse
bitwise, nonzero conservation, round trip, numpy fp64 matmul cross-check,
bf16 rounding against torch's conversion, for ``gate_stats`` brute force,
conservation against the TwELL counts and closed forms (all dead, all active,
one live neuron), for ``hybrid_to_dense`` the exact round trip through the
dense-to-hybrid direction and a hand-built example, and for ``compact_hybrid``
the hand example, the exact round trip and nonzero conservation, and for
``ffn_backward`` central finite differences of an independent numpy forward,
the matrix form with numpy matmuls, and a one-neuron closed form; for
``abs_sums`` pure-Python brute force and the closed form for non-negative
inputs (equal to the dot product itself).
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

VDTYPE = {"exact": -1, "f64": -1, "f32": 0, "bf16": 1}


def load(path: str = None):
    """Use the oracle library at `path` (default oracle/liboracle.so, built
    when missing) for every later call; returns it."""
    global _lib
    _lib = None
    return _load(path)


def set_threads(n: int):
    """Threads of the oracle's OpenMP loops (for timing; results do not depend on it)."""
    _load().orc_set_threads(int(n))


def max_threads() -> int:
    return int(_load().orc_max_threads())


def _load(path: str = None):
    global _lib
    if _lib is not None:
        return _lib
    path = path or _LIB_PATH
    if not os.path.exists(path):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(path)
    lib.orc_set_threads.argtypes = [ctypes.c_int]
    lib.orc_max_threads.restype = ctypes.c_int
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.orc_round_array.argtypes = [P, ctypes.c_int64, I, P]
    lib.orc_matmul_nt_rows.argtypes = [P, P, I, P, I, I, P]
    lib.orc_pack_twell.argtypes = [P, I, I, I, I, I, P, P, P]
    lib.orc_partition.argtypes = [P, I, I, I, P, P]
    lib.orc_partition.restype = I
    lib.orc_ffn_dense.argtypes = [P, P, P, I, I, I, I, P]
    lib.orc_gate_stats.argtypes = [P, I, I, I, P, P]
    lib.orc_ffn_backward.argtypes = [P, I, I, P, P, P, P, I, I, P, P, P, P, P]
    lib.orc_ffn_twell.argtypes = [P, P, P, I, I, I, I, P, P, P, I, I, P]
    lib.orc_ffn_active.argtypes = [P, I, I, P, P, P, I, I, P]
    _lib = lib
    return lib


def _p(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def _vd(v) -> int:
    if v is None:
        return -1
    return VDTYPE[v] if isinstance(v, str) else int(v)


# ---------------------------------------------------------------- projections
def gate(x: np.ndarray, wg_t: np.ndarray) -> np.ndarray:
    """z = x . W_g in fp64 (numpy matmul).  Exact for grid-mode inputs."""
    return _c(x, np.float64) @ _c(wg_t, np.float64).T


def up(x: np.ndarray, wu_t: np.ndarray) -> np.ndarray:
    """u = x . W_u in fp64 (numpy matmul)."""
    return _c(x, np.float64) @ _c(wu_t, np.float64).T


def abs_sums(x: np.ndarray, w_t: np.ndarray) -> np.ndarray:
    """M[t][j] = sum_k |x[t][k] * w_t[j][k]| in fp64 (numpy matmul of the
    absolute values).  Not a result of the method: it is the magnitude that
    bounds the rounding error of the dot product x[t] . w_t[j] in any
    summation order, |fl(x.w) - x.w| <= gamma(d) * M, gamma(n) = n u / (1 - n u)
    for unit roundoff u.  With W_g it is the tie band of the gate: an entry
    with |z| <= gamma(d) M may be active in one summation order and not in
    another."""
    return np.abs(_c(x, np.float64)) @ np.abs(_c(w_t, np.float64)).T


def gamma(n: int, unit: float = 2.0 ** -23) -> float:
    """n u / (1 - n u): the relative error bound of an n-term sum in floating
    point of unit roundoff u (default 2^-23, fp32 with any rounding mode)."""
    return n * unit / (1.0 - n * unit)


def matmul_rows(a: np.ndarray, rows, b_t: np.ndarray) -> np.ndarray:
    """out[r][j] = a[rows[r]] . b_t[j], fp64 scalar loops, ascending k."""
    lib = _load()
    a = _c(a, np.float32)
    b_t = _c(b_t, np.float32)
    rows = _c(np.asarray(rows), np.int32)
    out = np.empty((len(rows), b_t.shape[0]), np.float64)
    lib.orc_matmul_nt_rows(_p(a), _p(rows), len(rows), _p(b_t), b_t.shape[0], a.shape[1], _p(out))
    return out


def store_round(a: np.ndarray, vdtype) -> np.ndarray:
    """Values as held in storage of type vdtype ('f32', 'bf16' or 'exact')."""
    lib = _load()
    a = _c(a, np.float64)
    out = np.empty_like(a)
    lib.orc_round_array(_p(a), a.size, _vd(vdtype), _p(out))
    return out


# ---------------------------------------------------------------- TwELL
@dataclass
class TwELL:
    T: int
    F: int
    tile_w: int
    cap: int
    cnt: np.ndarray  # int32 [T][n_b], true counts
    val: np.ndarray  # float64 [T][n_b][cap], stored values, 0 in unused slots
    idx: np.ndarray  # uint8 [T][n_b][cap], tile-local columns, 0 in unused slots

    @property
    def n_b(self) -> int:
        return self.F // self.tile_w

    def kept(self) -> np.ndarray:
        """bool [T][n_b][cap]: slot s holds an entry iff s < min(cnt, cap)."""
        m = np.minimum(self.cnt, self.cap)
        return np.arange(self.cap)[None, None, :] < m[:, :, None]


def pack_twell(z: np.ndarray, tile_w: int, cap: int, vdtype) -> TwELL:
    lib = _load()
    z = _c(z, np.float64)
    T, F = z.shape
    assert F % tile_w == 0 and 1 <= cap <= tile_w <= 256
    n_b = F // tile_w
    cnt = np.empty((T, n_b), np.int32)
    val = np.empty((T, n_b, cap), np.float64)
    idx = np.empty((T, n_b, cap), np.uint8)
    lib.orc_pack_twell(_p(z), T, F, tile_w, cap, _vd(vdtype), _p(cnt), _p(val), _p(idx))
    return TwELL(T, F, tile_w, cap, cnt, val, idx)


def gate_stats(z: np.ndarray, tile_w: int):
    """Activation statistics of the gate (section 2.4's L1 activation penalty
    and dead neurons): per-neuron count of rows with z > 0 ([F] int64) and per
    (row, tile) sum of the active z values ([T][n_b] fp64, before rounding)."""
    lib = _load()
    z = _c(z, np.float64)
    T, F = z.shape
    cnt = np.zeros(F, dtype=np.int64)
    l1 = np.zeros((T, F // tile_w), dtype=np.float64)
    lib.orc_gate_stats(_p(z), T, F, tile_w, _p(cnt), _p(l1))
    return cnt, l1


def unpack_twell(tw: TwELL) -> np.ndarray:
    """Dense [T][F] array holding the kept entries (0 elsewhere)."""
    out = np.zeros((tw.T, tw.F), np.float64)
    kept = tw.kept()
    t, b, s = np.nonzero(kept)
    out[t, b * tw.tile_w + tw.idx[t, b, s].astype(np.int64)] = tw.val[t, b, s]
    return out


def hybrid_to_dense(tw: TwELL, ovf_rows, dense, max_ovf: int) -> np.ndarray:
    """Section 2.4's hybrid-to-dense conversion: [T][F] holding the TwELL
    entries of every row, with the first max_ovf overflow rows replaced by
    their dense backup rows (later overflow rows keep only their TwELL
    entries: the hybrid holds nothing more of them)."""
    out = unpack_twell(tw)
    for i, t in enumerate(np.asarray(ovf_rows)[:max_ovf]):
        out[int(t)] = np.asarray(dense[i], np.float64)
    return out


def compact_hybrid(tw: TwELL, row_ovf, ovf_rows, dense, max_ovf: int) -> dict:
    """Compacted hybrid storage (section 2.3: the sparse part stored compactly,
    the dense part sized by the rows that need it), in the reading of this
    library: the rows that fit keep exactly their entries, row by row in
    ascending column order (row_ptr [T+1], global column, value: no slot
    padding), overflow rows keep none there; the overflow rows are listed in
    ascending order with their dense rows (the first max_ovf of them held)."""
    T = tw.T
    row_ptr = np.zeros(T + 1, np.int64)
    cols, vals = [], []
    kept = tw.kept()
    for t in range(T):
        if not row_ovf[t]:
            b, sl = np.nonzero(kept[t])
            c = b * tw.tile_w + tw.idx[t, b, sl].astype(np.int64)
            cols.extend(c.tolist())
            vals.extend(tw.val[t, b, sl].tolist())
        row_ptr[t + 1] = len(cols)
    n = len(ovf_rows)
    m = min(n, max_ovf)
    return {"row_ptr": row_ptr, "col": np.asarray(cols, np.int64), "val": np.asarray(vals, np.float64),
            "ovf_rows": np.asarray(ovf_rows, np.int64), "n_ovf": n,
            "dense": np.asarray(dense, np.float64)[:m], "complete": m == n}


def compact_to_dense(c: dict, T: int, F: int) -> np.ndarray:
    """[T][F] from the compacted storage (zeros where nothing is held)."""
    out = np.zeros((T, F), np.float64)
    for t in range(T):
        a, b = c["row_ptr"][t], c["row_ptr"][t + 1]
        out[t, c["col"][a:b]] = c["val"][a:b]
    for i in range(len(c["dense"])):
        out[c["ovf_rows"][i]] = c["dense"][i]
    return out


def partition_overflow(cnt: np.ndarray, cap: int):
    """(row_ovf int32 [T], ovf_rows int32 [n_ovf] ascending, n_ovf)."""
    lib = _load()
    cnt = _c(cnt, np.int32)
    T, n_b = cnt.shape
    row_ovf = np.empty(T, np.int32)
    rows = np.empty(T, np.int32)
    n = lib.orc_partition(_p(cnt), T, n_b, cap, _p(row_ovf), _p(rows))
    return row_ovf, rows[:n].copy(), int(n)


def dense_backup(z: np.ndarray, ovf_rows, vdtype) -> np.ndarray:
    """[n_ovf][F]: stored ReLU(z) rows of the overflow tokens, ascending token order."""
    zr = np.asarray(z, np.float64)[np.asarray(ovf_rows, np.int64)]
    return store_round(np.where(zr > 0.0, zr, 0.0), vdtype)


# ---------------------------------------------------------------- FFN
def ffn_dense(z: np.ndarray, u: np.ndarray, wd: np.ndarray, hround=None) -> np.ndarray:
    lib = _load()
    z = _c(z, np.float64)
    u = _c(u, np.float64)
    wd = _c(wd, np.float32)
    T, F = z.shape
    d = wd.shape[1]
    y = np.empty((T, d), np.float64)
    lib.orc_ffn_dense(_p(z), _p(u), _p(wd), T, F, d, _vd(hround), _p(y))
    return y


def ffn_twell(tw: TwELL, x, wu_t, wd, skip_overflow: bool = True) -> np.ndarray:
    lib = _load()
    x = _c(x, np.float32)
    wu_t = _c(wu_t, np.float32)
    wd = _c(wd, np.float32)
    d = x.shape[1]
    y = np.empty((tw.T, d), np.float64)
    lib.orc_ffn_twell(_p(_c(tw.cnt, np.int32)), _p(_c(tw.val, np.float64)), _p(_c(tw.idx, np.uint8)),
                      tw.T, tw.F, tw.tile_w, tw.cap, _p(x), _p(wu_t), _p(wd), d,
                      1 if skip_overflow else 0, _p(y))
    return y


def ffn_active(z: np.ndarray, x, wu_t, wd, hround=None) -> np.ndarray:
    lib = _load()
    z = _c(z, np.float64)
    x = _c(x, np.float32)
    wu_t = _c(wu_t, np.float32)
    wd = _c(wd, np.float32)
    T, F = z.shape
    d = x.shape[1]
    y = np.empty((T, d), np.float64)
    lib.orc_ffn_active(_p(z), T, F, _p(x), _p(wu_t), _p(wd), d, _vd(hround), _p(y))
    return y


def ffn_backward(z: np.ndarray, x, wg_t, wu_t, wd, dy, hround=None):
    """Gradients (dx [T][d], dW_g^T, dW_u^T, dW_d [F][d], all fp64) of
    sum(y * dy) for the FFN of ``ffn_active``: section 2.4's backward pass,
    with the stored gate value h in the products and ReLU's derivative 1 on
    the active neurons (scalar C loops, ascending rows and neurons)."""
    lib = _load()
    z = _c(z, np.float64)
    x = _c(x, np.float32)
    wg_t, wu_t, wd = _c(wg_t, np.float32), _c(wu_t, np.float32), _c(wd, np.float32)
    dy = _c(dy, np.float64)
    T, F = z.shape
    d = x.shape[1]
    dx = np.empty((T, d), np.float64)
    dwg = np.empty((F, d), np.float64)
    dwu = np.empty((F, d), np.float64)
    dwd = np.empty((F, d), np.float64)
    lib.orc_ffn_backward(_p(z), T, F, _p(x), _p(wg_t), _p(wu_t), _p(wd), d, _vd(hround), _p(dy), _p(dx), _p(dwg),
                         _p(dwu), _p(dwd))
    return dx, dwg, dwu, dwd


def ffn_numpy(x, wg_t, wu_t, wd) -> np.ndarray:
    """Library cross-check: relu(x W_g) * (x W_u) @ W_d with numpy fp64 matmuls."""
    z = gate(x, wg_t)
    return (np.where(z > 0.0, z, 0.0) * up(x, wu_t)) @ _c(wd, np.float64)


# ---------------------------------------------------------------- one layer
@dataclass
class Reference:
    rows: np.ndarray       # token indices the reference covers
    z: np.ndarray          # [R][F] fp64
    tw: TwELL              # TwELL of those rows
    row_ovf: np.ndarray    # [R]
    ovf_local: np.ndarray  # positions (into rows) of overflow rows, ascending
    y_exact: np.ndarray    # [R][d] hybrid y from exact h (all active neurons)
    y_stored: np.ndarray   # [R][d] hybrid y from the stored (rounded) h
    y_fused: np.ndarray    # [R][d] fused-only y: overflow rows 0, stored h


def reference(wl, rows=None, use_blas: bool = True, with_y: bool = True) -> Reference:
    """Everything the path computes for `wl` (a workloads.Workload) on `rows`
    (with_y=False: the gate, TwELL and partition only; the y fields are None)."""
    if rows is None:
        rows = np.arange(wl.T)
    rows = np.asarray(rows, np.int64)
    x = wl.x[rows]
    z = gate(x, wl.wg_t) if use_blas else matmul_rows(x, np.arange(len(rows)), wl.wg_t)
    tw = pack_twell(z, wl.tile_w, wl.cap, wl.dtype)
    row_ovf, ovf_local, _ = partition_overflow(tw.cnt, wl.cap)
    if not with_y:
        return Reference(rows, z, tw, row_ovf, ovf_local, None, None, None)
    y_exact = ffn_active(z, x, wl.wu_t, wl.wd, None)
    y_stored = ffn_active(z, x, wl.wu_t, wl.wd, wl.dtype)
    y_fused = ffn_twell(tw, x, wl.wu_t, wl.wd, skip_overflow=True)
    return Reference(rows, z, tw, row_ovf, ovf_local, y_exact, y_stored, y_fused)
