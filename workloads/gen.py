"""Deterministic synthetic workloads, on an exact-accumulation grid (the
default, "grid" mode) or off it ("continuous" mode).

Every array is drawn from its own PCG64 stream,
``SeedSequence(0, spawn_key=(workload_id, layer, array_id))``, so changing one
array's shape never shifts another array's numbers.

Grid construction (what makes GPU and CPU agree bit for bit on z = x.W_g):

* x (all columns but the last): ``rint(16 * N(0,1)) / 16`` clipped to |m| <= 127,
  i.e. multiples of 2^-4 with at most 7 significant bits.
* every weight: ``rint(1024 * N(0, 1/d)) / 1024`` clipped to |m| <= 255, i.e.
  multiples of 2^-10 with at most 8 significant bits (exact in bf16).
* the last column of x is a "ones" column (1.0) or a per-token jitter value that
  is a bf16 number >= 2^-3 (so a multiple of 2^-10), and the last column of
  W_g^T holds the per-neuron bias: a bf16 number of magnitude >= 1 (so a
  multiple of 2^-7), or -inf for a dead neuron.
* hence every product x_k * w_k is a multiple of 2^-17; as long as every
  partial sum stays below 2^7 in magnitude, fp32 accumulation in ANY order is
  exact.  The tests check that bound for every workload (Cauchy-Schwarz on the
  non-bias part plus the bias term).

Continuous mode (``mode="continuous"``; the 0.5B and 2B layers, decode
windows and random small layers): x ~ N(0,1) and weights ~ N(0, 1/d) rounded
to the storage type (bf16, or plain fp32 values for fp32 layers), with the same
last-column / bias structure.  There fp32 sums depend on their order, so a gate
value near 0 may be active on one side only; tests compare such inputs within
the tie band instead of bit for bit.

All arrays are float32 holding values that are exactly representable in the
workload's dtype ("bf16" or "f32"); -inf appears only in W_g^T's last column.
Layouts: x [T][d]; W_g^T, W_u^T, W_d all [F][d] (one contiguous d-vector per
hidden neuron), row-major.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from statistics import NormalDist

import numpy as np

_ND = NormalDist()

# Workload ids used in the seed spawn keys.
WID_TINY, WID_0P5B, WID_2B, WID_DECODE, WID_STRESS, WID_RANDOM = 0, 1, 2, 3, 4, 5
# Array ids used in the seed spawn keys.
AID_X, AID_WG, AID_WU, AID_WD, AID_JITTER, AID_DEAD, AID_STRESS = 0, 1, 2, 3, 4, 5, 6


@dataclass
class Workload:
    name: str
    T: int
    d: int
    F: int
    dtype: str  # "bf16" or "f32": the type x, weights and TwELL values are held in
    tile_w: int
    cap: int
    x: np.ndarray
    wg_t: np.ndarray
    wu_t: np.ndarray
    wd: np.ndarray
    meta: dict = field(default_factory=dict)

    @property
    def n_b(self) -> int:
        return self.F // self.tile_w

    def rows(self, lo: int, hi: int) -> "Workload":
        """The same layer restricted to tokens [lo, hi) (weights shared)."""
        return Workload(f"{self.name}[{lo}:{hi}]", hi - lo, self.d, self.F, self.dtype,
                        self.tile_w, self.cap, self.x[lo:hi], self.wg_t, self.wu_t,
                        self.wd, dict(self.meta))


def _rng(wid: int, layer: int, aid: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(0, spawn_key=(wid, layer, aid))))


def round_to_bf16(a) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32.

    Input construction only (choosing representable biases / jitter values).
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    out = r.view(np.float32).copy()
    out[np.isnan(a)] = np.nan
    return out


def bf16_representable(a) -> bool:
    a = np.ascontiguousarray(a, dtype=np.float32)
    return bool(np.all((a.view(np.uint32) & 0xFFFF) == 0))


def _cont_x(rng, shape, dtype: str) -> np.ndarray:
    """Continuous mode: N(0,1) rounded to the storage type (no grid)."""
    a = rng.standard_normal(shape, dtype=np.float32)
    return round_to_bf16(a) if dtype == "bf16" else a


def _cont_w(rng, shape, d, dtype: str) -> np.ndarray:
    a = ((1.0 / np.sqrt(d)) * rng.standard_normal(shape, dtype=np.float32)).astype(np.float32)
    return round_to_bf16(a) if dtype == "bf16" else a


def _draw_x(rng, shape, mode: str, dtype: str) -> np.ndarray:
    if mode == "grid":
        return _grid_x(rng, shape)
    assert mode == "continuous", mode
    return _cont_x(rng, shape, dtype)


def _draw_w(rng, shape, d, mode: str, dtype: str) -> np.ndarray:
    if mode == "grid":
        return _grid_w(rng, shape, d)
    assert mode == "continuous", mode
    return _cont_w(rng, shape, d, dtype)


def _grid_x(rng, shape) -> np.ndarray:
    g = np.rint(16.0 * rng.standard_normal(shape, dtype=np.float32))
    np.clip(g, -127, 127, out=g)
    return (g / 16.0).astype(np.float32)


def _grid_w(rng, shape, d) -> np.ndarray:
    g = np.rint((1024.0 / np.sqrt(d)) * rng.standard_normal(shape, dtype=np.float32))
    np.clip(g, -255, 255, out=g)
    return (g / 1024.0).astype(np.float32)


def _threshold_for_rate(p: float, d: int) -> float:
    """tau with P(N(0,(d-1)/d) > tau) = p: the non-bias part of z has variance ~(d-1)/d."""
    return _ND.inv_cdf(1.0 - p) * np.sqrt((d - 1) / d)


def _bias_grid_f32(tau: float) -> np.float32:
    return np.float32(-np.rint(1024.0 * tau) / 1024.0)


def _bias_bf16(tau: float) -> np.float32:
    return round_to_bf16(np.array([-tau], np.float32))[0]


def make_tiny() -> Workload:
    """64 tokens, d=256, F=1024, fp32, P(active)=3%, tile 128, capacity 16."""
    T, d, F = 64, 256, 1024
    x = _grid_x(_rng(WID_TINY, 0, AID_X), (T, d))
    x[:, d - 1] = 1.0
    wg = _grid_w(_rng(WID_TINY, 0, AID_WG), (F, d), d)
    wu = _grid_w(_rng(WID_TINY, 0, AID_WU), (F, d), d)
    wd = _grid_w(_rng(WID_TINY, 0, AID_WD), (F, d), d)
    tau = _threshold_for_rate(0.03, d)
    wg[:, d - 1] = _bias_grid_f32(tau)
    return Workload("tiny", T, d, F, "f32", 128, 16, x, wg, wu, wd,
                    {"target_active_frac": 0.03, "tau": tau, "bias": float(wg[0, d - 1])})


def make_layer_0p5b(mode: str = "grid") -> Workload:
    """4096 tokens, d=1024, F=4096, bf16, ~1% active, tile 128, capacity 8."""
    T, d, F = 4096, 1024, 4096
    x = _draw_x(_rng(WID_0P5B, 0, AID_X), (T, d), mode, "bf16")
    x[:, d - 1] = 1.0
    wg = _draw_w(_rng(WID_0P5B, 0, AID_WG), (F, d), d, mode, "bf16")
    wu = _draw_w(_rng(WID_0P5B, 0, AID_WU), (F, d), d, mode, "bf16")
    wd = _draw_w(_rng(WID_0P5B, 0, AID_WD), (F, d), d, mode, "bf16")
    tau = _threshold_for_rate(0.01, d)
    wg[:, d - 1] = _bias_bf16(tau)
    return Workload("layer_0p5b" + _suffix(mode), T, d, F, "bf16", 128, 8, x, wg, wu, wd,
                    {"target_active_frac": 0.01, "tau": tau, "bias": float(wg[0, d - 1]), "mode": mode})


def _solve_tau_lognormal_jitter(target_mean: float, live: int, d: int, sigma_j: float) -> float:
    """tau0 with live * E_eps[ P(s > tau0 * exp(sigma_j * eps)) ] = target_mean.

    s ~ N(0, (d-1)/d) is the non-bias part of z; eps ~ N(0,1) clipped at +-4.
    """
    from math import erfc, sqrt
    sig = np.sqrt((d - 1) / d)
    eps = np.linspace(-4.0, 4.0, 16001)
    wts = np.exp(-0.5 * eps * eps)
    wts /= wts.sum()

    def mean(t):
        q = np.array([0.5 * erfc(t * np.exp(sigma_j * e) / sig / sqrt(2.0)) for e in eps[::10]])
        return live * float(np.sum(wts[::10] * q) / np.sum(wts[::10]))

    lo, hi = 0.5, 12.0
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        if mean(mid) > target_mean:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


_CACHE: dict = {}


def _suffix(mode: str) -> str:
    return "" if mode == "grid" else "_" + mode


def make_layer_2b(cache: bool = True, mode: str = "grid") -> Workload:
    """8192 tokens, d=2048, F=8192, bf16, mean ~29 active, lognormal jitter, 20% dead.

    Per-token threshold tau0 * exp(0.5 eps_t): the last column of x holds
    bf16(exp(0.5 eps_t)) and the last column of W_g^T holds bf16(-tau0), or -inf
    for the round(0.2 F) dead neurons.  Tile 256, capacity 16.
    """
    key = "2b" + _suffix(mode)
    if cache and key in _CACHE:
        return _CACHE[key]
    T, d, F = 8192, 2048, 8192
    x = _draw_x(_rng(WID_2B, 0, AID_X), (T, d), mode, "bf16")
    eps = np.clip(_rng(WID_2B, 0, AID_JITTER).standard_normal(T), -4.0, 4.0)
    x[:, d - 1] = round_to_bf16(np.exp(0.5 * eps).astype(np.float32))
    wg = _draw_w(_rng(WID_2B, 0, AID_WG), (F, d), d, mode, "bf16")
    wu = _draw_w(_rng(WID_2B, 0, AID_WU), (F, d), d, mode, "bf16")
    wd = _draw_w(_rng(WID_2B, 0, AID_WD), (F, d), d, mode, "bf16")
    n_dead = int(round(0.2 * F))
    dead = np.sort(_rng(WID_2B, 0, AID_DEAD).choice(F, n_dead, replace=False))
    tau0 = _solve_tau_lognormal_jitter(29.0, F - n_dead, d, 0.5)
    wg[:, d - 1] = _bias_bf16(tau0)
    wg[dead, d - 1] = -np.inf
    w = Workload("layer_2b" + _suffix(mode), T, d, F, "bf16", 256, 16, x, wg, wu, wd,
                 {"target_mean_active": 29.0, "tau0": tau0, "bias": float(_bias_bf16(tau0)),
                  "dead": dead, "jitter_sigma": 0.5, "mode": mode})
    if cache:
        _CACHE[key] = w
    return w


def make_decode_windows(T: int, max_windows: int = 512, mode: str = "grid"):
    """Disjoint consecutive windows of T tokens of the 2B-like layer (same weights)."""
    base = make_layer_2b(mode=mode)
    n = min(base.T // T, max_windows)
    out = []
    for i in range(n):
        w = base.rows(i * T, (i + 1) * T)
        w.name = f"decode_2b{_suffix(mode)}_T{T}[{i}]"
        out.append(w)
    return out


STRESS_LAYERS = 24


def stress_layer_mean(layer: int) -> float:
    """Target mean active count of the normal tokens of stress layer `layer` (10 .. 60)."""
    return 10.0 + 50.0 * (layer / (STRESS_LAYERS - 1)) ** 3


def make_stress_layer(layer: int, T: int = 16384) -> Workload:
    """One layer of the 24-layer overflow stress stack: d=2048, F=8192, bf16.

    Normal tokens: ones column, bias bf16(-tau_l) giving mean m_l active.
    2% of tokens (chosen by seed) get a target active fraction f ~ U(0.05, 0.30)
    through their last column, bf16(Phi^-1(1-f) * sigma / tau_l).  No dead neurons.
    Tile 256, capacity 16.
    """
    d, F = 2048, 8192
    sig = np.sqrt((d - 1) / d)
    m = stress_layer_mean(layer)
    x = _grid_x(_rng(WID_STRESS, layer, AID_X), (T, d))
    wg = _grid_w(_rng(WID_STRESS, layer, AID_WG), (F, d), d)
    wu = _grid_w(_rng(WID_STRESS, layer, AID_WU), (F, d), d)
    wd = _grid_w(_rng(WID_STRESS, layer, AID_WD), (F, d), d)
    tau = _threshold_for_rate(m / F, d)
    bias = _bias_bf16(tau)
    wg[:, d - 1] = bias
    rs = _rng(WID_STRESS, layer, AID_STRESS)
    n_stress = int(round(0.02 * T))
    stress = np.sort(rs.choice(T, n_stress, replace=False))
    f = rs.uniform(0.05, 0.30, n_stress)
    xl = np.array([_ND.inv_cdf(1.0 - fi) * sig / abs(float(bias)) for fi in f], np.float32)
    xl = round_to_bf16(xl)
    assert np.all(xl >= 0.125)
    x[:, d - 1] = 1.0
    x[stress, d - 1] = xl
    return Workload(f"stress_l{layer}", T, d, F, "bf16", 256, 16, x, wg, wu, wd,
                    {"layer": layer, "target_mean_active": m, "tau": tau, "bias": float(bias),
                     "stress_rows": stress, "stress_frac": f})


def make_random_small(T: int, d: int, F: int, tile_w: int, cap: int, dtype: str = "bf16",
                      active_frac: float = 0.05, seed: int = 0, jitter: float = 0.0,
                      n_dead: int = 0, mode: str = "grid") -> Workload:
    """A layer of any shape (tests): ones/jitter column + bias for `active_frac`."""
    assert d >= 2
    x = _draw_x(_rng(WID_RANDOM, seed, AID_X), (T, d), mode, dtype)
    wg = _draw_w(_rng(WID_RANDOM, seed, AID_WG), (F, d), max(d, 16), mode, dtype)
    wu = _draw_w(_rng(WID_RANDOM, seed, AID_WU), (F, d), max(d, 16), mode, dtype)
    wd = _draw_w(_rng(WID_RANDOM, seed, AID_WD), (F, d), max(d, 16), mode, dtype)
    sig = np.sqrt((d - 1) / max(d, 16))
    tau = max(_ND.inv_cdf(1.0 - active_frac) * sig, 1.0)
    if jitter > 0:
        eps = np.clip(_rng(WID_RANDOM, seed, AID_JITTER).standard_normal(T), -4.0, 4.0)
        x[:, d - 1] = round_to_bf16(np.exp(jitter * eps).astype(np.float32))
    else:
        x[:, d - 1] = 1.0
    wg[:, d - 1] = _bias_bf16(tau)
    if n_dead:
        dead = _rng(WID_RANDOM, seed, AID_DEAD).choice(F, n_dead, replace=False)
        wg[dead, d - 1] = -np.inf
    return Workload(f"random_T{T}_d{d}_F{F}_w{tile_w}_c{cap}_s{seed}{_suffix(mode)}", T, d, F, dtype, tile_w,
                    cap, x, wg, wu, wd, {"tau": tau, "mode": mode})


WORKLOADS = {
    "tiny": make_tiny,
    "layer_0p5b": make_layer_0p5b,
    "layer_2b": make_layer_2b,
}


def make_workload(name: str, **kw) -> Workload:
    if name in WORKLOADS:
        return WORKLOADS[name](**kw)
    if name.startswith("stress_l"):
        return make_stress_layer(int(name[len("stress_l"):]), **kw)
    if name.startswith("decode_"):  # decode_<T>: the first T tokens of the 2B-like layer
        return make_decode_windows(int(name[len("decode_"):]), max_windows=1)[0]
    raise KeyError(name)
