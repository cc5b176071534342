"""Pure-Python brute force of the same definitions, for tiny inputs only.

TEST INFRASTRUCTURE ONLY.  Written independently of ``twell_oracle.c`` (Python
floats are IEEE fp64) so the two can pin each other: every quantity is built
from nested lists with no numpy arithmetic.  Follows the gist.science summary
of "Sparser, Faster, Lighter Transformer Language Models", sections 2.1-2.3,
with the readings listed in ``oracle/__init__.py``.
"""

from __future__ import annotations

import struct


def _f32(v: float) -> float:
    return struct.unpack("<f", struct.pack("<f", v))[0]


def _bf16(v: float) -> float:
    """fp32 round-to-nearest-even, then keep 8 significant bits with ties to even."""
    f = _f32(v)
    if f != f or f in (float("inf"), float("-inf")) or f == 0.0:
        return f
    bits = struct.unpack("<I", struct.pack("<f", f))[0]
    lower = bits & 0xFFFF
    upper = bits >> 16
    if lower > 0x8000 or (lower == 0x8000 and (upper & 1)):
        upper += 1
    return struct.unpack("<f", struct.pack("<I", (upper << 16) & 0xFFFFFFFF))[0]


def stored(v: float, vdtype) -> float:
    if vdtype in (None, "exact", "f64"):
        return v
    if vdtype == "f32":
        return _f32(v)
    if vdtype == "bf16":
        return _bf16(v)
    raise ValueError(vdtype)


def matmul_nt(a, b_t):
    return [[sum(a[t][k] * b_t[j][k] for k in range(len(a[t]))) for j in range(len(b_t))]
            for t in range(len(a))]


def pack(z, w: int, cap: int, vdtype):
    """Per row, per tile: (true count, [stored value of kept entries], [tile-local col])."""
    out = []
    for row in z:
        tiles = []
        for b in range(len(row) // w):
            cols = [c for c in range(w) if row[b * w + c] > 0.0]
            kept = cols[:cap]
            tiles.append((len(cols), [stored(row[b * w + c], vdtype) for c in kept], kept))
        out.append(tiles)
    return out


def overflow_rows(packed, cap: int):
    return [t for t, tiles in enumerate(packed) if any(n > cap for n, _, _ in tiles)]


def ffn(x, wg_t, wu_t, wd, hround=None):
    """y[t] = sum over active j (ascending) of h * (x[t] . wu_t[j]) * wd[j]."""
    z = matmul_nt(x, wg_t)
    d = len(wd[0])
    y = []
    for t in range(len(x)):
        acc = [0.0] * d
        for j in range(len(wg_t)):
            if z[t][j] > 0.0:
                h = stored(z[t][j], hround)
                u = sum(x[t][k] * wu_t[j][k] for k in range(len(x[t])))
                for k in range(d):
                    acc[k] += (h * u) * wd[j][k]
        y.append(acc)
    return y


def gate_stats(z, w: int):
    """Per-neuron active counts and per (row, tile) sums of active values
    (section 2.4's L1 activation penalty), by nested loops over lists."""
    T, F = len(z), len(z[0])
    cnt = [0] * F
    l1 = [[0.0] * (F // w) for _ in range(T)]
    for t in range(T):
        for j in range(F):
            if z[t][j] > 0.0:
                cnt[j] += 1
                l1[t][j // w] += z[t][j]
    return cnt, l1
