"""The C ABI on the host (no GPU needed): the library loads, exports every
symbol include/twell.h declares, and rejects bad arguments before launching."""

import ctypes
import os
import re

import pytest

import unstructured_sparse_transformer_amd as tw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "twell.h")).read()
    return sorted(set(re.findall(r"TWELL_API\s+[\w\s\*]+?\b(twell_\w+)\s*\(", src)))


def test_exports_match_header():
    lib = tw.load()
    names = _declared()
    assert set(names) == set(tw.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.twell_version() == 201


def test_status_strings():
    lib = tw.load()
    for st in range(0, -8, -1):
        assert lib.twell_status_str(st)
    assert lib.twell_status_str(-99) == b"unknown status"


def _desc(T=16, F=512, w=128, cap=8, vd=1, val=256, idx=512, cnt=1024):
    return tw.TwellT(T, F, w, cap, vd, 0, val, idx, cnt)


GOOD = 4096  # an aligned, never dereferenced fake device address


def test_pack_gate_stats_validation():
    lib = tw.load()
    f = lib.twell_pack_gate_stats
    d = ctypes.byref(_desc())
    assert f(GOOD, GOOD, 64, None, GOOD, GOOD, None) == -1
    assert f(GOOD, GOOD, 64, d, None, GOOD, None) == -1                     # neuron_cnt NULL
    assert f(GOOD, GOOD, 64, d, GOOD, None, None) == -1                     # l1 NULL
    assert f(GOOD, GOOD, 64, d, GOOD + 2, GOOD, None) == -2                 # neuron_cnt misaligned
    assert f(GOOD, GOOD, 64, d, GOOD, GOOD + 1, None) == -2                 # l1 misaligned
    assert f(None, GOOD, 64, d, GOOD, GOOD, None) == -1                     # x NULL
    assert f(GOOD, GOOD, 65, d, GOOD, GOOD, None) == -3                     # d % 64
    assert f(GOOD, GOOD, 64, ctypes.byref(_desc(w=100)), GOOD, GOOD, None) == -4
    assert f(GOOD, GOOD, 64, ctypes.byref(_desc(T=0)), GOOD, GOOD, None) == 0  # nothing to do


def test_pack_gate_validation():
    lib = tw.load()
    f = lib.twell_pack_gate
    assert f(GOOD, GOOD, 64, None, None) == -1
    assert f(None, GOOD, 64, ctypes.byref(_desc()), None) == -1             # x NULL
    assert f(GOOD, None, 64, ctypes.byref(_desc()), None) == -1             # W_g NULL
    assert f(GOOD, GOOD, 64, ctypes.byref(_desc(val=0)), None) == -1        # val NULL
    assert f(GOOD + 8, GOOD, 64, ctypes.byref(_desc()), None) == -2         # x misaligned
    assert f(GOOD, GOOD, 64, ctypes.byref(_desc(cnt=1026)), None) == -2     # cnt misaligned
    assert f(GOOD, GOOD, 65, ctypes.byref(_desc()), None) == -3             # d % 64
    assert f(GOOD, GOOD, 64, ctypes.byref(_desc(F=500)), None) == -3        # F % w
    assert f(GOOD, GOOD, 64, ctypes.byref(_desc(F=96, w=32)), None) == -3   # F % 64
    assert f(GOOD, GOOD, 64, ctypes.byref(_desc(T=-1)), None) == -3
    assert f(GOOD, GOOD, 64, ctypes.byref(_desc(w=100)), None) == -4        # tile width
    assert f(GOOD, GOOD, 64, ctypes.byref(_desc(w=512, F=1024)), None) == -4
    assert f(GOOD, GOOD, 64, ctypes.byref(_desc(cap=0)), None) == -4
    assert f(GOOD, GOOD, 64, ctypes.byref(_desc(cap=129)), None) == -4
    assert f(GOOD, GOOD, 64, ctypes.byref(_desc(vd=2)), None) == -4
    assert f(GOOD, GOOD, 8192, ctypes.byref(_desc()), None) == -4           # bf16 row > 8 KiB
    assert f(GOOD, GOOD, 4096, ctypes.byref(_desc(vd=0)), None) == -4       # f32 row > 8 KiB
    assert f(GOOD, GOOD, 2048, ctypes.byref(_desc(T=1 << 20, F=8192, w=256, cap=16)), None) == -3  # x = 4 GiB
    assert f(GOOD, GOOD, 64, ctypes.byref(_desc(T=1 << 15, F=1 << 16, w=32, cap=32)), None) == -3  # 2^31 slots
    assert f(None, None, 64, ctypes.byref(_desc(T=0)), None) == 0           # T = 0: nothing to do


def test_fused_and_hybrid_validation():
    lib = tw.load()
    d = _desc()
    need_f = lib.twell_workspace_bytes(16, 512, 128, 8, 0, 64, 1)
    slots = 16 * 4 * 8                                                    # T * n_b * cap
    # row entry counts by row and in work order (256 B each here), each row's packed entries (neuron,
    # gate value: 8 B per slot) and (d / 64) partial dot products per slot
    assert need_f == 2 * 256 + slots * 8 + slots * 1 * 4
    f = lib.twell_ffn_fused
    r = ctypes.byref(d)
    assert f(r, None, GOOD, GOOD, GOOD, 64, None, GOOD, need_f, None) == -1       # y NULL
    assert f(r, None, GOOD, GOOD, GOOD + 4, 64, GOOD, GOOD, need_f, None) == -2
    assert f(r, None, GOOD, GOOD, GOOD, 60, GOOD, GOOD, need_f, None) == -3
    assert f(r, GOOD + 2, GOOD, GOOD, GOOD, 64, GOOD, GOOD, need_f, None) == -2   # order
    assert f(r, None, GOOD, GOOD, GOOD, 64, GOOD, None, need_f, None) == -6       # no workspace
    assert f(r, None, GOOD, GOOD, GOOD, 64, GOOD, GOOD, need_f - 1, None) == -6
    assert f(r, None, GOOD, GOOD, GOOD, 64, GOOD, GOOD + 16, need_f, None) == -2  # workspace 256-aligned
    hy = tw.TwellHybridT(d, 8, 0, GOOD, GOOD, GOOD, GOOD, GOOD)
    need = lib.twell_workspace_bytes(16, 512, 128, 8, 8, 64, 1)
    assert need > need_f
    assert lib.twell_ffn_hybrid(ctypes.byref(hy), GOOD, GOOD, GOOD, 64, GOOD, None, 0, None) == -6
    assert lib.twell_ffn_hybrid(ctypes.byref(hy), GOOD, GOOD, GOOD, 64, GOOD, GOOD, need - 1, None) == -6
    assert lib.twell_ffn_hybrid(ctypes.byref(hy), GOOD, GOOD, GOOD, 64, GOOD, GOOD + 16, need, None) == -2
    assert lib.twell_ffn_overflow(ctypes.byref(hy), GOOD, GOOD, GOOD, 64, GOOD, GOOD, need - 1, None) == -6
    bad = tw.TwellHybridT(d, -1, 0, GOOD, GOOD, GOOD, GOOD, GOOD)
    assert lib.twell_partition_overflow(GOOD, GOOD, 64, ctypes.byref(bad), None) == -3
    nod = tw.TwellHybridT(d, 8, 0, GOOD, GOOD, GOOD, None, GOOD)
    assert lib.twell_pack_gate_hybrid(GOOD, GOOD, 64, ctypes.byref(nod), None) == -1
    noo = tw.TwellHybridT(d, 8, 0, GOOD, GOOD, GOOD, GOOD, None)                 # order NULL
    assert lib.twell_partition_overflow(GOOD, GOOD, 64, ctypes.byref(noo), None) == -1
    odd = tw.TwellHybridT(d, 8, 0, GOOD, GOOD, GOOD, GOOD, GOOD + 2)             # order misaligned
    assert lib.twell_partition_overflow(GOOD, GOOD, 64, ctypes.byref(odd), None) == -2
    assert lib.twell_partition_overflow(GOOD, GOOD, 64, None, None) == -1
    # invalid sizes give 0
    assert lib.twell_workspace_bytes(-1, 512, 128, 8, 0, 64, 1) == 0
    assert lib.twell_workspace_bytes(16, 500, 128, 8, 0, 64, 1) == 0
    assert lib.twell_workspace_bytes(16, 512, 100, 8, 0, 64, 1) == 0
    assert lib.twell_workspace_bytes(16, 512, 128, 8, 0, 64, 2) == 0
    assert lib.twell_workspace_bytes(0, 512, 128, 8, 0, 64, 1) == 0                # nothing to hold


def test_ffn_forward_validation():
    """Every argument of the one-call layer is checked before its first launch."""
    lib = tw.load()
    f = lib.twell_ffn_forward
    d = _desc()
    hy = tw.TwellHybridT(d, 8, 0, GOOD, GOOD, GOOD, GOOD, GOOD)
    r = ctypes.byref(hy)
    need = lib.twell_workspace_bytes(16, 512, 128, 8, 8, 64, 1)
    assert f(GOOD, GOOD, GOOD, GOOD, 64, None, GOOD, GOOD, need, None) == -1          # hybrid NULL
    assert f(None, GOOD, GOOD, GOOD, 64, r, GOOD, GOOD, need, None) == -1             # x NULL
    assert f(GOOD, None, GOOD, GOOD, 64, r, GOOD, GOOD, need, None) == -1             # W_g NULL
    assert f(GOOD, GOOD, None, GOOD, 64, r, GOOD, GOOD, need, None) == -1             # W_u NULL
    assert f(GOOD, GOOD, GOOD, None, 64, r, GOOD, GOOD, need, None) == -1             # W_d NULL
    assert f(GOOD, GOOD, GOOD, GOOD, 64, r, None, GOOD, need, None) == -1             # y NULL
    assert f(GOOD, GOOD, GOOD + 2, GOOD, 64, r, GOOD, GOOD, need, None) == -2         # W_u misaligned
    assert f(GOOD, GOOD, GOOD, GOOD, 60, r, GOOD, GOOD, need, None) == -3             # d % 64
    assert f(GOOD, GOOD, GOOD, GOOD, 64, r, GOOD, None, 0, None) == -6                # no workspace
    assert f(GOOD, GOOD, GOOD, GOOD, 64, r, GOOD, GOOD, need - 1, None) == -6         # too small
    assert f(GOOD, GOOD, GOOD, GOOD, 64, r, GOOD, GOOD + 16, need, None) == -2        # not 256-aligned
    nod = tw.TwellHybridT(d, 8, 0, GOOD, GOOD, GOOD, None, GOOD)                     # dense NULL
    assert f(GOOD, GOOD, GOOD, GOOD, 64, ctypes.byref(nod), GOOD, GOOD, need, None) == -1
    noval = tw.TwellHybridT(_desc(val=0), 8, 0, GOOD, GOOD, GOOD, GOOD, GOOD)         # TwELL val NULL
    assert f(GOOD, GOOD, GOOD, GOOD, 64, ctypes.byref(noval), GOOD, GOOD, need, None) == -1
    empty = tw.TwellHybridT(_desc(T=0), 8, 0, None, None, None, None, None)
    assert f(None, None, None, None, 64, ctypes.byref(empty), None, None, 0, None) == 0  # T = 0
    g = lib.twell_ffn_from_gate  # same checks
    assert g(GOOD, GOOD, GOOD, GOOD, 64, None, GOOD, GOOD, need, None) == -1
    assert g(GOOD, None, GOOD, GOOD, 64, r, GOOD, GOOD, need, None) == -1
    assert g(GOOD, GOOD, GOOD, GOOD, 64, r, GOOD, GOOD, need - 1, None) == -6
    assert g(GOOD, GOOD, GOOD, GOOD, 64, r, GOOD + 4, GOOD, need, None) == -2
    assert g(None, None, None, None, 64, ctypes.byref(empty), None, None, 0, None) == 0


def test_ffn_decode_validation():
    lib = tw.load()
    f = lib.twell_ffn_decode
    hy = lambda **k: tw.TwellHybridT(_desc(**k), 8, 0, GOOD, GOOD, GOOD, GOOD, GOOD)  # noqa: E731
    need = lib.twell_ffn_decode_workspace_bytes(16, 512, 64, 128)
    assert need > 16 * 512 * 4
    assert lib.twell_ffn_decode_workspace_bytes(65, 512, 64, 128) == 0      # T > 64
    assert lib.twell_ffn_decode_workspace_bytes(16, 512, 64, 100) == 0      # tile width
    ok = hy()
    assert f(GOOD, GOOD, GOOD, GOOD, 64, None, GOOD, GOOD, need, None) == -1
    assert f(GOOD, GOOD, GOOD, GOOD, 64, ctypes.byref(ok), GOOD, None, need, None) == -1        # workspace NULL
    assert f(GOOD, GOOD, GOOD, GOOD, 64, ctypes.byref(ok), GOOD, GOOD + 16, need, None) == -2   # not 256-aligned
    assert f(GOOD, GOOD, GOOD, GOOD, 64, ctypes.byref(ok), GOOD, GOOD, need - 1, None) == -6
    assert f(GOOD, GOOD, None, GOOD, 64, ctypes.byref(ok), GOOD, GOOD, need, None) == -1        # W_u NULL
    assert f(GOOD, GOOD, GOOD, GOOD, 64, ctypes.byref(ok), GOOD + 4, GOOD, need, None) == -2    # y misaligned
    assert f(GOOD, GOOD, GOOD, GOOD, 64, ctypes.byref(hy(T=65)), GOOD, GOOD, need, None) == -4  # T > 64
    assert f(GOOD, GOOD, GOOD, GOOD, 64, ctypes.byref(hy(vd=0)), GOOD, GOOD, need, None) == -4  # fp32
    assert f(GOOD, GOOD, GOOD, GOOD, 64, ctypes.byref(hy(T=64, F=32768, w=256)), GOOD, GOOD, need,
             None) == -4                                                                        # T * F > 2^20
    assert f(GOOD, GOOD, GOOD, GOOD, 60, ctypes.byref(ok), GOOD, GOOD, need, None) == -3        # d % 64
    assert f(None, None, None, None, 64, ctypes.byref(hy(T=0)), None, None, 0, None) == 0       # nothing to do


def test_ffn_decode_noalloc_validation():
    """The same checks as twell_ffn_decode (no workspace argument), and a
    shape whose workspace exceeds the 16 MiB static scratch is rejected with
    TWELL_E_SCRATCH before anything touches the GPU."""
    lib = tw.load()
    f = lib.twell_ffn_decode_noalloc
    hy = lambda **k: tw.TwellHybridT(_desc(**k), 8, 0, GOOD, GOOD, GOOD, GOOD, GOOD)  # noqa: E731
    ok = hy()
    assert f(GOOD, GOOD, GOOD, GOOD, 64, None, GOOD, None) == -1
    assert f(GOOD, GOOD, None, GOOD, 64, ctypes.byref(ok), GOOD, None) == -1                    # W_u NULL
    assert f(GOOD, GOOD, GOOD, GOOD, 64, ctypes.byref(ok), GOOD + 4, None) == -2                # y misaligned
    assert f(GOOD + 8, GOOD, GOOD, GOOD, 64, ctypes.byref(ok), GOOD, None) == -2                # x misaligned
    assert f(GOOD, GOOD, GOOD, GOOD, 64, ctypes.byref(hy(T=65)), GOOD, None) == -4              # T > 64
    assert f(GOOD, GOOD, GOOD, GOOD, 64, ctypes.byref(hy(vd=0)), GOOD, None) == -4              # fp32
    assert f(GOOD, GOOD, GOOD, GOOD, 64, ctypes.byref(hy(T=64, F=32768, w=256)), GOOD, None) == -4
    assert f(GOOD, GOOD, GOOD, GOOD, 60, ctypes.byref(ok), GOOD, None) == -3                    # d % 64
    assert f(None, None, None, None, 64, ctypes.byref(hy(T=0)), None, None) == 0                # nothing to do
    # d = 4096, T = 17: the chunked layout's (1024 + T) partial rows of 16 KiB
    # exceed the 16 MiB scratch, and the two-kernel layout serves T <= 16 only
    assert noalloc_scratch_need(17, 512, 4096) > 16 << 20
    assert f(GOOD, GOOD, GOOD, GOOD, 4096, ctypes.byref(hy(T=17)), GOOD, None) == -7
    assert b"static" in lib.twell_status_str(-7)
    # d = 4096, T = 1: the two-kernel layout fits
    assert noalloc_scratch_need(1, 512, 4096) <= 16 << 20
    # every d <= 2048 shape the decode path accepts fits (largest: T * F = 2^20, d = 2048)
    assert noalloc_scratch_need(64, 16384, 2048) <= 16 << 20
    assert noalloc_scratch_need(1, 1 << 20, 2048) <= 16 << 20


def noalloc_scratch_need(T, F, d):
    """Bytes the allocation-free decode path carves from its static scratch
    (256-byte aligned sections): for T <= 16 the smaller of its two layouts.
    Two-kernel layout: z [T][F] fp32, the counter block, flags [T][F / 32] and
    T * F / 32 partial rows of d floats.  Chunked layout: z, the counter
    block, per-row sums [2T], the chunk table [T + 1] and (1024 + T) partial
    rows of d floats."""
    up = lambda b: (b + 255) & ~255  # noqa: E731
    chunked = up(T * F * 4) + 256 + up(T * 8) + up((T + 1) * 4) + up((1024 + T) * d * 4)
    if T > 16:
        return chunked
    two = up(T * F * 4) + 256 + up(T * (F // 32) * 4) + up(T * (F // 32) * d * 4)
    return two if two <= 16 << 20 else chunked


def test_conversion_validation():
    lib = tw.load()
    hy = tw.TwellHybridT(_desc(), 8, 0, GOOD, GOOD, GOOD, GOOD, GOOD)
    assert lib.twell_dense_to_hybrid(GOOD, None, None) == -1
    assert lib.twell_dense_to_hybrid(None, ctypes.byref(hy), None) == -1
    assert lib.twell_dense_to_hybrid(GOOD + 2, ctypes.byref(hy), None) == -2
    bad = tw.TwellHybridT(_desc(w=100), 8, 0, GOOD, GOOD, GOOD, GOOD, GOOD)
    assert lib.twell_dense_to_hybrid(GOOD, ctypes.byref(bad), None) == -4
    nod = tw.TwellHybridT(_desc(), 8, 0, GOOD, GOOD, GOOD, None, GOOD)      # dense NULL with max_ovf > 0
    assert lib.twell_dense_to_hybrid(GOOD, ctypes.byref(nod), None) == -1
    assert lib.twell_hybrid_to_dense(None, GOOD, None) == -1
    assert lib.twell_hybrid_to_dense(ctypes.byref(hy), None, None) == -1
    assert lib.twell_hybrid_to_dense(ctypes.byref(hy), GOOD + 8, None) == -2
    noval = tw.TwellHybridT(_desc(val=0), 8, 0, GOOD, GOOD, GOOD, GOOD, GOOD)
    assert lib.twell_hybrid_to_dense(ctypes.byref(noval), GOOD, None) == -1
    empty = tw.TwellHybridT(_desc(T=0), 8, 0, GOOD, GOOD, GOOD, GOOD, GOOD)
    assert lib.twell_hybrid_to_dense(ctypes.byref(empty), None, None) == 0
    assert lib.twell_dense_to_hybrid(None, ctypes.byref(empty), None) == 0


def test_compact_validation():
    import struct
    lib = tw.load()
    # the binding's header description matches the C struct's size
    assert struct.calcsize("<" + "".join(f for _, f in tw.COMPACT_HEADER)) == 80
    assert lib.twell_compact_min_bytes(16) == 256 + 256
    assert lib.twell_compact_min_bytes(100) == 256 + 512
    hy = tw.TwellHybridT(_desc(), 8, 0, GOOD, GOOD, GOOD, GOOD, GOOD)
    need = lib.twell_compact_min_bytes(16)
    assert lib.twell_compact_hybrid(None, GOOD, need, None) == -1
    assert lib.twell_compact_hybrid(ctypes.byref(hy), None, need, None) == -1
    assert lib.twell_compact_hybrid(ctypes.byref(hy), GOOD + 16, need, None) == -2
    assert lib.twell_compact_hybrid(ctypes.byref(hy), GOOD, need - 1, None) == -6
    big = tw.TwellHybridT(_desc(F=131072, w=256), 8, 0, GOOD, GOOD, GOOD, GOOD, GOOD)
    assert lib.twell_compact_hybrid(ctypes.byref(big), GOOD, need, None) == -4   # F > 65536
    assert lib.twell_compact_to_dense(GOOD, 16, 512, 2, GOOD, None) == -4      # dtype
    assert lib.twell_compact_to_dense(GOOD, 16, 500, 1, GOOD, None) == -3      # F % 64
    assert lib.twell_compact_to_dense(None, 16, 512, 1, GOOD, None) == -1
    assert lib.twell_compact_to_dense(GOOD + 64, 16, 512, 1, GOOD, None) == -2
    assert lib.twell_compact_to_dense(GOOD, 16, 512, 1, GOOD + 2, None) == -2
    assert lib.twell_compact_to_dense(None, 0, 512, 1, None, None) == 0


def test_binding_requires_library(tmp_path, monkeypatch):
    """No CPU fallback: a missing library is an error."""
    tw.load()
    monkeypatch.setattr(tw, "_lib", None)
    with pytest.raises(RuntimeError, match="libtwell.so not found"):
        tw.load(str(tmp_path / "missing.so"))


def test_ffn_backward_validation():
    """Host checks of twell_ffn_backward, including the bound on the entry
    scan's int32 count: T * n_b * cap + max_ovf * F must stay below 2^31."""
    lib = tw.load()
    f = lib.twell_ffn_backward

    def hy(max_ovf=8, **k):
        return tw.TwellHybridT(_desc(**k), max_ovf, 0, GOOD, GOOD, GOOD, GOOD, GOOD)

    def call(h, d=64, max_entries=16, ws=GOOD, ws_bytes=1 << 30):
        return f(ctypes.byref(h) if h is not None else None, GOOD, GOOD, GOOD, GOOD, d, GOOD, GOOD, GOOD, GOOD,
                 GOOD, max_entries, ws, ws_bytes, None)

    assert call(None) == -1
    assert call(hy(vd=0)) == -4                      # fp32
    assert call(hy(), d=4096) == -4                  # d > 2048
    assert call(hy(), max_entries=-1) == -3
    assert call(hy(), ws=None) == -1
    assert call(hy(), ws=GOOD + 16) == -2
    assert call(hy(), ws_bytes=0) == -6
    # 7 * 2^28 fitting-row slots (< 2^31 on their own) + 2^14 dense rows of 2^14 = 2^31 entries
    big = dict(T=1 << 19, F=16384, w=32, cap=7)
    assert call(hy(max_ovf=1 << 14, **big), d=2048, ws_bytes=0) == -3
    assert call(hy(max_ovf=(1 << 14) - 1, **big), d=2048, ws_bytes=0) == -6   # one row less: next check


def test_gate_dense_validation():
    lib = tw.load()
    f = lib.twell_gate_dense
    assert f(GOOD, GOOD, 64, 16, 512, 2, GOOD, None) == -4         # dtype
    assert f(GOOD, GOOD, 60, 16, 512, 1, GOOD, None) == -3         # d % 64
    assert f(GOOD, GOOD, 64, 16, 500, 1, GOOD, None) == -3         # F % 64
    assert f(GOOD, GOOD, 64, -1, 512, 1, GOOD, None) == -3
    assert f(None, GOOD, 64, 16, 512, 1, GOOD, None) == -1         # x NULL
    assert f(GOOD, GOOD + 8, 64, 16, 512, 1, GOOD, None) == -2     # W_g misaligned
    assert f(GOOD, GOOD, 64, 16, 512, 1, None, None) == -1         # h NULL
    assert f(GOOD, GOOD, 64, 16, 512, 1, GOOD + 1, None) == -2     # h not element-aligned
    assert f(GOOD, GOOD, 2048, 1 << 20, 512, 1, GOOD, None) == -3  # x = 4 GiB
    assert f(None, None, 64, 0, 512, 1, None, None) == 0           # T = 0
