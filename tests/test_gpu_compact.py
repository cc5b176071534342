"""GPU parity of the compacted hybrid storage (twell_compact_hybrid,
twell_compact_to_dense) against the oracle, through the C ABI: the header,
row offsets, columns, values, overflow ids and dense rows exactly, and the
expansion back to dense exactly."""

import numpy as np
import pytest

import oracle
from helpers import say, to_device
from test_gpu_convert import _matrix
from workloads import make_layer_2b

pytestmark = pytest.mark.gpu


def _a256(b):
    return (b + 255) & ~255


def _layout(T, F, n_entries, n_dense, esz):
    off_col = 256 + _a256((T + 1) * 4)
    off_val = off_col + _a256(n_entries * 2)
    off_ovf = off_val + _a256(n_entries * esz)
    off_dense = off_ovf + _a256(n_dense * 4)
    return off_col, off_val, off_ovf, off_dense, off_dense + n_dense * F * esz


def _compact(hy, T, F, dt, nbytes):
    import torch
    import unstructured_sparse_transformer_amd as tw
    buf = torch.full((max(nbytes, tw.twell_compact_min_bytes(T)),), 0xEE, dtype=torch.uint8, device="cuda")
    tw.twell_compact_hybrid(hy, buf)
    out = torch.full((T, F), -9.0, dtype=dt, device="cuda")
    tw.twell_compact_to_dense(buf, T, F, dt, out)
    torch.cuda.synchronize()
    return buf, tw.compact_header(buf), out.float().cpu().numpy()


def _check(h, hy, T, F, w, cap, dtype, max_ovf, label):
    import torch
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    esz = 2 if dtype == "bf16" else 4
    tw_ = oracle.pack_twell(h, w, cap, dtype)
    row_ovf, rows, n = oracle.partition_overflow(tw_.cnt, cap)
    ref = oracle.compact_hybrid(tw_, row_ovf, rows, oracle.dense_backup(h, rows[:max_ovf], dtype), max_ovf)
    n_e, n_d = int(ref["row_ptr"][-1]), len(ref["dense"])
    off_col, off_val, off_ovf, off_dense, total = _layout(T, F, n_e, n_d, esz)
    # a buffer one byte short (when the variable part is not empty): header and row offsets only
    if total > 256 + _a256((T + 1) * 4):
        buf, hdr, out = _compact(hy, T, F, dt, total - 1)
        assert hdr["fits"] == 0 and hdr["bytes"] == total, (label, hdr)
        assert not out.any(), f"{label}: a buffer that does not fit expands to zeros"
    # exactly enough
    buf, hdr, out = _compact(hy, T, F, dt, total)
    want = {"T": T, "F": F, "tile_w": w, "vdtype": 1 if dtype == "bf16" else 0, "n_entries": n_e, "n_ovf": n,
            "n_dense": n_d, "fits": 1, "off_row_ptr": 256, "off_col": off_col, "off_val": off_val,
            "off_ovf": off_ovf, "off_dense": off_dense, "bytes": total}
    assert hdr == want, (label, hdr, want)
    b = buf.cpu().numpy()
    row_ptr = b[256:256 + (T + 1) * 4].view(np.int32)
    np.testing.assert_array_equal(row_ptr, ref["row_ptr"], err_msg=f"{label}: row_ptr")
    col = b[off_col:off_col + n_e * 2].view(np.uint16)
    np.testing.assert_array_equal(col, ref["col"], err_msg=f"{label}: columns")
    vraw = b[off_val:off_val + n_e * esz]
    vals = (vraw.view(np.uint16).astype(np.uint32) << 16).view(np.float32) if esz == 2 else vraw.view(np.float32)
    np.testing.assert_array_equal(vals, ref["val"].astype(np.float32), err_msg=f"{label}: values")
    ids = b[off_ovf:off_ovf + n_d * 4].view(np.int32)
    np.testing.assert_array_equal(ids, ref["ovf_rows"][:n_d], err_msg=f"{label}: overflow ids")
    draw = b[off_dense:off_dense + n_d * F * esz]
    dense = ((draw.view(np.uint16).astype(np.uint32) << 16).view(np.float32) if esz == 2
             else draw.view(np.float32)).reshape(n_d, F)
    np.testing.assert_array_equal(dense, ref["dense"].astype(np.float32), err_msg=f"{label}: dense rows")
    np.testing.assert_array_equal(out, oracle.compact_to_dense(ref, T, F).astype(np.float32),
                                  err_msg=f"{label}: compact -> dense")
    if ref["complete"]:
        np.testing.assert_array_equal(out, np.where(h > 0, h, 0.0).astype(np.float32), err_msg=f"{label}: round trip")
    return hdr


CASES = [
    # (T, F, w, cap, dtype, frac, max_ovf)
    (300, 1024, 256, 16, "bf16", 0.03, 300),
    (257, 384, 128, 4, "bf16", 0.05, 257),
    (100, 1024, 32, 4, "f32", 0.1, 100),
    (128, 512, 128, 3, "bf16", 0.4, 5),     # n_ovf above max_ovf: not every overflow row is held
    (64, 512, 64, 3, "f32", 0.4, 0),        # max_ovf = 0
    (1, 64, 64, 8, "bf16", 0.2, 1),         # T = 1
]


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}_F{c[1]}_w{c[2]}_c{c[3]}_{c[4]}_m{c[6]}" for c in CASES])
def test_compact_random(gpu_lib, case):
    import torch
    import unstructured_sparse_transformer_amd as tw
    T, F, w, cap, dtype, frac, max_ovf = case
    h = _matrix(T, F, frac, dtype, seed=3 * T + F, heavy_rows=(0, T - 1))
    say(f"case compact {case}")
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    hy = tw.Hybrid.empty(T, F, w, cap, dt, max_ovf)
    tw.twell_dense_to_hybrid(torch.from_numpy(np.ascontiguousarray(h)).to("cuda").to(dt), hy)
    _check(h, hy, T, F, w, cap, dtype, max_ovf, str(case))


def test_compact_layer_2b(gpu_lib):
    """The gate's hybrid of the full 2B-like layer: its compact form against
    the oracle, and its size against TwELL and the dense activations."""
    import torch
    import unstructured_sparse_transformer_amd as tw
    wl = make_layer_2b()
    say(f"case compact layer_2b T={wl.T} F={wl.F}")
    dt, x, wg, _, _ = to_device(wl)
    hy = tw.Hybrid.empty(wl.T, wl.F, wl.tile_w, wl.cap, dt, 1024)
    tw.twell_pack_gate_hybrid(x, wg, hy)
    z = oracle.gate(wl.x, wl.wg_t)
    h = oracle.store_round(np.where(z > 0, z, 0.0), wl.dtype)
    hdr = _check(h, hy, wl.T, wl.F, wl.tile_w, wl.cap, wl.dtype, 1024, "layer_2b")
    twell_bytes = wl.T * (wl.F // wl.tile_w) * (4 + wl.cap * 3)
    say(f"  compact {hdr['bytes']} B vs TwELL {twell_bytes} B + dense backup, dense h {wl.T * wl.F * 2} B")
    assert hdr["bytes"] < 0.05 * wl.T * wl.F * 2


def test_compact_zero_rows(gpu_lib):
    """T = 0: the buffer holds a header and row_ptr[0] = 0; expansion is a no-op."""
    import torch
    import unstructured_sparse_transformer_amd as tw
    say("case compact T = 0")
    hy = tw.Hybrid.empty(0, 512, 128, 8, torch.bfloat16, 0)
    buf = torch.full((tw.twell_compact_min_bytes(0),), 0xEE, dtype=torch.uint8, device="cuda")
    tw.twell_compact_hybrid(hy, buf)
    hdr = tw.compact_header(buf)
    assert hdr["T"] == 0 and hdr["n_entries"] == 0 and hdr["n_ovf"] == 0 and hdr["fits"] == 1
    assert hdr["bytes"] == tw.twell_compact_min_bytes(0)
    out = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda")
    tw.twell_compact_to_dense(buf, 0, 512, torch.bfloat16, out)
    torch.cuda.synchronize()
