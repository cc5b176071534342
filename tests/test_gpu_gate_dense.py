"""twell_gate_dense (the gate GEMM with a plain dense epilogue) against the
oracle: h = ReLU(x . W_g) rounded to the storage type, bit for bit on the
exactness grid; and packing that dense h with twell_dense_to_hybrid gives
the TwELL twell_pack_gate writes from its epilogue, bit for bit."""

import numpy as np
import pytest
import torch

import oracle
from helpers import say, to_device
from workloads import make_layer_2b, make_random_small, make_tiny

pytestmark = pytest.mark.gpu

CASES = [("tiny", None), ("ragged", (300, 128, 512, 128, 8, "bf16")), ("f32", (90, 192, 640, 64, 8, "f32")),
         ("F64", (50, 64, 64, 64, 8, "bf16")), ("2b_rows", None)]


def _wl(name, shape):
    if name == "tiny":
        return make_tiny()
    if name == "2b_rows":
        return make_layer_2b().rows(0, 1024)
    T, d, F, w, cap, dt = shape
    return make_random_small(T, d, F, w, cap, dt, active_frac=0.08, seed=T + F, jitter=0.5, n_dead=3)


@pytest.mark.parametrize("name,shape", CASES, ids=[c[0] for c in CASES])
def test_gate_dense(gpu_lib, name, shape):
    tw = gpu_lib
    wl = _wl(name, shape)
    say(f"case gate_dense {wl.name}")
    dt, x, wg, _, _ = to_device(wl)
    h = torch.full((wl.T, wl.F), float("nan"), dtype=dt, device="cuda")
    tw.twell_gate_dense(x, wg, h)
    hy = tw.Hybrid.empty(wl.T, wl.F, wl.tile_w, wl.cap, dt, wl.T)
    tw.twell_dense_to_hybrid(h, hy)
    ref = tw.TwELL.empty(wl.T, wl.F, wl.tile_w, wl.cap, dt)
    tw.twell_pack_gate(x, wg, ref)
    torch.cuda.synchronize()
    z = oracle.gate(wl.x, wl.wg_t)
    want = oracle.dense_backup(z, np.arange(wl.T), wl.dtype)
    np.testing.assert_array_equal(h.float().cpu().numpy(), want.astype(np.float32), err_msg="dense gate values")
    for k in ("cnt", "idx", "val"):
        a, b = getattr(hy.ell, k), getattr(ref, k)
        assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), \
            f"dense_to_hybrid(gate_dense) differs from pack_gate in {k}"
