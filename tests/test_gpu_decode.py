"""GPU parity of the decode-shaped path (twell_ffn_decode, T <= 64) against the
oracle, through the C ABI: TwELL, overflow flags and list, dense backup and
work order exactly as for the batch path; every row of y, overflow rows
included, within 1e-2 of the exact-h oracle and 1e-4 of the stored-h oracle;
repeated calls bit-identical."""

import numpy as np
import pytest

import oracle
from helpers import compare_decode, run_decode, say
from workloads import make_decode_windows, make_layer_2b, make_random_small

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T", [1, 8, 64])
def test_decode_windows(gpu_lib, T):
    """Windows of the 2B layer: the first three and the five with the most actives."""
    wins = make_decode_windows(T, max_windows=512)
    base = make_layer_2b()
    z_sample = oracle.gate(base.x[: len(wins) * T], base.wg_t)
    act = (z_sample > 0).reshape(len(wins), T, -1).sum((1, 2))
    pick = sorted(set([0, 1, 2] + list(np.argsort(-act)[:5])))
    n_ovf_seen = 0
    for i in pick:
        wl = wins[i]
        say(f"case decode T={T} window={i}")
        out = run_decode(wl, calls=2)
        compare_decode(wl, out, label=f"decode T={T} w={i}")
        n_ovf_seen += out["n_ovf"]
    if T >= 8:
        assert n_ovf_seen > 0  # the busiest windows hold overflow rows


DEC_EDGE = [
    # (T, d, F, w, cap, frac, jitter, dead)
    (1, 64, 64, 64, 8, 0.2, 0.0, 0),          # smallest: one row, one tile
    (5, 128, 512, 32, 4, 0.1, 0.5, 0),        # w = 32
    (33, 256, 1024, 64, 2, 0.1, 0.5, 20),     # two row blocks, w = 64, dead neurons
    (64, 512, 2048, 128, 8, 0.05, 0.5, 0),    # w = 128
    (64, 4096, 512, 256, 16, 0.05, 0.5, 0),   # d = 4096 (largest bf16 row)
    (17, 192, 768, 256, 1, 0.2, 0.5, 0),      # cap = 1: nearly every row overflows
    (64, 128, 16384, 256, 16, 0.5, 0.2, 0),   # T * F = 2^20, half active: large gather chunks
    (40, 64, 320, 64, 64, 0.3, 0.5, 0),       # cap = w: no overflow possible
    # Windows of at most 16 rows take the two-kernel organisation (rows split
    # over 8, 4, 2 or 1 waves by T; 1, 2, 4 or 8 16-byte chunks per lane by d).
    (2, 1024, 2048, 256, 8, 0.1, 0.5, 0),     # T = 2: four waves per row, two chunks per lane
    (3, 4096, 1024, 128, 4, 0.1, 0.5, 0),     # T = 3: two waves per row, d = 4096 (no prefetch)
    (4, 1536, 1024, 64, 2, 0.1, 0.5, 5),      # T = 4: ragged last reduce block, dead neurons
    (16, 4096, 2048, 256, 4, 0.1, 0.5, 0),    # T = 16 at d = 4096: largest two-kernel window
    (16, 192, 768, 256, 1, 0.2, 0.5, 0),      # T = 16, cap = 1: the T = 17 case's twin below the switch
]


@pytest.mark.parametrize("case", DEC_EDGE, ids=[f"T{c[0]}_d{c[1]}_F{c[2]}_w{c[3]}_c{c[4]}" for c in DEC_EDGE])
def test_decode_edge_shapes(gpu_lib, case):
    T, d, F, w, cap, frac, jit, dead = case
    wl = make_random_small(T, d, F, w, cap, "bf16", active_frac=frac, seed=T + d + 3, jitter=jit, n_dead=dead)
    say(f"case decode edge {wl.name}")
    out = run_decode(wl, calls=2)
    compare_decode(wl, out, label=wl.name)


def test_decode_overflow_beyond_max_ovf(gpu_lib):
    """n_ovf > max_ovf: the first max_ovf overflow rows get a dense row; every
    row of y is still complete."""
    wl = make_random_small(48, 128, 1024, 128, 2, "bf16", active_frac=0.1, seed=21, jitter=0.6)
    say("case decode max_ovf below n_ovf")
    full = run_decode(wl)
    assert full["n_ovf"] > 4
    for m in (0, 3):
        out = run_decode(wl, max_ovf=m)
        assert out["n_ovf"] == full["n_ovf"]
        compare_decode(wl, out, label=f"max_ovf={m}")
        np.testing.assert_array_equal(out["y"], full["y"])


def test_decode_unaligned_twell_buffers(gpu_lib):
    wl = make_random_small(24, 256, 1024, 256, 16, "bf16", active_frac=0.1, seed=5, jitter=0.5)
    say("case decode unaligned TwELL buffers")
    out = run_decode(wl, unaligned=True)
    compare_decode(wl, out, label="unaligned")


def test_decode_matches_batch_twell(gpu_lib):
    """The decode path writes the same TwELL, partition and order as the batch
    path on the same rows (y agrees within the summation-order tolerance)."""
    from helpers import run_hip
    wl = make_decode_windows(64, max_windows=4)[1]
    say("case decode vs batch path, T=64")
    a = run_decode(wl)
    b = run_hip(wl)
    for k in ("cnt", "val", "idx", "row_ovf", "ovf_rows", "dense", "order"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    assert a["n_ovf"] == b["n_ovf"]
    ok = a["row_ovf"] == 0
    num = np.linalg.norm(a["y"][ok] - b["y"][ok], axis=1)
    den = np.linalg.norm(b["y"][ok], axis=1)
    assert (num <= 1e-4 * np.maximum(den, 1e-30)).all()


def test_decode_zero_rows_and_stream(gpu_lib):
    import torch
    import unstructured_sparse_transformer_amd as tw
    wl = make_random_small(12, 128, 512, 128, 8, "bf16", active_frac=0.1, seed=9, jitter=0.5)
    say("case decode on a side stream; T = 0")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = run_decode(wl, stream=s, calls=3)
    compare_decode(wl, out, label="side stream")
    hy = tw.Hybrid.empty(0, 512, 128, 8, torch.bfloat16, 0)
    y = torch.empty((0, 128), dtype=torch.float32, device="cuda")
    x = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    wg = torch.zeros((512, 128), dtype=torch.bfloat16, device="cuda")
    tw.twell_ffn_decode(x, wg, wg, wg, hy, y, tw.decode_workspace(0, 512, 128, 128))
