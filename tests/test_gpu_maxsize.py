"""GPU parity at the largest row count the library accepts for the 2B layer's
shape, through the C ABI (twell_pack_gate then twell_ffn_from_gate).

T = 2^20 - 64 rows, d = 2048, bf16: x is 4 GiB - 256 KiB, just under the 4 GiB
bound on a GEMM operand (T = 2^20 is rejected with TWELL_E_SHAPE), y is
8 GiB of fp32 and the TwELL holds 2^29 - 2^15 slots.  Row t of x is row
t mod 8192 of the 2B layer, so every result has a known expected value:
sampled rows (the first, around 2^19, the ragged last 320, overflow rows near
the end, random ones) are compared with the oracle on their base rows (TwELL,
flags and dense backup bit for bit, y within the usual tolerance), and the
whole overflow list with the base rows' flags repeated.  This is the check
that no row, slot or byte offset wraps at 32 bits."""

import numpy as np
import pytest
import torch

import oracle
from helpers import check_y_rows, say, to_device
from workloads import make_layer_2b

pytestmark = pytest.mark.gpu


def test_max_rows_layer_2b(gpu_lib):
    tw = gpu_lib
    base = make_layer_2b()
    B = base.T
    T = (1 << 20) - 64
    assert T * base.d * 2 < (1 << 32) <= (T + 64) * base.d * 2
    say(f"case max rows T={T} d={base.d} F={base.F} bf16 (x {T * base.d * 2 / 2**30:.3f} GiB)")

    # expected overflow flags of the base rows (oracle), repeated over T
    z = oracle.gate(base.x, base.wg_t)
    ref_all = oracle.pack_twell(z, base.tile_w, base.cap, base.dtype)
    base_ovf, _, _ = oracle.partition_overflow(ref_all.cnt, base.cap)
    del z
    want_list = np.nonzero(base_ovf[np.arange(T) % B])[0]
    max_ovf = 32768
    assert len(want_list) <= max_ovf

    dt, x0, wg, wu, wd = to_device(base)
    x = x0.repeat((T + B - 1) // B, 1)[:T]
    assert x.is_contiguous()
    hy = tw.Hybrid.empty(T, base.F, base.tile_w, base.cap, dt, max_ovf)
    ws = tw.hybrid_workspace(hy, base.d)
    y = torch.full((T, base.d), float("nan"), dtype=torch.float32, device="cuda")
    hy.ell.cnt.fill_(-7)
    hy.n_ovf.fill_(-7)
    tw.twell_pack_gate(x, wg, hy.ell)
    tw.twell_ffn_from_gate(x, wg, wu, wd, hy, y, ws)
    torch.cuda.synchronize()

    n_ovf = int(hy.n_ovf.item())
    assert n_ovf == len(want_list), f"n_ovf {n_ovf} vs {len(want_list)}"
    np.testing.assert_array_equal(hy.ovf_rows[:n_ovf].cpu().numpy(), want_list, err_msg="ovf_rows")
    order = hy.order
    assert torch.equal(torch.sort(order).values, torch.arange(T, dtype=order.dtype, device="cuda")), \
        "work order is not a permutation of the rows"
    assert not torch.isnan(y[-64:]).any() and not torch.isnan(y[:64]).any()

    rng = np.random.default_rng(20)
    tail_ovf = want_list[want_list >= T - 4 * B][-16:]
    rows = np.unique(np.concatenate([np.arange(64), np.arange((1 << 19) - 32, (1 << 19) + 32),
                                     np.arange(T - 320, T), tail_ovf, rng.choice(T, 256, replace=False)]))
    brows, inv = np.unique(rows % B, return_inverse=True)
    ref = oracle.reference(base, rows=brows)
    rd = torch.from_numpy(rows).to("cuda")
    cnt = hy.ell.cnt[rd].cpu().numpy()
    np.testing.assert_array_equal(cnt, ref.tw.cnt[inv], err_msg="TwELL counts")
    np.testing.assert_array_equal(hy.ell.idx[rd].cpu().numpy(), ref.tw.idx[inv], err_msg="TwELL indices")
    np.testing.assert_array_equal(hy.ell.val[rd].float().cpu().numpy(), ref.tw.val[inv].astype(np.float32),
                                  err_msg="TwELL values")
    np.testing.assert_array_equal(hy.row_ovf[rd].cpu().numpy(), ref.row_ovf[inv], err_msg="row_ovf")
    # dense backup rows of the sampled overflow rows
    pos = {int(t): i for i, t in enumerate(want_list)}
    n_dense = 0
    for k, t in enumerate(rows):
        if int(t) in pos:
            li = int(inv[k])
            want = oracle.dense_backup(ref.z[li:li + 1], [0], base.dtype)[0]
            got = hy.dense[pos[int(t)]].float().cpu().numpy()
            np.testing.assert_array_equal(got, want.astype(np.float32), err_msg=f"dense backup row {t}")
            n_dense += 1
    assert n_dense >= len(tail_ovf) > 0
    yr = y[rd].cpu().numpy().astype(np.float64)
    ref_y = oracle.reference(base, rows=brows[inv])  # the sampled rows' base rows, in sample order
    r_inf, r_bound = check_y_rows(base, yr, ref_y, np.ones(len(rows), bool), "max rows")
    say(f"  y: max |dy| {r_inf:.2e} of ||y_ref||_inf, {r_bound:.2f} of the rounding bound")
    say(f"  n_ovf={n_ovf} sampled rows={len(rows)} (dense-backup rows among them: {n_dense})")
