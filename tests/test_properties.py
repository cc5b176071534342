"""Property tests (hypothesis) on the CPU: the oracle's invariants over random
shapes, capacities and sparsity, and the C ABI's argument checks against a
model of the rules include/twell.h states.  Only arguments the model says are
rejected (or T = 0, nothing to do) are passed to the library, so no call here
can launch a kernel."""

import ctypes

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
import unstructured_sparse_transformer_amd as tw
from test_capi import noalloc_scratch_need
from workloads import make_random_small

SETTINGS = settings(max_examples=60, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow])


@st.composite
def layers(draw):
    w = draw(st.sampled_from([4, 8, 32, 64, 128]))
    n_b = draw(st.integers(1, 6))
    F = w * n_b
    d = draw(st.sampled_from([4, 8, 16, 32]))
    T = draw(st.integers(1, 24))
    cap = draw(st.integers(1, w))
    frac = draw(st.floats(0.01, 0.6))
    seed = draw(st.integers(0, 10_000))
    dt = draw(st.sampled_from(["bf16", "f32"]))
    return make_random_small(T, d, F, w, cap, dt, active_frac=frac, seed=seed, jitter=0.5)


@SETTINGS
@given(layers())
def test_oracle_invariants(wl):
    """TwELL of ReLU(x W_g): true counts = actives per tile; nonzeros are
    conserved by the hybrid; kept entries are the lowest active columns in
    ascending order with values = stored z; unpacking the rows that fit gives
    back h; the TwELL sum equals the dense sum bit for bit on those rows."""
    ref = oracle.reference(wl)
    z, t = ref.z, ref.tw
    act = (z > 0).reshape(wl.T, wl.n_b, wl.tile_w)
    np.testing.assert_array_equal(t.cnt, act.sum(2))
    kept = t.kept()
    for r in range(wl.T):
        for b in range(wl.n_b):
            cols = np.nonzero(act[r, b])[0][:wl.cap]
            m = len(cols)
            np.testing.assert_array_equal(t.idx[r, b, :m], cols)
            np.testing.assert_array_equal(t.val[r, b, :m], oracle.store_round(z[r, b * wl.tile_w + cols], wl.dtype))
            assert not t.idx[r, b, m:].any() and not t.val[r, b, m:].any()
    ovf = ref.row_ovf.astype(bool)
    np.testing.assert_array_equal(ovf, (t.cnt > wl.cap).any(1))
    dense = oracle.dense_backup(z, ref.ovf_local, wl.dtype)
    nnz = int(np.minimum(t.cnt, wl.cap)[~ovf].sum()) + int((dense != 0).sum())
    h = oracle.store_round(np.where(z > 0, z, 0.0), wl.dtype)
    assert nnz == int((h != 0).sum()) + int(((z > 0) & (h == 0)).sum())
    un = oracle.unpack_twell(t)
    np.testing.assert_array_equal(un[~ovf], h[~ovf])
    assert kept.sum() == np.minimum(t.cnt, wl.cap).sum()
    np.testing.assert_array_equal(ref.y_fused[~ovf], ref.y_stored[~ovf])
    assert not ref.y_fused[ovf].any()


GOOD = 4096


def _model_pack_gate(T, F, w, cap, vd, d, ptr):
    """The status twell_pack_gate must return (the header's rules, in the
    order the library checks them); None = accepted (would launch)."""
    if vd not in (0, 1):
        return -4
    if w not in (32, 64, 128, 256) or cap < 1 or cap > w:
        return -4
    if T < 0 or F <= 0 or F % w or F % 64 or d <= 0 or d % 64:
        return -3
    esz = 2 if vd == 1 else 4
    if d * esz > 8192:
        return -4
    if T * d * esz >= 1 << 32 or F * d * esz >= 1 << 32 or T * (F // w) * cap >= 1 << 31:
        return -3
    if T == 0:
        return 0
    for name in ("x", "wg"):
        if ptr[name] is None:
            return -1
        if ptr[name] % 16:
            return -2
    if ptr["val"] is None or ptr["idx"] is None or ptr["cnt"] is None:
        return -1
    if ptr["val"] % esz or ptr["cnt"] % 4:
        return -2
    return None


PTR = st.sampled_from([None, GOOD, GOOD + 1, GOOD + 2, GOOD + 4, GOOD + 8])


@SETTINGS
@given(T=st.sampled_from([-1, 0, 1, 7, 1 << 15, 1 << 20]), F=st.sampled_from([0, 96, 256, 500, 512, 1 << 16]),
       w=st.sampled_from([16, 32, 64, 100, 128, 256, 512]), cap=st.sampled_from([-1, 0, 1, 8, 64, 257]),
       vd=st.sampled_from([0, 1, 2]), d=st.sampled_from([0, 60, 64, 2048, 4096, 8192]),
       x=PTR, wg=PTR, val=PTR, idx=PTR, cnt=PTR)
def test_pack_gate_status_model(T, F, w, cap, vd, d, x, wg, val, idx, cnt):
    want = _model_pack_gate(T, F, w, cap, vd, d, {"x": x, "wg": wg, "val": val, "idx": idx, "cnt": cnt})
    if want is None:
        return  # valid: the library would launch; nothing to check without a GPU
    lib = tw.load()
    desc = tw.TwellT(T, F, w, cap, vd, 0, val, idx, cnt)
    assert lib.twell_pack_gate(x, wg, d, ctypes.byref(desc), None) == want


@SETTINGS
@given(T=st.sampled_from([0, 1, 8, 64, 65]), F=st.sampled_from([256, 8192, 16384, 32768]),
       w=st.sampled_from([32, 128, 256]), d=st.sampled_from([64, 1024, 2048, 4096]))
def test_decode_noalloc_scratch_rule(T, F, w, d):
    """twell_ffn_decode_noalloc rejects exactly the valid decode shapes whose
    workspace exceeds the 16 MiB scratch (TWELL_E_SCRATCH) and the shapes the
    decode path does not take (TWELL_E_UNSUPPORTED); the rest would launch."""
    lib = tw.load()
    if T > 64 or T * F > 1 << 20 or F // w > 512:
        want = -4
    elif T == 0:
        want = 0
    elif noalloc_scratch_need(T, F, d) > 16 << 20:
        want = -7
    else:
        return  # accepted: would launch
    hy = tw.TwellHybridT(tw.TwellT(T, F, w, 8, 1, 0, GOOD, GOOD, GOOD), 8, 0, GOOD, GOOD, GOOD, GOOD, GOOD)
    assert lib.twell_ffn_decode_noalloc(GOOD, GOOD, GOOD, GOOD, d, ctypes.byref(hy), GOOD, None) == want
