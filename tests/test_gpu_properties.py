"""Property test on the GPU (hypothesis): random shapes, tile widths,
capacities, element types and sparsity on the exactness grid, run through the
whole path (the separate calls, twell_ffn_forward, twell_pack_gate +
twell_ffn_from_gate) and compared with the oracle as in the parity tests.
Bounded: 40 derandomized examples, no shrinking, so the run stops at the
first failing case, which is printed before it runs."""

import pytest
from hypothesis import HealthCheck, Phase, given, settings
from hypothesis import strategies as st

from helpers import compare, grid_ok, run_hip, say
from workloads import make_random_small

pytestmark = pytest.mark.gpu


@st.composite
def gpu_layers(draw):
    dt = draw(st.sampled_from(["bf16", "bf16", "f32"]))
    w = draw(st.sampled_from([32, 64, 128, 256]))
    n_b = draw(st.integers(1, 12))
    F = w * n_b
    if F % 64:
        F *= 2
    d = 64 * draw(st.integers(1, 32 if dt == "bf16" else 16))
    T = draw(st.integers(1, 700))
    cap = draw(st.integers(1, min(w, 64)))
    frac = draw(st.floats(0.005, 0.5))
    jitter = draw(st.sampled_from([0.0, 0.3, 0.5]))  # last x column stays >= 2^-3
    dead = draw(st.integers(0, F // 8))
    seed = draw(st.integers(0, 1 << 20))
    return make_random_small(T, d, F, w, cap, dt, active_frac=frac, seed=seed, jitter=jitter, n_dead=dead)


@settings(max_examples=40, deadline=None, derandomize=True, phases=[Phase.explicit, Phase.generate],
          suppress_health_check=list(HealthCheck))
@given(gpu_layers())
def test_random_layers(gpu_lib, wl):
    grid_ok(wl)
    say(f"case property {wl.name}")
    out = run_hip(wl)
    compare(wl, out, label=wl.name)
