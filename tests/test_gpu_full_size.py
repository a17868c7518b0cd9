"""The full-size workloads' user side on their stress inputs under both phi,
with history outputs, against the CPU oracle on sampled users (users are
independent, so a sample is exact).  Bar: max|gpu - ref| <= 2e-2 max|ref|
per output tensor (per user)."""
import numpy as np
import pytest
import torch

import oracle.lime_oracle as O
import workloads as W
from parity_utils import assert_close, dev, dev_weights, host_f64, user_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import decoupled_linear_link_amd as lib
    return lib


def _users_for(w, off):
    """The longest user and one other (seeded)."""
    lens = np.diff(off)
    return sorted({int(np.argmax(lens)), int(np.random.default_rng(1).integers(0, w.B))})


@pytest.mark.parametrize("name", ["long", "large_m", "lifelong"])
@pytest.mark.parametrize("phi", ["softmax", "silu_mean"])
def test_xor_fwd_full_size_stress_both_phis(L, name, phi):
    """The full-size workloads on their stress inputs (unit-variance context
    links), under both phi, with hist_out: the kernel instantiations of the
    long, large-M and lifelong shapes checked on the oracle's sampled users
    (users are independent, so a sample is exact)."""
    w = W.workload(name)
    ui = user_inputs(name, stress=True)
    off = ui["hist_offsets"]
    print(f"xor_fwd full size {name} {phi} stress: B={w.B} total_N={int(off[-1])}", flush=True)
    lp, ho = L.xor_fwd(dev(ui["links_ctx"]), dev(ui["hist"]), dev(off), dev_weights(ui["weights"]),
                       heads=w.heads, phi=phi, scale=W.scale_for(w), max_N=int(np.diff(off).max()),
                       want_hist=True)
    torch.cuda.synchronize()
    users = _users_for(w, off)
    ref, href = O.xor_fwd(ui["links_ctx"], ui["hist"], off, ui["weights"], w.heads, W.scale_for(w), phi,
                          users=users)
    assert_close(host_f64(lp)[users], ref, w.dtype, f"L^P[{name},{phi},stress]")
    hg = host_f64(ho)
    for b, hr in zip(users, href):
        assert_close(hg[off[b]:off[b + 1]], hr, w.dtype, f"hist_out[{name},{phi},stress,user {b}]")
